// Sigmoid-score top-k router.
//
// Logits use one fixed fp32 order so that every implementation produces the
// same bits (the routing ids must match exactly): H splits into 64 contiguous
// chunks of L = H/64; chunk c is the fused-multiply-add chain over ascending k
// from 0; the 64 chunk sums are added as a perfect pairwise tree in index
// order; the bias is added last. Two kernels produce identical bits:
//   * router_wave: one wave per expert, lane c owns chunk c, the tree is an
//     xor-butterfly across lanes (xor 1 pairs chunks 2j and 2j+1, xor 2 pairs
//     those pairs, ...). Used for small token counts, where streaming Wr once
//     at full bandwidth is what matters.
//   * router_tiled: 64 tokens x 64 experts per workgroup, 4x4 per thread,
//     operands staged through LDS; each thread keeps a 6-slot pairwise stack
//     per output, pushing a chunk sum whenever a chunk ends (the carry chain
//     of a binary counter reproduces the pairwise tree exactly).
// Top-k: one wave per token; scores s = 1/(1 + exp(-l)); k rounds of a wave
// argmax keyed (score desc, expert asc); w_j = s_j / S with S accumulated
// left to right in slot order.
#include "common.h"
#include "kernels.h"

namespace {

template <typename XT>
__device__ __forceinline__ float load_x(const XT* p);
template <>
__device__ __forceinline__ float load_x<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_x<uint16_t>(const uint16_t* p) { return moe::bf16_bits_to_f32(*p); }

template <typename XT>
__device__ __forceinline__ void load_x4(const XT* p, float* o);
template <>
__device__ __forceinline__ void load_x4<float>(const float* p, float* o) {
  float4 v = *reinterpret_cast<const float4*>(p);
  o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
}
template <>
__device__ __forceinline__ void load_x4<uint16_t>(const uint16_t* p, float* o) {
  uint2 v = *reinterpret_cast<const uint2*>(p);
  o[0] = __uint_as_float(v.x << 16);
  o[1] = __uint_as_float(v.x & 0xffff0000u);
  o[2] = __uint_as_float(v.y << 16);
  o[3] = __uint_as_float(v.y & 0xffff0000u);
}

// ---------------------------------------------------------------------------
// One wave per expert; 4 experts per 256-thread workgroup.
// ---------------------------------------------------------------------------
template <typename XT>
__global__ __launch_bounds__(256) void router_wave_kernel(const XT* __restrict__ x, const float* __restrict__ wr,
                                                          const float* __restrict__ bias, float* __restrict__ logits,
                                                          int T, int H, int E) {
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int c = threadIdx.x & 63;
  if (e >= E) return;
  const int L = H >> 6;
  const float* wrow = wr + (size_t)e * H + (size_t)c * L;
  const float b = bias ? bias[e] : 0.0f;
  for (int t = 0; t < T; ++t) {
    const XT* xrow = x + (size_t)t * H + (size_t)c * L;
    float p = 0.0f;
    for (int i = 0; i < L; i += 4) {
      float xv[4];
      load_x4<XT>(xrow + i, xv);
      float4 wv = *reinterpret_cast<const float4*>(wrow + i);
      p = __builtin_fmaf(xv[0], wv.x, p);
      p = __builtin_fmaf(xv[1], wv.y, p);
      p = __builtin_fmaf(xv[2], wv.z, p);
      p = __builtin_fmaf(xv[3], wv.w, p);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) p = p + __shfl_xor(p, o, 64);
    if (c == 0) logits[(size_t)t * E + e] = bias ? p + b : p;
  }
}

// ---------------------------------------------------------------------------
// 64x64 tile per workgroup, 16x16 threads with 4x4 outputs each.
// ---------------------------------------------------------------------------
constexpr int RT = 64;   // tokens per tile
constexpr int RE = 64;   // experts per tile
constexpr int RK = 32;   // k per LDS stage

template <typename XT>
__global__ __launch_bounds__(256) void router_tiled_kernel(const XT* __restrict__ x, const float* __restrict__ wr,
                                                           const float* __restrict__ bias, float* __restrict__ logits,
                                                           int T, int H, int E) {
  __shared__ float xs[RK][RT + 4];
  __shared__ float ws[RK][RE + 4];
  const int t0 = blockIdx.y * RT, e0 = blockIdx.x * RE;
  const int tid = threadIdx.x;
  const int ty = tid >> 4, tx = tid & 15;
  const int L = H >> 6;

  float acc[4][4];
  float st[6][4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0f;

  // staging map: 64 rows x 32 k = 512 groups of 4 k; 2 groups per thread
  int chunk = 0, in_chunk = 0;
  for (int k0 = 0; k0 < H; k0 += RK) {
    __syncthreads();
#pragma unroll
    for (int rep = 0; rep < 2; ++rep) {
      int gidx = tid + rep * 256;
      int r = gidx >> 3, kq = (gidx & 7) * 4;
      float v[4] = {0.f, 0.f, 0.f, 0.f};
      if (t0 + r < T) load_x4<XT>(x + (size_t)(t0 + r) * H + k0 + kq, v);
      xs[kq + 0][r] = v[0]; xs[kq + 1][r] = v[1]; xs[kq + 2][r] = v[2]; xs[kq + 3][r] = v[3];
      float4 w4 = make_float4(0.f, 0.f, 0.f, 0.f);
      if (e0 + r < E) w4 = *reinterpret_cast<const float4*>(wr + (size_t)(e0 + r) * H + k0 + kq);
      ws[kq + 0][r] = w4.x; ws[kq + 1][r] = w4.y; ws[kq + 2][r] = w4.z; ws[kq + 3][r] = w4.w;
    }
    __syncthreads();
    for (int kk = 0; kk < RK; ++kk) {
      float4 xv = *reinterpret_cast<const float4*>(&xs[kk][ty * 4]);
      float4 wv = *reinterpret_cast<const float4*>(&ws[kk][tx * 4]);
      float xa[4] = {xv.x, xv.y, xv.z, xv.w};
      float wa[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = __builtin_fmaf(xa[a], wa[b], acc[a][b]);
      if (++in_chunk == L) {
        // push the finished chunk sums onto the pairwise stack
        in_chunk = 0;
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            float v = acc[a][b];
            acc[a][b] = 0.0f;
#pragma unroll
            for (int lv = 0; lv < 6; ++lv) {
              if ((chunk >> lv) & 1) {
                v = st[lv][a][b] + v;
              } else {
                st[lv][a][b] = v;
                break;
              }
            }
            if (chunk == 63) st[0][a][b] = v;  // the full tree sum
          }
        ++chunk;
      }
    }
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    int t = t0 + ty * 4 + a;
    if (t >= T) continue;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      int e = e0 + tx * 4 + b;
      if (e < E) logits[(size_t)t * E + e] = bias ? st[0][a][b] + bias[e] : st[0][a][b];
    }
  }
}

// ---------------------------------------------------------------------------
// Top-k + renormalization: one wave per token, 4 tokens per workgroup.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E, int K,
                                                   int32_t* __restrict__ ids, float* __restrict__ w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  constexpr int MAXPER = 16;  // E <= 1024
  float s[MAXPER];
  const int per = (E + 63) / 64;
#pragma unroll
  for (int i = 0; i < MAXPER; ++i) {
    int e = lane + 64 * i;
    s[i] = (i < per && e < E) ? moe::sigmoid_fixed(logits[(size_t)t * E + e]) : -1.0f;  // sigmoid >= 0
  }
  uint32_t taken = 0;
  float ssel[16];
  int isel[16];
  for (int j = 0; j < K; ++j) {
    // lane-local best: highest score, lowest index (i ascending = e ascending)
    float bv = -2.0f;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
      int e = lane + 64 * i;
      if (!((taken >> i) & 1) && s[i] > bv) { bv = s[i]; bi = e; }
    }
    // wave argmax
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      float ov = __shfl_xor(bv, o, 64);
      int oi = __shfl_xor(bi, o, 64);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    ssel[j] = bv;
    isel[j] = bi;
  }
  if (lane == 0) {
    float S = 0.0f;
    for (int j = 0; j < K; ++j) S = S + ssel[j];
    for (int j = 0; j < K; ++j) {
      ids[(size_t)t * K + j] = isel[j];
      w[(size_t)t * K + j] = (S == 0.0f) ? 1.0f / (float)K : ssel[j] / S;
    }
  }
}

}  // namespace

hipError_t moe_k_router_logits(int x_dtype, const void* x, const float* wr, const float* bias, float* logits,
                               int T, int H, int E, hipStream_t st) {
  if (T <= 64) {
    dim3 grid((E + 3) / 4);
    if (x_dtype == 0)
      router_wave_kernel<float><<<grid, 256, 0, st>>>((const float*)x, wr, bias, logits, T, H, E);
    else
      router_wave_kernel<uint16_t><<<grid, 256, 0, st>>>((const uint16_t*)x, wr, bias, logits, T, H, E);
  } else {
    dim3 grid((E + RE - 1) / RE, (T + RT - 1) / RT);
    if (x_dtype == 0)
      router_tiled_kernel<float><<<grid, 256, 0, st>>>((const float*)x, wr, bias, logits, T, H, E);
    else
      router_tiled_kernel<uint16_t><<<grid, 256, 0, st>>>((const uint16_t*)x, wr, bias, logits, T, H, E);
  }
  return hipGetLastError();
}

hipError_t moe_k_router_logits_variant(int variant, int x_dtype, const void* x, const float* wr, const float* bias,
                                       float* logits, int T, int H, int E, hipStream_t st) {
  if (variant == 0) {
    dim3 grid((E + 3) / 4);
    if (x_dtype == 0)
      router_wave_kernel<float><<<grid, 256, 0, st>>>((const float*)x, wr, bias, logits, T, H, E);
    else
      router_wave_kernel<uint16_t><<<grid, 256, 0, st>>>((const uint16_t*)x, wr, bias, logits, T, H, E);
  } else {
    dim3 grid((E + RE - 1) / RE, (T + RT - 1) / RT);
    if (x_dtype == 0)
      router_tiled_kernel<float><<<grid, 256, 0, st>>>((const float*)x, wr, bias, logits, T, H, E);
    else
      router_tiled_kernel<uint16_t><<<grid, 256, 0, st>>>((const uint16_t*)x, wr, bias, logits, T, H, E);
  }
  return hipGetLastError();
}

hipError_t moe_k_topk(const float* logits, int T, int E, int K, int32_t* ids, float* w, hipStream_t st) {
  topk_kernel<<<(T + 3) / 4, 256, 0, st>>>(logits, T, E, K, ids, w);
  return hipGetLastError();
}
