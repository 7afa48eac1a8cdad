// Sigmoid-score top-k router, and the fused kernels that finish routing.
//
// Logits use one fixed fp32 order so that every implementation produces the
// same bits (the routing ids must match exactly): H splits into 64 contiguous
// chunks of L = H/64; chunk c is the fused-multiply-add chain over ascending k
// from 0; the 64 chunk sums are added as a perfect pairwise tree in index
// order; the bias is added last.
//
// Large batches: the 64 chunks form 8 slices of 8 chunks. router_mfma (H a
// multiple of 1024) runs each output's chain on fp32 matrix cores, two fused
// multiply-adds per 32x32x2 MFMA in ascending k; router_partial (other H)
// on the VALU, a workgroup staging a (tokens x experts) tile's operands
// through LDS, each thread owning an RA x RB block of outputs. Both keep a
// 3-level pairwise stack per output, pushing a chunk sum whenever a chunk
// ends (the carry chain of a binary counter reproduces the tree exactly).
// The slice sums (tree level 3) go to partial[8][T][E]; the kernels below add
// the top three levels, ((S0+S1)+(S2+S3)) + ((S4+S5)+(S6+S7)), then the bias.
//
// Top-k: scores s = 1/(1 + exp(-l)); k rounds of a wave argmax keyed (score
// desc, expert asc); w_j = s_j / S with S accumulated left to right in slot
// order.
//
// Small batches (T <= 64) keep all 64 chunk sums, partial[64][T][E] (one
// chunk per workgroup, so each workgroup loads its operands once, and writes
// 64-byte runs of adjacent experts), and finish the whole tree in
// topk_quant_token, one workgroup per token; extra workgroups of the router's
// launch quantize x. Tiny batches (T <= 16, T E <= 4096) use 16 slices of 4
// chunks instead (a workgroup adds its 4 chunk sums as tree levels 1-2), and
// route_sort_small finishes the top four levels, selects every token's
// experts and sorts the pairs in one workgroup. Larger batches keep 8 slice
// sums; topk_quant uses one wave per token.
#include <algorithm>

#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "sort_dev.h"

namespace {

constexpr int NSLICE = 8;        // slices of large batches (8 chunks each)
constexpr int NSLICE_SMALL = 64;  // slices of small batches (1 chunk each)
constexpr int NSLICE_TINY = 16;   // slices of tiny batches (4 chunks each)
constexpr int RKS = 32;  // k per LDS stage

template <typename XT>
__device__ __forceinline__ void load4(const XT* p, float* o);
template <>
__device__ __forceinline__ void load4<float>(const float* p, float* o) {
  float4 v = *reinterpret_cast<const float4*>(p);
  o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
}
template <>
__device__ __forceinline__ void load4<uint16_t>(const uint16_t* p, float* o) {
  uint2 v = *reinterpret_cast<const uint2*>(p);
  o[0] = __uint_as_float(v.x << 16);
  o[1] = __uint_as_float(v.x & 0xffff0000u);
  o[2] = __uint_as_float(v.y << 16);
  o[3] = __uint_as_float(v.y & 0xffff0000u);
}

template <typename XT>
__device__ __forceinline__ float load1(const XT* p);
template <>
__device__ __forceinline__ float load1<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load1<uint16_t>(const uint16_t* p) { return moe::bf16_bits_to_f32(*p); }

// Quantize one row of x with one wave: int8 as FP8 (hi, lo) planes
// [2][K] + fp32 scale, or MXFP4 codes [K/2] + E8M0 scales [K/32]
// (K % 256 == 0). Compact loops: four four-element units per lane per batch.
template <typename XT>
__device__ __forceinline__ void wave_quant_row(const XT* __restrict__ row, int K, int mx, uint8_t* __restrict__ q,
                                            uint8_t* __restrict__ qs) {
  const int lane = threadIdx.x & 63;
  if (!mx) {
    const int nu = K >> 8;  // four-element units per lane
    float amax = 0.f;
#pragma unroll 1
    for (int u0 = 0; u0 < nu; u0 += 4) {
      float v[4][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) load4<XT>(row + ((size_t)min(u0 + u, nu - 1) * 64 + lane) * 4, v[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[u][0]), fabsf(v[u][1])), fmaxf(fabsf(v[u][2]), fabsf(v[u][3]))));
    }
    amax = moe::wave_max(amax);
    const float s = amax / 127.0f;
    if (lane == 0) *reinterpret_cast<float*>(qs) = s;
#pragma unroll 1
    for (int u = 0; u < nu; ++u) {
      float v[4];
      const size_t i = ((size_t)u * 64 + lane) * 4;
      load4<XT>(row + i, v);
      uint32_t hw = 0, lw = 0;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        float qq = 0.f;
        if (amax != 0.f) qq = fminf(fmaxf(__builtin_rintf(v[m] / s), -127.f), 127.f);
        int hi, lo;
        moe::split_int8((int)qq, hi, lo);
        hw |= moe::small_int_to_e4m3(hi) << (8 * m);
        lw |= moe::small_int_to_e4m3(lo) << (8 * m);
      }
      *reinterpret_cast<uint32_t*>(q + i) = hw;
      *reinterpret_cast<uint32_t*>(q + K + i) = lw;
    }
  } else {
#pragma unroll 1
    for (int b = lane; b < K / 32; b += 64) {
      float v[32];
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 32; i += 4) load4<XT>(row + b * 32 + i, v + i);
#pragma unroll
      for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
      const int e = amax > 0.f ? moe::mx_scale_exp(amax) : 0;
      *reinterpret_cast<uint4*>(q + b * 16) = amax > 0.f ? moe::mx_pack32(v, e) : make_uint4(0, 0, 0, 0);
      qs[b] = (uint8_t)e;
    }
  }
}

// Quantize one row of x with a whole 256-thread workgroup (the arithmetic of
// wave_quant_row): int8 in two passes over the row (amax, then the FP8 pair
// planes), float4 units with four loads in flight per thread; MXFP4 one
// 32-block per thread. red: 4 floats of LDS.
template <typename XT>
__device__ __forceinline__ void block_quant_row(const XT* __restrict__ row, int K, int mx, uint8_t* __restrict__ q,
                                                uint8_t* __restrict__ qs, float* red) {
  const int tid = threadIdx.x;
  if (mx) {
    for (int b = tid; b < K / 32; b += 256) {
      float v[32];
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 32; i += 4) load4<XT>(row + b * 32 + i, v + i);
#pragma unroll
      for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
      const int e = amax > 0.f ? moe::mx_scale_exp(amax) : 0;
      *reinterpret_cast<uint4*>(q + b * 16) = amax > 0.f ? moe::mx_pack32(v, e) : make_uint4(0, 0, 0, 0);
      qs[b] = (uint8_t)e;
    }
    return;
  }
  float amax = 0.f;
#pragma unroll 4
  for (int i = tid * 4; i < K; i += 1024) {
    float v[4];
    load4<XT>(row + i, v);
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
  }
  amax = moe::wave_max(amax);
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = amax / 127.0f;
  if (tid == 0) *reinterpret_cast<float*>(qs) = s;
#pragma unroll 4
  for (int i = tid * 4; i < K; i += 1024) {
    float v[4];
    load4<XT>(row + i, v);
    uint32_t hw = 0, lw = 0;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float qq = 0.f;
      if (amax != 0.f) qq = fminf(fmaxf(__builtin_rintf(v[m] / s), -127.f), 127.f);
      int hi, lo;
      moe::split_int8((int)qq, hi, lo);
      hw |= moe::small_int_to_e4m3(hi) << (8 * m);
      lw |= moe::small_int_to_e4m3(lo) << (8 * m);
    }
    *reinterpret_cast<uint32_t*>(q + i) = hw;
    *reinterpret_cast<uint32_t*>(q + K + i) = lw;
  }
}

// ---------------------------------------------------------------------------
// Partial logits over one H slice. 256 threads = 16 x 16; tile (16 RA) tokens
// x (16 RB) experts; KS k values per LDS stage; the next stage's global loads
// are in flight while the current stage is computed. Four waves a SIMD (at
// most 128 registers): the 16-output tile of large batches measured faster so
// than with three waves and no spill.
// ---------------------------------------------------------------------------
template <typename XT, int RA, int RB, int KS, int CPS>
__global__ __launch_bounds__(256, 4) void router_partial_kernel(const XT* __restrict__ x, const float* __restrict__ wr,
                                                             float* __restrict__ partial, int T, int H, int E,
                                                             int mx, uint8_t* __restrict__ xq_out,
                                                             uint8_t* __restrict__ xs_out) {
  static_assert(CPS == 1 || CPS == 4 || CPS == 8, "chunks per slice");
  constexpr int NSL = 64 / CPS;
  constexpr int TT = 16 * RA, TE = 16 * RB;
  constexpr int NX = TT * KS / 4 / 256, NW = TE * KS / 4 / 256;  // float4 groups per thread
  static_assert(NX >= 1 && NW >= 1, "tile too small for the stage");
  static_assert(KS % 4 == 0, "k groups of four");
  // rows padded to a 16-byte multiple: each thread reads its RA (RB) operands
  // of one k as 16-byte LDS loads, the 16 lanes of a row group contiguous
  __shared__ __attribute__((aligned(16))) float xs[KS][TT + 4];
  __shared__ __attribute__((aligned(16))) float ws[KS][TE + 4];
  const int e0 = blockIdx.x * TE, t0 = blockIdx.y * TT, slice = blockIdx.z;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  if (CPS < 8 && slice >= NSL) {
    // the quantization of x, which the routing does not need, in workgroups
    // of the same launch: one token row per workgroup
    __shared__ float red[4];
    const int t = (slice - NSL) * gridDim.x + blockIdx.x;
    if (t < T) {
      const size_t qrow = mx ? (size_t)H / 2 : (size_t)2 * H;
      const size_t srow = mx ? (size_t)H / 32 : 4;
      block_quant_row<XT>(x + (size_t)t * H, H, mx, xq_out + t * qrow, xs_out + t * srow, red);
    }
    return;
  }
  const int L = H >> 6;
  const int kbeg = slice * CPS * L, kend = kbeg + CPS * L;

  float acc[RA][RB], st0[RA][RB], st1[RA][RB], st2[RA][RB];
#pragma unroll
  for (int a = 0; a < RA; ++a)
#pragma unroll
    for (int b = 0; b < RB; ++b) { acc[a][b] = 0.f; st0[a][b] = 0.f; st1[a][b] = 0.f; st2[a][b] = 0.f; }

  // Register sets of fetched stages: D = 1 fetches the next stage while the
  // current one runs; the four-chunk tiny-batch slices (a multiple of four
  // stages: 4 L with L % 64 == 0) have four stages in flight at once, since
  // a stage computes for less than a memory latency.
  constexpr int D = CPS == 4 ? 4 : 1;
  // Raw bits in registers, converted to fp32 at the LDS store: a conversion
  // right after the load (or a load under a branch) makes the compiler wait
  // for it at once, and the prefetch would not overlap anything. Rows past T
  // or E read row 0: their outputs are never stored.
  using Raw = std::conditional_t<sizeof(XT) == 2, uint2, float4>;
  Raw xr[D][NX];
  float4 wrr[D][NW];
  auto fetch = [&](int set, int k0) {
#pragma unroll
    for (int n = 0; n < NX; ++n) {
      const int g = tid + n * 256, r = g / (KS / 4), kq = (g % (KS / 4)) * 4;
      const int row = t0 + r < T ? t0 + r : 0;
      xr[set][n] = *reinterpret_cast<const Raw*>(x + (size_t)row * H + k0 + kq);
    }
#pragma unroll
    for (int n = 0; n < NW; ++n) {
      const int g = tid + n * 256, r = g / (KS / 4), kq = (g % (KS / 4)) * 4;
      const int row = e0 + r < E ? e0 + r : 0;
      wrr[set][n] = *reinterpret_cast<const float4*>(wr + (size_t)row * H + k0 + kq);
    }
  };
  auto stash = [&](int set) {
#pragma unroll
    for (int n = 0; n < NX; ++n) {
      const int g = tid + n * 256, r = g / (KS / 4), kq = (g % (KS / 4)) * 4;
      float v[4];
      if constexpr (sizeof(XT) == 2) {
        const uint2 b = xr[set][n];
        v[0] = __uint_as_float(b.x << 16);
        v[1] = __uint_as_float(b.x & 0xffff0000u);
        v[2] = __uint_as_float(b.y << 16);
        v[3] = __uint_as_float(b.y & 0xffff0000u);
      } else {
        v[0] = xr[set][n].x; v[1] = xr[set][n].y; v[2] = xr[set][n].z; v[3] = xr[set][n].w;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) xs[kq + u][r] = v[u];
    }
#pragma unroll
    for (int n = 0; n < NW; ++n) {
      const int g = tid + n * 256, r = g / (KS / 4), kq = (g % (KS / 4)) * 4;
      ws[kq + 0][r] = wrr[set][n].x;
      ws[kq + 1][r] = wrr[set][n].y;
      ws[kq + 2][r] = wrr[set][n].z;
      ws[kq + 3][r] = wrr[set][n].w;
    }
  };

  int chunk = 0, in_chunk = 0;
  if constexpr (D == 1) fetch(0, kbeg);
  else {
#pragma unroll
    for (int i = 0; i < D; ++i) fetch(i, kbeg + i * KS);  // kend - kbeg >= D KS
  }
  for (int k0 = kbeg; k0 < kend; k0 += D * KS) {
#pragma unroll
   for (int i = 0; i < D; ++i) {
    const int ks = k0 + i * KS;  // this stage
    __syncthreads();
    stash(i);
    __syncthreads();
    if (ks + D * KS < kend) fetch(i, ks + D * KS);  // the stage D ahead
    // Four k per group (L % 4 == 0, so a chunk never ends inside a group):
    // the group's LDS reads are issued together, then its fmas run in
    // ascending k per output. Where L is a multiple of KS (the one-chunk
    // small-batch slices) a chunk can only end with a stage, so the stage
    // runs branch-free and fully unrolled; otherwise the chunk end is checked
    // after every group (unrolling the large-batch tiles measured slower: the
    // hoisted reads halve the occupancy).
    auto group = [&](int kk) {
      float xa[4][RA], wb[4][RB];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if constexpr (RA % 4 == 0) {
#pragma unroll
          for (int a = 0; a < RA; a += 4) {
            const float4 v = *reinterpret_cast<const float4*>(&xs[kk + u][ty * RA + a]);
            xa[u][a] = v.x; xa[u][a + 1] = v.y; xa[u][a + 2] = v.z; xa[u][a + 3] = v.w;
          }
        } else if constexpr (RA % 2 == 0) {
#pragma unroll
          for (int a = 0; a < RA; a += 2) {
            const float2 v = *reinterpret_cast<const float2*>(&xs[kk + u][ty * RA + a]);
            xa[u][a] = v.x; xa[u][a + 1] = v.y;
          }
        } else {
#pragma unroll
          for (int a = 0; a < RA; ++a) xa[u][a] = xs[kk + u][ty * RA + a];
        }
        if constexpr (RB % 4 == 0) {
#pragma unroll
          for (int b = 0; b < RB; b += 4) {
            const float4 v = *reinterpret_cast<const float4*>(&ws[kk + u][tx * RB + b]);
            wb[u][b] = v.x; wb[u][b + 1] = v.y; wb[u][b + 2] = v.z; wb[u][b + 3] = v.w;
          }
        } else {
#pragma unroll
          for (int b = 0; b < RB; ++b) wb[u][b] = ws[kk + u][tx * RB + b];
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int a = 0; a < RA; ++a)
#pragma unroll
          for (int b = 0; b < RB; ++b) acc[a][b] = __builtin_fmaf(xa[u][a], wb[u][b], acc[a][b]);
    };
    auto push = [&]() {
      // push the chunk sums: chunk index within the slice = 2- or 3-bit counter
      const bool b0 = chunk & 1, b1 = chunk & 2, b2 = chunk & 4;
#pragma unroll
      for (int a = 0; a < RA; ++a)
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          float v = acc[a][b];
          acc[a][b] = 0.f;
          if (CPS == 1) {
            st2[a][b] = v;  // the chunk sum itself (tree level 0)
          } else if (!b0) {
            st0[a][b] = v;
          } else {
            v = st0[a][b] + v;
            if (!b1) {
              st1[a][b] = v;
            } else {
              v = st1[a][b] + v;
              if (CPS == 4 || !b2) st2[a][b] = v;  // CPS 4: chunk 3, the slice total
              else st2[a][b] = st2[a][b] + v;      // CPS 8: chunk 7, the slice total
            }
          }
        }
      ++chunk;
    };
    if (CPS < 8 && L % KS == 0) {
#pragma unroll
      for (int kk = 0; kk < KS; kk += 4) group(kk);
      in_chunk += KS;
      if (in_chunk == L) {
        in_chunk = 0;
        push();
      }
    } else {
#pragma unroll 1
      for (int kk = 0; kk < KS; kk += 4) {
        group(kk);
        in_chunk += 4;
        if (in_chunk == L) {
          in_chunk = 0;
          push();
        }
      }
    }
   }
  }
#pragma unroll
  for (int a = 0; a < RA; ++a) {
    const int t = t0 + ty * RA + a;
    if (t >= T) continue;
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const int e = e0 + tx * RB + b;
      if (e < E) {
        partial[((size_t)slice * T + t) * E + e] = st2[a][b];
      }
    }
  }
}

// Logit of (t, e) from the NS slice sums of the slice-major layout
// [NS][T][E] (NS = 8, 16 or 64): the tree's remaining levels over the slices,
// then the bias. A wave's load of one slice reads adjacent experts.
template <int NS>
__device__ __forceinline__ float tree_sum(float* v) {
#pragma unroll
  for (int w = NS; w > 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w / 2; ++i) v[i] = v[2 * i] + v[2 * i + 1];
  return v[0];
}

template <int NS>
__device__ __forceinline__ float finish_logit(const float* __restrict__ partial, const float* __restrict__ bias, int T,
                                              int E, int t, int e) {
  float v[NS];
  const size_t st = (size_t)T * E, o = (size_t)t * E + e;
  // read through a pointer that is never null (partial stands in, unused,
  // when there is no bias), so the load needs no branch of its own and can
  // go out with the slice sums
  const float b = (bias ? bias : partial)[e];
#pragma unroll
  for (int i = 0; i < NS; ++i) v[i] = partial[i * st + o];
  const float l = tree_sum<NS>(v);
  return bias ? l + b : l;
}

// Wave-wide max / min of a uint32 by DPP: row shifts build each 16-lane
// row's prefix, the two row broadcasts carry it across rows, lane 63 ends with
// the result (read back as a scalar). Lanes without a DPP source contribute
// the operation's identity.
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false));  // row_shr:1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false));  // row_shr:2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false));  // row_shr:4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false));  // row_shr:8
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));  // row_bcast:15
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_umin(uint32_t v) {
  const int ident = -1;  // 0xffffffff
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(ident, (int)v, 0x111, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(ident, (int)v, 0x112, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(ident, (int)v, 0x114, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(ident, (int)v, 0x118, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(ident, (int)v, 0x142, 0xa, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(ident, (int)v, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Top-k of one token's scores (sc[0..E), E <= 64 NK, scores >= 0) by one
// wave: K rounds of a wave argmax keyed (score desc, expert asc), the same
// selection and slot order as a full sort. Lane l keeps experts l, l+64, ...
// in NK registers as keys fp32 bits + 1 (scores are non-negative, so the bits
// order like the values; 0 marks a taken or absent expert). A round is two
// wave reductions: the largest key, then the lowest expert holding it.
// Lane 0 writes slot j of sel_id / sel_s.
template <int NK>
__device__ __forceinline__ void wave_topk_n(const float* __restrict__ sc, int E, int K, int* sel_id, float* sel_s) {
  const int lane = threadIdx.x & 63;
  uint32_t key[NK];
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? __float_as_uint(sc[e]) + 1u : 0u;
  }
#pragma unroll 1
  for (int j = 0; j < K; ++j) {
    uint32_t bk = key[0];
    int be = lane;
#pragma unroll
    for (int i = 1; i < NK; ++i)
      if (key[i] > bk) {  // strictly greater: the lower expert wins a tie
        bk = key[i];
        be = lane + 64 * i;
      }
    const uint32_t top = wave_umax(bk);
    const int e = (int)wave_umin(bk == top ? (uint32_t)be : 0xffffffffu);
#pragma unroll
    for (int i = 0; i < NK; ++i)
      if (lane + 64 * i == e) key[i] = 0u;
    if (lane == 0) {
      sel_id[j] = e;
      sel_s[j] = __uint_as_float(top - 1u);
    }
  }
}

// The above with NK = the fewest registers that hold E experts (E <= 1024).
__device__ __forceinline__ void wave_topk(const float* __restrict__ sc, int E, int K, int* sel_id, float* sel_s) {
  if (E <= 64) wave_topk_n<1>(sc, E, K, sel_id, sel_s);
  else if (E <= 128) wave_topk_n<2>(sc, E, K, sel_id, sel_s);
  else if (E <= 256) wave_topk_n<4>(sc, E, K, sel_id, sel_s);
  else if (E <= 512) wave_topk_n<8>(sc, E, K, sel_id, sel_s);
  else wave_topk_n<16>(sc, E, K, sel_id, sel_s);
}

// Renormalized weights of the K selected scores: S accumulated left to right
// over the slots, w_j = s_j / S (1/K if S == 0).
__device__ __forceinline__ float renorm_weight(const float* sel_s, int K, int j) {
  float S = 0.0f;
  for (int i = 0; i < K; ++i) S = S + sel_s[i];
  return (S == 0.0f) ? 1.0f / (float)K : sel_s[j] / S;
}

// ---------------------------------------------------------------------------
// Small batches: one 256-thread workgroup per token. Threads finish the
// logits of the token's experts from the NS slice sums (the tree's top
// levels), the sigmoid scores go to LDS, wave 0 selects the top k, and all
// four waves quantize the token's row of x (int8 rows only).
// ---------------------------------------------------------------------------
template <typename XT, int NS>
__global__ __launch_bounds__(256) void topk_quant_token_kernel(const float* __restrict__ partial,
                                                               const float* __restrict__ bias, const XT* __restrict__ x,
                                                               int T, int H, int E, int K, int quant, int mx,
                                                               int32_t* __restrict__ ids_out,
                                                               float* __restrict__ w_out, uint8_t* __restrict__ xq,
                                                               uint8_t* __restrict__ xs) {
  __shared__ float sc[1024];
  __shared__ float red[4];
  __shared__ int sel_id[16];
  __shared__ float sel_s[16];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const XT* row = x + (size_t)t * H;
  // int8 rows of up to 4096 values: each thread's 16 values are loaded first,
  // so the row and the chunk sums are in flight together
  const bool regs = quant && !mx && H <= 4096 && (H & 1023) == 0;
  const int nu = H >> 10;
  float v[4][4];
  if (regs) {
#pragma unroll
    for (int u = 0; u < 4; ++u) load4<XT>(row + ((size_t)min(u, nu - 1) * 256 + tid) * 4, v[u]);
  }
#pragma unroll 1
  for (int e = tid; e < E; e += 256) sc[e] = moe::sigmoid_fixed(finish_logit<NS>(partial, bias, T, E, t, e));
  float amax = 0.f;
  if (regs) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int m = 0; m < 4; ++m) amax = fmaxf(amax, fabsf(v[u][m]));
    amax = moe::wave_max(amax);
    if (lane == 0) red[wave] = amax;
  }
  __syncthreads();
  if (wave == 0) wave_topk(sc, E, K, sel_id, sel_s);
  __syncthreads();
  if (tid < K) {
    ids_out[(size_t)t * K + tid] = sel_id[tid];
    w_out[(size_t)t * K + tid] = renorm_weight(sel_s, K, tid);
  }
  if (!quant) return;
  if (!regs) {
    if (wave == 1) {
      const size_t qrow = mx ? (size_t)H / 2 : (size_t)2 * H;
      const size_t srow = mx ? (size_t)H / 32 : 4;
      wave_quant_row<XT>(row, H, mx, xq + t * qrow, xs + t * srow);
    }
    return;
  }
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = amax / 127.0f;
  if (tid == 0) reinterpret_cast<float*>(xs)[t] = s;
  uint8_t* q = xq + (size_t)t * 2 * H;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (u >= nu) break;
    uint32_t hw = 0, lw = 0;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float qq = 0.f;
      if (amax != 0.f) qq = fminf(fmaxf(__builtin_rintf(v[u][m] / s), -127.f), 127.f);
      int hi, lo;
      moe::split_int8((int)qq, hi, lo);
      hw |= moe::small_int_to_e4m3(hi) << (8 * m);
      lw |= moe::small_int_to_e4m3(lo) << (8 * m);
    }
    const size_t i = ((size_t)u * 256 + tid) * 4;
    *reinterpret_cast<uint32_t*>(q + i) = hw;
    *reinterpret_cast<uint32_t*>(q + H + i) = lw;
  }
}

// ---------------------------------------------------------------------------
// One wave per token: top-k and (optionally) the quantization of the token.
// ---------------------------------------------------------------------------
template <typename XT>
__global__ __launch_bounds__(256) void topk_quant_kernel(const float* __restrict__ partial,
                                                         const float* __restrict__ bias, const XT* __restrict__ x,
                                                         int T, int H, int E, int K, int quant, int mx,
                                                         int32_t* __restrict__ ids_out, float* __restrict__ w_out,
                                                         uint8_t* __restrict__ xq, uint8_t* __restrict__ xs) {
  __shared__ float sc[4][1024];
  __shared__ int sel_id[4][16];
  __shared__ float sel_s[4][16];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
#pragma unroll 1
  for (int e = lane; e < E; e += 64) sc[wave][e] = moe::sigmoid_fixed(finish_logit<NSLICE>(partial, bias, T, E, t, e));
  // a wave reads only its own LDS rows: wave-level ordering suffices
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  wave_topk(sc[wave], E, K, sel_id[wave], sel_s[wave]);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (lane < K) {
    ids_out[(size_t)t * K + lane] = sel_id[wave][lane];
    w_out[(size_t)t * K + lane] = renorm_weight(sel_s[wave], K, lane);
  }
  if (quant) {
    const size_t qrow = mx ? (size_t)H / 2 : (size_t)2 * H;
    const size_t srow = mx ? (size_t)H / 32 : 4;
    wave_quant_row<XT>(x + (size_t)t * H, H, mx, xq + (size_t)t * qrow, xs + (size_t)t * srow);
  }
}

// ---------------------------------------------------------------------------
// Small batches, routing and sort in one 1024-thread workgroup (no hand-over
// between workgroups): the logits of all T x E (token, expert) items from the
// 16 four-chunk slice sums, their sigmoid scores in LDS, the top k of token t by wave
// t % 16, then the stable expert sort of the P = T k pairs with the
// arithmetic of the one-workgroup sort kernel. Dynamic LDS: max(T E scores,
// the sort's E ceil(P / 32) mask words), then tot[E], offs[E + 1], tmp[1024].
// ---------------------------------------------------------------------------
constexpr int RS_MAX_TE = 4096;  // scores of a tiny batch (4 per thread)

// Sigmoid scores of items tid, tid + 1024, ... (NI of them, NI * 1024 >= TE)
// into sc[TE].
template <int NI>
__device__ __forceinline__ void score_items(const float* __restrict__ partial, const float* __restrict__ bias, int TE,
                                            int E, float* sc) {
  const int tid = threadIdx.x;
  float v[NI][NSLICE_TINY], b[NI];
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int ic = min(u * 1024 + tid, TE - 1);
    b[u] = (bias ? bias : partial)[ic % E];  // pointer never null, as in finish_logit
#pragma unroll
    for (int sl = 0; sl < NSLICE_TINY; ++sl) v[u][sl] = partial[(size_t)sl * TE + ic];
  }
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int i = u * 1024 + tid;
    if (i < TE) {
      const float l = tree_sum<NSLICE_TINY>(v[u]);
      sc[i] = moe::sigmoid_fixed(bias ? l + b[u] : l);
    }
  }
}

__global__ __launch_bounds__(1024) void route_sort_small_kernel(
    const float* __restrict__ partial, const float* __restrict__ bias, int T, int E, int K, int block_m,
    int32_t* __restrict__ ids_out, float* __restrict__ w_out, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted, int32_t* __restrict__ pos,
    int32_t* __restrict__ tile_expert, int32_t* __restrict__ n_tiles, int32_t* __restrict__ wide,
    int32_t* __restrict__ n_wide) {
  extern __shared__ int smem[];
  __shared__ int ids_lds[moe::SB];
  __shared__ int sel_id[16][16];
  __shared__ float sel_s[16][16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int TE = T * E, P = T * K, W = (P + 31) >> 5;
  float* sc = reinterpret_cast<float*>(smem);
  int* tot = smem + max(TE, E * W);
  int* offs = tot + E;
  int* tmp = offs + E + 1;

  // scores: the items of a thread have all their slice loads in flight
  // together (indices clamped, so no load is conditional)
  if (TE > 2048) score_items<4>(partial, bias, TE, E, sc);
  else if (TE > 1024) score_items<2>(partial, bias, TE, E, sc);
  else score_items<1>(partial, bias, TE, E, sc);
  __syncthreads();

  for (int t = wave; t < T; t += 16) {
    wave_topk(sc + (size_t)t * E, E, K, sel_id[wave], sel_s[wave]);
    // lane 0 wrote the wave's own LDS rows: wave-level ordering suffices
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lane < K) {
      const int id = sel_id[wave][lane];
      ids_out[(size_t)t * K + lane] = id;
      w_out[(size_t)t * K + lane] = renorm_weight(sel_s[wave], K, lane);
      ids_lds[t * K + lane] = id;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  __syncthreads();

  // the sort (the score region is reused for the expert bitmasks)
  const bool valid = tid < P;
  const int id = valid ? ids_lds[tid] : 0;
  int rank;
  moe::block_rank(id, valid, P, E, reinterpret_cast<uint32_t*>(smem), tot, rank);
  moe::scan_offsets(tot, E, block_m, offs, tmp);
  if (valid) {
    const int p = offs[id] + rank;
    sorted[p] = tid;
    pos[tid] = p;
  }
  for (int e = tid; e < E; e += blockDim.x) counts[e] = tot[e];
  for (int e = tid; e <= E; e += blockDim.x) offsets[e] = offs[e];
  moe::write_tiles_and_padding(tot, offs, E, P, block_m, sorted, tile_expert, n_tiles);
  if (wide) moe::write_wide_tiles(offs, E, block_m, tmp, wide, n_wide);
}

// ---------------------------------------------------------------------------
// Partial logits of large batches on the fp32 matrix cores, fed straight from
// memory. The 32x32x2 fp32 MFMA adds two products to each accumulator per
// instruction as two chained IEEE fused multiply-adds, k slot 0 then slot 1
// (checked bit for bit on the GPU), so issuing it over ascending k pairs is
// the chunk's chain, at twice the non-packed VALU rate. Each wave owns 64
// tokens x 32 experts of one 8-chunk slice as two accumulators (token blocks
// 0..31 and 32..63: two independent chains a wave) plus the 3-level pairwise
// stack of every output. Lanes l and l + 32 read the two halves of the same
// row's 16-k batch (8 consecutive k each), so one load touches 32 cache lines
// and no lane re-reads what its partner holds; a v_permlane32_swap per
// register pair then puts k 2m in the low half and k 2m + 1 in the high half
// of one register, the MFMA's k slots. Plain vector loads from L2, double-
// buffered in registers: no LDS, no barriers. Chunks are whole batches
// (L % 16 == 0: H % 1024 == 0; other widths take router_partial_kernel).
// ---------------------------------------------------------------------------
constexpr int RM_KB = 16;  // k per batch (32 measured no faster)
constexpr int RM_NBUF = 2;  // register sets: batch b + 2 is loaded while batch b runs

// NV consecutive values as fp32 (16-byte aligned, NV % 8 == 0).
template <typename XT, int NV>
__device__ __forceinline__ void load_row(const XT* p, float* o) {
  if constexpr (sizeof(XT) == 4) {
#pragma unroll
    for (int i = 0; i < NV / 4; ++i) {
      const float4 v = reinterpret_cast<const float4*>(p)[i];
      o[4 * i] = v.x; o[4 * i + 1] = v.y; o[4 * i + 2] = v.z; o[4 * i + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < NV / 8; ++i) {
      const uint4 v = reinterpret_cast<const uint4*>(p)[i];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
        o[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
      }
    }
  }
}

// In: lane half h holds k NV h + i of the batch in r[i]. Out: r[2m] holds k 2m
// (low half) and 2m + 1 (high half), r[2m + 1] holds k NV + 2m and NV + 2m + 1:
// the swap exchanges the high half of r[2m] with the low half of r[2m + 1].
template <int NV>
__device__ __forceinline__ void pair_k(float* r) {
#pragma unroll
  for (int m = 0; m < NV / 2; ++m) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(r[2 * m]), __float_as_uint(r[2 * m + 1]), false,
                                                    false);
    r[2 * m] = __uint_as_float(s[0]);
    r[2 * m + 1] = __uint_as_float(s[1]);
  }
}

template <typename XT>
__global__ __launch_bounds__(256, 2) void router_mfma_kernel(const XT* __restrict__ x, const float* __restrict__ wr,
                                                             float* __restrict__ partial, int T, int H, int E) {
  constexpr int KB = RM_KB, NV = KB / 2;  // NV: values a lane loads per row and batch
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, h = lane >> 5, r = lane & 31;
  const int e0 = (blockIdx.x * 4 + wave) * 32, t0 = blockIdx.y * 64, slice = blockIdx.z;
  const int L = H >> 6;
  const int kbeg = slice * NSLICE * L, nb = NSLICE * L / KB;  // batches in the slice (even)
  const int e = e0 + r;
  const bool ev = e < E;
  // Rows past T or E read row 0 instead: an MFMA output depends only on its
  // own A row and B column, and those outputs are not stored.
  const int ta = t0 + r < T ? t0 + r : 0, tb = t0 + 32 + r < T ? t0 + 32 + r : 0;
  const XT* xr0 = x + (size_t)ta * H + kbeg + NV * h;
  const XT* xr1 = x + (size_t)tb * H + kbeg + NV * h;
  const float* wrow = wr + (size_t)(ev ? e : 0) * H + kbeg + NV * h;

  v16f acc[2] = {}, st0[2] = {}, st1[2] = {}, st2[2] = {};
  float xa[RM_NBUF][2][NV], wb[RM_NBUF][NV];
  auto fetch = [&](int set, int b) {
    b = b < nb ? b : nb - 1;  // past the end: re-read the last batch (branch-free)
    load_row<XT, NV>(xr0 + b * KB, xa[set][0]);
    load_row<XT, NV>(xr1 + b * KB, xa[set][1]);
    load_row<float, NV>(wrow + b * KB, wb[set]);
  };
  int chunk = 0, in_chunk = 0;
  auto push = [&]() {
    // chunk index within the slice as a 3-bit counter (wave-uniform): the
    // pairwise tree, only the adds this chunk needs
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      if (!(chunk & 1)) {
        st0[blk] = acc[blk];
      } else {
        const v16f a1 = st0[blk] + acc[blk];  // level 1
        if (!(chunk & 2)) {
          st1[blk] = a1;
        } else {
          const v16f a2 = st1[blk] + a1;  // level 2
          st2[blk] = (chunk & 4) ? st2[blk] + a2 : a2;  // level 3 at chunk 7
        }
      }
      acc[blk] = (v16f){};
    }
    ++chunk;
  };
  auto batch = [&](int set, int b) {
    pair_k<NV>(xa[set][0]);
    pair_k<NV>(xa[set][1]);
    pair_k<NV>(wb[set]);
#pragma unroll
    for (int s = 0; s < NV; ++s) {
      const int reg = s < NV / 2 ? 2 * s : 2 * (s - NV / 2) + 1;  // k 2s, 2s + 1
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(xa[set][0][reg], wb[set][reg], acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(xa[set][1][reg], wb[set][reg], acc[1], 0, 0, 0);
    }
    fetch(set, b + RM_NBUF);
    in_chunk += KB;
    if (in_chunk == L) {
      in_chunk = 0;
      push();
    }
  };
  // Sets are issued in the order the loop consumes them, here as on the loop's
  // back edge, so that the wait before a set's first use counts only that
  // set's loads (with the prologue's loads in another order the waits at the
  // loop head covered both sets).
#pragma unroll
  for (int i = 0; i < RM_NBUF; ++i) {
    fetch(i, i);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int b = 0; b < nb; b += RM_NBUF) {  // nb % RM_NBUF == 0: every pass runs every set
#pragma unroll
    for (int i = 0; i < RM_NBUF; ++i) batch(i, b + i);
  }
  // block blk: token t0 + 32 blk + 8 (v / 4) + 4 (lane / 32) + v % 4, expert e0 + lane % 32
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int tt = t0 + 32 * blk + 8 * (v >> 2) + 4 * h + (v & 3);
      if (tt < T && ev) partial[((size_t)slice * T + tt) * E + e] = st2[blk][v];
    }
}

// logits[t][e] from the NS slice sums: one thread per (t, e).
template <int NS>
__global__ __launch_bounds__(256) void finish_logits_kernel(const float* __restrict__ partial,
                                                            const float* __restrict__ bias, int T, int E,
                                                            float* __restrict__ logits) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)T * E) return;
  const int t = (int)(i / E), e = (int)(i % E);
  logits[i] = finish_logit<NS>(partial, bias, T, E, t, e);
}

template <typename XT>
hipError_t launch_partial(const XT* x, const float* wr, float* partial, int T, int H, int E, int ns, int mx,
                          uint8_t* xq, uint8_t* xs, hipStream_t st) {
  if (ns == NSLICE_TINY) {
    // four chunks per workgroup (T <= 16 here), one LDS stage (64 k) per
    // chunk sub-range, so that each stage runs branch-free (stages of 256 k
    // took the per-group chunk-end checks and measured slower); with xq,
    // slices 16.. quantize x (a token row each)
    const int ex = (E + 15) / 16;
    dim3 grid(ex, 1, NSLICE_TINY + (xq ? (T + ex - 1) / ex : 0));
    router_partial_kernel<XT, 1, 1, 64, 4><<<grid, 256, 0, st>>>(x, wr, partial, T, H, E, mx, xq, xs);
  } else if (ns == NSLICE_SMALL) {
    // one chunk per workgroup, one LDS stage (64 k) per chunk sub-range; with
    // xq, slices 64.. quantize x (one token row per workgroup)
    auto go = [&](auto ra, auto rb) {
      constexpr int RA = decltype(ra)::value, RB = decltype(rb)::value;
      const int ex = (E + 16 * RB - 1) / (16 * RB);
      dim3 grid(ex, 1, NSLICE_SMALL + (xq ? (T + ex - 1) / ex : 0));
      router_partial_kernel<XT, RA, RB, 64, 1><<<grid, 256, 0, st>>>(x, wr, partial, T, H, E, mx, xq, xs);
    };
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I4 = std::integral_constant<int, 4>;
    // above 32 tokens 64 x 32 tiles (8 outputs a thread, fewer LDS bytes per
    // fma): 10.4 -> 8.9 us at 64 tokens; 64 x 64 spills, and 32 x 32 tiles
    // at 17..32 tokens measured no faster than 32 x 16
    if (T <= 16) go(I1{}, I1{});
    else if (T <= 32) go(I2{}, I1{});
    else go(I4{}, I2{});
  } else {
    if (xq) return hipErrorInvalidValue;  // large batches quantize x in the top-k kernel
    if ((H / 64) % RM_KB == 0) {
      // four waves a workgroup, each 64 tokens x 32 experts
      dim3 grid((E + 127) / 128, (T + 63) / 64, NSLICE);
      router_mfma_kernel<XT><<<grid, 256, 0, st>>>(x, wr, partial, T, H, E);
    } else {
      dim3 grid((E + 63) / 64, (T + 63) / 64, NSLICE);
      router_partial_kernel<XT, 4, 4, 32, 8><<<grid, 256, 0, st>>>(x, wr, partial, T, H, E, 0, nullptr, nullptr);
    }
  }
  return hipGetLastError();
}

}  // namespace

int moe_k_router_slices(int T, int H, int E, int K) {
  const int L = H / 64;
  if (!(T <= 64 && L % 64 == 0 && L <= 256)) return NSLICE;
  return (T <= 16 && T * E <= RS_MAX_TE && K <= 16 && E <= 1024) ? NSLICE_TINY : NSLICE_SMALL;
}

size_t moe_k_router_partial_bytes(int T, int H, int E, int K) {
  return (size_t)moe_k_router_slices(T, H, E, K) * T * E * 4;
}

hipError_t moe_k_router_partial(int x_dtype, const void* x, const float* wr, float* partial, int T, int H, int E,
                                int K, int mx, uint8_t* xq, uint8_t* xs, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  const int ns = moe_k_router_slices(T, H, E, K);
  if (x_dtype == 0) return launch_partial<float>((const float*)x, wr, partial, T, H, E, ns, mx, xq, xs, st);
  return launch_partial<uint16_t>((const uint16_t*)x, wr, partial, T, H, E, ns, mx, xq, xs, st);
}

int moe_k_router_quantizes_x(int T, int H, int E, int K) { return moe_k_router_slices(T, H, E, K) != NSLICE; }

hipError_t moe_k_topk_quant(int x_dtype, const float* partial, const float* bias, const void* x, int T, int H, int E,
                            int K, int quant, int mx, int32_t* ids, float* w, uint8_t* xq, uint8_t* xs,
                            hipStream_t st) {
  if (T <= 0) return hipSuccess;
  const int ns = moe_k_router_slices(T, H, E, K);
  if (ns != NSLICE) {
    // per-token workgroups
    if (x_dtype == 0) {
      if (ns == NSLICE_TINY)
        topk_quant_token_kernel<float, NSLICE_TINY><<<T, 256, 0, st>>>(partial, bias, (const float*)x, T, H, E, K,
                                                                       quant, mx, ids, w, xq, xs);
      else
        topk_quant_token_kernel<float, NSLICE_SMALL><<<T, 256, 0, st>>>(partial, bias, (const float*)x, T, H, E, K,
                                                                        quant, mx, ids, w, xq, xs);
    } else {
      if (ns == NSLICE_TINY)
        topk_quant_token_kernel<uint16_t, NSLICE_TINY><<<T, 256, 0, st>>>(partial, bias, (const uint16_t*)x, T, H, E,
                                                                          K, quant, mx, ids, w, xq, xs);
      else
        topk_quant_token_kernel<uint16_t, NSLICE_SMALL><<<T, 256, 0, st>>>(partial, bias, (const uint16_t*)x, T, H,
                                                                           E, K, quant, mx, ids, w, xq, xs);
    }
    return hipGetLastError();
  }
  const int blocks = (T + 3) / 4;
  if (x_dtype == 0)
    topk_quant_kernel<float><<<blocks, 256, 0, st>>>(partial, bias, (const float*)x, T, H, E, K, quant, mx, ids, w, xq,
                                                     xs);
  else
    topk_quant_kernel<uint16_t><<<blocks, 256, 0, st>>>(partial, bias, (const uint16_t*)x, T, H, E, K, quant, mx, ids,
                                                        w, xq, xs);
  return hipGetLastError();
}

int moe_k_route_sort_fits(int T, int H, int E, int K) { return moe_k_router_slices(T, H, E, K) == NSLICE_TINY; }

hipError_t moe_k_route_sort_small(const float* partial, const float* bias, int T, int E, int K, int block_m,
                                  int32_t* ids, float* w, int32_t* counts, int32_t* offsets, int32_t* sorted,
                                  int32_t* pos, int32_t* tile_expert, int32_t* n_tiles, int32_t* wide,
                                  int32_t* n_wide, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  if (T * K > moe::SB || K > 16 || E > 1024 || T * E > RS_MAX_TE) return hipErrorInvalidValue;
  // above 64 KB of LDS a kernel must opt in (gfx950: 160 KB per workgroup)
  static std::atomic<bool> lds_opt_in[moe::kMaxDevices];
  const hipError_t e = moe::once_per_device(lds_opt_in, [] {
    return hipFuncSetAttribute((const void*)route_sort_small_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                               150 * 1024);
  });
  if (e != hipSuccess) return e;
  const int P = T * K, W = (P + 31) / 32;
  const size_t lds = (size_t)(std::max(T * E, E * W) + E + E + 1 + 1024) * 4;
  route_sort_small_kernel<<<1, 1024, lds, st>>>(partial, bias, T, E, K, block_m, ids, w, counts, offsets, sorted, pos,
                                                tile_expert, n_tiles, wide, n_wide);
  return hipGetLastError();
}

hipError_t moe_k_finish_logits(const float* partial, const float* bias, int T, int H, int E, int K, float* logits,
                               hipStream_t st) {
  if (T <= 0) return hipSuccess;
  const int ns = moe_k_router_slices(T, H, E, K);
  const unsigned blocks = (unsigned)(((size_t)T * E + 255) / 256);
  if (ns == NSLICE_TINY)
    finish_logits_kernel<NSLICE_TINY><<<blocks, 256, 0, st>>>(partial, bias, T, E, logits);
  else if (ns == NSLICE_SMALL)
    finish_logits_kernel<NSLICE_SMALL><<<blocks, 256, 0, st>>>(partial, bias, T, E, logits);
  else
    finish_logits_kernel<NSLICE><<<blocks, 256, 0, st>>>(partial, bias, T, E, logits);
  return hipGetLastError();
}
