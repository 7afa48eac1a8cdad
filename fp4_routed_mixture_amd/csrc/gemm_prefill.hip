// Large-M (prefill) grouped expert GEMMs on the gfx950 scaled FP4 MFMA.
//
// The pages accelerate prefill with MFMA kernels and "improved packed-weight
// reuse" (abstract of "DeepSeek-V4-Flash on AMD gfx90a: Correctness Recovery
// and Inference Performance Engineering"). Here both operands are MXFP4
// (E2M1 codes + E8M0 per 32) and go to V_MFMA_SCALE_F32_32X32X64_F8F6F4
// directly: weights are A (32 rows), token rows are B (32 columns).
//
// Work item: (block of JB weight row tiles -- gate/up tile pairs for W13 --,
// sort tile q of 128 pairs of one expert). Wave w owns pair rows
// q*128 + w*32 .. +32; every wave reuses each weight tile across its 32 rows,
// and the four waves of a workgroup read the same weight tiles (L1/L2 hits),
// so each weight byte is fetched once per 128 rows.
// Epilogue W13: a = (g * sigmoid(g)) * u, then MXFP4 requantization of each
// 32-block along I (a 32-row gate tile is exactly one block): lanes l and
// l^32 hold the block's two halves, one shuffle gives the block amax.
// Epilogue W2: y[pair][H] in fp32.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int JB = 4;       // weight row tiles per workgroup
constexpr int BM = 128;     // pair rows per sort tile

template <int U>
__device__ __forceinline__ v16f mfma44(const v4i& a, const v4i& b, v16f acc, uint32_t sa, uint32_t sb) {
  v8i a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  v8i b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  return MFMA_FP4_FP4(a8, b8, acc, U, (int)sa, U, (int)sb);
}

template <bool GATE_UP>
__global__ __launch_bounds__(256) void prefill_gemm_kernel(
    const uint8_t* __restrict__ wq, const uint8_t* __restrict__ wsc, const uint8_t* __restrict__ act_codes,
    const uint8_t* __restrict__ act_scales, const int32_t* __restrict__ sorted,
    const int32_t* __restrict__ tile_expert, const int32_t* __restrict__ n_tiles, int K, int NT, int top_k, int P,
    int rows_are_tokens, uint8_t* __restrict__ aq, uint8_t* __restrict__ as, float* __restrict__ y, int out_n) {
  constexpr int S = GATE_UP ? 2 : 1;
  const int jb0 = blockIdx.x * JB, q = blockIdx.y;
  if (q >= *n_tiles) return;
  const int e = tile_expert[q];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int KT = K >> 6, G = (KT + 3) >> 2, KB = K >> 5;
  const int c = lane & 31, h = lane >> 5;

  // B operand: token row of this lane's column
  const int p = q * BM + wave * 32 + c;
  const int pair = sorted[p];
  const bool valid = pair < P;
  const int row = rows_are_tokens ? (valid ? pair / top_k : 0) : p;
  const uint8_t* bptr = act_codes + (size_t)row * (K >> 1) + h * 16;
  const uint8_t* bsp = act_scales + (size_t)row * KB + h;

  // A operands: JB tiles (x S)
  const uint8_t* aptr = wq + ((size_t)e * NT + jb0) * KT * (S * 1024) + lane * 16;
  const size_t a_tile_stride = (size_t)KT * S * 1024;
  const uint32_t* sptr = reinterpret_cast<const uint32_t*>(wsc + ((size_t)e * NT + jb0) * G * (S * 256)) + lane;
  const size_t s_tile_stride = (size_t)G * S * 64;

  v16f acc[JB][S];
#pragma unroll
  for (int jb = 0; jb < JB; ++jb)
#pragma unroll
    for (int s = 0; s < S; ++s) acc[jb][s] = (v16f){};

  for (int g = 0; g < G; ++g) {
    // B scales of four K-tiles: bytes (kt*2 + h) for kt = 4g..4g+3
    uint32_t sb = 0x7f7f7f7fu;
    v4i b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) b[u] = (v4i){0, 0, 0, 0};
    if (valid) {
      sb = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int kt = g * 4 + u;
        uint32_t byte = 127;
        if (kt < KT) {
          byte = bsp[kt * 2];
          b[u] = *reinterpret_cast<const v4i*>(bptr + (size_t)kt * 32);
        }
        sb |= byte << (8 * u);
      }
    }
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) {
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const uint32_t sa = sptr[jb * s_tile_stride + (size_t)g * S * 64 + s * 64];
        v4i a[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int kt = g * 4 + u;
          a[u] = (v4i){0, 0, 0, 0};
          if (kt < KT) a[u] = *reinterpret_cast<const v4i*>(aptr + jb * a_tile_stride + (size_t)kt * S * 1024 + s * 1024);
        }
        acc[jb][s] = mfma44<0>(a[0], b[0], acc[jb][s], sa, sb);
        acc[jb][s] = mfma44<1>(a[1], b[1], acc[jb][s], sa, sb);
        acc[jb][s] = mfma44<2>(a[2], b[2], acc[jb][s], sa, sb);
        acc[jb][s] = mfma44<3>(a[3], b[3], acc[jb][s], sa, sb);
      }
    }
  }

  if (!valid) return;  // no cross-lane traffic below involves invalid columns' partners? (see note)
  // note: lanes l and l^32 share the column c, hence the same validity.
  if (GATE_UP) {
    const int I = out_n;
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) {
      float a[16];
      float amax = 0.0f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float gg = acc[jb][0][v], uu = acc[jb][S - 1][v];
        a[v] = (gg * moe::sigmoid_fixed(gg)) * uu;
        amax = fmaxf(amax, fabsf(a[v]));
      }
      amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
      const int ex = amax > 0.0f ? moe::mx_scale_exp(amax) : 0;
      uint8_t* dst = aq + (size_t)p * (I >> 1) + (size_t)(jb0 + jb) * 16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t packed = 0;
        if (amax > 0.0f) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const float vs = __builtin_ldexpf(a[i * 4 + jj], 127 - ex);
            const uint32_t code = moe::e2m1_mag_code(fabsf(vs)) | ((__float_as_uint(vs) >> 31) << 3);
            packed |= code << (4 * jj);
          }
        }
        // rows 8i + 4h .. +3 -> bytes 4i + 2h, 4i + 2h + 1
        *reinterpret_cast<uint16_t*>(dst + 4 * i + 2 * h) = (uint16_t)packed;
      }
      if (h == 0) as[(size_t)p * (I >> 5) + jb0 + jb] = (uint8_t)ex;
    }
  } else {
    const int H = out_n;
    float* yrow = y + (size_t)pair * H;
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = (jb0 + jb) * 32 + 8 * i + 4 * h;
        *reinterpret_cast<float4*>(yrow + n) =
            make_float4(acc[jb][0][4 * i], acc[jb][0][4 * i + 1], acc[jb][0][4 * i + 2], acc[jb][0][4 * i + 3]);
      }
  }
}

}  // namespace

int moe_k_prefill_block_m() { return BM; }
int moe_k_prefill_jb() { return JB; }

hipError_t moe_k_prefill_gemm(int gate_up, const uint8_t* wq, const uint8_t* wsc, const uint8_t* act_codes,
                              const uint8_t* act_scales, const int32_t* sorted, const int32_t* tile_expert,
                              const int32_t* n_tiles, int max_tiles, int K, int NT, int top_k, int P,
                              int rows_are_tokens, uint8_t* aq, uint8_t* as, float* y, int out_n, hipStream_t st) {
  if (max_tiles <= 0) return hipSuccess;
  dim3 grid(NT / JB, max_tiles);
  if (gate_up)
    prefill_gemm_kernel<true><<<grid, 256, 0, st>>>(wq, wsc, act_codes, act_scales, sorted, tile_expert, n_tiles, K,
                                                    NT, top_k, P, rows_are_tokens, aq, as, y, out_n);
  else
    prefill_gemm_kernel<false><<<grid, 256, 0, st>>>(wq, wsc, act_codes, act_scales, sorted, tile_expert, n_tiles,
                                                     K, NT, top_k, P, rows_are_tokens, aq, as, y, out_n);
  return hipGetLastError();
}
