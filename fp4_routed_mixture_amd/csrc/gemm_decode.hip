// Low-M (decode) expert GEMMs: packed E2M1 weights x int8 activations.
//
// The pages' CDNA2 decode kernel used dot-product instructions on int8
// activations ("INT8 activation quantization", "CDNA2 dot-product
// instructions", abstract of "DeepSeek-V4-Flash on AMD gfx90a: Correctness
// Recovery and Inference Performance Engineering"); on gfx950 the FP4
// operand goes to the scaled MFMA unchanged, so there is no format mismatch:
// each int8 activation q is given to the FP4 x FP8 scaled MFMA as the exact
// pair q = 16*hi + lo (hi, lo small integers in E4M3), the hi columns carrying
// an E8M0 scale of 2^4. Every product and partial sum is then an exactly
// representable dyadic rational, so the block-scaled sum is exact and equals
// the integer block sums of the definition.
//
// Work item: (row tile j of 32 weight rows -- a gate/up tile pair for W13 --,
// sort tile q of 16 pairs of one expert). B columns 0..15 are the hi parts of
// the 16 pair rows, 16..31 the lo parts. The four waves of a workgroup split
// K into contiguous ranges of four-K-tile groups and reduce through LDS in a
// fixed order. Weights stream straight from HBM into MFMA registers: the
// prepacked layout makes each wave's load of a 32x64 tile one contiguous
// 1 KB (16 B per lane).
// Epilogue W13: a = (g * sigmoid(g)) * u in fp32 into a[pos][I].
// Epilogue W2 : y[pair][H] = s_a * sum.
#include "common.h"
#include "kernels.h"

namespace {

template <int U>
__device__ __forceinline__ v16f mfma_fp4_fp8(const v4i& a, const v8i& b, v16f acc, uint32_t sa, uint32_t sb) {
  v8i a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  return MFMA_FP4_FP8(a8, b, acc, U, (int)sa, 0, (int)sb);
}

template <bool GATE_UP>
__global__ __launch_bounds__(256) void decode_gemm_kernel(
    const uint8_t* __restrict__ wq, const uint8_t* __restrict__ wsc, const uint8_t* __restrict__ act8,
    const float* __restrict__ act_s, const int32_t* __restrict__ sorted, const int32_t* __restrict__ tile_expert,
    const int32_t* __restrict__ n_tiles, int K, int NT, int top_k, int P, int rows_are_tokens,
    float* __restrict__ out, int out_ld) {
  constexpr int S = GATE_UP ? 2 : 1;
  __shared__ float red[4][S][16][64];
  const int j = blockIdx.x, q = blockIdx.y;
  if (q >= *n_tiles) return;
  const int e = tile_expert[q];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int KT = K >> 6, G = (KT + 3) >> 2;

  // B operand
  const int c = lane & 31, h = lane >> 5;
  const int slot = c & 15, part = c >> 4;
  const int p = q * 16 + slot;
  const int pair = sorted[p];
  const bool valid = pair < P;
  const int row = rows_are_tokens ? (valid ? pair / top_k : 0) : p;
  const uint8_t* bptr = act8 + ((size_t)row * 2 + part) * K + h * 16;
  const uint32_t sb = part ? 0x7f7f7f7fu : 0x83838383u;  // lo: 2^0, hi: 2^4

  // A operand
  const size_t tile = (size_t)e * NT + j;
  const uint8_t* aptr = wq + tile * KT * (S * 1024) + lane * 16;
  const uint32_t* sptr = reinterpret_cast<const uint32_t*>(wsc + tile * G * (S * 256)) + lane;

  const int g0 = (G * wave) >> 2, g1 = (G * (wave + 1)) >> 2;
  v16f acc0 = {}, acc1 = {};
  for (int g = g0; g < g1; ++g) {
    const uint32_t sa0 = sptr[(size_t)g * S * 64];
    const uint32_t sa1 = GATE_UP ? sptr[(size_t)g * S * 64 + 64] : 0u;
    v4i a0[4], a1[4];
    v8i b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kt = g * 4 + u;
      a0[u] = (v4i){0, 0, 0, 0};
      a1[u] = (v4i){0, 0, 0, 0};
      b[u] = (v8i){0, 0, 0, 0, 0, 0, 0, 0};
      if (kt < KT) {
        a0[u] = *reinterpret_cast<const v4i*>(aptr + (size_t)kt * S * 1024);
        if (GATE_UP) a1[u] = *reinterpret_cast<const v4i*>(aptr + (size_t)kt * S * 1024 + 1024);
        if (valid) {
          v4i lo = *reinterpret_cast<const v4i*>(bptr + (size_t)kt * 64);
          v4i hi = *reinterpret_cast<const v4i*>(bptr + (size_t)kt * 64 + 32);
          b[u] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
      }
    }
    // padded K-tiles (kt >= KT) carry zero operands: they add exactly 0
    acc0 = mfma_fp4_fp8<0>(a0[0], b[0], acc0, sa0, sb);
    acc0 = mfma_fp4_fp8<1>(a0[1], b[1], acc0, sa0, sb);
    acc0 = mfma_fp4_fp8<2>(a0[2], b[2], acc0, sa0, sb);
    acc0 = mfma_fp4_fp8<3>(a0[3], b[3], acc0, sa0, sb);
    if (GATE_UP) {
      acc1 = mfma_fp4_fp8<0>(a1[0], b[0], acc1, sa1, sb);
      acc1 = mfma_fp4_fp8<1>(a1[1], b[1], acc1, sa1, sb);
      acc1 = mfma_fp4_fp8<2>(a1[2], b[2], acc1, sa1, sb);
      acc1 = mfma_fp4_fp8<3>(a1[3], b[3], acc1, sa1, sb);
    }
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    red[wave][0][v][lane] = acc0[v];
    if (GATE_UP) red[wave][S - 1][v][lane] = acc1[v];
  }
  __syncthreads();

  // thread t: lane l = t & 63 with (l & 31) < 16 (hi column of its slot), four v
  const int l = threadIdx.x & 63, vq = threadIdx.x >> 6;
  if ((l & 31) >= 16) return;
  const int oslot = l & 15;
  const int op = q * 16 + oslot;
  const int opair = sorted[op];
  if (opair >= P) return;
  const int orow = rows_are_tokens ? opair / top_k : op;
  const float s = act_s[orow];
#pragma unroll
  for (int vv = 0; vv < 4; ++vv) {
    const int v = vq * 4 + vv;
    const int n_local = 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
    float t0 = 0.0f, t1 = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) t0 = t0 + (red[w][0][v][l] + red[w][0][v][l + 16]);
    if (GATE_UP) {
#pragma unroll
      for (int w = 0; w < 4; ++w) t1 = t1 + (red[w][S - 1][v][l] + red[w][S - 1][v][l + 16]);
      const float gg = s * t0, uu = s * t1;
      const float a = (gg * moe::sigmoid_fixed(gg)) * uu;
      out[(size_t)op * out_ld + j * 32 + n_local] = a;
    } else {
      out[(size_t)opair * out_ld + j * 32 + n_local] = s * t0;
    }
  }
}

}  // namespace

hipError_t moe_k_decode_gemm(int gate_up, const uint8_t* wq, const uint8_t* wsc, const uint8_t* act8,
                             const float* act_s, const int32_t* sorted, const int32_t* tile_expert,
                             const int32_t* n_tiles, int max_tiles, int K, int NT, int top_k, int P,
                             int rows_are_tokens, float* out, int out_ld, hipStream_t st) {
  if (max_tiles <= 0) return hipSuccess;
  dim3 grid(NT, max_tiles);
  if (gate_up)
    decode_gemm_kernel<true><<<grid, 256, 0, st>>>(wq, wsc, act8, act_s, sorted, tile_expert, n_tiles, K, NT, top_k,
                                                   P, rows_are_tokens, out, out_ld);
  else
    decode_gemm_kernel<false><<<grid, 256, 0, st>>>(wq, wsc, act8, act_s, sorted, tile_expert, n_tiles, K, NT, top_k,
                                                    P, rows_are_tokens, out, out_ld);
  return hipGetLastError();
}
