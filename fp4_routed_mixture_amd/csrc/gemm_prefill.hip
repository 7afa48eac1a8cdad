// Large-M (prefill) grouped expert GEMMs on the gfx950 scaled FP4 MFMA.
//
// The pages accelerate prefill with MFMA kernels and "improved packed-weight
// reuse" (abstract of "DeepSeek-V4-Flash on AMD gfx90a: Correctness Recovery
// and Inference Performance Engineering"). Here both operands are MXFP4
// (E2M1 codes + E8M0 per 32) and go to V_MFMA_SCALE_F32_32X32X64_F8F6F4
// unchanged: weights are A (32-row tiles), pair rows are B (32 columns).
//
// Workgroup tile: BM = 128 pair rows (one sort tile of one expert) x 256
// weight rows (4 gate/up tile pairs of W13, or 8 row tiles of W2). Four waves
// in a 2 x 2 grid; a wave owns 4 weight tiles x 2 pair tiles (8 MFMA
// accumulators). K advances 128 per stage (two 64-K MFMA steps); each stage's
// weight tiles (16 KB, copied in prepacked order, so every lane's 16-byte
// operand read is conflict-free) and gathered pair rows (8 KB, transposed into
// the operand layout) are double-buffered in LDS, the next stage's global
// loads in flight while the current stage runs. Scale dwords (four K-tiles
// each) go straight to registers; the MFMA's byte select picks the K-tile.
// Launch order puts the sort tiles of one expert for one weight block 16
// workgroups apart, i.e. on the same XCD close in time, so the re-reads of a
// weight block by an expert's sort tiles hit that XCD's L2.
//
// Epilogue W13: a = (g * sigmoid(g)) * u, then MXFP4 requantization of each
// 32-block along I (a 32-row gate tile is exactly one block): lanes l and
// l^32 hold the block's two halves, one shuffle gives the block amax.
// Epilogue W2: y[pair][H] in fp32.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace {

constexpr int BM = 128;          // pair rows per sort tile
constexpr int WT = 8;            // 32-row weight tiles per workgroup
constexpr int A_STAGE = WT * 2 * 1024;   // 16 KB
constexpr int B_STAGE = 4 * 2 * 1024;    // 8 KB

template <int OA, int OB>
__device__ __forceinline__ v16f mfma44(const v4i& a, const v4i& b, v16f acc, uint32_t sa, uint32_t sb) {
  v8i a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  v8i b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  return MFMA_FP4_FP4(a8, b8, acc, OA, (int)sa, OB, (int)sb);
}

// bytes h, h+2, h+4, h+6 of the 8 scale bytes of a 4-K-tile group -> one dword
__device__ __forceinline__ uint32_t pick_scales(uint32_t vx, uint32_t vy, int h) {
  const uint2 v = make_uint2(vx, vy);
  const uint32_t lo = h ? (v.x >> 8) : v.x, hi = h ? (v.y >> 8) : v.y;
  return (lo & 0xffu) | ((lo >> 8) & 0xff00u) | ((hi & 0xffu) << 16) | ((hi << 8) & 0xff000000u);
}

template <bool GATE_UP>
__global__ __launch_bounds__(256, 1) void prefill_gemm_kernel(
    const uint8_t* __restrict__ wq, const uint8_t* __restrict__ wsc, const uint8_t* __restrict__ act_codes,
    const uint8_t* __restrict__ act_scales, const int32_t* __restrict__ sorted,
    const int32_t* __restrict__ tile_expert, const int32_t* __restrict__ n_tiles, int K, int NT, int top_k, int P,
    int rows_are_tokens, uint8_t* __restrict__ aq, uint8_t* __restrict__ as, float* __restrict__ y, int out_n) {
  constexpr int S = GATE_UP ? 2 : 1;
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][A_STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][B_STAGE];
  const int nb = blockIdx.x, q = blockIdx.y;
  if (q >= *n_tiles) return;
  const int e = tile_expert[q];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wn = wave & 1, wm = wave >> 1;
  const int KT = K >> 6, G = (KT + 3) >> 2, KB = K >> 5;
  const int NS = KT >> 1;  // stages (K % 128 == 0)
  const int c = lane & 31, h = lane >> 5;

  // ---- staging loads: uniform base pointers + 32-bit per-thread offsets ----
  // weights: 4 instructions of 4 KB. W13: instruction i = tile pair j0+i,
  // contiguous [kt][gate/up][lane][16]. W2: instruction i covers tiles 2i,
  // 2i+1 (128 threads each), contiguous [kt][lane][16] per tile.
  const int j0 = nb * (WT / S);  // first tile (pair) index of this block
  const uint8_t* a_base = wq + ((size_t)e * NT + j0) * KT * (S * 1024);
  const uint32_t a_tile_stride = (uint32_t)KT * (S * 1024);  // bytes between tiles (pairs)
  const uint32_t a_thr = GATE_UP ? tid * 16 : (tid >> 7) * a_tile_stride + (tid & 127) * 16;
  const uint32_t a_instr_stride = GATE_UP ? a_tile_stride : 2 * a_tile_stride;
  const int a_dst0 = GATE_UP ? tid * 16 : (tid >> 7) * 2048 + (tid & 127) * 16;
  const int a_dst_stride = GATE_UP ? 4096 : 4096;  // LDS bytes between instructions
  const uint32_t a_stage_stride = GATE_UP ? 4096 : 2048;  // bytes per stage within a tile (pair)
  // pair rows: 2 instructions of 64 rows x 64 bytes
  uint32_t b_off[2];
  bool b_ok[2];
  const int c4 = tid & 3;
  const int b_dst0 = ((tid >> 2) >> 5) * 2048 + (c4 >> 1) * 1024 + ((c4 & 1) * 32 + ((tid >> 2) & 31)) * 16;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int r = m * 64 + (tid >> 2);
    const int pr = sorted[q * BM + r];
    b_ok[m] = pr < P;
    const int row = b_ok[m] ? (rows_are_tokens ? pr / top_k : q * BM + r) : 0;
    b_off[m] = (uint32_t)row * (uint32_t)(K >> 1) + (c4 >> 1) * 32 + (c4 & 1) * 16;
  }

  // ---- MFMA operands of this wave ---------------------------------------------
  // weight tile t (0..3) of the wave: W13 pair 2*wn + t/2, half t%2; W2 tile 4*wn + t
  // LDS offset of (t, kt_local): W13 pi*4096 + kl*2048 + s*1024; W2 ti*2048 + kl*1024
  const uint32_t* sa_base =
      reinterpret_cast<const uint32_t*>(wsc + ((size_t)e * NT + j0) * G * (S * 256)) + lane;
  // pair tiles of the wave: 2*wm, 2*wm+1; scale-row offsets of this lane's rows
  uint32_t sb_off[2];
  bool sb_ok[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int r = (2 * wm + u) * 32 + c;
    const int pr = sorted[q * BM + r];
    sb_ok[u] = pr < P;
    const int row = sb_ok[u] ? (rows_are_tokens ? pr / top_k : q * BM + r) : 0;
    sb_off[u] = (uint32_t)row * (uint32_t)KB;
  }

  v16f acc[4][2];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int u = 0; u < 2; ++u) acc[t][u] = (v16f){};

  // two register staging sets: stages st+1 and st+2 are in flight while
  // stage st is computed
  v4i ra[2][4], rb[2][2];
  auto gload = [&](int set, int st) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ra[set][i] = *reinterpret_cast<const v4i*>(a_base + a_thr + i * a_instr_stride + (uint32_t)st * a_stage_stride);
#pragma unroll
    for (int m = 0; m < 2; ++m)
      rb[set][m] =
          b_ok[m] ? *reinterpret_cast<const v4i*>(act_codes + b_off[m] + (uint32_t)st * 64) : (v4i){0, 0, 0, 0};
  };
  auto lstore = [&](int set, int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<v4i*>(&lds_a[buf][a_dst0 + i * a_dst_stride]) = ra[set][i];
#pragma unroll
    for (int m = 0; m < 2; ++m) *reinterpret_cast<v4i*>(&lds_b[buf][b_dst0 + m * 4096]) = rb[set][m];
  };
  uint32_t sa[4], sb[2];
  auto load_scales = [&](int g) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      // W13: pair 2wn + t/2, half t%2 -> dword (pair * G + g) * 128 + half * 64; W2: (tile * G + g) * 64
      const uint32_t idx = GATE_UP ? ((uint32_t)(2 * wn + (t >> 1)) * G + g) * 128 + (t & 1) * 64
                                   : ((uint32_t)(4 * wn + t) * G + g) * 64;
      sa[t] = sa_base[idx];
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      // a group's 8 bytes; K-tiles beyond KT (K % 256 == 128) do not exist
      const uint32_t* p = reinterpret_cast<const uint32_t*>(act_scales + sb_off[u] + g * 8);
      const uint32_t vx = sb_ok[u] ? p[0] : 0x7f7f7f7fu;
      const uint32_t vy = (sb_ok[u] && 4 * g + 2 < KT) ? p[1] : 0x7f7f7f7fu;
      sb[u] = pick_scales(vx, vy, h);
    }
  };
  // one stage: two 64-K steps with byte selects (O0, O0+1)
  auto compute = [&](int buf, auto o0) {
    constexpr int O0 = decltype(o0)::value;
#pragma unroll
    for (int kl = 0; kl < 2; ++kl) {
      v4i av[4], bv[2];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int off = GATE_UP ? (2 * wn + (t >> 1)) * 4096 + kl * 2048 + (t & 1) * 1024
                                : (4 * wn + t) * 2048 + kl * 1024;
        av[t] = *reinterpret_cast<const v4i*>(&lds_a[buf][off + lane * 16]);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
        bv[u] = *reinterpret_cast<const v4i*>(&lds_b[buf][((2 * wm + u) * 2 + kl) * 1024 + lane * 16]);
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          if (kl == 0)
            acc[t][u] = mfma44<O0, O0>(av[t], bv[u], acc[t][u], sa[t], sb[u]);
          else
            acc[t][u] = mfma44<O0 + 1, O0 + 1>(av[t], bv[u], acc[t][u], sa[t], sb[u]);
        }
    }
  };

  // stage st lives in LDS buffer st&1 and register set st&1 (before its store)
  gload(0, 0);
  if (NS > 1) gload(1, 1);
  lstore(0, 0);
  __syncthreads();
  for (int st = 0; st < NS; st += 2) {
    // stage st: K-tiles 2st, 2st+1 -> byte selects 0, 1; buffer 0
    load_scales(st >> 1);
    if (st + 2 < NS) gload(0, st + 2);
    compute(0, std::integral_constant<int, 0>());
    if (st + 1 >= NS) break;
    lstore(1, 1);
    __syncthreads();
    // stage st+1: byte selects 2, 3; buffer 1
    if (st + 3 < NS) gload(1, st + 3);
    compute(1, std::integral_constant<int, 2>());
    if (st + 2 < NS) {
      lstore(0, 0);  // buffer 0 was last read before the barrier above
      __syncthreads();
    }
  }

  // ---- epilogue ------------------------------------------------------------
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int r = (2 * wm + u) * 32 + c;
    const int p = q * BM + r;
    const int pair = sorted[p];
    if (pair >= P) continue;  // lanes l and l^32 share the row, hence the validity
    if (GATE_UP) {
      const int I = out_n;
#pragma unroll
      for (int pi = 0; pi < 2; ++pi) {
        const int jp = j0 + 2 * wn + pi;  // global tile pair = 32-block of I
        float av[16];
        float amax = 0.0f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float gg = acc[2 * pi][u][v], uu = acc[2 * pi + 1][u][v];
          av[v] = (gg * moe::sigmoid_fixed(gg)) * uu;
          amax = fmaxf(amax, fabsf(av[v]));
        }
        amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
        const int ex = amax > 0.0f ? moe::mx_scale_exp(amax) : 0;
        uint8_t* dst = aq + (size_t)p * (I >> 1) + (size_t)jp * 16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t packed = 0;
          if (amax > 0.0f) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              const float vs = __builtin_ldexpf(av[i * 4 + jj], 127 - ex);
              const uint32_t code = moe::e2m1_mag_code(fabsf(vs)) | ((__float_as_uint(vs) >> 31) << 3);
              packed |= code << (4 * jj);
            }
          }
          // rows 8i + 4h .. +3 -> bytes 4i + 2h, 4i + 2h + 1
          *reinterpret_cast<uint16_t*>(dst + 4 * i + 2 * h) = (uint16_t)packed;
        }
        if (h == 0) as[(size_t)p * (I >> 5) + jp] = (uint8_t)ex;
      }
    } else {
      const int H = out_n;
      float* yrow = y + (size_t)pair * H;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = (j0 + 4 * wn + t) * 32 + 8 * i + 4 * h;
          *reinterpret_cast<float4*>(yrow + n) =
              make_float4(acc[t][u][4 * i], acc[t][u][4 * i + 1], acc[t][u][4 * i + 2], acc[t][u][4 * i + 3]);
        }
    }
  }
}

}  // namespace

int moe_k_prefill_block_m() { return BM; }

hipError_t moe_k_prefill_gemm(int gate_up, const uint8_t* wq, const uint8_t* wsc, const uint8_t* act_codes,
                              const uint8_t* act_scales, const int32_t* sorted, const int32_t* tile_expert,
                              const int32_t* n_tiles, int max_tiles, int K, int NT, int top_k, int P,
                              int rows_are_tokens, uint8_t* aq, uint8_t* as, float* y, int out_n, hipStream_t st) {
  if (max_tiles <= 0) return hipSuccess;
  // NT: tile pairs (W13) or row tiles (W2); a workgroup covers 4 pairs / 8 tiles
  const int per_wg = gate_up ? WT / 2 : WT;
  dim3 grid(NT / per_wg, max_tiles);
  if (gate_up)
    prefill_gemm_kernel<true><<<grid, 256, 0, st>>>(wq, wsc, act_codes, act_scales, sorted, tile_expert, n_tiles, K,
                                                    NT, top_k, P, rows_are_tokens, aq, as, y, out_n);
  else
    prefill_gemm_kernel<false><<<grid, 256, 0, st>>>(wq, wsc, act_codes, act_scales, sorted, tile_expert, n_tiles,
                                                     K, NT, top_k, P, rows_are_tokens, aq, as, y, out_n);
  return hipGetLastError();
}
