// Large-M (prefill) grouped expert GEMMs on the gfx950 scaled FP4 MFMA.
//
// The pages accelerate prefill with MFMA kernels and better reuse of the
// packed weights (abstract of "DeepSeek-V4-Flash on AMD gfx90a: Correctness
// Recovery and Inference Performance Engineering"). Here both operands are
// MXFP4 (E2M1 codes + E8M0 per 32) and go to V_MFMA_SCALE_F32_32X32X64_F8F6F4
// unchanged: weights are A (32-row tiles), pair rows are B (32 columns).
//
// Workgroup tile: BM = 32 NU pair rows (one sort tile of one expert) x 4
// waves, each wave owning 8/NU weight tiles of 32 rows (gate/up tile pairs
// of W13, or row tiles of W2) against all NU pair tiles: 8 accumulators, half
// the accumulation register file, so that two workgroups share a CU and one's
// prologue and epilogue (SiLU, requantization, stores) run under the other's
// MFMAs. NU = 2 (64-row sort tiles, 4 weight tiles per wave) measures faster
// than NU = 4 on the Zipf prefill workloads and wastes less padding on small
// experts. Weight tiles are used by one wave only, so they go from HBM
// straight into the MFMA operand registers: the prepacked layout stores each
// 64-K step of a tile as 64 lanes x 16 bytes, one fully coalesced load per
// tile and K-step, kept PF K-steps ahead in a register ring. The gathered pair
// rows are shared by the 4 waves and go through LDS: the two 128-K stages of
// the next 4-step group are loaded into registers one group ahead and
// transposed into the operand layout on their LDS store, into a 4-stage ring,
// so that a group needs one barrier (the two barriers of a double buffer per
// group measured about 1% slower).
//
// Scale dwords (four K-steps each) are loaded one group ahead; the MFMA's
// byte select picks the K-step. The main loop has no branch between a load
// and its consumer, so the compiler's memory-counter waits stay partial;
// prefetches past the end re-read the last step (cache hits) instead.
// Launch order: blockIdx.x = weight block, so the sort tiles of one expert
// for one weight block land on the same XCD and share its L2.
//
// Weights in the canonical row-major layout (CANON) take the same path with
// another address map: lane l reads 16 bytes of its tile row l % 32 at K
// offset 32 kt + 16 (l / 32) (32 rows x 32 bytes a load instead of one
// contiguous 1 KB), and builds its scale dword from the row's eight E8M0
// bytes of the group.
//
// Epilogue W13: a = (g * sigmoid(g)) * u, then MXFP4 requantization of each
// 32-block along I (a 32-row gate tile is exactly one block): lanes l and
// l^32 hold the block's two halves, one shuffle gives the block amax.
// Epilogue W2: y[pair][H] in fp32, transposed through LDS so that stores
// write whole row segments.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace {

#ifndef MOE_PREFILL_NU
#define MOE_PREFILL_NU 2
#endif
constexpr int NU = MOE_PREFILL_NU;       // 32-row pair tiles per sort tile (2 or 4)
constexpr int BM = 32 * NU;              // pair rows per sort tile
constexpr int WTW = 8 / NU;              // 32-row weight tiles per wave (4 or 2)
constexpr int NWAVE = 4;
#ifndef MOE_PREFILL_PF
#define MOE_PREFILL_PF 4
#endif
constexpr int PF = MOE_PREFILL_PF;       // weight prefetch depth in 64-K steps (2 or 4)
constexpr int B_STAGE = NU * 2 * 1024;   // BM pair rows x 128 K, operand layout
constexpr int NBL = BM * 4 / (NWAVE * 64);  // 16-byte pair-row loads per thread and stage
static_assert(PF == 2 || PF == 4, "ring slots are K-step % PF within a 4-step scale group");
static_assert(NBL >= 1 && WTW % 2 == 0, "whole pair-row loads, whole gate/up pairs");

template <int OA, int OB>
__device__ __forceinline__ v16f mfma44(const v4i& a, const v4i& b, v16f acc, uint32_t sa, uint32_t sb) {
  v8i a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  v8i b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  return MFMA_FP4_FP4(a8, b8, acc, OA, (int)sa, OB, (int)sb);
}

// bytes h, h+2, h+4, h+6 of the 8 scale bytes of a 4-K-step group -> one dword
__device__ __forceinline__ uint32_t pick_scales(uint32_t vx, uint32_t vy, int h) {
  const uint2 v = make_uint2(vx, vy);
  const uint32_t lo = h ? (v.x >> 8) : v.x, hi = h ? (v.y >> 8) : v.y;
  return (lo & 0xffu) | ((lo >> 8) & 0xff00u) | ((hi & 0xffu) << 16) | ((hi << 8) & 0xff000000u);
}

// A canonical weight row's scale dword for group g: its E8M0 bytes 8g..8g+7,
// of which a last group with two K-steps (K % 256 == 128) has only the first
// four (the other two steps are never selected; they get scale 1).
__device__ __forceinline__ uint32_t canon_row_scales(const uint8_t* row_scales, int g, int KT, int h) {
  const uint32_t* p = reinterpret_cast<const uint32_t*>(row_scales + 8 * g);
  return pick_scales(p[0], (4 * g + 2 < KT) ? p[1] : 0x7f7f7f7fu, h);
}

// The sort tile's pair-row scales (KD dwords a row) into LDS rows of KD + 1
// dwords: eight loads in flight per thread before their stores.
__device__ __forceinline__ void stage_row_scales(const uint8_t* __restrict__ act_scales, const int* lds_row, int rows,
                                                 int KD, int KB, int nthreads, uint32_t* dst) {
  const int total = rows * KD;
  for (int i0 = threadIdx.x; i0 < total; i0 += 8 * nthreads) {
    uint32_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = i0 + j * nthreads, ic = i < total ? i : 0;
      const int r = ic / KD, d = ic - r * KD;
      v[j] = reinterpret_cast<const uint32_t*>(act_scales + (size_t)lds_row[r] * KB)[d];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = i0 + j * nthreads;
      if (i < total) {
        const int r = i / KD, d = i - r * KD;
        dst[r * (KD + 1) + d] = v[j];
      }
    }
  }
}

template <bool GATE_UP, bool CANON>
__global__ __launch_bounds__(256, 2) void prefill_gemm_kernel(
    const uint8_t* __restrict__ wq, const uint8_t* __restrict__ wsc, const uint8_t* __restrict__ act_codes,
    const uint8_t* __restrict__ act_scales, const int32_t* __restrict__ sorted,
    const int32_t* __restrict__ tile_expert, const int32_t* __restrict__ n_tiles, int K, int NT, int top_k, int P,
    int rows_are_tokens, uint8_t* __restrict__ aq, uint8_t* __restrict__ as, float* __restrict__ y, int out_n) {
  constexpr int S = GATE_UP ? 2 : 1;           // 32-row tiles per NT unit (gate/up pair or one W2 tile)
  constexpr int UPW = WTW / S;                 // NT units per wave
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[4][B_STAGE];
  extern __shared__ uint32_t lds_s[];  // pair-row scales (BM x (K/128 + 1) dwords), later the y staging
  __shared__ int lds_row[BM];
  __shared__ int lds_pair[BM];
  const int nb = blockIdx.x, q = blockIdx.y;
  if (q >= *n_tiles) return;
  const int e = tile_expert[q];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int KT = K >> 6, G = (KT + 3) >> 2, KB = K >> 5;
  const int NS = KT >> 1;  // stages of 128 K (K % 128 == 0)
  const int c = lane & 31, h = lane >> 5;

  // ---- this wave's weight tiles (NT % UPW == 0: all valid or none) ----------
  const int unit0 = (nb * NWAVE + wave) * UPW;
  const bool w_valid = unit0 < NT;
  const int ubase = w_valid ? unit0 : 0;  // invalid waves compute a real block and store nothing
  // canonical rows: W13 tile t = gate/up half t%2 of pair ubase + t/2, row
  // (t%2) N/2 + (ubase + t/2) 32 + c of N = 64 NT; W2 tile t: row (ubase + t) 32 + c
  const int NR = GATE_UP ? NT * 64 : NT * 32;
  auto canon_row = [&](int t) -> uint32_t {
    return GATE_UP ? (uint32_t)((t & 1) * (NR >> 1) + (ubase + (t >> 1)) * 32) : (uint32_t)((ubase + t) * 32);
  };
  const uint8_t* a_base = CANON ? wq + ((size_t)e * NR + c) * (K >> 1) + h * 16
                                : wq + ((size_t)e * NT + ubase) * KT * (S * 1024) + lane * 16;
  // tile t: W13 pair t/2, half t%2; W2 tile t
  auto a_ptr = [&](int t, int kt) {
    const uint32_t off = CANON ? canon_row(t) * (uint32_t)(K >> 1) + (uint32_t)kt * 32
                         : GATE_UP ? (uint32_t)(t >> 1) * KT * 2048 + (t & 1) * 1024 + (uint32_t)kt * 2048
                                   : (uint32_t)t * KT * 1024 + (uint32_t)kt * 1024;
    return reinterpret_cast<const v4i*>(a_base + off);
  };
  const uint32_t* sa_base = reinterpret_cast<const uint32_t*>(wsc + ((size_t)e * NT + ubase) * G * (S * 256)) + lane;
  const uint8_t* sa_canon = wsc + ((size_t)e * NR + c) * KB;

  // ---- gathered pair rows: NBL loads of 64 rows x 64 bytes per stage -------
  // load m: thread -> row 64m + tid/4, 16-byte chunk tid%4 of the stage's 64 bytes
  const int c4 = tid & 3;
  const int b_dst = (((tid >> 2) >> 5) * 2 + (c4 >> 1)) * 1024 + ((c4 & 1) * 32 + ((tid >> 2) & 31)) * 16;
  uint32_t b_off[NBL];
#pragma unroll
  for (int m = 0; m < NBL; ++m) {
    const int br = m * 64 + (tid >> 2);
    const int pr = sorted[q * BM + br];
    const int row = pr < P ? (rows_are_tokens ? pr / top_k : q * BM + br) : 0;  // padding reads row 0
    b_off[m] = (uint32_t)row * (uint32_t)(K >> 1) + c4 * 16;
  }
  // The pair rows' E8M0 scales (K/32 bytes a row) are staged in LDS once:
  // read in the main loop straight from global memory, every lane would
  // touch its own cache line per load (one gathered row per lane), which
  // costs the vector memory path more than the weight stream. Row stride
  // K/128 + 1 dwords keeps the per-lane reads on distinct banks.
  const int KD = K >> 7;  // scale dwords per row
  if (tid < BM) {
    const int pr = sorted[q * BM + tid];
    lds_row[tid] = pr < P ? (rows_are_tokens ? pr / top_k : q * BM + tid) : 0;  // padding reads row 0
    lds_pair[tid] = pr;
  }
  __syncthreads();
  stage_row_scales(act_scales, lds_row, BM, KD, KB, NWAVE * 64, lds_s);

  v16f acc[WTW][NU];
#pragma unroll
  for (int t = 0; t < WTW; ++t)
#pragma unroll
    for (int u = 0; u < NU; ++u) acc[t][u] = (v16f){};

  v4i ra[PF][WTW];      // weight ring: slot kt % PF
  v4i rb[2][NBL];       // pair-row staging of the next group, set = its stage
  uint32_t sa[WTW], sx[NU], sy[NU], na[WTW], nx[NU], ny[NU];

  auto aload = [&](int slot, int kt) {
    kt = kt < KT ? kt : KT - 1;
#pragma unroll
    for (int t = 0; t < WTW; ++t) ra[slot][t] = *a_ptr(t, kt);
  };
  auto bload = [&](int set, int st) {
    st = st < NS ? st : NS - 1;
#pragma unroll
    for (int m = 0; m < NBL; ++m) rb[set][m] = *reinterpret_cast<const v4i*>(act_codes + b_off[m] + (uint32_t)st * 64);
  };
  auto bstore = [&](int set, int buf) {
#pragma unroll
    for (int m = 0; m < NBL; ++m) *reinterpret_cast<v4i*>(&lds_b[buf][b_dst + m * 4096]) = rb[set][m];
  };
  auto load_scales = [&](uint32_t* da, uint32_t* dx, uint32_t* dy, int g) {
    g = g < G ? g : G - 1;
#pragma unroll
    for (int t = 0; t < WTW; ++t) {
      if (CANON) {
        da[t] = canon_row_scales(sa_canon + canon_row(t) * (uint32_t)KB, g, KT, h);
      } else {
        // W13: (pair * G + g) * 128 + half * 64; W2: (tile * G + g) * 64
        const uint32_t idx = GATE_UP ? ((uint32_t)(t >> 1) * G + g) * 128 + (t & 1) * 64 : ((uint32_t)t * G + g) * 64;
        da[t] = sa_base[idx];
      }
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      // a group's 8 bytes; when K % 256 == 128 the last group has only 2
      // K-steps and its second dword is never selected (re-read the first)
      const uint32_t* p = lds_s + (u * 32 + c) * (KD + 1) + 2 * g;
      dx[u] = p[0];
      dy[u] = p[(4 * g + 2 < KT) ? 1 : 0];
    }
  };
  // one stage (two 64-K steps: byte selects B0, B0+1 of the current scale
  // group) from LDS buffer buf with weight ring slots J0, J0+1; refills those
  // slots with K-steps kt_next, kt_next+1 once their MFMAs are issued
  auto stage = [&](int buf, auto j0, auto b0, int kt_next, bool refill) {
    constexpr int J0 = decltype(j0)::value, B0 = decltype(b0)::value;
    uint32_t sb[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) sb[u] = pick_scales(sx[u], sy[u], h);
    v4i bv[2][NU];
#pragma unroll
    for (int kl = 0; kl < 2; ++kl)
#pragma unroll
      for (int u = 0; u < NU; ++u)
        bv[kl][u] = *reinterpret_cast<const v4i*>(&lds_b[buf][(u * 2 + kl) * 1024 + lane * 16]);
#pragma unroll
    for (int kl = 0; kl < 2; ++kl) {
#pragma unroll
      for (int t = 0; t < WTW; ++t)
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          if (kl == 0)
            acc[t][u] = mfma44<B0, B0>(ra[J0][t], bv[0][u], acc[t][u], sa[t], sb[u]);
          else
            acc[t][u] = mfma44<B0 + 1, B0 + 1>(ra[J0 + 1][t], bv[1][u], acc[t][u], sa[t], sb[u]);
        }
      if (refill) aload(J0 + kl, kt_next + kl);
    }
  };
  auto rotate_scales = [&]() {
#pragma unroll
    for (int t = 0; t < WTW; ++t) sa[t] = na[t];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      sx[u] = nx[u];
      sy[u] = ny[u];
    }
  };

  // prologue: K-steps 0..PF-1, pair-row stages 0 and 1 (group 0) stored,
  // then scale group 0 (the barrier also publishes the staged pair-row scales)
#pragma unroll
  for (int j = 0; j < PF; ++j) aload(j, j);
  bload(0, 0);
  bload(1, 1);
  bstore(0, 0);
  bstore(1, 1);
  __syncthreads();
  load_scales(sa, sx, sy, 0);
  // group g = K-steps 4g..4g+3 = stages 2g (buffer 0) and 2g+1 (buffer 1);
  // K-step kt sits in ring slot kt % PF
  using I0 = std::integral_constant<int, 0>;
  using I2 = std::integral_constant<int, 2>;
  using J2 = std::integral_constant<int, 2 % PF>;
  const int NG2 = NS >> 1;  // full groups
  // group g reads buffers 2(g&1), 2(g&1)+1 and writes the next group's two
  // stages into the other pair, read last in group g-1 (before the barrier
  // that ended it): one barrier per group
  for (int g = 0; g < NG2; ++g) {
    const int st = 2 * g, cur = 2 * (g & 1), nxt = 2 - cur;
    load_scales(na, nx, ny, g + 1);
    bload(0, st + 2);
    bload(1, st + 3);
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetches ahead of the MFMAs
    stage(cur, I0(), I0(), 4 * g + PF, true);
    stage(cur + 1, J2(), I2(), 4 * g + 2 + PF, true);
    bstore(0, nxt);
    bstore(1, nxt + 1);
    __syncthreads();
    rotate_scales();
  }
  if (NS & 1) stage(2 * (NG2 & 1), I0(), I0(), 0, false);  // last half group (K % 256 == 128)

  // ---- epilogue ------------------------------------------------------------
  if (!GATE_UP) {
    // y through LDS: each 32 x 32 tile goes in as the MFMA result layout and
    // comes out row-contiguous, so a store instruction writes whole 128-byte
    // row segments of 8 rows instead of 32-byte pieces of 32 rows. Each wave
    // uses its own 4.5 KB of the scale-staging LDS, free after the barrier.
    __syncthreads();
    if (!w_valid) return;
    float* stg = reinterpret_cast<float*>(lds_s) + wave * (32 * 36);
    const int H = out_n;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      int prow[4];
#pragma unroll
      for (int sr = 0; sr < 4; ++sr) prow[sr] = lds_pair[u * 32 + (lane >> 3) + 8 * sr];
#pragma unroll
      for (int t = 0; t < WTW; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<float4*>(&stg[c * 36 + 8 * i + 4 * h]) =
              make_float4(acc[t][u][4 * i], acc[t][u][4 * i + 1], acc[t][u][4 * i + 2], acc[t][u][4 * i + 3]);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int sr = 0; sr < 4; ++sr) {
          const int r = (lane >> 3) + 8 * sr;
          const float4 v = *reinterpret_cast<const float4*>(&stg[r * 36 + (lane & 7) * 4]);
          if (prow[sr] < P)
            *reinterpret_cast<float4*>(y + (size_t)prow[sr] * H + (unit0 + t) * 32 + (lane & 7) * 4) = v;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
    }
    return;
  }
  if (!w_valid) return;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int r = u * 32 + c;
    const int p = q * BM + r;
    const int pair = sorted[p];
    if (pair >= P) continue;  // lanes l and l^32 share the row, hence the validity
    if (GATE_UP) {
      const int I = out_n;
#pragma unroll
      for (int pi = 0; pi < UPW; ++pi) {
        const int jp = unit0 + pi;  // global tile pair = 32-block of I
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
        // gfx950's scaled FP4 pack conversion divides by the (power-of-two)
        // scale and rounds to nearest-even on the E2M1 grid with saturation
        // at 6 and the sign kept -- the OCP rule, checked bit for bit against
        // the software encoder below on 2^21 values including every midpoint.
        // Scales that would be denormal or near the exponent limits take the
        // software path.
        const bool hw = ex >= 2 && ex <= 252;
        const float scale = __uint_as_float((uint32_t)(hw ? ex : 127) << 23);
        uint32_t packed[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          packed[i] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, av[i * 4], av[i * 4 + 1], scale, 0);
          packed[i] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed[i], av[i * 4 + 2], av[i * 4 + 3], scale, 1);
        }
        // the software encoder only where a block's scale is out of the
        // conversion's range; a wave-uniform test keeps it a real branch
        if (__builtin_amdgcn_ballot_w64(!hw) != 0 && !hw) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            packed[i] = 0;
            if (amax > 0.0f) {
#pragma unroll
              for (int jj = 0; jj < 4; ++jj) {
                const float vs = __builtin_ldexpf(av[i * 4 + jj], 127 - ex);
                const uint32_t code = moe::e2m1_mag_code(fabsf(vs)) | ((__float_as_uint(vs) >> 31) << 3);
                packed[i] |= code << (4 * jj);
              }
            }
          }
        }
        uint32_t word[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // rows 8i + 4h .. +3 are bytes 4i + 2h, 4i + 2h + 1 of the block:
          // the lane with h = 0 gathers its partner's half into one dword
          const uint32_t other = (uint32_t)__shfl_xor((int)packed[i], 32, 64);
          word[i] = (packed[i] & 0xffffu) | (other << 16);
        }
        if (h == 0) {
          *reinterpret_cast<uint4*>(dst) = make_uint4(word[0], word[1], word[2], word[3]);
          as[(size_t)p * (I >> 5) + jp] = (uint8_t)ex;
        }
      }
    }
  }
}

}  // namespace

int moe_k_prefill_block_m() { return BM; }

hipError_t moe_k_prefill_gemm(int gate_up, int canon, const uint8_t* wq, const uint8_t* wsc, const uint8_t* act_codes,
                              const uint8_t* act_scales, const int32_t* sorted, const int32_t* tile_expert,
                              const int32_t* n_tiles, int max_tiles, int K, int NT, int top_k, int P,
                              int rows_are_tokens, uint8_t* aq, uint8_t* as, float* y, int out_n, hipStream_t st) {
  if (max_tiles <= 0) return hipSuccess;
  // NT: tile pairs (W13) or row tiles (W2); a workgroup covers 8 pairs / 16 tiles
  const int per_wg = NWAVE * (gate_up ? WTW / 2 : WTW);
  dim3 grid((NT + per_wg - 1) / per_wg, max_tiles);
  // dynamic LDS: the pair-row scales, or the down GEMM's y staging (4 waves
  // x 32 rows x 36 floats), whichever is larger
  const size_t lds = std::max<size_t>((size_t)BM * (K / 128 + 1) * 4, gate_up ? 0 : (size_t)NWAVE * 32 * 36 * 4);
  // above 64 KB of dynamic LDS a kernel must opt in; the static arrays
  // (pair-row stages, row maps) share the 160 KB
  static std::atomic<bool> lds_opt_in[moe::kMaxDevices];
  const hipError_t e = moe::once_per_device(lds_opt_in, [] {
    const int cap = 160 * 1024 - 4 * B_STAGE - 2 * BM * 4 - 1024;
    const void* fns[4] = {(const void*)prefill_gemm_kernel<true, false>, (const void*)prefill_gemm_kernel<false, false>,
                          (const void*)prefill_gemm_kernel<true, true>, (const void*)prefill_gemm_kernel<false, true>};
    hipError_t r = hipSuccess;
    for (int i = 0; i < 4 && r == hipSuccess; ++i)
      r = hipFuncSetAttribute(fns[i], hipFuncAttributeMaxDynamicSharedMemorySize, cap);
    return r;
  });
  if (e != hipSuccess) return e;
#define MOE_PREFILL_LAUNCH(G1, CN)                                                                                 \
  prefill_gemm_kernel<G1, CN><<<grid, 256, lds, st>>>(wq, wsc, act_codes, act_scales, sorted, tile_expert, n_tiles, \
                                                      K, NT, top_k, P, rows_are_tokens, aq, as, y, out_n)
  if (gate_up) {
    if (canon) MOE_PREFILL_LAUNCH(true, true);
    else MOE_PREFILL_LAUNCH(true, false);
  } else {
    if (canon) MOE_PREFILL_LAUNCH(false, true);
    else MOE_PREFILL_LAUNCH(false, false);
  }
#undef MOE_PREFILL_LAUNCH
  return hipGetLastError();
}
