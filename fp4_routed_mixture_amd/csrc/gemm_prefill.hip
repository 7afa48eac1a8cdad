// Large-M (prefill) grouped expert GEMMs on the gfx950 scaled FP4 MFMA.
//
// The pages accelerate prefill with MFMA kernels and better reuse of the
// packed weights (abstract of "DeepSeek-V4-Flash on AMD gfx90a: Correctness
// Recovery and Inference Performance Engineering"). Here both operands are
// MXFP4 (E2M1 codes + E8M0 per 32) and go to V_MFMA_SCALE_F32_32X32X64_F8F6F4
// unchanged: weights are A (32-row tiles), pair rows are B (32 columns).
//
// Workgroup tile: up to BM = 128 pair rows -- two consecutive 64-row sort
// tiles of one expert, or one when the expert has no second tile left (a
// half tile, which skips the MFMAs and loads of the missing half), from the
// sort's list of such wide tiles, so that no workgroup of the grid is empty
// (a grid over single tiles whose odd ones exit at once left a third of the
// workgroup slots unfilled) -- against
// 4 waves x WTW = 2 weight tiles of 32 rows (one gate/up tile pair of W13, or
// two row tiles of W2). Each wave keeps 2 x 4 = 8 accumulators (half the
// accumulation registers), so two workgroups share a CU and one's prologue
// and epilogue (SiLU, requantization, stores) run under the other's MFMAs.
// A weight tile feeds four pair tiles: 256 bytes of weights per MFMA, half
// of what two pair tiles need, and the weight stream through the vector
// memory path is what bounds these kernels.
//
// Weight tiles are used by one wave only, so they go from memory straight
// into the MFMA operand registers: the prepacked layout stores each 64-K step
// of a tile as 64 lanes x 16 bytes, one fully coalesced load per tile and
// K-step, kept PF K-steps ahead in a register ring. The gathered pair rows are
// shared by the 4 waves and go through LDS in the operand layout, in a ring of
// three four-K-step groups: the rows of group g + 2 are loaded during group g
// and stored at its end, so one barrier per group suffices and the operands
// of the next K-step (even across the barrier) are read from LDS one K-step
// ahead of their MFMAs.
//
// Scale dwords (four K-steps each) are loaded one group ahead; the MFMA's
// byte select picks the K-step. The main loop has no branch between a load
// and its consumer, so the compiler's memory-counter waits stay partial;
// prefetches past the end re-read the last step (cache hits) instead.
// Launch order: blockIdx.x = weight block, so the tiles of one expert for one
// weight block land on the same XCD and share its L2.
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

constexpr int SUB = 64;                 // rows of a sort tile (the sort's block_m)
constexpr int NU = 4;                   // 32-row pair tiles of a full workgroup tile
constexpr int BM = 32 * NU;             // pair rows of a full workgroup tile (two sort tiles)
constexpr int WTW = 2;                  // 32-row weight tiles per wave
constexpr int NWAVE = 4;
constexpr int PF = 4;                   // weight prefetch depth in 64-K steps (one scale group)
constexpr int B_STAGE = NU * 2 * 1024;  // BM pair rows x 128 K, operand layout
constexpr int RING = 3;                 // groups of pair-row stages in the LDS ring
constexpr int NBL = BM * 4 / (NWAVE * 64);  // 16-byte pair-row loads per thread and stage (2)
static_assert(NBL == 2, "one load per sort tile and stage per thread");

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

// The tile's pair-row scales (KD dwords a row) into LDS rows of KD + 1
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

template <int N>
using IC = std::integral_constant<int, N>;

// Everything the main loop of one workgroup tile needs; the loop is a
// template on the number of active pair tiles (4, or 2 for a half tile).
template <bool GATE_UP, bool CANON>
struct Tile {
  const uint8_t* a_base;       // lane's weight byte base
  const uint32_t* sa_base;     // lane's prepacked scale dword base
  const uint8_t* sa_canon;     // lane's canonical scale row base
  const uint8_t* act_codes;
  uint32_t b_off[NBL];         // this thread's pair-row byte offsets (+ chunk)
  int b_dst;                   // its LDS destination within a stage
  int K, KT, G, NS, KD, KB, NR, ubase, h, c;
};

template <bool GATE_UP, bool CANON, int NUA>
__device__ __forceinline__ void mainloop(const Tile<GATE_UP, CANON>& tl, uint8_t (*lds_b)[B_STAGE],
                                         const uint32_t* lds_s, v16f (&acc)[WTW][NU]) {
  const int lane = threadIdx.x & 63, h = tl.h, c = tl.c;
  const int KT = tl.KT, G = tl.G, NS = tl.NS, KD = tl.KD;
  // tile t of this wave: W13 t = 0 gate, 1 up of pair ubase; W2 row tile ubase + t
  auto a_ptr = [&](int t, int kt) {
    const uint32_t off =
        CANON ? (GATE_UP ? (uint32_t)(t * (tl.NR >> 1) + tl.ubase * 32) : (uint32_t)((tl.ubase + t) * 32)) *
                        (uint32_t)(tl.K >> 1) +
                    (uint32_t)kt * 32
              : GATE_UP ? (uint32_t)t * 1024 + (uint32_t)kt * 2048 : (uint32_t)t * KT * 1024 + (uint32_t)kt * 1024;
    return reinterpret_cast<const v4i*>(tl.a_base + off);
  };
  v4i ra[PF][WTW];     // weight ring: slot = K-step % PF
  v4i rb[2][NBL];      // pair rows of the stages of group g + 2
  v4i bv[2][NU];       // operands of the current and the next K-step
  // weight scale dwords (this and the next group), the pair-row scale bytes
  // of the next group as read from LDS, and the B scale dwords of this and
  // the next group (the byte select picks the K-step)
  uint32_t sa[WTW], na[WTW], nx[NU], ny[NU], sb[NU], nsb[NU];

  auto aload = [&](int slot, int kt) {
    kt = kt < KT ? kt : KT - 1;
#pragma unroll
    for (int t = 0; t < WTW; ++t) ra[slot][t] = *a_ptr(t, kt);
  };
  auto bload = [&](int set, int st) {
    st = st < NS ? st : NS - 1;
#pragma unroll
    for (int m = 0; m < (NUA == NU ? NBL : 1); ++m)
      rb[set][m] = *reinterpret_cast<const v4i*>(tl.act_codes + tl.b_off[m] + (uint32_t)st * 64);
  };
  auto bstore = [&](int set, int buf) {
#pragma unroll
    for (int m = 0; m < (NUA == NU ? NBL : 1); ++m)
      *reinterpret_cast<v4i*>(&lds_b[buf][tl.b_dst + m * 4096]) = rb[set][m];
  };
  auto load_wscales = [&](uint32_t* da, int g) {
    g = g < G ? g : G - 1;
#pragma unroll
    for (int t = 0; t < WTW; ++t) {
      if (CANON) {
        const uint32_t row = GATE_UP ? (uint32_t)(t * (tl.NR >> 1) + tl.ubase * 32) : (uint32_t)((tl.ubase + t) * 32);
        da[t] = canon_row_scales(tl.sa_canon + row * (uint32_t)tl.KB, g, KT, h);
      } else {
        // W13: (pair * G + g) * 128 + half * 64; W2: (tile * G + g) * 64
        const uint32_t idx = GATE_UP ? (uint32_t)g * 128 + t * 64 : ((uint32_t)t * G + g) * 64;
        da[t] = tl.sa_base[idx];
      }
    }
  };
  auto load_rscales = [&](uint32_t* dx, uint32_t* dy, int g) {
    g = g < G ? g : G - 1;
#pragma unroll
    for (int u = 0; u < NUA; ++u) {
      // a group's 8 bytes; when K % 256 == 128 the last group has only 2
      // K-steps and its second dword is never selected (re-read the first)
      const uint32_t* p = lds_s + (u * 32 + c) * (KD + 1) + 2 * g;
      dx[u] = p[0];
      dy[u] = p[(4 * g + 2 < KT) ? 1 : 0];
    }
  };
  // the operands of K-step kl (0 or 1) of stage buffer buf
  auto bread = [&](int set, int buf, int kl) {
#pragma unroll
    for (int u = 0; u < NUA; ++u) bv[set][u] = *reinterpret_cast<const v4i*>(&lds_b[buf][(u * 2 + kl) * 1024 + lane * 16]);
  };
  // K-step kk (0..3) of a group: MFMAs on bv[kk & 1], weight slot kk, scale
  // byte kk; then the slot is refilled with K-step kt_next
  auto kstep = [&](auto kk_c, int kt_next, bool refill) {
    constexpr int kk = decltype(kk_c)::value;
#pragma unroll
    for (int t = 0; t < WTW; ++t)
#pragma unroll
      for (int u = 0; u < NUA; ++u) acc[t][u] = mfma44<kk, kk>(ra[kk][t], bv[kk & 1][u], acc[t][u], sa[t], sb[u]);
    if (refill) aload(kk, kt_next);
  };
  // the next group's B scale dwords, built once per group after its last
  // MFMAs are issued (the LDS reads of its bytes were issued at the group's
  // start), then both sets rotate in
  auto pick_next = [&]() {
#pragma unroll
    for (int u = 0; u < NUA; ++u) nsb[u] = pick_scales(nx[u], ny[u], h);
  };
  auto rotate_scales = [&]() {
#pragma unroll
    for (int t = 0; t < WTW; ++t) sa[t] = na[t];
#pragma unroll
    for (int u = 0; u < NUA; ++u) sb[u] = nsb[u];
  };

  // prologue: the weight scales of group 0 first (so that on entering the
  // loop they are older than every weight and pair-row load, and the loop's
  // wait for the previous group's scales stays partial on both of its
  // paths), then K-steps 0..PF-1 of the weights and the stages of groups 0
  // and 1 (ring slots 0 and 1); the barrier also publishes the row scales
  load_wscales(sa, 0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < PF; ++j) aload(j, j);
  bload(0, 0);
  bload(1, 1);
  bstore(0, 0);
  bstore(1, 1);
  bload(0, 2);
  bload(1, 3);
  bstore(0, 2);
  bstore(1, 3);
  __syncthreads();
  load_rscales(nx, ny, 0);
  pick_next();
#pragma unroll
  for (int u = 0; u < NUA; ++u) sb[u] = nsb[u];
  bread(0, 0, 0);

  // group g = K-steps 4g..4g+3 = stages 2g, 2g+1 in ring slot g % 3 (LDS
  // buffers 2 (g % 3), +1). During group g the stages of group g + 2 are
  // loaded and, after the group's last MFMAs, stored into slot (g + 2) % 3,
  // last read in group g - 1, before the barrier that ended it; the one
  // barrier of the group publishes them for group g + 2. The operands of the
  // next K-step are read before the current K-step's MFMAs are issued.
  const int NG = NS >> 1;  // full groups
  int cur = 0;
  for (int g = 0; g < NG; ++g) {
    const int nxt = cur == RING - 1 ? 0 : cur + 1;
    const int fut = nxt == RING - 1 ? 0 : nxt + 1;
    load_wscales(na, g + 1);
    load_rscales(nx, ny, g + 1);
    bload(0, 2 * g + 4);
    bload(1, 2 * g + 5);
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetches ahead of the MFMAs
    // Each K-step's operand reads are issued before the previous K-step's
    // MFMAs; the scheduling barriers keep the compiler from sinking them to
    // their own MFMAs (where it would share the two operand sets' registers
    // and expose every LDS read's latency).
    bread(1, 2 * cur, 1);
    __builtin_amdgcn_sched_barrier(0);
    kstep(IC<0>(), 4 * g + PF, true);
    bread(0, 2 * cur + 1, 0);
    __builtin_amdgcn_sched_barrier(0);
    kstep(IC<1>(), 4 * g + 1 + PF, true);
    bread(1, 2 * cur + 1, 1);
    __builtin_amdgcn_sched_barrier(0);
    kstep(IC<2>(), 4 * g + 2 + PF, true);
    bread(0, 2 * nxt, 0);  // group g + 1, published by the barrier that ended group g - 1
    __builtin_amdgcn_sched_barrier(0);
    kstep(IC<3>(), 4 * g + 3 + PF, true);
    pick_next();
    bstore(0, 2 * fut);
    bstore(1, 2 * fut + 1);
    __syncthreads();
    rotate_scales();
    cur = nxt;
  }
  if (NS & 1) {  // last half group (K % 256 == 128): K-steps 4 NG, 4 NG + 1
    bread(1, 2 * cur, 1);
    kstep(IC<0>(), 0, false);
    kstep(IC<1>(), 0, false);
  }
}

template <bool GATE_UP, bool CANON>
__global__ __launch_bounds__(256, 2) void prefill_gemm_kernel(
    const uint8_t* __restrict__ wq, const uint8_t* __restrict__ wsc, const uint8_t* __restrict__ act_codes,
    const uint8_t* __restrict__ act_scales, const int32_t* __restrict__ sorted,
    const int32_t* __restrict__ tile_expert, const int32_t* __restrict__ wide, const int32_t* __restrict__ n_wide,
    int K, int NT, int top_k, int P, int rows_are_tokens, uint8_t* __restrict__ aq, uint8_t* __restrict__ as,
    float* __restrict__ y, int out_n) {
  constexpr int S = GATE_UP ? 2 : 1;  // 32-row tiles per NT unit (gate/up pair or one W2 tile)
  constexpr int UPW = WTW / S;        // NT units per wave
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2 * RING][B_STAGE];
  extern __shared__ uint32_t lds_s[];  // pair-row scales (BM x (K/128 + 1) dwords), later the y staging
  __shared__ int lds_row[BM];
  __shared__ int lds_pair[BM];
  const int nb = blockIdx.x, wi = blockIdx.y;
  // Wide tile wi: sort tile q and, if the sort paired it, tile q + 1 of the
  // same expert (the grid covers the bound on the list's length; the
  // entries past n_wide are never read).
  if (wi >= *n_wide) return;
  const int wt = wide[wi];
  const int q = wt >> 1, nsub = 1 + (wt & 1);
  const int e = tile_expert[q];
  const int rows = nsub * SUB;
  const int p0 = q * SUB;  // sorted position of the tile's first row
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c = lane & 31, h = lane >> 5;

  Tile<GATE_UP, CANON> tl;
  tl.K = K;
  tl.KT = K >> 6;
  tl.G = (tl.KT + 3) >> 2;
  tl.KB = K >> 5;
  tl.NS = tl.KT >> 1;  // stages of 128 K (K % 128 == 0)
  tl.KD = K >> 7;      // scale dwords per row
  tl.h = h;
  tl.c = c;
  tl.act_codes = act_codes;

  // ---- this wave's weight tiles (NT % UPW == 0: all valid or none) ----------
  const int unit0 = (nb * NWAVE + wave) * UPW;
  const bool w_valid = unit0 < NT;
  tl.ubase = w_valid ? unit0 : 0;  // invalid waves compute a real block and store nothing
  tl.NR = GATE_UP ? NT * 64 : NT * 32;
  tl.a_base = CANON ? wq + ((size_t)e * tl.NR + c) * (K >> 1) + h * 16
                    : wq + ((size_t)e * NT + tl.ubase) * tl.KT * (S * 1024) + lane * 16;
  tl.sa_base = reinterpret_cast<const uint32_t*>(wsc + ((size_t)e * NT + tl.ubase) * tl.G * (S * 256)) + lane;
  tl.sa_canon = wsc + ((size_t)e * tl.NR + c) * tl.KB;

  // ---- gathered pair rows: load m covers row 64 m + tid / 4, 16-byte chunk
  // tid % 4 of a stage's 64 bytes (rows past the tile read row 0) ------------
  const int c4 = tid & 3;
  tl.b_dst = (((tid >> 2) >> 5) * 2 + (c4 >> 1)) * 1024 + ((c4 & 1) * 32 + ((tid >> 2) & 31)) * 16;
  if (tid < BM) {
    const int pr = tid < rows ? sorted[p0 + tid] : P;
    lds_row[tid] = pr < P ? (rows_are_tokens ? pr / top_k : p0 + tid) : 0;  // padding reads row 0
    lds_pair[tid] = pr;
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < NBL; ++m) tl.b_off[m] = (uint32_t)lds_row[m * 64 + (tid >> 2)] * (uint32_t)(K >> 1) + c4 * 16;
  // The pair rows' E8M0 scales (K/32 bytes a row) are staged in LDS once:
  // read in the main loop straight from global memory, every lane would
  // touch its own cache line per load (one gathered row per lane). Row
  // stride K/128 + 1 dwords keeps the per-lane reads on distinct banks.
  stage_row_scales(act_scales, lds_row, rows, tl.KD, tl.KB, NWAVE * 64, lds_s);

  v16f acc[WTW][NU];
#pragma unroll
  for (int t = 0; t < WTW; ++t)
#pragma unroll
    for (int u = 0; u < NU; ++u) acc[t][u] = (v16f){};
  if (nsub == 2)
    mainloop<GATE_UP, CANON, NU>(tl, lds_b, lds_s, acc);
  else
    mainloop<GATE_UP, CANON, NU / 2>(tl, lds_b, lds_s, acc);
  const int nua = nsub * 2;  // active pair tiles

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
      if (u >= nua) break;
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
  const int I = out_n;
  const int jp = unit0;  // this wave's gate/up tile pair = 32-block of I
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    if (u >= nua) break;
    const int r = u * 32 + c;
    const int p = p0 + r;
    if (lds_pair[r] >= P) continue;  // lanes l and l^32 share the row, hence the validity
    float av[16];
    float amax = 0.0f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float gg = acc[0][u][v], uu = acc[1][u][v];
      av[v] = (gg * moe::sigmoid_fixed(gg)) * uu;
      amax = fmaxf(amax, fabsf(av[v]));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
    const int ex = amax > 0.0f ? moe::mx_scale_exp(amax) : 0;
    uint8_t* dst = aq + (size_t)p * (I >> 1) + (size_t)jp * 16;
    // gfx950's scaled FP4 pack conversion divides by the (power-of-two)
    // scale and rounds to nearest-even on the E2M1 grid with saturation at 6
    // and the sign kept -- the OCP rule, checked bit for bit against the
    // software encoder below on 2^21 values including every midpoint. Scales
    // that would be denormal or near the exponent limits take the software
    // path.
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
      // rows 8i + 4h .. +3 are bytes 4i + 2h, 4i + 2h + 1 of the block: the
      // lane with h = 0 gathers its partner's half into one dword
      const uint32_t other = (uint32_t)__shfl_xor((int)packed[i], 32, 64);
      word[i] = (packed[i] & 0xffffu) | (other << 16);
    }
    if (h == 0) {
      *reinterpret_cast<uint4*>(dst) = make_uint4(word[0], word[1], word[2], word[3]);
      as[(size_t)p * (I >> 5) + jp] = (uint8_t)ex;
    }
  }
}

}  // namespace

int moe_k_prefill_block_m() { return SUB; }

hipError_t moe_k_prefill_gemm(int gate_up, int canon, const uint8_t* wq, const uint8_t* wsc, const uint8_t* act_codes,
                              const uint8_t* act_scales, const int32_t* sorted, const int32_t* tile_expert,
                              const int32_t* wide, const int32_t* n_wide, int max_wide, int K, int NT, int top_k,
                              int P, int rows_are_tokens, uint8_t* aq, uint8_t* as, float* y, int out_n,
                              hipStream_t st) {
  if (max_wide <= 0) return hipSuccess;
  // NT: tile pairs (W13) or row tiles (W2); a workgroup covers 4 pairs / 8 tiles
  const int per_wg = NWAVE * (gate_up ? WTW / 2 : WTW);
  dim3 grid((NT + per_wg - 1) / per_wg, max_wide);
  // dynamic LDS: the pair-row scales, or the down GEMM's y staging (4 waves
  // x 32 rows x 36 floats), whichever is larger
  const size_t lds = std::max<size_t>((size_t)BM * (K / 128 + 1) * 4, gate_up ? 0 : (size_t)NWAVE * 32 * 36 * 4);
  // above 64 KB of dynamic LDS a kernel must opt in; the static arrays
  // (pair-row stages, row maps) share the 160 KB
  static std::atomic<bool> lds_opt_in[moe::kMaxDevices];
  const hipError_t e = moe::once_per_device(lds_opt_in, [] {
    const int cap = 160 * 1024 - 2 * RING * B_STAGE - 2 * BM * 4 - 1024;
    const void* fns[4] = {(const void*)prefill_gemm_kernel<true, false>, (const void*)prefill_gemm_kernel<false, false>,
                          (const void*)prefill_gemm_kernel<true, true>, (const void*)prefill_gemm_kernel<false, true>};
    hipError_t r = hipSuccess;
    for (int i = 0; i < 4 && r == hipSuccess; ++i)
      r = hipFuncSetAttribute(fns[i], hipFuncAttributeMaxDynamicSharedMemorySize, cap);
    return r;
  });
  if (e != hipSuccess) return e;
#define MOE_PREFILL_LAUNCH(G1, CN)                                                                                  \
  prefill_gemm_kernel<G1, CN><<<grid, 256, lds, st>>>(wq, wsc, act_codes, act_scales, sorted, tile_expert, wide, \
                                                      n_wide, K, NT, top_k, P, rows_are_tokens, aq, as, y, out_n)
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
