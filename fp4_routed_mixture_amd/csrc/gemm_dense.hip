// Block-scaled FP8 dense projection on the gfx950 scaled MFMA.
//
// The model's dense projections run in FP8 (DeepSeek-V4-Flash on AMD gfx90a:
// Correctness Recovery and Inference Performance Engineering, abstract: "FP8
// dense projections"; DeepSeek V4 Flash on 8x AMD gfx1201, What we set out to
// do: FP8 block quantization). The block layout is not on the pages; this
// library reads it as OCP MX FP8: E4M3 elements with one E8M0 scale per 32
// consecutive elements along K, for the weights W [N][K] and for the
// activations, quantized per token. gfx950 executes that format natively:
// V_MFMA_SCALE_F32_32X32X64_F8F6F4 with both operands in E4M3 and the E8M0
// bytes as its per-lane block scales, so no dequantization pass exists.
//
// Y[m][n] = sum_k x[m][k] w[n][k] (fp32 accumulation in the matrix cores).
//
// Workgroup tile: 64 token rows (two 32-row tiles, the A operand, shared by
// the 4 waves through LDS) x 256 output features (4 waves x 2 weight tiles of
// 32, the B operand, each wave's straight from memory into registers, a
// 4-K-step ring). Operand layout of a 32x32x64 FP8 MFMA: lane l holds row
// l % 32; its 32 bytes are k = 16h .. 16h+15 and 32+16h .. 47+16h of the
// K-step (h = l / 32), and its E8M0 byte scales K-block h (k = 32h .. 32h+31)
// of that row. The activation rows go through a three-group LDS ring in that
// layout (one barrier a group, the next K-step's operands read one K-step
// ahead), as in the prefill expert GEMM.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace {

constexpr int DBM = 64;                      // token rows of a workgroup tile
constexpr int DNU = DBM / 32;                // 32-row token tiles (A operand)
constexpr int DWT = 2;                       // 32-row weight tiles per wave (B operand)
constexpr int DNW = 4;                       // waves
constexpr int DBN = DNW * DWT * 32;          // output features of a workgroup tile (256)
constexpr int DPF = 4;                       // weight ring depth in K-steps
constexpr int DSTAGE = DNU * 2 * 2048;       // 64 rows x 128 K in the operand layout (8 KB)
constexpr int DRING = 3;                     // groups of stages in the LDS ring
constexpr int DNBL = DBM * 128 / (16 * DNW * 64);  // 16-byte activation loads per thread and stage (2)
static_assert(DNBL == 2, "two 16-byte pieces per thread and stage");

template <int OA, int OB>
__device__ __forceinline__ v16f mfma88(const v8i& a, const v8i& b, v16f acc, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, OA, (int)sa, OB, (int)sb);
}

__device__ __forceinline__ uint32_t pick4(uint32_t vx, uint32_t vy, int h) {
  const uint32_t lo = h ? (vx >> 8) : vx, hi = h ? (vy >> 8) : vy;
  return (lo & 0xffu) | ((lo >> 8) & 0xff00u) | ((hi & 0xffu) << 16) | ((hi << 8) & 0xff000000u);
}

// A row's E8M0 dword for group g (K-steps 4g..4g+3): bytes 8g..8g+7 hold
// blocks (step, half) = 2 step + half; lane half h takes h, h+2, h+4, h+6. A
// last group with two K-steps (K % 256 == 128) has only four bytes.
__device__ __forceinline__ uint32_t row_scale_dword(const uint8_t* row, int g, int KT, int h) {
  const uint32_t* p = reinterpret_cast<const uint32_t*>(row + 8 * g);
  return pick4(p[0], (4 * g + 2 < KT) ? p[1] : 0x7f7f7f7fu, h);
}

template <int N>
using DIC = std::integral_constant<int, N>;

template <int NUA>
__device__ __forceinline__ void dense_mainloop(const uint8_t* __restrict__ w_row, const uint8_t* __restrict__ ws_row,
                                               int w_stride, const uint8_t* __restrict__ xq, const uint32_t* b_off,
                                               int b_dst, int K, uint8_t (*lds_x)[DSTAGE], const uint32_t* lds_s,
                                               v16f (&acc)[DNU][DWT]) {
  const int lane = threadIdx.x & 63, h = lane >> 5, c = lane & 31;
  const int KT = K >> 6, G = (KT + 3) >> 2, NS = KT >> 1, KD = K >> 7;
  // weight tile t of this wave: row w_row + t * 32 * w_stride (lane row c
  // included), K-step kt: bytes kt*64 + 16h and kt*64 + 32 + 16h
  v8i ra[DPF][DWT];
  v4i rb[2][DNBL];
  v8i bx[2][DNU];  // A operands of the current and the next K-step
  uint32_t sw[DWT], nw[DWT], nx[DNU], ny[DNU], sx[DNU], nsx[DNU];
  auto aload = [&](int slot, int kt) {
    kt = kt < KT ? kt : KT - 1;
#pragma unroll
    for (int t = 0; t < DWT; ++t) {
      const uint8_t* p = w_row + (size_t)t * 32 * w_stride + kt * 64;
      const v4i lo = *reinterpret_cast<const v4i*>(p);
      const v4i hi = *reinterpret_cast<const v4i*>(p + 32);
      ra[slot][t] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  };
  auto bload = [&](int set, int st) {
    st = st < NS ? st : NS - 1;
#pragma unroll
    for (int m = 0; m < (NUA == DNU ? DNBL : 1); ++m)
      rb[set][m] = *reinterpret_cast<const v4i*>(xq + b_off[m] + (uint32_t)st * 128);
  };
  auto bstore = [&](int set, int buf) {
#pragma unroll
    for (int m = 0; m < (NUA == DNU ? DNBL : 1); ++m)
      *reinterpret_cast<v4i*>(&lds_x[buf][b_dst + m * 4096]) = rb[set][m];
  };
  auto load_wscales = [&](uint32_t* dst, int g) {
    g = g < G ? g : G - 1;
#pragma unroll
    for (int t = 0; t < DWT; ++t) dst[t] = row_scale_dword(ws_row + (size_t)t * 32 * (K >> 5), g, KT, h);
  };
  auto load_xscales = [&](int g) {
    g = g < G ? g : G - 1;
#pragma unroll
    for (int u = 0; u < NUA; ++u) {
      const uint32_t* p = lds_s + (u * 32 + c) * (KD + 1) + 2 * g;
      nx[u] = p[0];
      ny[u] = p[(4 * g + 2 < KT) ? 1 : 0];
    }
  };
  auto pick_next = [&]() {
#pragma unroll
    for (int u = 0; u < NUA; ++u) nsx[u] = pick4(nx[u], ny[u], h);
  };
  // the A operands (token rows) of K-step kl of stage buffer buf: the lane's
  // 32 bytes sit at (tile, kl) slot offset + lane * 32
  auto bread = [&](int set, int buf, int kl) {
#pragma unroll
    for (int u = 0; u < NUA; ++u) bx[set][u] = *reinterpret_cast<const v8i*>(&lds_x[buf][(u * 2 + kl) * 2048 + lane * 32]);
  };
  auto kstep = [&](auto kk_c, int kt_next, bool refill) {
    constexpr int kk = decltype(kk_c)::value;
#pragma unroll
    for (int u = 0; u < NUA; ++u)
#pragma unroll
      for (int t = 0; t < DWT; ++t) acc[u][t] = mfma88<kk, kk>(bx[kk & 1][u], ra[kk][t], acc[u][t], sx[u], sw[t]);
    if (refill) aload(kk, kt_next);
  };
  auto rotate = [&]() {
#pragma unroll
    for (int t = 0; t < DWT; ++t) sw[t] = nw[t];
#pragma unroll
    for (int u = 0; u < NUA; ++u) sx[u] = nsx[u];
  };

  load_wscales(sw, 0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < DPF; ++j) aload(j, j);
  bload(0, 0);
  bload(1, 1);
  bstore(0, 0);
  bstore(1, 1);
  bload(0, 2);
  bload(1, 3);
  bstore(0, 2);
  bstore(1, 3);
  __syncthreads();
  load_xscales(0);
  pick_next();
#pragma unroll
  for (int u = 0; u < NUA; ++u) sx[u] = nsx[u];
  bread(0, 0, 0);

  const int NG = NS >> 1;
  int cur = 0;
  for (int g = 0; g < NG; ++g) {
    const int nxt = cur == DRING - 1 ? 0 : cur + 1;
    const int fut = nxt == DRING - 1 ? 0 : nxt + 1;
    load_wscales(nw, g + 1);
    load_xscales(g + 1);
    bload(0, 2 * g + 4);
    bload(1, 2 * g + 5);
    __builtin_amdgcn_sched_barrier(0);
    bread(1, 2 * cur, 1);
    __builtin_amdgcn_sched_barrier(0);
    kstep(DIC<0>(), 4 * g + DPF, true);
    bread(0, 2 * cur + 1, 0);
    __builtin_amdgcn_sched_barrier(0);
    kstep(DIC<1>(), 4 * g + 1 + DPF, true);
    bread(1, 2 * cur + 1, 1);
    __builtin_amdgcn_sched_barrier(0);
    kstep(DIC<2>(), 4 * g + 2 + DPF, true);
    bread(0, 2 * nxt, 0);
    __builtin_amdgcn_sched_barrier(0);
    kstep(DIC<3>(), 4 * g + 3 + DPF, true);
    pick_next();
    bstore(0, 2 * fut);
    bstore(1, 2 * fut + 1);
    __syncthreads();
    rotate();
    cur = nxt;
  }
  if (NS & 1) {  // last half group (K % 256 == 128)
    bread(1, 2 * cur, 1);
    kstep(DIC<0>(), 0, false);
    kstep(DIC<1>(), 0, false);
  }
}

__global__ __launch_bounds__(256, 2) void dense_fp8_gemm_kernel(const uint8_t* __restrict__ xq,
                                                                const uint8_t* __restrict__ xs,
                                                                const uint8_t* __restrict__ wq,
                                                                const uint8_t* __restrict__ ws, int M, int N, int K,
                                                                float* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_x[2 * DRING][DSTAGE];
  extern __shared__ uint32_t lds_s[];  // token-row scales: DBM x (K/128 + 1) dwords
  const int nb = blockIdx.x, mt = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c = lane & 31, h = lane >> 5;
  const int m0 = mt * DBM;
  const int rows = min(DBM, M - m0);
  const int KD = K >> 7, KB = K >> 5;

  // activation rows: load m covers row 32 m + tid / 8 ... a stage holds 64
  // rows x 128 bytes (two K-steps); thread tid loads 16-byte chunk tid % 8 of
  // row tid / 8 (rows 0..31) and of row 32 + tid / 8; chunk j of a K-step's 64
  // bytes goes to lane half (j % 2) piece j / 2 of the operand layout
  const int r0 = tid >> 3, ch = tid & 7;
  const int kl = ch >> 2, j = ch & 3;  // K-step within the stage, 16-byte chunk within the K-step
  const int lh = j & 1, piece = j >> 1;
  const int b_dst = kl * 2048 + (lh * 32 + r0) * 32 + piece * 16;  // tile 0; tile 1 at + 4096
  uint32_t b_off[DNBL];
#pragma unroll
  for (int m = 0; m < DNBL; ++m) {
    const int r = m * 32 + r0;
    const int row = m0 + (r < rows ? r : rows - 1);  // rows past M read the last row; never stored
    b_off[m] = (uint32_t)row * (uint32_t)K + kl * 64 + j * 16;
  }
  // token-row scales into LDS rows of KD + 1 dwords
  for (int i = tid; i < DBM * KD; i += DNW * 64) {
    const int r = i / KD, d = i - r * KD;
    const int row = m0 + (r < rows ? r : rows - 1);
    lds_s[r * (KD + 1) + d] = reinterpret_cast<const uint32_t*>(xs + (size_t)row * KB)[d];
  }

  const int n_base = nb * DBN + wave * (DWT * 32);
  const uint8_t* w_row = wq + (size_t)(n_base + c) * K + h * 16;
  const uint8_t* ws_row = ws + (size_t)(n_base + c) * KB;
  v16f acc[DNU][DWT];
#pragma unroll
  for (int u = 0; u < DNU; ++u)
#pragma unroll
    for (int t = 0; t < DWT; ++t) acc[u][t] = (v16f){};
  if (rows > 32)
    dense_mainloop<DNU>(w_row, ws_row, K, xq, b_off, b_dst, K, lds_x, lds_s, acc);
  else
    dense_mainloop<1>(w_row, ws_row, K, xq, b_off, b_dst, K, lds_x, lds_s, acc);

  // epilogue: lane l of tile (u, t) holds column n = n_base + 32t + l % 32 and
  // rows m = m0 + 32u + 8(v/4) + 4h + v%4; for each v a half wave writes 128
  // contiguous bytes of one row
#pragma unroll
  for (int u = 0; u < DNU; ++u)
#pragma unroll
    for (int t = 0; t < DWT; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 32 * u + 8 * (v >> 2) + 4 * h + (v & 3);
        if (r < rows) y[(size_t)(m0 + r) * N + n_base + 32 * t + c] = acc[u][t][v];
      }
}

// ---------------------------------------------------------------------------
// Small batches (M <= 32, the decode regime): the whole batch is one 32-row A
// tile, so the weights are read once and the kernel is bound by that stream.
// A workgroup owns 32 output features (one B tile); its 4 waves split the
// workgroup's K range into contiguous quarters, each streaming its weight
// rows and token rows straight into registers through an 8-K-step ring (at
// N = K = 4096 the whole weight matrix is in flight at once), and the four
// partial tiles are added in wave order through LDS. gridDim.y = S splits K
// across workgroups when N / 32 alone gives too few of them; then the
// workgroup sums go to part[S][M][N] and dense_reduce_kernel adds them in
// ascending s.
// ---------------------------------------------------------------------------
constexpr int GPF = 8;

__global__ __launch_bounds__(256) void dense_fp8_small_kernel(const uint8_t* __restrict__ xq,
                                                              const uint8_t* __restrict__ xs,
                                                              const uint8_t* __restrict__ wq,
                                                              const uint8_t* __restrict__ ws, int M, int N, int K,
                                                              float* __restrict__ out) {
  __shared__ float red[3][16][64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c = lane & 31, h = lane >> 5;
  const int n0 = blockIdx.x * 32, s = blockIdx.y, S = gridDim.y;
  const int KT = K >> 6, KB = K >> 5;
  const int wb = (int)((int64_t)KT * s / S), we = (int)((int64_t)KT * (s + 1) / S);
  const int k0 = wb + (we - wb) * wave / 4, k1 = wb + (we - wb) * (wave + 1) / 4;
  const int xrow = c < M ? c : M - 1;  // rows past M read the last row; never stored
  const uint8_t* xp = xq + (size_t)xrow * K + h * 16;
  const uint8_t* wp = wq + (size_t)(n0 + c) * K + h * 16;
  const uint8_t* xsp = xs + (size_t)xrow * KB + h;
  const uint8_t* wsp = ws + (size_t)(n0 + c) * KB + h;
  v16f acc = (v16f){};
  if (k1 > k0) {
    v8i xa[GPF], wa[GPF];
    uint32_t sx[GPF], sw[GPF];
    auto load = [&](int j, int kt) {
      kt = kt < k1 ? kt : k1 - 1;
      const v4i wl = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wp + kt * 64));
      const v4i wh = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wp + kt * 64 + 32));
      const v4i xl = *reinterpret_cast<const v4i*>(xp + kt * 64);
      const v4i xh = *reinterpret_cast<const v4i*>(xp + kt * 64 + 32);
      wa[j] = (v8i){wl[0], wl[1], wl[2], wl[3], wh[0], wh[1], wh[2], wh[3]};
      xa[j] = (v8i){xl[0], xl[1], xl[2], xl[3], xh[0], xh[1], xh[2], xh[3]};
      sw[j] = wsp[2 * kt];
      sx[j] = xsp[2 * kt];
    };
#pragma unroll
    for (int j = 0; j < GPF; ++j) load(j, k0 + j);
    for (int kb = k0; kb < k1; kb += GPF) {
#pragma unroll
      for (int j = 0; j < GPF; ++j) {
        if (kb + j < k1) {
          acc = mfma88<0, 0>(xa[j], wa[j], acc, sx[j], sw[j]);
          load(j, kb + j + GPF);
        }
      }
    }
  }
  if (wave > 0)
#pragma unroll
    for (int v = 0; v < 16; ++v) red[wave - 1][v][lane] = acc[v];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] += red[w][v][lane];
  float* o = out + (size_t)s * M * N;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int r = 8 * (v >> 2) + 4 * h + (v & 3);
    if (r < M) o[(size_t)r * N + n0 + c] = acc[v];
  }
}

// y[i] = part[0][i] + part[1][i] + ... + part[S-1][i], four elements a thread.
__global__ __launch_bounds__(256) void dense_reduce_kernel(const float* __restrict__ part, int S, int n4,
                                                           float* __restrict__ y) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const v4f* p = reinterpret_cast<const v4f*>(part);
  v4f a = p[i];
  for (int s = 1; s < S; ++s) a += p[(size_t)s * n4 + i];
  reinterpret_cast<v4f*>(y)[i] = a;
}

// ---------------------------------------------------------------------------
// MXFP8 quantization of activation rows: one workgroup per row, 16 values a
// thread (two threads a 32-block). Scale exponent e = clamp(floor(log2 amax)
// - 8 + 127, 0, 254); each value is scaled by 2^(127 - e) (exact) and rounded
// to the nearest E4M3 value, ties to even, saturating at 448.
// ---------------------------------------------------------------------------
// Nearest-even E4M3 magnitude code of a >= 0 (finite). Below 2^-6 the grid
// is the subnormal step 2^-9 (q = rint(a * 2^9) in 0..8; 8 is the smallest
// normal, code 8); above, with E = floor(log2 a), q = rint(a * 2^(3 - E)) in
// 8..16 and the code ((E + 7) << 3) + q - 8 carries into the exponent when
// q = 16. Values from 464 (the midpoint above 448) up saturate.
__device__ __forceinline__ uint32_t e4m3_code_mag(float a) {
  if (a >= 464.0f) return 126u;
  if (a < 0x1p-6f) return (uint32_t)__builtin_rintf(a * 512.0f);
  int ex = 0;
  (void)__builtin_frexpf(a, &ex);
  const int E = ex - 1;
  const int q = (int)__builtin_rintf(__builtin_ldexpf(a, 3 - E));
  return (uint32_t)(((E + 7) << 3) + q - 8);
}

template <typename TIN>
__global__ __launch_bounds__(256) void quant_mxfp8_kernel(const TIN* __restrict__ v, int K, uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  const int row = blockIdx.x;
  const TIN* src = v + (size_t)row * K;
  for (int base = threadIdx.x * 16; base < K; base += 256 * 16) {
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if constexpr (std::is_same<TIN, float>::value) x[i] = src[base + i];
      else x[i] = moe::bf16_bits_to_f32(src[base + i]);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));  // the block's other half
    int e = 0;
    if (amax > 0.0f) {
      int ex = 0;
      (void)__builtin_frexpf(amax, &ex);
      e = (ex - 1) - 8 + 127;
      e = e < 0 ? 0 : (e > 254 ? 254 : e);
    }
    uint32_t w[4] = {0, 0, 0, 0};
    if (amax > 0.0f) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float vs = __builtin_ldexpf(x[i], 127 - e);
        const uint32_t code = e4m3_code_mag(fabsf(vs)) | ((__float_as_uint(vs) >> 31) << 7);
        w[i >> 2] |= code << (8 * (i & 3));
      }
    }
    *reinterpret_cast<uint4*>(codes + (size_t)row * K + base) = make_uint4(w[0], w[1], w[2], w[3]);
    if ((threadIdx.x & 1) == 0) scales[(size_t)row * (K >> 5) + (base >> 5)] = (uint8_t)e;
  }
}

}  // namespace

int moe_k_dense_block_n() { return DBN; }

// Workgroups the small-batch kernel splits K over: the smallest power of two
// that gives N / 32 * S >= 256 workgroups, keeping at least two K-steps a wave.
int moe_k_dense_split(int M, int N, int K) {
  if (M > 32) return 1;
  int S = 1;
  while ((N / 32) * S < 256 && (K / 64) / (4 * 2 * S) >= 2) S *= 2;
  return S;
}

size_t moe_k_dense_partial_bytes(int M, int N, int K) {
  const int S = moe_k_dense_split(M, N, K);
  return S > 1 ? (size_t)S * M * N * 4 : 0;
}

hipError_t moe_k_quant_mxfp8(int in_dtype, const void* v, int rows, int K, uint8_t* codes, uint8_t* scales,
                             hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (in_dtype == 0)
    quant_mxfp8_kernel<float><<<rows, 256, 0, st>>>((const float*)v, K, codes, scales);
  else
    quant_mxfp8_kernel<uint16_t><<<rows, 256, 0, st>>>((const uint16_t*)v, K, codes, scales);
  return hipGetLastError();
}

hipError_t moe_k_dense_fp8_gemm(const uint8_t* xq, const uint8_t* xs, const uint8_t* wq, const uint8_t* ws, int M,
                                int N, int K, float* y, float* part, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  if (M <= 32) {
    const int S = moe_k_dense_split(M, N, K);
    dense_fp8_small_kernel<<<dim3(N / 32, S), 256, 0, st>>>(xq, xs, wq, ws, M, N, K, S > 1 ? part : y);
    if (S > 1) {
      const int n4 = M * N / 4;
      dense_reduce_kernel<<<(n4 + 255) / 256, 256, 0, st>>>(part, S, n4, y);
    }
    return hipGetLastError();
  }
  dim3 grid(N / DBN, (M + DBM - 1) / DBM);
  const size_t lds = (size_t)DBM * (K / 128 + 1) * 4;
  static std::atomic<bool> lds_opt_in[moe::kMaxDevices];
  const hipError_t e = moe::once_per_device(lds_opt_in, [] {
    return hipFuncSetAttribute((const void*)dense_fp8_gemm_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                               160 * 1024 - 2 * DRING * DSTAGE - 1024);
  });
  if (e != hipSuccess) return e;
  dense_fp8_gemm_kernel<<<grid, 256, lds, st>>>(xq, xs, wq, ws, M, N, K, y);
  return hipGetLastError();
}
