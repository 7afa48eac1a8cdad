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
// Y[m][n] = sum_k x[m][k] w[n][k], summed by the matrix cores: measured on
// gfx950, each MFMA adds its products in groups of 8 consecutive k, every
// product truncated toward zero at 2^-13 of the group's largest exponent sum,
// and the group sums in fp32.
//
// Operand layout of a 32x32x64 FP8 MFMA: lane l holds row l % 32; its 32
// bytes are k = 16h .. 16h+15 and 32+16h .. 47+16h of the K-step (h = l / 32),
// and its E8M0 byte scales K-block h (k = 32h .. 32h+31) of that row.
//
// Batches above 32 tokens (dense_fp8_wide_kernel): a workgroup computes 256
// tokens x 256 output features with 4 waves, each 128 x 128 (4 x 4 MFMA
// tiles, 256 accumulators). The token rows (A operand) go through a
// three-slot LDS ring of two-K-step groups in the operand layout (one barrier
// a group; each wave reads the next K-step's operands while the current
// K-step's 16 MFMAs run); each wave streams its weight rows (B operand)
// straight from memory into registers two K-steps ahead. blockIdx.x is the
// output-feature block, so the workgroups that share a weight block run on
// one XCD (linear id mod 8) and find it in that XCD's L2.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace {

constexpr int WFT = 4;                     // 32-row weight tiles per wave (B operand)
constexpr int WBN = 2 * WFT * 32;          // output features of a workgroup tile (256)
constexpr int WRING = 3;                   // groups in the LDS ring
// WNU = 32-row token tiles per wave (A operand): 4 (workgroup tile 256 tokens)
// or 2 (128 tokens, for batches that would leave CUs idle)
template <int WNU>
struct WideTile {
  static constexpr int BM = 2 * WNU * 32;                // token rows of a workgroup tile
  static constexpr int SLOT = (BM / 32) * 2 * 2048;      // one group (two K-steps) of token rows, operand layout
  static constexpr int XL = BM * 128 / (16 * 256);       // 16-byte token loads per thread and group
};

template <int OA, int OB>
__device__ __forceinline__ v16f mfma88(const v8i& a, const v8i& b, v16f acc, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, OA, (int)sa, OB, (int)sb);
}

__device__ __forceinline__ uint32_t pick4(uint32_t vx, uint32_t vy, int h) {
  const uint32_t lo = h ? (vx >> 8) : vx, hi = h ? (vy >> 8) : vy;
  return (lo & 0xffu) | ((lo >> 8) & 0xff00u) | ((hi & 0xffu) << 16) | ((hi << 8) & 0xff000000u);
}

// A row's E8M0 bytes 4g .. 4g+3 hold blocks (K-step, half) of K-steps 2g and
// 2g+1; lane half h takes bytes h and 2 + h (op_sel 0 and 1): one byte
// permute with the lane's selector sel2(h) (selector byte 0x0c gives zero).
__device__ __forceinline__ uint32_t sel2(int h) { return 0x0c0c0200u + 0x0101u * (uint32_t)h; }
__device__ __forceinline__ uint32_t pick2(uint32_t d, uint32_t sel) { return __builtin_amdgcn_perm(0u, d, sel); }

template <int N>
using DIC = std::integral_constant<int, N>;

template <bool PW, int WNU>
__global__ __launch_bounds__(256, 1) void dense_fp8_wide_kernel(const uint8_t* __restrict__ xq,
                                                                const uint8_t* __restrict__ xs,
                                                                const uint8_t* __restrict__ wq,
                                                                const uint8_t* __restrict__ ws, int M, int N, int K,
                                                                float* __restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];  // WRING slots of WSLOT bytes
  constexpr int WBM = WideTile<WNU>::BM, WSLOT = WideTile<WNU>::SLOT, WXL = WideTile<WNU>::XL;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ti = wave & 1, fi = wave >> 1;  // token half, feature half of the workgroup tile
  const int c = lane & 31, h = lane >> 5;
  const int n0 = blockIdx.x * WBN + fi * (WFT * 32), m0 = blockIdx.y * WBM;
  const int rows = min(WBM, M - m0);
  const int KT = K >> 6, KB = K >> 5, NG = K >> 7;
  const uint32_t psel = sel2(h);

  // token loads: load m covers rows 32 m + tid / 8, 16-byte chunk tid % 8 of
  // the group's 128 bytes (K-step ch / 4, chunk j = ch % 4 of it), stored at
  // lane half j % 2, piece j / 2 of the operand layout
  const int r0 = tid >> 3, ch = tid & 7, kl = ch >> 2, j = ch & 3;
  const int x_dst = kl * 2048 + ((j & 1) * 32 + r0) * 32 + (j >> 1) * 16;
  const uint8_t* x_src = xq + kl * 64 + j * 16;
  // the wave's token rows (scales; rows past M read the last row, never stored)
  uint32_t xs_off[WNU];
#pragma unroll
  for (int u = 0; u < WNU; ++u) {
    const int r = ti * (WNU * 32) + u * 32 + c;
    xs_off[u] = (uint32_t)(m0 + (r < rows ? r : rows - 1)) * (uint32_t)KB;
  }
  // weights: the lane's canonical rows (tile t: + 32 t rows), or the packed
  // tiles n0 / 32 + t (K-step kt at kt * 2048, plane p at p * 1024, the
  // lane's 16 bytes at lane * 16; scale dword of four K-steps per lane)
  const int G4 = (KT + 3) >> 2;
  const uint8_t* w_row = PW ? wq + (size_t)(n0 >> 5) * KT * 2048 + lane * 16 : wq + (size_t)(n0 + c) * K + h * 16;
  const uint8_t* ws_row = PW ? ws + ((size_t)(n0 >> 5) * G4 * 64 + lane) * 4 : ws + (size_t)(n0 + c) * KB;
  const size_t w_tile = PW ? (size_t)KT * 2048 : (size_t)32 * K;
  const size_t ws_tile = PW ? (size_t)G4 * 256 : (size_t)32 * KB;

  v16f acc[WNU][WFT];
#pragma unroll
  for (int u = 0; u < WNU; ++u)
#pragma unroll
    for (int t = 0; t < WFT; ++t) acc[u][t] = (v16f){};
  v8i ra[2][WFT];   // weight operands of K-steps of parity 0 and 1
  v8i bx[2][WNU];   // token operands of the current and the next K-step
  v4i rb[WXL];      // token bytes of a future group on their way to LDS
  uint32_t sxc[WNU], swc[WFT], sxn[WNU], swn[WFT];

  auto aload = [&](int par, int kt) {
    kt = kt < KT ? kt : KT - 1;
#pragma unroll
    for (int t = 0; t < WFT; ++t) {
      const uint8_t* p = w_row + t * w_tile + (PW ? (size_t)kt * 2048 : (size_t)kt * 64);
      const v4i lo = *reinterpret_cast<const v4i*>(p);
      const v4i hi = *reinterpret_cast<const v4i*>(p + (PW ? 1024 : 32));
      ra[par][t] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  };
  auto xload = [&](int g) {
    g = g < NG ? g : NG - 1;
#pragma unroll
    for (int m = 0; m < WXL; ++m) {
      const int r = m * 32 + r0;
      const uint32_t off = (uint32_t)(m0 + (r < rows ? r : rows - 1)) * (uint32_t)K + (uint32_t)g * 128;
      rb[m] = *reinterpret_cast<const v4i*>(x_src + off);
    }
  };
  auto xstore = [&](int slot) {
#pragma unroll
    for (int m = 0; m < WXL; ++m) *reinterpret_cast<v4i*>(&lds[slot * WSLOT + x_dst + m * 4096]) = rb[m];
  };
  auto load_scales = [&](uint32_t* sx, uint32_t* sw, int g) {
    g = g < NG ? g : NG - 1;
#pragma unroll
    for (int u = 0; u < WNU; ++u) sx[u] = *reinterpret_cast<const uint32_t*>(xs + xs_off[u] + 4 * g);
#pragma unroll
    for (int t = 0; t < WFT; ++t) {
      if constexpr (PW) {  // the dword of four K-steps; the pair's half is picked at use
        sw[t] = *reinterpret_cast<const uint32_t*>(ws_row + t * ws_tile + (size_t)(g >> 1) * 256);
      } else {
        sw[t] = *reinterpret_cast<const uint32_t*>(ws_row + t * ws_tile + 4 * g);
      }
    }
  };
  auto bread = [&](int set, int slot, int k) {
#pragma unroll
    for (int u = 0; u < WNU; ++u)
      bx[set][u] = *reinterpret_cast<const v8i*>(&lds[slot * WSLOT + ((ti * WNU + u) * 2 + k) * 2048 + lane * 32]);
  };
  // (scales are picked here, not where they are loaded: an operation on a
  // just-loaded value would wait for that load within the group)
  auto kstep = [&](auto k_c, int kt_next, uint32_t wsh) {
    constexpr int k = decltype(k_c)::value;
    uint32_t sa[WNU], sb[WFT];
#pragma unroll
    for (int u = 0; u < WNU; ++u) sa[u] = pick2(sxc[u], psel);
#pragma unroll
    for (int t = 0; t < WFT; ++t) sb[t] = PW ? swc[t] >> wsh : pick2(swc[t], psel);
#pragma unroll
    for (int u = 0; u < WNU; ++u)
#pragma unroll
      for (int t = 0; t < WFT; ++t) acc[u][t] = mfma88<k, k>(bx[k][u], ra[k][t], acc[u][t], sa[u], sb[t]);
    aload(k, kt_next);
  };

  load_scales(sxc, swc, 0);
  __builtin_amdgcn_sched_barrier(0);
  aload(0, 0);
  aload(1, 1);
  xload(0);
  xstore(0);
  xload(1);
  xstore(1);
  __syncthreads();
  bread(0, 0, 0);

  int cur = 0;
  for (int g = 0; g < NG; ++g) {
    const int nxt = cur == WRING - 1 ? 0 : cur + 1;
    const int fut = nxt == WRING - 1 ? 0 : nxt + 1;
    load_scales(sxn, swn, g + 1);
    xload(g + 2);
    __builtin_amdgcn_sched_barrier(0);
    bread(1, cur, 1);
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t wsh = 16u * (uint32_t)(g & 1);  // packed weights: this group's half of the scale dword
    kstep(DIC<0>(), 2 * g + 2, wsh);
    bread(0, nxt, 0);
    __builtin_amdgcn_sched_barrier(0);
    kstep(DIC<1>(), 2 * g + 3, wsh);
    xstore(fut);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < WNU; ++u) sxc[u] = sxn[u];
#pragma unroll
    for (int t = 0; t < WFT; ++t) swc[t] = swn[t];
    cur = nxt;
  }

  // epilogue: lane l of tile (u, t) holds feature n0 + 32 t + l % 32 of rows
  // 32 u + 8 (v / 4) + 4 h + v % 4 of the wave's 128
#pragma unroll
  for (int u = 0; u < WNU; ++u)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = ti * (WNU * 32) + 32 * u + 8 * (v >> 2) + 4 * h + (v & 3);
      if (r < rows) {
        float* yr = y + (size_t)(m0 + r) * N + n0 + c;
#pragma unroll
        for (int t = 0; t < WFT; ++t) yr[32 * t] = acc[u][t][v];
      }
    }
}

// ---------------------------------------------------------------------------
// Small batches (M <= 32, the decode regime): the whole batch is one 32-row A
// tile, so the weights are read once and the kernel is bound by that stream.
// The token rows arrive operand-packed (one 32-row tile: 2 KB a K-step, one
// scale dword per lane and group of four K-steps), the weights operand-packed
// (PW) or canonical. A workgroup owns 32 output features (one B tile); its 8
// waves split the workgroup's K range into contiguous runs of 4-K-step chunks,
// each wave streaming its weight and token operands straight into registers
// one chunk ahead of the MFMAs (every load of a packed operand is 1 KB
// contiguous; no conditional inside the loop, so the next chunk's loads stay
// in flight), and the eight partial tiles are added in wave order through
// LDS. gridDim.y = S splits K across workgroups when N / 32 alone gives too
// few of them; then the workgroup sums go to part[S][M][N] and
// dense_reduce_kernel adds them in ascending s. With K % 256 == 128 the last
// two K-steps are taken by the last wave after its chunks.
// ---------------------------------------------------------------------------
constexpr int SWV = 8;  // waves per workgroup
constexpr int SCH = 4;  // K-steps per chunk

template <bool PW>
__global__ __launch_bounds__(SWV * 64) void dense_fp8_small_kernel(const uint8_t* __restrict__ xp,
                                                                   const uint8_t* __restrict__ xsp,
                                                                   const uint8_t* __restrict__ wq,
                                                                   const uint8_t* __restrict__ ws, int M, int N,
                                                                   int K, float* __restrict__ out) {
  __shared__ float red[SWV - 1][16][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, h = lane >> 5;
  const int n0 = blockIdx.x * 32, s = blockIdx.y, S = gridDim.y;
  const int KT = K >> 6, KB = K >> 5, G = (KT + 3) >> 2;
  const int C = KT / SCH, parts = SWV * S, part = s * SWV + wave;
  const int c0 = (int)((int64_t)C * part / parts), c1 = (int)((int64_t)C * (part + 1) / parts);
  // packed token tile: K-step kt at kt * 2048, lane's 16 bytes of plane p at p * 1024 + lane * 16
  const uint8_t* xl = xp + lane * 16;
  const uint32_t* xsl = reinterpret_cast<const uint32_t*>(xsp) + lane;
  // weights: packed tile blockIdx.x, or the lane's canonical row
  const uint8_t* wl = PW ? wq + (size_t)blockIdx.x * KT * 2048 + lane * 16 : wq + (size_t)(n0 + c) * K + h * 16;
  const uint8_t* wsrow = ws + (size_t)(n0 + c) * KB;
  const uint32_t* wsl = reinterpret_cast<const uint32_t*>(ws) + (size_t)blockIdx.x * G * 64 + lane;
  v16f acc = (v16f){};
  v8i xa[2][SCH], wa[2][SCH];
  uint32_t sxr[2], swr[2];  // a chunk's E8M0 bytes (one a K-step) of the lane's rows
  uint2 swc[2];             // canonical weights: the row's 8 bytes of the chunk
  auto load_step = [&](v8i& xr, v8i& wr, int kt) {
    v4i w0, w1;
    if constexpr (PW) {
      w0 = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wl + (size_t)kt * 2048));
      w1 = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wl + (size_t)kt * 2048 + 1024));
    } else {
      w0 = *reinterpret_cast<const v4i*>(wl + kt * 64);
      w1 = *reinterpret_cast<const v4i*>(wl + kt * 64 + 32);
    }
    const v4i x0 = *reinterpret_cast<const v4i*>(xl + kt * 2048);
    const v4i x1 = *reinterpret_cast<const v4i*>(xl + kt * 2048 + 1024);
    wr = (v8i){w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
    xr = (v8i){x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
  };
  auto load = [&](int buf, int ch) {
#pragma unroll
    for (int j = 0; j < SCH; ++j) load_step(xa[buf][j], wa[buf][j], ch * SCH + j);
    if constexpr (PW) swr[buf] = wsl[ch * 64];
    else swc[buf] = *reinterpret_cast<const uint2*>(wsrow + 8 * ch);
    sxr[buf] = xsl[ch * 64];
    __builtin_amdgcn_sched_barrier(0);
  };
  auto comp = [&](int buf) {
    const uint32_t sw4 = PW ? swr[buf] : pick4(swc[buf].x, swc[buf].y, h), sx4 = sxr[buf];
    acc = mfma88<0, 0>(xa[buf][0], wa[buf][0], acc, sx4, sw4);
    acc = mfma88<1, 1>(xa[buf][1], wa[buf][1], acc, sx4, sw4);
    acc = mfma88<2, 2>(xa[buf][2], wa[buf][2], acc, sx4, sw4);
    acc = mfma88<3, 3>(xa[buf][3], wa[buf][3], acc, sx4, sw4);
    __builtin_amdgcn_sched_barrier(0);
  };
  if (c1 > c0) {
    load(0, c0);
    int ch = c0;
    for (; ch + 2 <= c1; ch += 2) {
      load(1, ch + 1);
      comp(0);
      load(0, ch + 2 < c1 ? ch + 2 : c1 - 1);
      comp(1);
    }
    if (ch < c1) comp(0);
  }
  if (part == parts - 1 && C * SCH < KT) {  // the two K-steps of a last half group
    load_step(xa[0][0], wa[0][0], C * SCH);
    load_step(xa[0][1], wa[0][1], C * SCH + 1);
    const uint32_t sx4 = xsl[C * 64];
    const uint32_t sw4 = PW ? wsl[C * 64] : (uint32_t)wsrow[2 * C * SCH + h] | ((uint32_t)wsrow[2 * C * SCH + 2 + h] << 8);
    acc = mfma88<0, 0>(xa[0][0], wa[0][0], acc, sx4, sw4);
    acc = mfma88<1, 1>(xa[0][1], wa[0][1], acc, sx4, sw4);
  }
  if (wave > 0)
#pragma unroll
    for (int v = 0; v < 16; ++v) red[wave - 1][v][lane] = acc[v];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < SWV - 1; ++w)
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

// PACKED: codes and scales go to the operand-packed layout of a 32-row tile
// (rows 32 blockIdx.x / 32 ..), rows >= rows_valid get zero codes and scale
// bytes 127: element (row, k) sits in plane p = (k % 64) / 32, lane
// 32 ((k % 32) / 16) + row % 32, byte k % 16 of K-step k / 64; the E8M0 byte of
// block 2 kt + p goes to byte kt % 4 of lane (32 p + row % 32)'s dword of
// group kt / 4.
template <typename TIN, bool PACKED>
__global__ __launch_bounds__(256) void quant_mxfp8_kernel(const TIN* __restrict__ v, int K, int rows_valid,
                                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int row = blockIdx.x;
  const bool live = row < rows_valid;
  const TIN* src = v + (size_t)(live ? row : 0) * K;
  const int KT = K >> 6, G = (KT + 3) >> 2;
  for (int base = threadIdx.x * 16; base < K; base += 256 * 16) {
    float x[16];
    if (live) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if constexpr (std::is_same<TIN, float>::value) x[i] = src[base + i];
        else x[i] = moe::bf16_bits_to_f32(src[base + i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = 0.0f;
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
    if constexpr (PACKED) {
      const int kt = base >> 6, o = base & 63, pl = o >> 5, hh = (o >> 4) & 1, c = row & 31;
      const size_t tile = row >> 5;
      *reinterpret_cast<uint4*>(codes + (((tile * KT + kt) * 2 + pl) * 64 + 32 * hh + c) * 16) =
          make_uint4(w[0], w[1], w[2], w[3]);
      if (hh == 0) scales[((tile * G + (kt >> 2)) * 64 + 32 * pl + c) * 4 + (kt & 3)] = (uint8_t)(live ? e : 127);
    } else {
      *reinterpret_cast<uint4*>(codes + (size_t)row * K + base) = make_uint4(w[0], w[1], w[2], w[3]);
      if ((threadIdx.x & 1) == 0) scales[(size_t)row * (K >> 5) + (base >> 5)] = (uint8_t)e;
    }
  }
}

// Canonical <-> operand-packed layout of R rows (R % 32 == 0) x K of E4M3
// codes [R][K] and E8M0 scales [R][K/32]. Packed codes: [R/32][K/64][2][64][16]
// (tile, K-step, plane, lane, byte: row 32 tile + lane % 32, k = 64 kt +
// 32 plane + 16 (lane / 32) + byte); packed scales: [R/32][G][64] dwords
// (G = ceil(K/256)), byte j of lane l = block 2 (4 g + j) + l / 32 of row
// 32 tile + l % 32, 127 past the last K-step. Canonical rows >= rows_valid
// are read as zero codes with scale 127 when packing. One thread per 16-byte
// chunk of codes, then one per scale dword.
template <bool TO_PACKED>
__global__ __launch_bounds__(256) void dense_pack_kernel(const uint8_t* __restrict__ src_c,
                                                         const uint8_t* __restrict__ src_s, int R, int rows_valid,
                                                         int K, uint8_t* __restrict__ dst_c,
                                                         uint8_t* __restrict__ dst_s) {
  const int KT = K >> 6, G = (KT + 3) >> 2, KB = K >> 5;
  const size_t nchunks = (size_t)R * K / 16, nsc = (size_t)(R / 32) * G * 64;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < nchunks + nsc; i += (size_t)gridDim.x * 256) {
    if (i < nchunks) {
      const int l = (int)(i & 63);
      const size_t q = i >> 6;
      const int pl = (int)(q & 1);
      const size_t tk = q >> 1;
      const int kt = (int)(tk % KT);
      const size_t tile = tk / KT;
      const int row = (int)(tile * 32 + (l & 31));
      const size_t canon = (size_t)row * K + kt * 64 + 32 * pl + 16 * (l >> 5);
      if (TO_PACKED) {
        const uint4 v = row < rows_valid ? *reinterpret_cast<const uint4*>(src_c + canon) : make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(dst_c + i * 16) = v;
      } else {
        *reinterpret_cast<uint4*>(dst_c + canon) = *reinterpret_cast<const uint4*>(src_c + i * 16);
      }
    } else {
      const size_t d = i - nchunks;
      const int l = (int)(d & 63);
      const size_t tg = d >> 6;
      const int g = (int)(tg % G);
      const size_t tile = tg / G;
      const int row = (int)(tile * 32 + (l & 31));
      if (TO_PACKED) {
        uint32_t v = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kt = 4 * g + j;
          const uint32_t b = (kt < KT && row < rows_valid) ? src_s[(size_t)row * KB + 2 * kt + (l >> 5)] : 127u;
          v |= b << (8 * j);
        }
        reinterpret_cast<uint32_t*>(dst_s)[d] = v;
      } else {
        const uint32_t v = reinterpret_cast<const uint32_t*>(src_s)[d];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kt = 4 * g + j;
          if (kt < KT) dst_s[(size_t)row * KB + 2 * kt + (l >> 5)] = (uint8_t)(v >> (8 * j));
        }
      }
    }
  }
}

}  // namespace

int moe_k_dense_block_n() { return WBN; }

// Workgroups the small-batch kernel splits K over: the smallest power of two
// that gives N / 32 * S >= 128 workgroups (of 8 waves), keeping at least one
// chunk of K-steps a wave.
int moe_k_dense_split(int M, int N, int K) {
  if (M > 32) return 1;
  const int C = (K / 64) / SCH;
  int S = 1;
  while ((N / 32) * S < 128 && C / (SWV * 2 * S) >= 1) S *= 2;
  return S;
}

// Token rows of the wide kernel's workgroup tile: 256, unless 128-row tiles
// fill the 256 CUs (one workgroup each) in fewer rounds relative to the work,
// counting a 128-row workgroup as 0.6 of a 256-row one in time.
int moe_k_dense_wide_rows(int M, int N) {
  const long nb = N / WBN;
  const long w256 = nb * ((M + 255) / 256), w128 = nb * ((M + 127) / 128);
  const double t256 = (double)((w256 + 255) / 256), t128 = 0.6 * (double)((w128 + 255) / 256);
  return t128 < t256 ? 128 : 256;
}

size_t moe_k_dense_partial_bytes(int M, int N, int K) {
  const int S = moe_k_dense_split(M, N, K);
  return S > 1 ? (size_t)S * M * N * 4 : 0;
}

size_t moe_k_dense_packed_scale_bytes(int R, int K) { return (size_t)(R / 32) * ((K / 64 + 3) / 4) * 256; }

hipError_t moe_k_quant_mxfp8(int in_dtype, const void* v, int rows, int K, int packed, uint8_t* codes,
                             uint8_t* scales, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const int grid = packed ? (rows + 31) / 32 * 32 : rows;
  if (in_dtype == 0) {
    if (packed)
      quant_mxfp8_kernel<float, true><<<grid, 256, 0, st>>>((const float*)v, K, rows, codes, scales);
    else
      quant_mxfp8_kernel<float, false><<<grid, 256, 0, st>>>((const float*)v, K, rows, codes, scales);
  } else {
    if (packed)
      quant_mxfp8_kernel<uint16_t, true><<<grid, 256, 0, st>>>((const uint16_t*)v, K, rows, codes, scales);
    else
      quant_mxfp8_kernel<uint16_t, false><<<grid, 256, 0, st>>>((const uint16_t*)v, K, rows, codes, scales);
  }
  return hipGetLastError();
}

hipError_t moe_k_dense_pack(int to_packed, int R, int rows_valid, int K, const uint8_t* src_c, const uint8_t* src_s,
                            uint8_t* dst_c, uint8_t* dst_s, hipStream_t st) {
  if (R <= 0) return hipSuccess;
  const size_t work = (size_t)R * K / 16 + moe_k_dense_packed_scale_bytes(R, K) / 4;
  const unsigned blocks = (unsigned)std::min<size_t>((work + 255) / 256, 65536);
  if (to_packed)
    dense_pack_kernel<true><<<blocks, 256, 0, st>>>(src_c, src_s, R, rows_valid, K, dst_c, dst_s);
  else
    dense_pack_kernel<false><<<blocks, 256, 0, st>>>(src_c, src_s, R, rows_valid, K, dst_c, dst_s);
  return hipGetLastError();
}

hipError_t moe_k_dense_fp8_gemm(int packed_w, const uint8_t* xq, const uint8_t* xs, const uint8_t* wq,
                                const uint8_t* ws, int M, int N, int K, float* y, float* part, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  if (M <= 32) {
    const int S = moe_k_dense_split(M, N, K);
    float* o = S > 1 ? part : y;
    if (packed_w)
      dense_fp8_small_kernel<true><<<dim3(N / 32, S), SWV * 64, 0, st>>>(xq, xs, wq, ws, M, N, K, o);
    else
      dense_fp8_small_kernel<false><<<dim3(N / 32, S), SWV * 64, 0, st>>>(xq, xs, wq, ws, M, N, K, o);
    if (S > 1) {
      const int n4 = M * N / 4;
      dense_reduce_kernel<<<(n4 + 255) / 256, 256, 0, st>>>(part, S, n4, y);
    }
    return hipGetLastError();
  }
  static std::atomic<bool> lds_opt_in[moe::kMaxDevices];
  const hipError_t e = moe::once_per_device(lds_opt_in, [] {
    const void* fns[4] = {(const void*)dense_fp8_wide_kernel<true, 4>, (const void*)dense_fp8_wide_kernel<false, 4>,
                          (const void*)dense_fp8_wide_kernel<true, 2>, (const void*)dense_fp8_wide_kernel<false, 2>};
    for (int i = 0; i < 4; ++i) {
      const hipError_t r =
          hipFuncSetAttribute(fns[i], hipFuncAttributeMaxDynamicSharedMemorySize, WRING * WideTile<4>::SLOT);
      if (r != hipSuccess) return r;
    }
    return hipSuccess;
  });
  if (e != hipSuccess) return e;
  if (moe_k_dense_wide_rows(M, N) == WideTile<4>::BM) {
    const dim3 grid(N / WBN, (M + WideTile<4>::BM - 1) / WideTile<4>::BM);
    const size_t lds = WRING * WideTile<4>::SLOT;
    if (packed_w)
      dense_fp8_wide_kernel<true, 4><<<grid, 256, lds, st>>>(xq, xs, wq, ws, M, N, K, y);
    else
      dense_fp8_wide_kernel<false, 4><<<grid, 256, lds, st>>>(xq, xs, wq, ws, M, N, K, y);
  } else {
    const dim3 grid(N / WBN, (M + WideTile<2>::BM - 1) / WideTile<2>::BM);
    const size_t lds = WRING * WideTile<2>::SLOT;
    if (packed_w)
      dense_fp8_wide_kernel<true, 2><<<grid, 256, lds, st>>>(xq, xs, wq, ws, M, N, K, y);
    else
      dense_fp8_wide_kernel<false, 2><<<grid, 256, lds, st>>>(xq, xs, wq, ws, M, N, K, y);
  }
  return hipGetLastError();
}
