// Low-M (decode) expert GEMMs: packed E2M1 weights x int8 activations.
//
// The CDNA2 decode kernel of DeepSeek-V4-Flash on AMD gfx90a: Correctness
// Recovery and Inference Performance Engineering (abstract) multiplies int8
// activations with dot-product instructions; on gfx950 the FP4
// operand goes to the scaled MFMA unchanged, so there is no format mismatch:
// each int8 activation q is given to the FP4 x FP8 scaled MFMA as the exact
// pair q = 16*hi + lo (hi, lo small integers in E4M3), the hi columns carrying
// an E8M0 scale of 2^4. Every product and partial sum is then an exactly
// representable dyadic rational, so the block-scaled sum is exact and equals
// the integer block sums of the definition.
//
// Work item: (two 32-row weight tiles -- a gate/up tile pair of W13, or two
// consecutive row tiles of W2 --, sort tile q of 16 pairs of one expert). B columns 0..15 are the hi parts of
// the 16 pair rows, 16..31 the lo parts. The four waves of a workgroup split
// K into contiguous ranges of four-K-tile groups and reduce through LDS in a
// fixed order. Weights stream straight from HBM into MFMA registers: the
// prepacked layout makes each wave's load of a 32x64 tile one contiguous
// 1 KB (16 B per lane), loaded non-temporally (each weight byte is used by
// one workgroup only).
//
// Weights are read in either layout: the prepacked one (each wave's load of
// a 32x64 tile is one contiguous 1 KB) or the canonical row-major one, where
// lane l reads 16 bytes of row l % 32 at K offset (l / 32) * 32 of each
// K-step (32 rows x 32 bytes a load, a 128-byte line per row over a group of
// four K-steps) and picks its four scale bytes out of the row's eight bytes
// for the group.
//
// Epilogues write plain fp32 results; the steps that need whole rows or all
// of a token's pairs run as separate small kernels after the kernel boundary:
//   gate/up: a = (g * sigmoid(g)) * u into a[pos][I]  (then requant_rows)
//   down   : y[pair][H] = s_a * sum                    (then the combine)
// Handing the data to another workgroup inside the kernel would need
// device-coherent stores and a counter per tile, and every workgroup would
// wait for its stores to complete while holding its CU: measured slower than
// the two extra launches.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int DM = 16;  // pair rows per sort tile

template <int U>
__device__ __forceinline__ v16f mfma_fp4_fp8(const v4i& a, const v8i& b, v16f acc, uint32_t sa, uint32_t sb) {
  v8i a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  return MFMA_FP4_FP8(a8, b, acc, U, (int)sa, 0, (int)sb);
}

constexpr int NW = 4;  // waves per workgroup (K split)

template <int S>
struct Group {
  v4i a0[4], a1[4];
  v8i b[4];
  uint32_t sa0, sa1;
};

// Prepacked tiles are read once, nontemporally. A canonical row is read in
// 32-byte pieces, four K-steps to a 128-byte line: plain loads keep the line
// for the next pieces (nontemporal ones measured slower there).
template <bool CANON>
__device__ __forceinline__ v4i ld_weights(const uint8_t* p) {
  if constexpr (CANON) return *reinterpret_cast<const v4i*>(p);
  else return __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p));
}

// The scale dword of a canonical row for K-step group g (K-steps 4g..4g+3):
// the row's E8M0 bytes 8g..8g+7 hold blocks (step, half) = 2 step + half, so
// lane half h takes bytes h, h+2, h+4, h+6. A last group with two K-steps
// (K % 256 == 128) reads only its four bytes and gives the missing steps
// scale 1 (their operands are zero).
__device__ __forceinline__ uint32_t canon_scale_dword(const uint8_t* row_scales, int g, int KT, int h) {
  const uint32_t* p = reinterpret_cast<const uint32_t*>(row_scales + 8 * g);
  const uint32_t lo = p[0], hi = (4 * g + 2 < KT) ? p[1] : 0x7f7f7f7fu;
  const uint32_t a = h ? (lo >> 8) : lo, b = h ? (hi >> 8) : hi;
  return (a & 0xffu) | ((a >> 8) & 0xff00u) | ((b & 0xffu) << 16) | ((b << 8) & 0xff000000u);
}

// S = 2: a second 32-row tile, the up half of a W13 tile pair (interleaved
// per K-step: a_step = 2048, a1 at +1024, scales at +64 dwords) or the next
// W2 row tile (a_step = 1024, a1 at +KT*1024, scales at +G*64 dwords).
// CANON: aptr / sptr are the lane's canonical code row (+ 16 h) and scale
// row; a_step = 32, a1_off / s1_off the distance to the second row in bytes.
template <int S, bool CANON>
__device__ __forceinline__ void load_group(Group<S>& G, const uint8_t* aptr, const uint32_t* sptr, const uint8_t* bptr,
                                           bool valid, int g, int KT, uint32_t a_step, uint32_t a1_off,
                                           uint32_t s_step, uint32_t s1_off) {
  if (CANON) {
    const uint8_t* srow = reinterpret_cast<const uint8_t*>(sptr);
    const int h = (threadIdx.x >> 5) & 1;
    G.sa0 = canon_scale_dword(srow, g, KT, h);
    G.sa1 = S == 2 ? canon_scale_dword(srow + s1_off, g, KT, h) : 0u;
  } else {
    G.sa0 = sptr[(size_t)g * s_step];
    G.sa1 = S == 2 ? sptr[(size_t)g * s_step + s1_off] : 0u;
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int kt = g * 4 + u;
    G.a0[u] = (v4i){0, 0, 0, 0};
    G.a1[u] = (v4i){0, 0, 0, 0};
    G.b[u] = (v8i){0, 0, 0, 0, 0, 0, 0, 0};
    if (kt < KT) {
      G.a0[u] = ld_weights<CANON>(aptr + (size_t)kt * a_step);
      if (S == 2) G.a1[u] = ld_weights<CANON>(aptr + (size_t)kt * a_step + a1_off);
      if (valid) {
        const v4i lo = *reinterpret_cast<const v4i*>(bptr + (size_t)kt * 64);
        const v4i hi = *reinterpret_cast<const v4i*>(bptr + (size_t)kt * 64 + 32);
        G.b[u] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    }
  }
}

template <int S>
__device__ __forceinline__ void mma_group(const Group<S>& G, v16f& acc0, v16f& acc1, uint32_t sb) {
  // padded K-tiles (kt >= KT) carry zero operands: they add exactly 0
  acc0 = mfma_fp4_fp8<0>(G.a0[0], G.b[0], acc0, G.sa0, sb);
  acc0 = mfma_fp4_fp8<1>(G.a0[1], G.b[1], acc0, G.sa0, sb);
  acc0 = mfma_fp4_fp8<2>(G.a0[2], G.b[2], acc0, G.sa0, sb);
  acc0 = mfma_fp4_fp8<3>(G.a0[3], G.b[3], acc0, G.sa0, sb);
  if (S == 2) {
    acc1 = mfma_fp4_fp8<0>(G.a1[0], G.b[0], acc1, G.sa1, sb);
    acc1 = mfma_fp4_fp8<1>(G.a1[1], G.b[1], acc1, G.sa1, sb);
    acc1 = mfma_fp4_fp8<2>(G.a1[2], G.b[2], acc1, G.sa1, sb);
    acc1 = mfma_fp4_fp8<3>(G.a1[3], G.b[3], acc1, G.sa1, sb);
  }
}

// Main loop + cross-wave reduction. On return red[w][s][v][lane] holds every
// wave's partial sums (read by the epilogue after __syncthreads()).
// PAIRED: the two tiles are a W13 gate/up pair (tile pair j of NT pairs);
// otherwise S tiles S*j .. S*j+S-1 of the NT row tiles of W2.
template <int S, bool PAIRED, bool CANON>
__device__ __forceinline__ void decode_mainloop(const uint8_t* __restrict__ wq, const uint8_t* __restrict__ wsc,
                                                const uint8_t* __restrict__ act8, int row, bool valid, int part, int e,
                                                int j, int K, int NT, float (*red)[S][16][64]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int KT = K >> 6, G = (KT + 3) >> 2;
  const int h = lane >> 5;
  const uint8_t* bptr = act8 + ((size_t)row * 2 + part) * K + h * 16;
  const uint32_t sb = part ? 0x7f7f7f7fu : 0x83838383u;  // lo: 2^0, hi: 2^4
  constexpr int TS = PAIRED ? 2 : 1;  // 32-row tiles per NT unit
  const uint8_t* aptr;
  const uint32_t* sptr;
  uint32_t a_step, a1_off, s_step, s1_off;
  if (CANON) {
    // rows: W13 gate j*32 + c and up I + j*32 + c (N = 2I = 64 NT);
    // W2 (2j)*32 + c and (2j+1)*32 + c (N = 32 NT)
    const int N = PAIRED ? NT * 64 : NT * 32, c = lane & 31;
    const int r0 = (PAIRED ? j : S * j) * 32 + c;
    const int dr = PAIRED ? N / 2 : 32;
    aptr = wq + ((size_t)e * N + r0) * (K >> 1) + h * 16;
    sptr = reinterpret_cast<const uint32_t*>(wsc + ((size_t)e * N + r0) * (K >> 5));
    a_step = 32;
    a1_off = (uint32_t)dr * (K >> 1);
    s_step = 0;
    s1_off = (uint32_t)dr * (K >> 5);
  } else {
    const size_t tile = (size_t)e * NT + (PAIRED ? j : (size_t)S * j);
    aptr = wq + tile * KT * (TS * 1024) + lane * 16;
    sptr = reinterpret_cast<const uint32_t*>(wsc + tile * G * (TS * 256)) + lane;
    a_step = TS * 1024;
    a1_off = PAIRED ? 1024u : (uint32_t)KT * 1024;
    s_step = TS * 64;
    s1_off = PAIRED ? 64u : (uint32_t)G * 64;
  }
  const int g0 = (G * wave) / NW, g1 = (G * (wave + 1)) / NW;
  v16f acc0 = {}, acc1 = {};
  for (int g = g0; g < g1; ++g) {
    Group<S> cur;
    load_group<S, CANON>(cur, aptr, sptr, bptr, valid, g, KT, a_step, a1_off, s_step, s1_off);
    mma_group<S>(cur, acc0, acc1, sb);
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    red[wave][0][v][lane] = acc0[v];
    if (S == 2) red[wave][S - 1][v][lane] = acc1[v];
  }
  __syncthreads();
}

// Sum over waves (fixed order) of hi and lo columns for lane l (hi column,
// l % 32 < 16), element v.
template <int S>
__device__ __forceinline__ float reduced(float (*red)[S][16][64], int s, int v, int l) {
  float t = 0.0f;
#pragma unroll
  for (int w = 0; w < NW; ++w) t = t + (red[w][s][v][l] + red[w][s][v][l + 16]);
  return t;
}

template <bool CANON>
__global__ __launch_bounds__(64 * NW) void decode_gate_up_kernel(
    const uint8_t* __restrict__ wq, const uint8_t* __restrict__ wsc, const uint8_t* __restrict__ x8,
    const float* __restrict__ xs, const int32_t* __restrict__ sorted, const int32_t* __restrict__ tile_expert,
    const int32_t* __restrict__ n_tiles, int K, int NT, int top_k, int P, float* __restrict__ a, int I) {
  __shared__ float red[NW][2][16][64];
  const int j = blockIdx.x, q = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int c = lane & 31, part = c >> 4;
  // The tile count, the tile's expert and its pair ids are loaded together
  // (q < max_tiles: within both arrays, whose entries past n_tiles are never
  // used), and the pair row's scale before the main loop: every index load
  // waited for in turn would delay the start of the weight stream.
  const int nt = *n_tiles;
  const int e = tile_expert[q];
  const int pair = sorted[q * DM + (c & 15)];
  // (an empty asm reading the three values: otherwise the compiler sinks the
  // second and third load below the exit test and waits for each in turn)
  asm volatile("" ::"s"(nt), "s"(e), "v"(pair));
  if (q >= nt) return;
  const bool valid = pair < P;
  const int row = valid ? pair / top_k : 0;
  const float s = xs[row];
  decode_mainloop<2, true, CANON>(wq, wsc, x8, row, valid, part, e, j, K, NT, red);

  // a = (g * sigmoid(g)) * u for the hi-column lanes' rows (lane l: sort row
  // q DM + l % 16, the pair loaded above)
  const int l = lane, vq = threadIdx.x >> 6;
  if ((l & 31) >= 16 || !valid) return;
  const int op = q * DM + (l & 15);
  float* arow = a + (size_t)op * I + j * 32;
#pragma unroll
  for (int vv = 0; vv < 4; ++vv) {
    const int v = vq * 4 + vv;
    const float gg = s * reduced<2>(red, 0, v, l), uu = s * reduced<2>(red, 1, v, l);
    arow[8 * (v >> 2) + 4 * (l >> 5) + (v & 3)] = (gg * moe::sigmoid_fixed(gg)) * uu;
  }
}

template <bool CANON>
__global__ __launch_bounds__(64 * NW) void decode_down_kernel(
    const uint8_t* __restrict__ wq, const uint8_t* __restrict__ wsc, const uint8_t* __restrict__ aq8,
    const float* __restrict__ as, const int32_t* __restrict__ sorted, const int32_t* __restrict__ tile_expert,
    const int32_t* __restrict__ n_tiles, int K, int NT, int top_k, int P, float* __restrict__ y, int H) {
  __shared__ float red[NW][2][16][64];
  const int j = blockIdx.x, q = blockIdx.y;  // j: pair of row tiles 2j, 2j+1
  const int lane = threadIdx.x & 63;
  const int c = lane & 31, part = c >> 4;
  const int p = q * DM + (c & 15);
  // loaded together, as in the gate/up kernel (q < max_tiles, p < capacity)
  const int nt = *n_tiles;
  const int e = tile_expert[q];
  const int pair = sorted[p];
  const float s = as[p];
  asm volatile("" ::"s"(nt), "s"(e), "v"(pair), "v"(s));
  if (q >= nt) return;
  const bool valid = pair < P;
  decode_mainloop<2, false, CANON>(wq, wsc, aq8, p, valid, part, e, j, K, NT, red);

  const int l = lane, vq = threadIdx.x >> 6;
  if ((l & 31) >= 16 || !valid) return;  // lane l: sort row p, its pair above
  float* yrow = y + (size_t)pair * H + j * 64;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int vv = 0; vv < 4; ++vv) {
      const int v = vq * 4 + vv;
      yrow[t * 32 + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3)] = s * reduced<2>(red, t, v, l);
    }
}

// int8 requantization of the activation rows of the valid pairs: one
// 256-thread workgroup per pair i (its row p = pos[i] in sort order), each
// thread holds I/256 values (loads issued together), s = amax / 127,
// q = clamp(rint(a / s), +-127) stored as FP8 hi/lo planes [2][I].
__global__ __launch_bounds__(256) void requant_rows_kernel(const float* __restrict__ a, int I,
                                                           const int32_t* __restrict__ pos,
                                                           uint8_t* __restrict__ aq8, float* __restrict__ as) {
  __shared__ float red[4];
  const int p = pos[blockIdx.x], tid = threadIdx.x;
  const float* arow = a + (size_t)p * I;
  const int nu = I >> 10;  // four-element units per thread (I % 1024 == 0), else fallback below
  float v[4][4];
  float amax = 0.f;
  if (nu >= 1 && nu <= 4 && (I & 1023) == 0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float4 t = *reinterpret_cast<const float4*>(arow + ((size_t)min(u, nu - 1) * 256 + tid) * 4);
      v[u][0] = t.x; v[u][1] = t.y; v[u][2] = t.z; v[u][3] = t.w;
#pragma unroll
      for (int m = 0; m < 4; ++m) amax = fmaxf(amax, fabsf(v[u][m]));
    }
  } else {
    for (int i = tid; i < I; i += 256) amax = fmaxf(amax, fabsf(arow[i]));
  }
  amax = moe::wave_max(amax);
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = amax / 127.0f;
  if (tid == 0) as[p] = s;
  uint8_t* dst = aq8 + (size_t)p * 2 * I;
  auto quant1 = [&](float x) -> int {
    float qq = 0.f;
    if (amax != 0.f) qq = fminf(fmaxf(__builtin_rintf(x / s), -127.f), 127.f);
    return (int)qq;
  };
  if (nu >= 1 && nu <= 4 && (I & 1023) == 0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (u >= nu) break;
      uint32_t hw = 0, lw = 0;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        int hi, lo;
        moe::split_int8(quant1(v[u][m]), hi, lo);
        hw |= moe::small_int_to_e4m3(hi) << (8 * m);
        lw |= moe::small_int_to_e4m3(lo) << (8 * m);
      }
      const size_t i = ((size_t)u * 256 + tid) * 4;
      *reinterpret_cast<uint32_t*>(dst + i) = hw;
      *reinterpret_cast<uint32_t*>(dst + I + i) = lw;
    }
  } else {
    for (int i = tid; i < I; i += 256) {
      int hi, lo;
      moe::split_int8(quant1(arow[i]), hi, lo);
      dst[i] = (uint8_t)moe::small_int_to_e4m3(hi);
      dst[I + i] = (uint8_t)moe::small_int_to_e4m3(lo);
    }
  }
}

}  // namespace

int moe_k_decode_block_m() { return DM; }

hipError_t moe_k_decode_gate_up(int canon, const uint8_t* wq, const uint8_t* wsc, const uint8_t* x8, const float* xs,
                                const int32_t* sorted, const int32_t* tile_expert, const int32_t* n_tiles,
                                int max_tiles, int H, int I, int top_k, int P, float* a, hipStream_t st) {
  if (max_tiles <= 0) return hipSuccess;
  dim3 grid(I / 32, max_tiles);
  if (canon)
    decode_gate_up_kernel<true><<<grid, 64 * NW, 0, st>>>(wq, wsc, x8, xs, sorted, tile_expert, n_tiles, H, I / 32,
                                                          top_k, P, a, I);
  else
    decode_gate_up_kernel<false><<<grid, 64 * NW, 0, st>>>(wq, wsc, x8, xs, sorted, tile_expert, n_tiles, H, I / 32,
                                                           top_k, P, a, I);
  return hipGetLastError();
}

hipError_t moe_k_requant_rows(const float* a, int I, const int32_t* pos, int P, uint8_t* aq8, float* as,
                              hipStream_t st) {
  if (P <= 0) return hipSuccess;
  requant_rows_kernel<<<P, 256, 0, st>>>(a, I, pos, aq8, as);
  return hipGetLastError();
}

hipError_t moe_k_decode_down(int canon, const uint8_t* wq, const uint8_t* wsc, const uint8_t* aq8, const float* as,
                             const int32_t* sorted, const int32_t* tile_expert, const int32_t* n_tiles, int max_tiles,
                             int H, int I, int top_k, int P, float* y, hipStream_t st) {
  if (max_tiles <= 0) return hipSuccess;
  dim3 grid(H / 64, max_tiles);  // two 32-row tiles per workgroup (H % 256 == 0)
  if (canon)
    decode_down_kernel<true><<<grid, 64 * NW, 0, st>>>(wq, wsc, aq8, as, sorted, tile_expert, n_tiles, I, H / 32,
                                                       top_k, P, y, H);
  else
    decode_down_kernel<false><<<grid, 64 * NW, 0, st>>>(wq, wsc, aq8, as, sorted, tile_expert, n_tiles, I, H / 32,
                                                        top_k, P, y, H);
  return hipGetLastError();
}
