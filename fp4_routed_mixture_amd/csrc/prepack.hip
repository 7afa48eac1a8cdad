// Load-time relayout of packed FP4 expert weights into the operand order of
// the gfx950 32x32x64 scaled MFMA; it also carries the load-time layout
// repair of DeepSeek-V4-Flash on AMD gfx90a: Correctness Recovery and
// Inference Performance Engineering (abstract).
//
// Canonical layout: codes [E][N][K/2] (low nibble = even k), E8M0 scales
// [E][N][K/32].
// Prepacked layout (NT = N/32 row tiles, or I/32 gate/up tile pairs for W13;
// KT = K/64; G = ceil(KT/4)):
//   codes : [E][NT][KT][S][64 lanes][16 B]      S = 2 for W13 (gate, up), 1 for W2
//           lane l holds row (tile row base + l%32), k = kt*64 + (l/32)*32 .. +32,
//           i.e. 16 consecutive canonical bytes.
//   scales: [E][NT][G][S][64 lanes][4 B]
//           byte q of lane l = scale of (row, k-block 2*(4g+q) + l/32); 127 where
//           4g+q >= KT.
// For W13 tile pair j covers gate rows j*32.. and up rows I + j*32.. .
// Both directions are a bijection on bytes (apart from the scale padding).
#include "common.h"
#include "kernels.h"

namespace {

struct PackGeom {
  int E, N, K, S, NT, KT, G, rows_half;  // rows_half: I for W13, unused for W2
};

__device__ __forceinline__ int canon_row(const PackGeom& g, int j, int s, int l) {
  // row in canonical order for tile (pair) j, sub-matrix s, lane l
  return (g.S == 2 ? s * g.rows_half : 0) + j * 32 + (l & 31);
}

// One thread per 16-byte chunk of packed codes.
__global__ void pack_codes_kernel(PackGeom g, const uint8_t* __restrict__ src, const int32_t* __restrict__ perm,
                                  uint8_t* __restrict__ dst, int to_packed) {
  size_t chunks = (size_t)g.E * g.N * (g.K / 32);  // 16 B = 32 codes per chunk
  for (size_t c = blockIdx.x * (size_t)blockDim.x + threadIdx.x; c < chunks; c += (size_t)gridDim.x * blockDim.x) {
    // decompose packed chunk index: [e][j][kt][s][l]
    size_t t = c;
    int l = t % 64; t /= 64;
    int s = t % g.S; t /= g.S;
    int kt = t % g.KT; t /= g.KT;
    int j = t % g.NT; t /= g.NT;
    int e = (int)t;
    int r = canon_row(g, j, s, l);
    int k0 = kt * 64 + (l / 32) * 32;
    size_t canon = ((size_t)e * g.N + r) * (g.K / 2) + k0 / 2;
    const uint4* ps;
    uint4* pd;
    if (to_packed) {
      int rs = perm ? perm[r] : r;
      size_t csrc = ((size_t)e * g.N + rs) * (g.K / 2) + k0 / 2;
      ps = reinterpret_cast<const uint4*>(src + csrc);
      pd = reinterpret_cast<uint4*>(dst + c * 16);
    } else {
      ps = reinterpret_cast<const uint4*>(src + c * 16);
      pd = reinterpret_cast<uint4*>(dst + canon);
    }
    *pd = *ps;
  }
}

// One thread per packed scale dword.
__global__ void pack_scales_kernel(PackGeom g, const uint8_t* __restrict__ src, const int32_t* __restrict__ perm,
                                   uint8_t* __restrict__ dst, int to_packed) {
  size_t words = (size_t)g.E * g.NT * g.G * g.S * 64;
  int KB = g.K / 32;
  for (size_t w = blockIdx.x * (size_t)blockDim.x + threadIdx.x; w < words; w += (size_t)gridDim.x * blockDim.x) {
    size_t t = w;
    int l = t % 64; t /= 64;
    int s = t % g.S; t /= g.S;
    int gi = t % g.G; t /= g.G;
    int j = t % g.NT; t /= g.NT;
    int e = (int)t;
    int r = canon_row(g, j, s, l);
    if (to_packed) {
      int rs = perm ? perm[r] : r;
      uint32_t word = 0;
      for (int q = 0; q < 4; ++q) {
        int kt = gi * 4 + q;
        uint32_t b = 127;
        if (kt < g.KT) b = src[((size_t)e * g.N + rs) * KB + kt * 2 + (l / 32)];
        word |= b << (8 * q);
      }
      reinterpret_cast<uint32_t*>(dst)[w] = word;
    } else {
      uint32_t word = reinterpret_cast<const uint32_t*>(src)[w];
      for (int q = 0; q < 4; ++q) {
        int kt = gi * 4 + q;
        if (kt < g.KT) dst[((size_t)e * g.N + r) * KB + kt * 2 + (l / 32)] = (uint8_t)(word >> (8 * q));
      }
    }
  }
}

PackGeom geom(int which, int E, int N, int K) {
  PackGeom g;
  g.E = E; g.N = N; g.K = K;
  g.S = which == 0 ? 2 : 1;
  g.rows_half = which == 0 ? N / 2 : 0;
  g.NT = which == 0 ? (N / 2) / 32 : N / 32;
  g.KT = K / 64;
  g.G = (g.KT + 3) / 4;
  return g;
}

}  // namespace

size_t moe_k_packed_scale_bytes(int which, int E, int N, int K) {
  PackGeom g = geom(which, E, N, K);
  return (size_t)g.E * g.NT * g.G * g.S * 64 * 4;
}

static int grid_for(size_t n) { size_t b = (n + 255) / 256; return (int)(b < 65536 ? (b ? b : 1) : 65536); }

hipError_t moe_k_pack(int which, int E, int N, int K, const uint8_t* codes, const uint8_t* scales,
                      const int32_t* perm, uint8_t* pcodes, uint8_t* pscales, hipStream_t st) {
  PackGeom g = geom(which, E, N, K);
  pack_codes_kernel<<<grid_for((size_t)E * N * (K / 32)), 256, 0, st>>>(g, codes, perm, pcodes, 1);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  pack_scales_kernel<<<grid_for((size_t)g.E * g.NT * g.G * g.S * 64), 256, 0, st>>>(g, scales, perm, pscales, 1);
  return hipGetLastError();
}

hipError_t moe_k_unpack(int which, int E, int N, int K, const uint8_t* pcodes, const uint8_t* pscales,
                        uint8_t* codes, uint8_t* scales, hipStream_t st) {
  PackGeom g = geom(which, E, N, K);
  pack_codes_kernel<<<grid_for((size_t)E * N * (K / 32)), 256, 0, st>>>(g, pcodes, nullptr, codes, 0);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  pack_scales_kernel<<<grid_for((size_t)g.E * g.NT * g.G * g.S * 64), 256, 0, st>>>(g, pscales, nullptr, scales, 0);
  return hipGetLastError();
}
