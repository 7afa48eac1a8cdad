// Shared device helpers for the gfx950 routed-MoE kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

#define MOE_WAVE 64

namespace moe {

// Host: run set() once for each device it is called on (the attributes that
// let a kernel use more than 64 KB of LDS belong to the device current when
// they are set). done: one flag per device id. Concurrent first calls on a
// device may both run set(), which only repeats the same settings.
constexpr int kMaxDevices = 64;
template <typename F>
inline hipError_t once_per_device(std::atomic<bool>* done, F set) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (done[dev].load(std::memory_order_acquire)) return hipSuccess;
  e = set();
  if (e == hipSuccess) done[dev].store(true, std::memory_order_release);
  return e;
}

// ---------------------------------------------------------------------------
// fp32 exp and sigmoid built from IEEE operations only, so the same bits come
// out of every conforming implementation: n = rint(z log2 e); r = z - n ln2
// with ln 2 split in two (Cody-Waite; the high part has 15 significant bits so
// n * hi is exact for |n| <= 256); exp(r) by its degree-7 Taylor polynomial in
// Horner form with fused multiply-adds; then scaling by 2^n with ldexp.
// Inputs above the largest z with a finite result give +inf, inputs below
// ln(2^-150) give 0.
// ---------------------------------------------------------------------------
// The polynomial path is evaluated for every input and the out-of-range
// results are selected afterwards (no branches: the three range tests as
// branches cost more than the polynomial). For z outside the range the
// evaluated value is discarded, so the result is the same for every input.
__device__ __forceinline__ float exp_fixed(float z) {
  const float kLog2e = 0x1.715476p+0f;
  const float kLn2Hi = 0x1.62e4p-1f;
  const float kLn2Lo = 0x1.7f7d1cp-20f;
  const float zc = __builtin_fminf(__builtin_fmaxf(z, -0x1.9fe36ap+6f), 0x1.62e42ep+6f);  // keeps n in range
  float n = __builtin_rintf(zc * kLog2e);
  float r = __builtin_fmaf(-n, kLn2Hi, zc);
  r = __builtin_fmaf(-n, kLn2Lo, r);
  float p = 0x1.a01a02p-13f;                 // 1/7!
  p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f);  // 1/6!
  p = __builtin_fmaf(p, r, 0x1.111112p-7f);   // 1/5!
  p = __builtin_fmaf(p, r, 0x1.555556p-5f);   // 1/4!
  p = __builtin_fmaf(p, r, 0x1.555556p-3f);   // 1/3!
  p = __builtin_fmaf(p, r, 0.5f);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  float e = __builtin_ldexpf(p, (int)n);
  e = z > 0x1.62e42ep+6f ? __builtin_inff() : e;
  e = z < -0x1.9fe36ap+6f ? 0.0f : e;
  return z != z ? z : e;
}

// IEEE division (hipcc lowers '/' on fp32 to the correctly rounded sequence;
// the library is built without fast-math and with contraction off).
__device__ __forceinline__ float sigmoid_fixed(float z) { return 1.0f / (1.0f + exp_fixed(-z)); }

// ---------------------------------------------------------------------------
// E2M1 (OCP MX v1.0): nearest-even rounding of |v| (already divided by the
// block scale) onto {0, .5, 1, 1.5, 2, 3, 4, 6}, saturating at 6. Decision
// points are the midpoints; at a midpoint the code with mantissa bit 0 wins.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e2m1_mag_code(float a) {
  uint32_t c;
  if (a <= 0.25f) c = 0;        // 0.25 -> 0 (even)
  else if (a < 0.75f) c = 1;    // (0.25, 0.75) -> 0.5
  else if (a <= 1.25f) c = 2;   // [0.75, 1.25] -> 1 (0.75 and 1.25 tie to 1)
  else if (a < 1.75f) c = 3;    // -> 1.5
  else if (a <= 2.5f) c = 4;    // [1.75, 2.5] -> 2
  else if (a < 3.5f) c = 5;     // -> 3
  else if (a <= 5.0f) c = 6;    // [3.5, 5] -> 4
  else c = 7;                   // -> 6 (saturating)
  return c;
}

// Shared E8M0 exponent of an MXFP4 block with maximum magnitude amax > 0:
// floor(log2 amax) - 2 + 127, clamped to [0, 254]. floor(log2) is read from
// the fp32 exponent field (frexp semantics), with subnormal amax normalized.
__device__ __forceinline__ int mx_scale_exp(float amax) {
  int ex = 0;
  float m = __builtin_frexpf(amax, &ex);  // amax = m * 2^ex, m in [0.5, 1)
  (void)m;
  int e = (ex - 1) - 2 + 127;
  return e < 0 ? 0 : (e > 254 ? 254 : e);
}

// One MXFP4 block: 32 values with block exponent e (amax > 0) -> 16 bytes of
// E2M1 codes, value 2i in the low nibble of byte i. gfx950's scaled FP4 pack
// conversion divides by the power-of-two scale 2^(e-127) and rounds as the
// OCP rule above does (nearest-even, saturating at 6, sign kept: checked bit
// for bit against e2m1_mag_code on 2^21 values including every midpoint);
// scales outside its normal range take the compare ladder.
__device__ __forceinline__ uint4 mx_pack32(const float* v, int e) {
  uint32_t w[4];
  if (e >= 2 && e <= 252) {
    const float scale = __uint_as_float((uint32_t)e << 23);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[8 * i], v[8 * i + 1], scale, 0);
      p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[8 * i + 2], v[8 * i + 3], scale, 1);
      p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[8 * i + 4], v[8 * i + 5], scale, 2);
      p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[8 * i + 6], v[8 * i + 7], scale, 3);
      w[i] = p;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float vs = __builtin_ldexpf(v[i], 127 - e);
      const uint32_t c = e2m1_mag_code(fabsf(vs)) | ((__float_as_uint(vs) >> 31) << 3);
      w[i / 8] |= c << ((i % 8) * 4);
    }
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// int8 in [-8, 8] -> OCP FP8 E4M3 bit pattern (exact). For 1 <= a <= 8 the
// fp32 encoding of a has exponent field 127 + e and a mantissa whose top
// three bits are E4M3's mantissa; E4M3 wants exponent field 7 + e, so the
// code is (fp32 bits >> 20) - (120 << 3). Pure ALU: a lookup table would be
// read from memory on every call.
__device__ __forceinline__ uint32_t small_int_to_e4m3(int v) {
  const uint32_t a = (uint32_t)(v < 0 ? -v : v);
  const uint32_t mag = a ? (__float_as_uint((float)a) >> 20) - 960u : 0u;
  return (v < 0 ? 0x80u : 0u) | mag;
}

// Split an int8 value q in [-127, 127] into hi, lo with q = 16 * hi + lo,
// lo in [-8, 7], hi in [-8, 8]: both are exact in FP8 E4M3.
__device__ __forceinline__ void split_int8(int q, int& hi, int& lo) {
  lo = ((q + 8) & 15) - 8;
  hi = (q - lo) >> 4;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

}  // namespace moe

// Scaled MFMA wrappers (gfx950). Formats: 4 = FP4 E2M1, 0 = FP8 E4M3.
// Operand layout (32x32x64): lane l holds row/col (l % 32); for FP4 its 32
// elements are k = (l/32)*32 + i (byte i/2, low nibble first); for FP8 its
// first 16 bytes are k = (l/32)*16 + i and its last 16 are k = 32 + (l/32)*16 + i.
// The E8M0 scale byte of a lane (selected by OPSEL) scales block (l/32) of
// row/col (l % 32). Result: lane l, element v -> column l % 32,
// row 8*(v/4) + 4*(l/32) + (v%4).
#define MFMA_FP4_FP4(a, b, c, opa, sa, opb, sb) \
  __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4((a), (b), (c), 4, 4, (opa), (sa), (opb), (sb))
#define MFMA_FP4_FP8(a, b, c, opa, sa, opb, sb) \
  __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4((a), (b), (c), 4, 0, (opa), (sa), (opb), (sb))
