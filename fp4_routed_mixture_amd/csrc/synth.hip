// Device side of the seeded input generator (not part of the layer): fills
// packed E2M1 code bytes and E8M0 scale bytes with the SplitMix64 counter
// stream described in synth.py (Steele, Lea and Flood 2014): output i of the
// stream with key K is mix(K + (i + 1) * 0x9E3779B97F4A7C15), each output
// gives eight little-endian bytes; a scale byte is 121 + (byte mod 5).
// Used to place the 43-layer stack (about 147 GB) in HBM without a host copy.
// For the tests it also evaluates the layer's own device exp and sigmoid
// (common.h) on an array, so that their bits can be compared with the CPU
// oracle's over the whole input range.
// The same benchmark-support library holds two probes: a plain streaming read
// (the practical HBM read ceiling that the weight-streaming kernels are set
// beside) and a scaled-MFMA issue loop on random FP4 or FP8 operands with the
// shader clock read in-kernel (the matrix rate the chip sustains under that
// load).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace {

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__global__ void fill_kernel(uint64_t key, uint64_t first_word, uint64_t nwords, int scale_mode, uint64_t* __restrict__ out) {
  for (uint64_t i = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; i < nwords; i += (uint64_t)gridDim.x * blockDim.x) {
    uint64_t v = mix64(key + (first_word + i + 1) * 0x9E3779B97F4A7C15ull);
    if (scale_mode) {
      uint64_t r = 0;
#pragma unroll
      for (int b = 0; b < 8; ++b) r |= (uint64_t)(121 + ((v >> (8 * b)) & 0xFF) % 5) << (8 * b);
      v = r;
    }
    out[i] = v;
  }
}

// Every thread reads 16-byte words nontemporally in a grid-stride loop and
// folds them with xor; one word per workgroup is written so that the loads
// are kept. nwords16 = bytes / 16.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, uint64_t nwords16,
                                                          u32x4* __restrict__ sink) {
  u32x4 acc = {0, 0, 0, 0};
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  uint64_t i = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x;
  for (; i + 3 * stride < nwords16; i += 4 * stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u];
  }
  for (; i < nwords16; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  __shared__ u32x4 red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    u32x4 t = {0, 0, 0, 0};
    for (int k = 0; k < 256; ++k) t ^= red[k];
    sink[blockIdx.x] = t;
  }
}

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Eight independent accumulators per wave, each fed one
// V_MFMA_SCALE_F32_32X32X64_F8F6F4 (131,072 FLOP) per iteration on operands
// drawn from a per-lane xorshift stream, scale 1: FP8 = false, FP4 x FP4
// (random E2M1 codes in the first four dwords); FP8 = true, E4M3 x E4M3
// (codes with the top two bits cleared: exponent fields 0..7, all finite).
// Every wave records its shader-clock and 100 MHz constant-clock deltas.
template <bool FP8>
__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, uint32_t seed, float* __restrict__ out,
                                                         uint64_t* __restrict__ clocks) {
  uint32_t st = seed ^ (blockIdx.x * 256u + threadIdx.x) * 0x9E3779B9u;
  auto next = [&]() {
    st ^= st << 13;
    st ^= st >> 17;
    st ^= st << 5;
    return (int)st;
  };
  i32x8 a[2], b[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      a[u][k] = FP8 ? (next() & 0x3f3f3f3f) : (k < 4 ? next() : 0);
      b[u][k] = FP8 ? (next() & 0x3f3f3f3f) : (k < 4 ? next() : 0);
    }
  f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = (f32x16){};
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[j & 1], b[(j >> 1) & 1], acc[j], FP8 ? 0 : 4,
                                                               FP8 ? 0 : 4, 0, 127, 0, 127);
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) sum += acc[j][v];
  out[blockIdx.x * 256 + threadIdx.x] = sum;
  if ((threadIdx.x & 63) == 0) {
    const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
    clocks[2 * w] = t1 - t0;
    clocks[2 * w + 1] = r1 - r0;
  }
}

// The same probe on the fp32 matrix cores (32x32x2 f32, 4,096 FLOP an
// instruction) with random fp32 operands: magnitudes in [1, 2) with random
// mantissas and signs, as the router's products are.
__global__ __launch_bounds__(256) void mfma_probe_f32_kernel(int iters, uint32_t seed, float* __restrict__ out,
                                                             uint64_t* __restrict__ clocks) {
  uint32_t st = seed ^ (blockIdx.x * 256u + threadIdx.x) * 0x9E3779B9u;
  auto next = [&]() {
    st ^= st << 13;
    st ^= st >> 17;
    st ^= st << 5;
    return st;
  };
  float a[2], b[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    a[u] = __uint_as_float(0x3f800000u | (next() & 0x807fffffu));
    b[u] = __uint_as_float(0x3f800000u | (next() & 0x807fffffu));
  }
  f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = (f32x16){};
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j & 1], b[(j >> 1) & 1], acc[j], 0, 0, 0);
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) sum += acc[j][v];
  out[blockIdx.x * 256 + threadIdx.x] = sum;
  if ((threadIdx.x & 63) == 0) {
    const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
    clocks[2 * w] = t1 - t0;
    clocks[2 * w + 1] = r1 - r0;
  }
}

__global__ void exp_sigmoid_kernel(const float* __restrict__ z, int n, float* __restrict__ e, float* __restrict__ s) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  e[i] = moe::exp_fixed(z[i]);
  s[i] = moe::sigmoid_fixed(z[i]);
}

}  // namespace

extern "C" {

// exp_fixed and sigmoid_fixed of the layer's kernels on n values (device arrays).
int synth_exp_sigmoid(const float* z, int n, float* e, float* s, void* stream) {
  if (n < 0 || (n && (!z || !e || !s))) return 1;
  if (n == 0) return 0;
  exp_sigmoid_kernel<<<(n + 255) / 256, 256, 0, (hipStream_t)stream>>>(z, n, e, s);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// The MFMA rate probe: blocks workgroups of 4 waves, iters iterations of 8
// MFMAs per wave, FP4 (fp8 == 0) or FP8 operands. out: blocks * 256 floats;
// clocks: blocks * 4 * 2 uint64 (shader-clock and 100 MHz-clock deltas of
// each wave).
// fmt: 0 FP4 x FP4, 1 FP8 x FP8 (scaled 32x32x64), 2 fp32 (32x32x2).
int synth_mfma_probe_fmt(int blocks, int iters, int fmt, void* out, void* clocks, void* stream) {
  if (blocks < 1 || iters < 1 || !out || !clocks || fmt < 0 || fmt > 2) return 1;
  if (fmt == 2)
    mfma_probe_f32_kernel<<<blocks, 256, 0, (hipStream_t)stream>>>(iters, 0x2545F491u, (float*)out,
                                                                   (uint64_t*)clocks);
  else if (fmt == 1)
    mfma_probe_kernel<true><<<blocks, 256, 0, (hipStream_t)stream>>>(iters, 0x2545F491u, (float*)out,
                                                                    (uint64_t*)clocks);
  else
    mfma_probe_kernel<false><<<blocks, 256, 0, (hipStream_t)stream>>>(iters, 0x2545F491u, (float*)out,
                                                                     (uint64_t*)clocks);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int synth_mfma_probe(int blocks, int iters, void* out, void* clocks, void* stream) {
  return synth_mfma_probe_fmt(blocks, iters, 0, out, clocks, stream);
}

// Streaming read of nbytes (multiple of 16, 16-byte aligned) at src with
// `blocks` workgroups of 256 threads; sink receives `blocks` 16-byte words.
int synth_stream_read(const void* src, uint64_t nbytes, int blocks, void* sink, void* stream) {
  if (!src || !sink || (nbytes & 15) || ((uintptr_t)src & 15) || ((uintptr_t)sink & 15) || blocks < 1) return 1;
  stream_read_kernel<<<blocks, 256, 0, (hipStream_t)stream>>>((const u32x4*)src, nbytes / 16, (u32x4*)sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

uint64_t synth_stream_key(int seed, int layer, int tensor) {
  uint64_t z = ((uint64_t)seed << 40) | ((uint64_t)layer << 16) | (uint64_t)tensor;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Fill nbytes (multiple of 8) at dst with bytes [first_byte, first_byte + nbytes)
// of the (seed, layer, tensor) stream; scale_mode != 0 maps bytes to 121..125.
int synth_fill(int seed, int layer, int tensor, uint64_t first_byte, uint64_t nbytes, int scale_mode, void* dst,
               void* stream) {
  if ((first_byte & 7) || (nbytes & 7) || !dst || ((uintptr_t)dst & 7)) return 1;
  uint64_t nwords = nbytes / 8;
  if (!nwords) return 0;
  uint64_t blocks = (nwords + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  fill_kernel<<<(unsigned)blocks, 256, 0, (hipStream_t)stream>>>(synth_stream_key(seed, layer, tensor), first_byte / 8,
                                                                 nwords, scale_mode, (uint64_t*)dst);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
