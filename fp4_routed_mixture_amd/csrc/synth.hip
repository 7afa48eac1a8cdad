// Device side of the seeded input generator (not part of the layer): fills
// packed E2M1 code bytes and E8M0 scale bytes with the SplitMix64 counter
// stream described in synth.py (Steele, Lea and Flood 2014): output i of the
// stream with key K is mix(K + (i + 1) * 0x9E3779B97F4A7C15), each output
// gives eight little-endian bytes; a scale byte is 121 + (byte mod 5).
// Used to place the 43-layer stack (about 147 GB) in HBM without a host copy.
// The same benchmark-support library holds a plain streaming-read probe, the
// practical HBM read ceiling that the weight-streaming kernels are set beside.
#include <hip/hip_runtime.h>
#include <stdint.h>

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

}  // namespace

extern "C" {

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
