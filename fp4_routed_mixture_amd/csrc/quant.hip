// Activation quantization (int8 rows as in the decode path of DeepSeek-V4-
// Flash on AMD gfx90a: Correctness Recovery and Inference Performance
// Engineering, abstract; MXFP4 per the OCP Microscaling v1.0 rules).
//
// int8 rows: s = amax / 127, q = clamp(rint(v / s), -127, 127); amax = 0 gives
// s = 0, q = 0. Besides plain int8 output, the forward path stores each q as
// the exact FP8 E4M3 pair (hi, lo) with q = 16*hi + lo, which is how the
// decode GEMM feeds int8 activations to the FP4 x FP8 scaled MFMA: layout
// [row][2][K] (hi plane, then lo plane).
// MXFP4 blocks of 32: e = clamp(floor(log2 amax) - 2 + 127, 0, 254); codes are
// nearest-even E2M1 of v * 2^(127 - e), saturated at 6, sign from the sign bit.
#include "common.h"
#include "kernels.h"

namespace {

template <typename XT>
__device__ __forceinline__ float ld(const XT* p, size_t i);
template <>
__device__ __forceinline__ float ld<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p, size_t i) { return moe::bf16_bits_to_f32(p[i]); }

// One 256-thread workgroup per row. OUT: 0 = int8 [row][K]; 1 = FP8 hi/lo
// planes [row][2][K]. If sorted != nullptr rows are padded sort positions and
// rows whose pair is the sentinel (>= P) are skipped; rows beyond *n_rows
// (device) are skipped.
template <typename XT, int OUT>
__global__ __launch_bounds__(256) void quant_int8_kernel(const XT* __restrict__ v, int K, void* __restrict__ q,
                                                         float* __restrict__ scales, const int32_t* __restrict__ sorted,
                                                         int P, const int32_t* __restrict__ n_rows) {
  const int row = blockIdx.x;
  if (n_rows && row >= *n_rows) return;
  if (sorted && sorted[row] >= P) return;
  const XT* src = v + (size_t)row * K;
  __shared__ float red[4];
  float amax = 0.0f;
  for (int i = threadIdx.x; i < K; i += 256) amax = fmaxf(amax, fabsf(ld<XT>(src, i)));
  amax = moe::wave_max(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = amax / 127.0f;
  if (threadIdx.x == 0) scales[row] = s;
  for (int i = threadIdx.x; i < K; i += 256) {
    float qq = 0.0f;
    if (amax != 0.0f) {
      qq = __builtin_rintf(ld<XT>(src, i) / s);
      qq = fminf(fmaxf(qq, -127.0f), 127.0f);
    }
    int qi = (int)qq;
    if (OUT == 0) {
      reinterpret_cast<int8_t*>(q)[(size_t)row * K + i] = (int8_t)qi;
    } else {
      int hi, lo;
      moe::split_int8(qi, hi, lo);
      uint8_t* d = reinterpret_cast<uint8_t*>(q) + (size_t)row * 2 * K;
      d[i] = (uint8_t)moe::small_int_to_e4m3(hi);
      d[K + i] = (uint8_t)moe::small_int_to_e4m3(lo);
    }
  }
}

// One thread per block of 32 values.
template <typename XT>
__global__ __launch_bounds__(256) void quant_mxfp4_kernel(const XT* __restrict__ v, int rows, int K,
                                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const size_t nb = (size_t)rows * (K / 32);
  for (size_t b = blockIdx.x * (size_t)blockDim.x + threadIdx.x; b < nb; b += (size_t)gridDim.x * blockDim.x) {
    const XT* src = v + b * 32;
    float x[32];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      x[i] = ld<XT>(src, i);
      amax = fmaxf(amax, fabsf(x[i]));
    }
    int e = amax > 0.0f ? moe::mx_scale_exp(amax) : 0;
    *reinterpret_cast<uint4*>(codes + b * 16) = amax > 0.0f ? moe::mx_pack32(x, e) : make_uint4(0, 0, 0, 0);
    scales[b] = (uint8_t)e;
  }
}

// Decode FP8 hi/lo planes back to int8 rows, gathered by pair order.
__global__ void fp8pair_to_int8_kernel(const uint8_t* __restrict__ src, const float* __restrict__ src_s, int K,
                                       const int32_t* __restrict__ row_of, int nrows, int8_t* __restrict__ q,
                                       float* __restrict__ s) {
  const int r = blockIdx.x;
  if (r >= nrows) return;
  const int sr = row_of ? row_of[r] : r;
  const uint8_t* hi = src + (size_t)sr * 2 * K;
  const uint8_t* lo = hi + K;
  for (int i = threadIdx.x; i < K; i += blockDim.x) {
    auto dec = [](uint32_t b) -> int {
      if ((b & 0x7f) == 0) return 0;
      int e = (b >> 3) & 15, m = b & 7;
      int mag = ((8 + m) << e) >> 10;  // (1 + m/8) * 2^(e-7), integer for e >= 7
      return (b & 0x80) ? -mag : mag;
    };
    q[(size_t)r * K + i] = (int8_t)(16 * dec(hi[i]) + dec(lo[i]));
  }
  if (threadIdx.x == 0) s[r] = src_s[sr];
}

__global__ void gather_rows_kernel(const uint8_t* __restrict__ src, int row_bytes, const int32_t* __restrict__ row_of,
                                   int nrows, uint8_t* __restrict__ dst) {
  const int r = blockIdx.x;
  if (r >= nrows) return;
  const uint8_t* s = src + (size_t)row_of[r] * row_bytes;
  for (int i = threadIdx.x; i < row_bytes; i += blockDim.x) dst[(size_t)r * row_bytes + i] = s[i];
}

int grid_for(size_t n) {
  size_t b = (n + 255) / 256;
  return (int)(b < 65536 ? (b ? b : 1) : 65536);
}

}  // namespace

hipError_t moe_k_quant_int8(int in_dtype, const void* v, int rows, int K, int out_fp8pair, void* q, float* scales,
                            const int32_t* sorted, int P, const int32_t* n_rows, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (in_dtype == 0) {
    if (out_fp8pair)
      quant_int8_kernel<float, 1><<<rows, 256, 0, st>>>((const float*)v, K, q, scales, sorted, P, n_rows);
    else
      quant_int8_kernel<float, 0><<<rows, 256, 0, st>>>((const float*)v, K, q, scales, sorted, P, n_rows);
  } else {
    if (out_fp8pair)
      quant_int8_kernel<uint16_t, 1><<<rows, 256, 0, st>>>((const uint16_t*)v, K, q, scales, sorted, P, n_rows);
    else
      quant_int8_kernel<uint16_t, 0><<<rows, 256, 0, st>>>((const uint16_t*)v, K, q, scales, sorted, P, n_rows);
  }
  return hipGetLastError();
}

hipError_t moe_k_quant_mxfp4(int in_dtype, const void* v, int rows, int K, uint8_t* codes, uint8_t* scales,
                             hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  int g = grid_for((size_t)rows * (K / 32));
  if (in_dtype == 0)
    quant_mxfp4_kernel<float><<<g, 256, 0, st>>>((const float*)v, rows, K, codes, scales);
  else
    quant_mxfp4_kernel<uint16_t><<<g, 256, 0, st>>>((const uint16_t*)v, rows, K, codes, scales);
  return hipGetLastError();
}

hipError_t moe_k_fp8pair_to_int8(const uint8_t* src, const float* src_s, int K, const int32_t* row_of, int nrows,
                                 int8_t* q, float* s, hipStream_t st) {
  if (nrows <= 0) return hipSuccess;
  fp8pair_to_int8_kernel<<<nrows, 256, 0, st>>>(src, src_s, K, row_of, nrows, q, s);
  return hipGetLastError();
}

hipError_t moe_k_gather_rows(const void* src, int row_bytes, const int32_t* row_of, int nrows, void* dst,
                             hipStream_t st) {
  if (nrows <= 0) return hipSuccess;
  gather_rows_kernel<<<nrows, 256, 0, st>>>((const uint8_t*)src, row_bytes, row_of, nrows, (uint8_t*)dst);
  return hipGetLastError();
}
