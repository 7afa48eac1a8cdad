// Weighted combine of the routed experts' outputs, and the two helpers of the
// stacked-layer residual stream.
//   combine : out[t][n] = fma chain over slots j = 0..k-1 of w[t][j] * y[t*k+j][n],
//             starting from 0 (y rows are indexed by pair, so a token's k rows
//             are adjacent).
//   rmsnorm : out = x / sqrt(ss / H + 1e-6), ss in the router's fixed order
//             (64 chunk chains, pairwise tree), one wave per row.
//   residual: x += y.
//   combine_residual_norm: the three above fused for stacked layers.
#include "common.h"
#include "kernels.h"

namespace {

// One instance per top-k K: every slot's weight and y column are loaded
// before the first fma, so a column waits for memory once rather than once a
// slot (with a runtime K the loads sat under branches, each waited for alone).
template <int K>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, const float* __restrict__ w, int T,
                                                      int H, float* __restrict__ out) {
  const size_t n4 = (size_t)T * (H >> 2);
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n4; i += (size_t)gridDim.x * blockDim.x) {
    const size_t t = i / (H >> 2);
    const int n = (int)(i - t * (H >> 2)) * 4;
    float wj[K];
    v4f v[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      wj[j] = w[t * K + j];
      // y is read exactly once: keep it out of the caches
      v[j] = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(y + (t * K + j) * (size_t)H + n));
    }
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < K; ++j) {
      acc.x = __builtin_fmaf(wj[j], v[j][0], acc.x);
      acc.y = __builtin_fmaf(wj[j], v[j][1], acc.y);
      acc.z = __builtin_fmaf(wj[j], v[j][2], acc.z);
      acc.w = __builtin_fmaf(wj[j], v[j][3], acc.w);
    }
    *reinterpret_cast<float4*>(out + t * H + n) = acc;
  }
}

__global__ __launch_bounds__(64) void rmsnorm_kernel(const float* __restrict__ x, int H, float* __restrict__ out) {
  const int t = blockIdx.x, c = threadIdx.x;
  const int L = H >> 6;
  const float* row = x + (size_t)t * H;
  const float* chunk = row + (size_t)c * L;
  float p = 0.0f;
  for (int i = 0; i < L; ++i) p = __builtin_fmaf(chunk[i], chunk[i], p);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) p = p + __shfl_xor(p, o, 64);
  const float r = __builtin_sqrtf(p / (float)H + 1e-6f);
  for (int i = c; i < H; i += 64) out[(size_t)t * H + i] = row[i] / r;
}

__global__ __launch_bounds__(256) void residual_kernel(float* __restrict__ x, const float* __restrict__ y, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    x[i] = x[i] + y[i];
}

// Stacked layers: the combine of layer l, the residual update and the RMSNorm
// of layer l+1's input in one pass per token (one workgroup of min(H/4, 1024)
// threads per token, a float4 column per thread and pass), with the
// arithmetic of combine_kernel, residual_kernel and rmsnorm_kernel in sequence:
//   out = fma chain over slots of w_j * y_j   (stored to layer_out if given)
//   x   = x + out
//   xn  = x / sqrt(ss / H + 1e-6)              (if xn is given)
// All slot rows of a column are loaded before the first fma, so a pass waits
// for memory once. The updated row is kept in LDS with one pad float per 64 so
// that the 64 chunk chains of the sum of squares read distinct banks.
__global__ __launch_bounds__(1024) void combine_residual_norm_kernel(const float* __restrict__ y,
                                                                     const float* __restrict__ w, int H, int K,
                                                                     float* __restrict__ x,
                                                                     float* __restrict__ layer_out,
                                                                     float* __restrict__ xn) {
  extern __shared__ float row[];  // H + H/64 floats
  __shared__ float r_sh;
  const int t = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
  const float* wt = w + (size_t)t * K;
  const float* yt = y + (size_t)t * K * H;
  float* xr = x + (size_t)t * H;
  for (int n = tid * 4; n < H; n += nt * 4) {
    v4f v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < K) v[j] = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(yt + (size_t)j * H + n));
    float4 xv = *reinterpret_cast<const float4*>(xr + n);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j < K) {
        const float wj = wt[j];
        acc.x = __builtin_fmaf(wj, v[j][0], acc.x);
        acc.y = __builtin_fmaf(wj, v[j][1], acc.y);
        acc.z = __builtin_fmaf(wj, v[j][2], acc.z);
        acc.w = __builtin_fmaf(wj, v[j][3], acc.w);
      }
    }
    if (layer_out) *reinterpret_cast<float4*>(layer_out + (size_t)t * H + n) = acc;
    xv.x = xv.x + acc.x;
    xv.y = xv.y + acc.y;
    xv.z = xv.z + acc.z;
    xv.w = xv.w + acc.w;
    *reinterpret_cast<float4*>(xr + n) = xv;
    float* rr = row + n + (n >> 6);
    rr[0] = xv.x; rr[1] = xv.y; rr[2] = xv.z; rr[3] = xv.w;
  }
  if (!xn) return;
  __syncthreads();
  if (tid < 64) {
    const int L = H >> 6;
    float p = 0.0f;
    for (int i = 0; i < L; ++i) {
      const int el = tid * L + i;  // element el sits at el + el / 64
      const float v = row[el + (el >> 6)];
      p = __builtin_fmaf(v, v, p);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) p = p + __shfl_xor(p, o, 64);
    if (tid == 0) r_sh = __builtin_sqrtf(p / (float)H + 1e-6f);
  }
  __syncthreads();
  const float r = r_sh;
  for (int n = tid; n < H; n += nt) xn[(size_t)t * H + n] = row[n + (n >> 6)] / r;
}

int grid_for(size_t n) {
  size_t b = (n + 255) / 256;
  return (int)(b < 65536 ? (b ? b : 1) : 65536);
}

// The combine instance for top-k K (1..16).
template <int KK>
hipError_t launch_combine(const float* y, const float* w, int T, int H, int K, float* out, hipStream_t st) {
  if (K == KK) {
    combine_kernel<KK><<<grid_for((size_t)T * (H >> 2)), 256, 0, st>>>(y, w, T, H, out);
    return hipGetLastError();
  }
  if constexpr (KK < 16) return launch_combine<KK + 1>(y, w, T, H, K, out, st);
  else return hipErrorInvalidValue;
}

}  // namespace

hipError_t moe_k_combine(const float* y, const float* w, int T, int H, int K, float* out, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  return launch_combine<1>(y, w, T, H, K, out, st);
}

hipError_t moe_k_rmsnorm(const float* x, int T, int H, float* out, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  rmsnorm_kernel<<<T, 64, 0, st>>>(x, H, out);
  return hipGetLastError();
}

hipError_t moe_k_residual(float* x, const float* y, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  residual_kernel<<<grid_for((size_t)n), 256, 0, st>>>(x, y, n);
  return hipGetLastError();
}

hipError_t moe_k_combine_residual_norm(const float* y, const float* w, int T, int H, int K, float* x,
                                       float* layer_out, float* xn, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  const size_t lds = (size_t)(H + H / 64) * 4;
  // above 64 KB of dynamic LDS a kernel must opt in; static LDS (r_sh) counts
  // against the same 160 KB, so ask for what H <= 16384 needs
  static std::atomic<bool> lds_opt_in[moe::kMaxDevices];
  const hipError_t e = moe::once_per_device(lds_opt_in, [] {
    return hipFuncSetAttribute((const void*)combine_residual_norm_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (16384 + 256) * 4);
  });
  if (e != hipSuccess) return e;
  const int threads = H / 4 < 1024 ? H / 4 : 1024;  // H % 256 == 0: whole waves
  combine_residual_norm_kernel<<<T, threads, lds, st>>>(y, w, H, K, x, layer_out, xn);
  return hipGetLastError();
}
