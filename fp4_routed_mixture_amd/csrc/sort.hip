// Expert sort (retuned for prefill in DeepSeek-V4-Flash on AMD gfx90a:
// Correctness Recovery and Inference Performance Engineering, abstract):
// a stable counting sort of the P = T*k (token, slot) pairs by expert, each
// expert segment padded to a multiple of block_m, plus the tile -> expert map
// the grouped GEMMs walk. Integers only, so it is bit-exact by construction.
//
// Inside a block of up to 1024 pairs the stable rank of a pair is the number
// of earlier pairs with its expert, read from a per-expert bitmask of the
// block's pairs. Blocks are ordered by pair index, so adding the counts of
// earlier blocks keeps the global order stable.
//
// Small P (<= 1024): one 1024-thread workgroup does everything.
// Large P: sort_count (per 1024-pair block: stable local ranks + per-expert
// counts) -> sort_scan (one workgroup: totals, padded offsets, per-block
// bases, tiles, padding sentinels) -> sort_scatter.
#include "common.h"
#include "kernels.h"
#include "sort_dev.h"

namespace {

constexpr size_t kScanLdsMax = 156 * 1024;  // dynamic LDS of the scan with the histogram staged


// P <= moe::SB: everything in one workgroup.
__global__ __launch_bounds__(1024) void sort_small_kernel(const int32_t* __restrict__ ids, int P, int E, int block_m,
                                                          int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ sorted, int32_t* __restrict__ pos,
                                                          int32_t* __restrict__ tile_expert,
                                                          int32_t* __restrict__ n_tiles, int32_t* __restrict__ wide,
                                                          int32_t* __restrict__ n_wide) {
  extern __shared__ int smem[];
  const int W = (P + 31) >> 5;
  uint32_t* mask = reinterpret_cast<uint32_t*>(smem);  // E * W
  int* tot = smem + E * W;                              // E
  int* offs = tot + E;                                  // E + 1
  int* tmp = offs + E + 1;                              // 1024
  const bool valid = (int)threadIdx.x < P;
  const int id = valid ? ids[threadIdx.x] : 0;
  int rank;
  moe::block_rank(id, valid, P, E, mask, tot, rank);
  moe::scan_offsets(tot, E, block_m, offs, tmp);
  const int tid = threadIdx.x;
  if (valid) {
    int p = offs[id] + rank;
    sorted[p] = tid;
    pos[tid] = p;
  }
  for (int e = tid; e < E; e += blockDim.x) counts[e] = tot[e];
  for (int e = tid; e <= E; e += blockDim.x) offsets[e] = offs[e];
  moe::write_tiles_and_padding(tot, offs, E, P, block_m, sorted, tile_expert, n_tiles);
  if (wide) moe::write_wide_tiles(offs, E, block_m, tmp, wide, n_wide);
}

// Large P, step 1: per block local ranks and per-expert block counts.
__global__ __launch_bounds__(1024) void sort_count_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                          int32_t* __restrict__ local_rank,
                                                          int32_t* __restrict__ block_hist) {
  extern __shared__ int smem[];
  const int n = min(moe::SB, P - (int)blockIdx.x * moe::SB);
  uint32_t* mask = reinterpret_cast<uint32_t*>(smem);  // E * ceil(n / 32)
  int* tot = smem + E * ((n + 31) >> 5);               // E
  const int i = blockIdx.x * moe::SB + threadIdx.x;
  const bool valid = i < P;
  const int id = valid ? ids[i] : 0;
  int rank;
  moe::block_rank(id, valid, n, E, mask, tot, rank);
  if (valid) local_rank[i] = rank;
  for (int e = threadIdx.x; e < E; e += blockDim.x) block_hist[(size_t)blockIdx.x * E + e] = tot[e];
}

// Large P, step 2: one workgroup. block_hist becomes per-block exclusive
// bases (offset of the expert segment plus earlier blocks' counts). With
// HIST_LDS the whole [nblocks][E] matrix is first copied into LDS (every
// load in flight at once) and written back at the end; otherwise the runs
// below walk it in global memory.
template <bool HIST_LDS>
__global__ __launch_bounds__(1024) void sort_scan_kernel(int nblocks, int P, int E, int block_m,
                                                         int32_t* __restrict__ block_hist,
                                                         int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ sorted,
                                                         int32_t* __restrict__ tile_expert,
                                                         int32_t* __restrict__ n_tiles, int32_t* __restrict__ wide,
                                                         int32_t* __restrict__ n_wide) {
  extern __shared__ int smem[];
  int* tot = smem;            // E
  int* offs = tot + E;        // E + 1
  int* tmp = offs + E + 1;    // 1024
  int* lh = tmp + 1024;       // nblocks * E (HIST_LDS)
  int32_t* hist = HIST_LDS ? lh : block_hist;
  const int tid = threadIdx.x;
  const int nh = nblocks * E;
  if (HIST_LDS) {
    for (int i0 = tid; i0 < nh; i0 += 8 * 1024) {
      int v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = i0 + j * 1024;
        v[j] = i < nh ? block_hist[i] : 0;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = i0 + j * 1024;
        if (i < nh) lh[i] = v[j];
      }
    }
    __syncthreads();
  }
  // Per expert, an exclusive scan over the blocks. With E <= 256 each expert
  // gets 1024 / E' threads (E' = E rounded up to a power of two) that scan
  // contiguous runs of blocks, then add the sums of the runs before them.
  int split = 1;
  while (split * 2 * E <= 1024 && split < 16) split *= 2;
  int* part = tmp;  // 1024 run sums
  {
    const int e = tid / split, r = tid % split;
    const int b0 = (nblocks * r) / split, b1 = (nblocks * (r + 1)) / split;
    int run = 0;
    if (e < E)
      for (int b = b0; b < b1; ++b) run += hist[(size_t)b * E + e];
    part[tid] = run;
    __syncthreads();
    int base = 0, total = 0;
    if (e < E) {
      for (int i = 0; i < split; ++i) {
        const int v = part[e * split + i];
        if (i < r) base += v;
        total += v;
      }
      if (r == 0) tot[e] = total;
    }
    __syncthreads();  // part[] is reused by scan_offsets
    if (e < E) {
      run = base;
      for (int b = b0; b < b1; ++b) {
        const int c = hist[(size_t)b * E + e];
        hist[(size_t)b * E + e] = run;
        run += c;
      }
    }
  }
  __syncthreads();
  moe::scan_offsets(tot, E, block_m, offs, tmp);
  {
    const int e = tid / split, r = tid % split;
    const int b0 = (nblocks * r) / split, b1 = (nblocks * (r + 1)) / split;
    if (e < E) {
      if (r == 0) counts[e] = tot[e];
      for (int b = b0; b < b1; ++b) hist[(size_t)b * E + e] += offs[e];
    }
  }
  if (HIST_LDS) {
    __syncthreads();
    for (int i = tid; i < nh; i += 1024) block_hist[i] = lh[i];
  }
  for (int e = tid; e <= E; e += blockDim.x) offsets[e] = offs[e];
  moe::write_tiles_and_padding(tot, offs, E, P, block_m, sorted, tile_expert, n_tiles);
  if (wide) moe::write_wide_tiles(offs, E, block_m, tmp, wide, n_wide);
}

// Routing given by a caller: ids clamped into [0, E), weights copied.
__global__ __launch_bounds__(256) void copy_routing_kernel(const int32_t* __restrict__ ids_in,
                                                           const float* __restrict__ w_in, int P, int E,
                                                           int32_t* __restrict__ ids, float* __restrict__ w) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= P) return;
  const int e = ids_in[i];
  ids[i] = e < 0 ? 0 : (e >= E ? E - 1 : e);
  w[i] = w_in[i];
}

// Large P, step 3: scatter.
__global__ __launch_bounds__(256) void sort_scatter_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                           const int32_t* __restrict__ local_rank,
                                                           const int32_t* __restrict__ block_base,
                                                           int32_t* __restrict__ sorted, int32_t* __restrict__ pos) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= P) return;
  const int b = i / moe::SB;
  const int p = block_base[(size_t)b * E + ids[i]] + local_rank[i];
  sorted[p] = i;
  pos[i] = p;
}

}  // namespace

hipError_t moe_k_copy_routing(const int32_t* ids_in, const float* w_in, int P, int E, int32_t* ids, float* w,
                              hipStream_t st) {
  if (P <= 0) return hipSuccess;
  copy_routing_kernel<<<(P + 255) / 256, 256, 0, st>>>(ids_in, w_in, P, E, ids, w);
  return hipGetLastError();
}

size_t moe_k_sort_scratch_bytes(int P, int E) {
  if (P <= moe::SB) return 0;
  size_t nb = (P + moe::SB - 1) / moe::SB;
  return ((size_t)P * 4 + 255) / 256 * 256 + (nb * E * 4 + 255) / 256 * 256;
}

hipError_t moe_k_sort(const int32_t* ids, int P, int E, int block_m, int32_t* counts, int32_t* offsets,
                      int32_t* sorted, int32_t* pos, int32_t* tile_expert, int32_t* n_tiles, int32_t* wide,
                      int32_t* n_wide, void* scratch, hipStream_t st) {
  // gfx950 has 160 KB of LDS per workgroup; above 64 KB a kernel must opt in
  static std::atomic<bool> lds_opt_in[moe::kMaxDevices];
  const hipError_t eo = moe::once_per_device(lds_opt_in, [] {
    hipError_t e1 = hipFuncSetAttribute((const void*)sort_small_kernel,
                                        hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    hipError_t e2 = hipFuncSetAttribute((const void*)sort_count_kernel,
                                        hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    hipError_t e3 = hipFuncSetAttribute((const void*)sort_scan_kernel<true>,
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)kScanLdsMax);
    return e1 != hipSuccess ? e1 : (e2 != hipSuccess ? e2 : e3);
  });
  if (eo != hipSuccess) return eo;
  if (P <= moe::SB) {
    size_t lds = (size_t)(E * ((P + 31) / 32) + E + E + 1 + 1024) * 4;
    sort_small_kernel<<<1, 1024, lds, st>>>(ids, P, E, block_m, counts, offsets, sorted, pos, tile_expert, n_tiles,
                                            wide, n_wide);
    return hipGetLastError();
  }
  int nb = (P + moe::SB - 1) / moe::SB;
  int32_t* local_rank = (int32_t*)scratch;
  int32_t* block_hist = (int32_t*)((char*)scratch + ((size_t)P * 4 + 255) / 256 * 256);
  sort_count_kernel<<<nb, 1024, (size_t)(E * (moe::SB / 32) + E) * 4, st>>>(ids, P, E, local_rank, block_hist);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t scan_lds = (size_t)(E + E + 1 + 1024) * 4, hist_lds = (size_t)nb * E * 4;
  if (scan_lds + hist_lds <= kScanLdsMax)
    sort_scan_kernel<true><<<1, 1024, scan_lds + hist_lds, st>>>(nb, P, E, block_m, block_hist, counts, offsets,
                                                                 sorted, tile_expert, n_tiles, wide, n_wide);
  else
    sort_scan_kernel<false><<<1, 1024, scan_lds, st>>>(nb, P, E, block_m, block_hist, counts, offsets, sorted,
                                                       tile_expert, n_tiles, wide, n_wide);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  sort_scatter_kernel<<<(P + 255) / 256, 256, 0, st>>>(ids, P, E, local_rank, block_hist, sorted, pos);
  return hipGetLastError();
}
