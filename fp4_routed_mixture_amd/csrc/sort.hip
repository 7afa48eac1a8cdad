// Expert sort ("retuned expert sorting", abstract of "DeepSeek-V4-Flash on
// AMD gfx90a: Correctness Recovery and Inference Performance Engineering"):
// a stable counting sort of the P = T*k (token, slot) pairs by expert, each
// expert segment padded to a multiple of block_m, plus the tile -> expert map
// the grouped GEMMs walk. Integers only, so it is bit-exact by construction.
//
// Stability inside a wave comes from a match loop: the lanes holding the
// lowest-numbered unprocessed expert vote (ballot), each learns its rank from
// the popcount of the voting lanes below it, and they retire together. Waves
// (and blocks) are ordered by pair index, so adding the counts of earlier
// waves (blocks) keeps the global order stable.
//
// Small P (<= 1024): one 1024-thread workgroup does everything.
// Large P: sort_count (per 1024-pair block: stable local ranks + per-expert
// counts) -> sort_scan (one workgroup: totals, padded offsets, per-block
// bases, tiles, padding sentinels) -> sort_scatter.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int SB = 1024;  // pairs per block

// Stable rank of each lane's id among lanes of this wave with the same id,
// and (for the lane that is lowest in its group) the group size.
__device__ __forceinline__ void wave_match_rank(int id, bool valid, int& rank, int& group_count, bool& leader) {
  const int lane = threadIdx.x & 63;
  uint64_t active = __ballot(valid);
  rank = 0;
  group_count = 0;
  leader = false;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  while (active) {
    int first = __ffsll((unsigned long long)active) - 1;
    int fid = __shfl(id, first, 64);
    uint64_t m = __ballot(valid && id == fid);
    if (valid && id == fid) {
      rank = __popcll(m & below);
      group_count = __popcll(m);
      leader = lane == first;
    }
    active &= ~m;
  }
}

// Per block of SB pairs: local stable rank of each pair and per-expert counts.
// wcnt: LDS [16 waves][E]
__device__ void block_rank(const int32_t* __restrict__ ids, int P, int E, int base, int* wcnt, int& my_rank,
                           int& my_id, bool& my_valid) {
  const int tid = threadIdx.x, wave = tid >> 6;
  for (int i = tid; i < 16 * E; i += blockDim.x) wcnt[i] = 0;
  __syncthreads();
  const int i = base + tid;
  my_valid = i < P;
  my_id = my_valid ? ids[i] : 0;
  int rank, cnt;
  bool leader;
  wave_match_rank(my_id, my_valid, rank, cnt, leader);
  if (leader) wcnt[wave * E + my_id] = cnt;
  __syncthreads();
  // exclusive prefix over waves, per expert (in place), then local rank
  for (int e = tid; e < E; e += blockDim.x) {
    int run = 0;
    for (int w = 0; w < 16; ++w) {
      int c = wcnt[w * E + e];
      wcnt[w * E + e] = run;
      run += c;
    }
    wcnt[16 * E + e] = run;  // block total for e
  }
  __syncthreads();
  my_rank = my_valid ? wcnt[wave * E + my_id] + rank : 0;
}

// Block-wide exclusive scan of padded counts over E experts (E <= 1024,
// 1024 threads): writes offsets[0..E].
__device__ void scan_offsets(const int* counts_lds, int E, int block_m, int* offs_lds, int* tmp) {
  const int tid = threadIdx.x;
  int v = 0;
  if (tid < E) v = (counts_lds[tid] + block_m - 1) / block_m * block_m;
  tmp[tid] = v;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    int add = tid >= o ? tmp[tid - o] : 0;
    __syncthreads();
    tmp[tid] += add;
    __syncthreads();
  }
  if (tid < E) offs_lds[tid + 1] = tmp[tid];
  if (tid == 0) offs_lds[0] = 0;
  __syncthreads();
}

__device__ void write_tiles_and_padding(const int* counts, const int* offs, int E, int P, int block_m,
                                        int32_t* __restrict__ sorted, int32_t* __restrict__ tile_expert,
                                        int32_t* __restrict__ n_tiles) {
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += blockDim.x) {
    for (int p = offs[e] + counts[e]; p < offs[e + 1]; ++p) sorted[p] = P;
    for (int q = offs[e] / block_m; q < offs[e + 1] / block_m; ++q) tile_expert[q] = e;
  }
  if (tid == 0) *n_tiles = offs[E] / block_m;
}

// P <= SB: everything in one workgroup.
__global__ __launch_bounds__(1024) void sort_small_kernel(const int32_t* __restrict__ ids, int P, int E, int block_m,
                                                          int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ sorted, int32_t* __restrict__ pos,
                                                          int32_t* __restrict__ tile_expert,
                                                          int32_t* __restrict__ n_tiles) {
  extern __shared__ int smem[];
  int* wcnt = smem;                  // 17 * E
  int* offs = wcnt + 17 * E;         // E + 1
  int* tmp = offs + E + 1;           // 1024
  int rank, id;
  bool valid;
  block_rank(ids, P, E, 0, wcnt, rank, id, valid);
  const int* tot = wcnt + 16 * E;
  scan_offsets(tot, E, block_m, offs, tmp);
  const int tid = threadIdx.x;
  if (valid) {
    int p = offs[id] + rank;
    sorted[p] = tid;
    pos[tid] = p;
  }
  for (int e = tid; e < E; e += blockDim.x) counts[e] = tot[e];
  for (int e = tid; e <= E; e += blockDim.x) offsets[e] = offs[e];
  write_tiles_and_padding(tot, offs, E, P, block_m, sorted, tile_expert, n_tiles);
}

// Large P, step 1: per block local ranks and per-expert block counts.
__global__ __launch_bounds__(1024) void sort_count_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                          int32_t* __restrict__ local_rank,
                                                          int32_t* __restrict__ block_hist) {
  extern __shared__ int smem[];
  int rank, id;
  bool valid;
  block_rank(ids, P, E, blockIdx.x * SB, smem, rank, id, valid);
  const int i = blockIdx.x * SB + threadIdx.x;
  if (valid) local_rank[i] = rank;
  for (int e = threadIdx.x; e < E; e += blockDim.x) block_hist[(size_t)blockIdx.x * E + e] = smem[16 * E + e];
}

// Large P, step 2: one workgroup. block_hist becomes per-block exclusive
// bases (offset of the expert segment plus earlier blocks' counts).
__global__ __launch_bounds__(1024) void sort_scan_kernel(int nblocks, int P, int E, int block_m,
                                                         int32_t* __restrict__ block_hist,
                                                         int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ sorted,
                                                         int32_t* __restrict__ tile_expert,
                                                         int32_t* __restrict__ n_tiles) {
  extern __shared__ int smem[];
  int* tot = smem;            // E
  int* offs = tot + E;        // E + 1
  int* tmp = offs + E + 1;    // 1024
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += blockDim.x) {
    int run = 0;
    for (int b = 0; b < nblocks; ++b) {
      int c = block_hist[(size_t)b * E + e];
      block_hist[(size_t)b * E + e] = run;
      run += c;
    }
    tot[e] = run;
  }
  __syncthreads();
  scan_offsets(tot, E, block_m, offs, tmp);
  for (int e = tid; e < E; e += blockDim.x) {
    counts[e] = tot[e];
    for (int b = 0; b < nblocks; ++b) block_hist[(size_t)b * E + e] += offs[e];
  }
  for (int e = tid; e <= E; e += blockDim.x) offsets[e] = offs[e];
  write_tiles_and_padding(tot, offs, E, P, block_m, sorted, tile_expert, n_tiles);
}

// Large P, step 3: scatter.
__global__ __launch_bounds__(256) void sort_scatter_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                           const int32_t* __restrict__ local_rank,
                                                           const int32_t* __restrict__ block_base,
                                                           int32_t* __restrict__ sorted, int32_t* __restrict__ pos) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= P) return;
  const int b = i / SB;
  const int p = block_base[(size_t)b * E + ids[i]] + local_rank[i];
  sorted[p] = i;
  pos[i] = p;
}

}  // namespace

size_t moe_k_sort_scratch_bytes(int P, int E) {
  if (P <= SB) return 0;
  size_t nb = (P + SB - 1) / SB;
  return ((size_t)P * 4 + 255) / 256 * 256 + (nb * E * 4 + 255) / 256 * 256;
}

hipError_t moe_k_sort(const int32_t* ids, int P, int E, int block_m, int32_t* counts, int32_t* offsets,
                      int32_t* sorted, int32_t* pos, int32_t* tile_expert, int32_t* n_tiles, void* scratch,
                      hipStream_t st) {
  // gfx950 has 160 KB of LDS per workgroup; above 64 KB a kernel must opt in
  static bool lds_opt_in = false;
  if (!lds_opt_in) {
    hipError_t e1 = hipFuncSetAttribute((const void*)sort_small_kernel,
                                        hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    hipError_t e2 = hipFuncSetAttribute((const void*)sort_count_kernel,
                                        hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e1 != hipSuccess) return e1;
    if (e2 != hipSuccess) return e2;
    lds_opt_in = true;
  }
  if (P <= SB) {
    size_t lds = (size_t)(17 * E + E + 1 + 1024) * 4;
    sort_small_kernel<<<1, 1024, lds, st>>>(ids, P, E, block_m, counts, offsets, sorted, pos, tile_expert, n_tiles);
    return hipGetLastError();
  }
  int nb = (P + SB - 1) / SB;
  int32_t* local_rank = (int32_t*)scratch;
  int32_t* block_hist = (int32_t*)((char*)scratch + ((size_t)P * 4 + 255) / 256 * 256);
  sort_count_kernel<<<nb, 1024, (size_t)17 * E * 4, st>>>(ids, P, E, local_rank, block_hist);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  sort_scan_kernel<<<1, 1024, (size_t)(E + E + 1 + 1024) * 4, st>>>(nb, P, E, block_m, block_hist, counts, offsets,
                                                                    sorted, tile_expert, n_tiles);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  sort_scatter_kernel<<<(P + 255) / 256, 256, 0, st>>>(ids, P, E, local_rank, block_hist, sorted, pos);
  return hipGetLastError();
}
