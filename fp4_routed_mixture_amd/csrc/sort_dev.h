// Device building blocks of the stable expert sort, shared by the sort
// kernels and the fused single-workgroup route kernel.
#pragma once
#include "common.h"

namespace moe {

constexpr int SB = 1024;  // pairs per sort block (one 1024-thread workgroup)

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

// Per block of up to SB pairs (thread i holds pair base + i): stable local
// rank of each pair and per-expert counts. wcnt: LDS [17][E]; row 16 receives
// the block's per-expert totals.
__device__ inline void block_rank(int my_id, bool my_valid, int E, int* wcnt, int& my_rank) {
  const int tid = threadIdx.x, wave = tid >> 6;
  for (int i = tid; i < 16 * E; i += blockDim.x) wcnt[i] = 0;
  __syncthreads();
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
// blockDim.x == 1024): writes offsets[0..E]. A scan inside each wave
// (shuffles), the wave totals scanned by wave 0, then one add: two barriers.
__device__ inline void scan_offsets(const int* counts_lds, int E, int block_m, int* offs_lds, int* tmp) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int v = 0;
  if (tid < E) v = (counts_lds[tid] + block_m - 1) / block_m * block_m;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(v, o, 64);
    if (lane >= o) v += n;
  }
  if (lane == 63) tmp[wave] = v;  // inclusive wave totals
  __syncthreads();
  if (wave == 0) {
    int t = lane < 16 ? tmp[lane] : 0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int n = __shfl_up(t, o, 64);
      if (lane >= o) t += n;
    }
    if (lane < 16) tmp[16 + lane] = t - tmp[lane];  // exclusive base of each wave
  }
  __syncthreads();
  if (tid < E) offs_lds[tid + 1] = v + tmp[16 + wave];
  if (tid == 0) offs_lds[0] = 0;
  __syncthreads();
}

__device__ inline void write_tiles_and_padding(const int* counts, const int* offs, int E, int P, int block_m,
                                        int32_t* __restrict__ sorted, int32_t* __restrict__ tile_expert,
                                        int32_t* __restrict__ n_tiles) {
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += blockDim.x) {
    for (int p = offs[e] + counts[e]; p < offs[e + 1]; ++p) sorted[p] = P;
    for (int q = offs[e] / block_m; q < offs[e + 1] / block_m; ++q) tile_expert[q] = e;
  }
  if (tid == 0) *n_tiles = offs[E] / block_m;
}

}  // namespace moe
