// Device building blocks of the stable expert sort, shared by the sort
// kernels and the fused single-workgroup route kernel.
#pragma once
#include "common.h"

namespace moe {

constexpr int SB = 1024;  // pairs per sort block (one 1024-thread workgroup)

// Per block of n <= SB pairs (thread i holds pair base + i, blockDim.x >= n):
// stable local rank of each pair and the block's per-expert counts, from
// bitmasks. Expert e owns W = ceil(n / 32) LDS words; bit i is set (an LDS
// atomic OR: the result does not depend on the order of the ORs) when pair i
// goes to e. The rank of pair i is the number of set bits below bit i in its
// expert's words, the count of e the number of all its set bits.
// mask: LDS [E][W] words; tot: LDS [E] (the block's totals on return).
__device__ inline void block_rank(int my_id, bool my_valid, int n, int E, uint32_t* mask, int* tot, int& my_rank) {
  const int tid = threadIdx.x;
  const int W = (n + 31) >> 5;
  for (int i = tid; i < E * W; i += blockDim.x) mask[i] = 0u;
  __syncthreads();
  if (my_valid) atomicOr(&mask[my_id * W + (tid >> 5)], 1u << (tid & 31));
  __syncthreads();
  my_rank = 0;
  if (my_valid) {
    const uint32_t* m = mask + my_id * W;
    const int wi = tid >> 5;
    int r = __popc(m[wi] & ((1u << (tid & 31)) - 1u));
    for (int w = 0; w < wi; ++w) r += __popc(m[w]);
    my_rank = r;
  }
  for (int e = tid; e < E; e += blockDim.x) {
    int c = 0;
    for (int w = 0; w < W; ++w) c += __popc(mask[e * W + w]);
    tot[e] = c;
  }
  __syncthreads();
}

// Inclusive prefix sum over a wave by DPP, in registers: row shifts 1, 2, 4, 8
// scan each 16-lane row (a lane without a source adds 0), then the row
// broadcasts of lanes 15 and 31 carry the row totals into the later rows.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return v;
}

// Block-wide exclusive scan of padded counts over E experts (E <= 1024,
// blockDim.x == 1024): writes offsets[0..E]. A scan inside each wave, the
// wave totals scanned by wave 0, then one add: two barriers.
__device__ inline void scan_offsets(const int* counts_lds, int E, int block_m, int* offs_lds, int* tmp) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int v = 0;
  if (tid < E) v = (counts_lds[tid] + block_m - 1) / block_m * block_m;
  v = wave_incl_scan(v);
  if (lane == 63) tmp[wave] = v;  // inclusive wave totals
  __syncthreads();
  if (wave == 0) {
    const int t = wave_incl_scan(lane < 16 ? tmp[lane] : 0);
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
  // padding slots: g = blockDim.x / E threads per expert (E <= blockDim.x)
  // stride over that expert's padding [offs + count, offs[e + 1]) only: one
  // division per thread rather than one per (expert, slot) candidate
  if (block_m > 1) {
    const int g = (int)blockDim.x / E;
    if (tid < g * E) {
      const int e = tid / g;
      const int end = offs[e + 1];
      for (int p = offs[e] + counts[e] + (tid - e * g); p < end; p += g) sorted[p] = P;
    }
  }
  for (int e = tid; e < E; e += blockDim.x)
    for (int q = offs[e] / block_m; q < offs[e + 1] / block_m; ++q) tile_expert[q] = e;
  if (tid == 0) *n_tiles = offs[E] / block_m;
}

// Wide tiles of the prefill GEMMs: expert e's padded segment holds
// n_e = (offs[e + 1] - offs[e]) / block_m sort tiles, covered in order by
// ceil(n_e / 2) wide tiles of two (the last one of an odd n_e holds one).
// wide[w] = (first sort tile << 1) | (1 if a second tile follows);
// *n_wide = their number. blockDim.x == 1024, E <= 1024; tmp: 32 LDS ints,
// free (scan_offsets leaves them so after its last barrier).
__device__ inline void write_wide_tiles(const int* offs, int E, int block_m, int* tmp, int32_t* __restrict__ wide,
                                        int32_t* __restrict__ n_wide) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int n = 0, m = 0;
  if (tid < E) {
    n = (offs[tid + 1] - offs[tid]) / block_m;
    m = (n + 1) >> 1;
  }
  const int v = wave_incl_scan(m);
  if (lane == 63) tmp[wave] = v;
  __syncthreads();
  if (wave == 0) {
    const int t = wave_incl_scan(lane < 16 ? tmp[lane] : 0);
    if (lane < 16) tmp[16 + lane] = t - tmp[lane];
  }
  __syncthreads();
  if (tid < E) {
    const int base = v - m + tmp[16 + wave];
    const int t0 = offs[tid] / block_m;
    for (int i = 0; i < m; ++i) wide[base + i] = ((t0 + 2 * i) << 1) | (2 * i + 1 < n ? 1 : 0);
    if (tid == E - 1) *n_wide = base + m;
  }
}

}  // namespace moe
