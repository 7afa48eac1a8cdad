// Internal launchers (host side). Every launcher enqueues on `st` and returns
// the launch status; argument checking happens in the C-ABI layer (api.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

// prepack.hip
size_t moe_k_packed_scale_bytes(int which, int E, int N, int K);
hipError_t moe_k_pack(int which, int E, int N, int K, const uint8_t* codes, const uint8_t* scales,
                      const int32_t* perm, uint8_t* pcodes, uint8_t* pscales, hipStream_t st);
hipError_t moe_k_unpack(int which, int E, int N, int K, const uint8_t* pcodes, const uint8_t* pscales,
                        uint8_t* codes, uint8_t* scales, hipStream_t st);

// route.hip
int moe_k_router_slices(int T, int H, int E, int K);
size_t moe_k_router_partial_bytes(int T, int H, int E, int K);
// With xq non-NULL (small batches only: moe_k_router_quantizes_x) the same
// launch also quantizes x (int8 FP8-pair rows + scale, or MXFP4 if mx).
hipError_t moe_k_router_partial(int x_dtype, const void* x, const float* wr, float* partial, int T, int H, int E,
                                int K, int mx, uint8_t* xq, uint8_t* xs, hipStream_t st);
int moe_k_router_quantizes_x(int T, int H, int E, int K);
// logits[T][E] from the partial sums (the tree's remaining levels + bias).
hipError_t moe_k_finish_logits(const float* partial, const float* bias, int T, int H, int E, int K, float* logits,
                               hipStream_t st);
// Tiny batches (moe_k_router_slices == 16): routing and the expert sort (the
// outputs of moe_k_sort) in one single-workgroup kernel.
int moe_k_route_sort_fits(int T, int H, int E, int K);
hipError_t moe_k_route_sort_small(const float* partial, const float* bias, int T, int E, int K, int block_m,
                                  int32_t* ids, float* w, int32_t* counts, int32_t* offsets, int32_t* sorted,
                                  int32_t* pos, int32_t* tile_expert, int32_t* n_tiles, int32_t* wide,
                                  int32_t* n_wide, hipStream_t st);
hipError_t moe_k_topk_quant(int x_dtype, const float* partial, const float* bias, const void* x, int T, int H, int E,
                            int K, int quant, int mx, int32_t* ids, float* w, uint8_t* xq, uint8_t* xs,
                            hipStream_t st);

// sort.hip. wide / n_wide (nullable): the prefill GEMMs' list of wide tiles,
// (first tile << 1) | (a second tile of the same expert follows), and its
// length: at most (n_tiles + E) / 2 + 1 entries.
size_t moe_k_sort_scratch_bytes(int P, int E);
hipError_t moe_k_sort(const int32_t* ids, int P, int E, int block_m, int32_t* counts, int32_t* offsets,
                      int32_t* sorted, int32_t* pos, int32_t* tile_expert, int32_t* n_tiles, int32_t* wide,
                      int32_t* n_wide, void* scratch, hipStream_t st);

hipError_t moe_k_copy_routing(const int32_t* ids_in, const float* w_in, int P, int E, int32_t* ids, float* w,
                              hipStream_t st);

// quant.hip
hipError_t moe_k_quant_int8(int in_dtype, const void* v, int rows, int K, int out_fp8pair, void* q, float* scales,
                            const int32_t* sorted, int P, const int32_t* n_rows, hipStream_t st);
hipError_t moe_k_quant_mxfp4(int in_dtype, const void* v, int rows, int K, uint8_t* codes, uint8_t* scales,
                             hipStream_t st);
hipError_t moe_k_fp8pair_to_int8(const uint8_t* src, const float* src_s, int K, const int32_t* row_of, int nrows,
                                 int8_t* q, float* s, hipStream_t st);
hipError_t moe_k_gather_rows(const void* src, int row_bytes, const int32_t* row_of, int nrows, void* dst,
                             hipStream_t st);

// gemm_decode.hip (canon: weights in the canonical row-major layout instead
// of the prepacked one)
int moe_k_decode_block_m();
hipError_t moe_k_decode_gate_up(int canon, const uint8_t* wq, const uint8_t* wsc, const uint8_t* x8, const float* xs,
                                const int32_t* sorted, const int32_t* tile_expert, const int32_t* n_tiles,
                                int max_tiles, int H, int I, int top_k, int P, float* a, hipStream_t st);
hipError_t moe_k_requant_rows(const float* a, int I, const int32_t* pos, int P, uint8_t* aq8, float* as,
                              hipStream_t st);
hipError_t moe_k_decode_down(int canon, const uint8_t* wq, const uint8_t* wsc, const uint8_t* aq8, const float* as,
                             const int32_t* sorted, const int32_t* tile_expert, const int32_t* n_tiles, int max_tiles,
                             int H, int I, int top_k, int P, float* y, hipStream_t st);

// gemm_prefill.hip
int moe_k_prefill_block_m();
// (wide / n_wide: the sort's wide-tile list; max_wide: the grid's bound on its
// length)
hipError_t moe_k_prefill_gemm(int gate_up, int canon, const uint8_t* wq, const uint8_t* wsc, const uint8_t* act_codes,
                              const uint8_t* act_scales, const int32_t* sorted, const int32_t* tile_expert,
                              const int32_t* wide, const int32_t* n_wide, int max_wide, int K, int NT, int top_k,
                              int P, int rows_are_tokens, uint8_t* aq, uint8_t* as, float* y, int out_n,
                              hipStream_t st);

// combine.hip
hipError_t moe_k_combine(const float* y, const float* w, int T, int H, int K, float* out, hipStream_t st);
hipError_t moe_k_rmsnorm(const float* x, int T, int H, float* out, hipStream_t st);
hipError_t moe_k_residual(float* x, const float* y, int64_t n, hipStream_t st);
hipError_t moe_k_combine_residual_norm(const float* y, const float* w, int T, int H, int K, float* x,
                                       float* layer_out, float* xn, hipStream_t st);

// gemm_dense.hip: block-scaled FP8 (MXFP8) dense projection y[M][N] =
// x[M][K] w[N][K]^T. M <= 32 runs the small-batch kernel on an operand-packed
// token tile (moe_k_quant_mxfp8 with packed, or moe_k_dense_pack; 32 rows)
// and needs part (moe_k_dense_partial_bytes) when it splits K over
// workgroups; larger M runs the wide kernel on canonical token rows. packed_w:
// weights in the operand-packed layout of moe_k_dense_pack.
int moe_k_dense_block_n();
int moe_k_dense_split(int M, int N, int K);
int moe_k_dense_wide_rows(int M, int N);
size_t moe_k_dense_partial_bytes(int M, int N, int K);
size_t moe_k_dense_packed_scale_bytes(int R, int K);
hipError_t moe_k_quant_mxfp8(int in_dtype, const void* v, int rows, int K, int packed, uint8_t* codes,
                             uint8_t* scales, hipStream_t st);
hipError_t moe_k_dense_pack(int to_packed, int R, int rows_valid, int K, const uint8_t* src_c, const uint8_t* src_s,
                            uint8_t* dst_c, uint8_t* dst_s, hipStream_t st);
hipError_t moe_k_dense_fp8_gemm(int packed_w, const uint8_t* xq, const uint8_t* xs, const uint8_t* wq,
                                const uint8_t* ws, int M, int N, int K, float* y, float* part, hipStream_t st);
