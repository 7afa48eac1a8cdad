// C ABI of the routed-MoE layer: argument checks, workspace plan, launches.
// Everything here runs on the host; every computation runs in the kernels.
#include <string.h>

#include <mutex>

#include "../../include/fp4moe.h"
#include "kernels.h"

// Scratch of moe_forward_noalloc: one fixed array per device, allocated with
// the code object when the library is loaded on that device and held until
// the process ends. Host code never uses this name as an address; it uses
// the per-device address from hipGetSymbolAddress (scratch_address below).
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return MOE_ERR_HIP;
}

#define MOE_TRY(call)                            \
  do {                                           \
    hipError_t e_ = (call);                      \
    if (e_ != hipSuccess) return hip_fail(e_);   \
  } while (0)

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
size_t up256(size_t n) { return (n + 255) / 256 * 256; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

int check_shape(const moe_config* c) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->x_dtype != MOE_X_F32 && c->x_dtype != MOE_X_BF16) return MOE_ERR_INVALID_ARG;
  if (c->act_mode != MOE_ACT_INT8 && c->act_mode != MOE_ACT_MXFP4) return MOE_ERR_INVALID_ARG;
  if (c->weight_layout != MOE_LAYOUT_CANONICAL && c->weight_layout != MOE_LAYOUT_PREPACKED) return MOE_ERR_INVALID_ARG;
  const int bm = c->act_mode == MOE_ACT_MXFP4 ? moe_k_prefill_block_m() : moe_k_decode_block_m();
  if (c->block_m != 0 && c->block_m != bm) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (c->T < 0 || c->T > (1 << 20)) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (c->H < 256 || c->H > 16384 || c->H % 256) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (c->I < 128 || c->I > 16384 || c->I % 128) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (c->E < 1 || c->E > 1024) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (c->top_k < 1 || c->top_k > 16 || c->top_k > c->E) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (c->act_mode == MOE_ACT_MXFP4) {
    // the prefill GEMMs address activation rows with 32-bit byte offsets:
    // tokens x H/2 (gate/up) and padded pair rows x I/2 (down) stay below 2^32
    const uint64_t P = (uint64_t)c->T * c->top_k;
    const uint64_t cap = P + (uint64_t)(c->E < (int64_t)P ? c->E : P) * (bm - 1);
    if ((uint64_t)c->T * (c->H / 2) >= (1ull << 32) || cap * (c->I / 2) >= (1ull << 32))
      return MOE_ERR_UNSUPPORTED_SHAPE;
  }
  return MOE_OK;
}

// Workspace plan of one layer call.
struct Plan {
  int block_m, P, cap, max_tiles, max_wide;
  size_t logits, ids, w, xq, xs, counts, offsets, sorted, pos, tiles, ntiles, wide, nwide, sort_scratch, a, aq, as, y,
      total;
};

Plan make_plan(const moe_config* c) {
  Plan p;
  const int T = c->T, H = c->H, I = c->I, E = c->E, k = c->top_k;
  const bool mx = c->act_mode == MOE_ACT_MXFP4;
  p.block_m = mx ? moe_k_prefill_block_m() : moe_k_decode_block_m();
  p.P = T * k;
  p.cap = p.P + (E < p.P ? E : p.P) * (p.block_m - 1);
  p.max_tiles = p.cap / p.block_m;
  // wide tiles of the prefill GEMMs: ceil(tiles / 2) per expert with pairs
  p.max_wide = mx ? (p.max_tiles + (E < p.P ? E : p.P)) / 2 + 1 : 0;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += up256(bytes);
    return o;
  };
  p.logits = take(moe_k_router_partial_bytes(T, H, E, k));
  p.ids = take((size_t)p.P * 4);
  p.w = take((size_t)p.P * 4);
  p.xq = take(mx ? (size_t)T * H / 2 : (size_t)T * 2 * H);
  p.xs = take(mx ? (size_t)T * H / 32 : (size_t)T * 4);
  p.counts = take((size_t)E * 4);
  p.offsets = take((size_t)(E + 1) * 4);
  p.sorted = take((size_t)p.cap * 4);
  p.pos = take((size_t)p.P * 4);
  p.tiles = take((size_t)(p.max_tiles + 1) * 4);
  p.ntiles = take(4);
  p.wide = take((size_t)(p.max_wide + 1) * 4);
  p.nwide = take(4);
  p.sort_scratch = take(moe_k_sort_scratch_bytes(p.P, E));
  p.a = take(mx ? 0 : (size_t)p.cap * I * 4);
  p.aq = take(mx ? (size_t)p.cap * I / 2 : (size_t)p.cap * 2 * I);
  p.as = take(mx ? (size_t)p.cap * I / 32 : (size_t)p.cap * 4);
  p.y = take((size_t)p.P * H * 4);
  p.total = off;
  return p;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(ws) + off);
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return FP4MOE_ABI_VERSION; }

const char* moe_status_string(int s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case MOE_ERR_ALIGNMENT: return "misaligned pointer";
    case MOE_ERR_ALIAS: return "output overlaps an input";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

int moe_last_hip_error(void) { return g_last_hip_error; }

int moe_workspace_size(const moe_config* cfg, size_t* bytes) {
  int st = check_shape(cfg);
  if (st) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = make_plan(cfg).total;
  return MOE_OK;
}

int moe_prepacked_size(int32_t which, int32_t E, int32_t N, int32_t K, size_t* code_bytes, size_t* scale_bytes) {
  if (which != MOE_W13 && which != MOE_W2) return MOE_ERR_INVALID_ARG;
  if (!code_bytes || !scale_bytes) return MOE_ERR_INVALID_ARG;
  if (E < 1 || N < 32 || K < 64 || K % 64) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (which == MOE_W13 ? (N % 64) : (N % 32)) return MOE_ERR_UNSUPPORTED_SHAPE;
  *code_bytes = (size_t)E * N * K / 2;
  *scale_bytes = moe_k_packed_scale_bytes(which, E, N, K);
  return MOE_OK;
}

int moe_prepack(int32_t which, int32_t E, int32_t N, int32_t K, const uint8_t* codes, const uint8_t* scales,
                const int32_t* row_perm, uint8_t* packed_codes, uint8_t* packed_scales, void* stream) {
  size_t cb, sb;
  int st = moe_prepacked_size(which, E, N, K, &cb, &sb);
  if (st) return st;
  if (!codes || !scales || !packed_codes || !packed_scales) return MOE_ERR_INVALID_ARG;
  if (!aligned16(codes) || !aligned16(packed_codes) || !aligned16(packed_scales)) return MOE_ERR_ALIGNMENT;
  if (overlaps(codes, cb, packed_codes, cb) || overlaps(scales, (size_t)E * N * K / 32, packed_scales, sb))
    return MOE_ERR_ALIAS;
  MOE_TRY(moe_k_pack(which, E, N, K, codes, scales, row_perm, packed_codes, packed_scales, (hipStream_t)stream));
  return MOE_OK;
}

int moe_unpack(int32_t which, int32_t E, int32_t N, int32_t K, const uint8_t* packed_codes,
               const uint8_t* packed_scales, uint8_t* codes, uint8_t* scales, void* stream) {
  size_t cb, sb;
  int st = moe_prepacked_size(which, E, N, K, &cb, &sb);
  if (st) return st;
  if (!codes || !scales || !packed_codes || !packed_scales) return MOE_ERR_INVALID_ARG;
  if (!aligned16(codes) || !aligned16(packed_codes) || !aligned16(packed_scales)) return MOE_ERR_ALIGNMENT;
  if (overlaps(codes, cb, packed_codes, cb) || overlaps(scales, (size_t)E * N * K / 32, packed_scales, sb))
    return MOE_ERR_ALIAS;
  MOE_TRY(moe_k_unpack(which, E, N, K, packed_codes, packed_scales, codes, scales, (hipStream_t)stream));
  return MOE_OK;
}

int moe_route(const moe_config* cfg, const void* x, const float* router_w, const float* router_bias,
              int32_t* topk_ids, float* topk_w, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_shape(cfg);
  if (st) return st;
  if (cfg->T == 0) return MOE_OK;
  if (!x || !router_w || !topk_ids || !topk_w || !workspace) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(router_w) || ((uintptr_t)workspace & 255)) return MOE_ERR_ALIGNMENT;
  Plan p = make_plan(cfg);
  if (workspace_bytes < p.logits + moe_k_router_partial_bytes(cfg->T, cfg->H, cfg->E, cfg->top_k))
    return MOE_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t s = (hipStream_t)stream;
  float* partial = at<float>(workspace, p.logits);
  MOE_TRY(moe_k_router_partial(cfg->x_dtype, x, router_w, partial, cfg->T, cfg->H, cfg->E, cfg->top_k, 0, nullptr,
                               nullptr, s));
  MOE_TRY(moe_k_topk_quant(cfg->x_dtype, partial, router_bias, x, cfg->T, cfg->H, cfg->E, cfg->top_k, 0, 0, topk_ids,
                           topk_w, nullptr, nullptr, s));
  return MOE_OK;
}

int moe_router_logits(const moe_config* cfg, const void* x, const float* router_w, const float* router_bias,
                      float* logits, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_shape(cfg);
  if (st) return st;
  if (cfg->T == 0) return MOE_OK;
  if (!x || !router_w || !logits || !workspace) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(router_w) || ((uintptr_t)workspace & 255)) return MOE_ERR_ALIGNMENT;
  Plan p = make_plan(cfg);
  const size_t need = p.logits + moe_k_router_partial_bytes(cfg->T, cfg->H, cfg->E, cfg->top_k);
  if (workspace_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (overlaps(workspace, need, logits, (size_t)cfg->T * cfg->E * 4)) return MOE_ERR_ALIAS;
  hipStream_t s = (hipStream_t)stream;
  float* partial = at<float>(workspace, p.logits);
  MOE_TRY(moe_k_router_partial(cfg->x_dtype, x, router_w, partial, cfg->T, cfg->H, cfg->E, cfg->top_k, 0, nullptr,
                               nullptr, s));
  MOE_TRY(moe_k_finish_logits(partial, router_bias, cfg->T, cfg->H, cfg->E, cfg->top_k, logits, s));
  return MOE_OK;
}

int moe_sort(const moe_config* cfg, int32_t block_m, const int32_t* topk_ids, int32_t* counts, int32_t* offsets,
             int32_t* sorted_pairs, int32_t* pair_pos, int32_t* tile_expert, int32_t* n_tiles, void* workspace,
             size_t workspace_bytes, void* stream) {
  int st = check_shape(cfg);
  if (st) return st;
  if (block_m < 1 || block_m > 1024) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (!counts || !offsets || !tile_expert || !n_tiles) return MOE_ERR_INVALID_ARG;
  const int P = cfg->T * cfg->top_k;
  if (P > 0 && (!topk_ids || !sorted_pairs || !pair_pos)) return MOE_ERR_INVALID_ARG;
  size_t scratch = moe_k_sort_scratch_bytes(P, cfg->E);
  if (scratch && !workspace) return MOE_ERR_INVALID_ARG;
  if (scratch && ((uintptr_t)workspace & 255)) return MOE_ERR_ALIGNMENT;
  if (workspace_bytes < scratch) return MOE_ERR_WORKSPACE_TOO_SMALL;
  MOE_TRY(moe_k_sort(topk_ids, P, cfg->E, block_m, counts, offsets, sorted_pairs, pair_pos, tile_expert, n_tiles,
                     nullptr, nullptr,
                     workspace, (hipStream_t)stream));
  return MOE_OK;
}

int moe_quantize(const moe_config* cfg, int32_t rows, int32_t K, int32_t in_dtype, const void* v, void* q,
                 void* scales, void* stream) {
  if (!cfg) return MOE_ERR_INVALID_ARG;
  if (cfg->act_mode != MOE_ACT_INT8 && cfg->act_mode != MOE_ACT_MXFP4) return MOE_ERR_INVALID_ARG;
  if (in_dtype != MOE_X_F32 && in_dtype != MOE_X_BF16) return MOE_ERR_INVALID_ARG;
  if (rows < 0 || K < 64 || K % 64 || K > 65536) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (rows == 0) return MOE_OK;
  if (!v || !q || !scales) return MOE_ERR_INVALID_ARG;
  if (!aligned16(v) || !aligned16(q)) return MOE_ERR_ALIGNMENT;
  hipStream_t s = (hipStream_t)stream;
  if (cfg->act_mode == MOE_ACT_INT8)
    MOE_TRY(moe_k_quant_int8(in_dtype, v, rows, K, 0, q, (float*)scales, nullptr, 0, nullptr, s));
  else
    MOE_TRY(moe_k_quant_mxfp4(in_dtype, v, rows, K, (uint8_t*)q, (uint8_t*)scales, s));
  return MOE_OK;
}

namespace {
// The layer; with combine == false it stops after the down GEMM, leaving y
// (per pair) and the routing weights in the workspace (the stack fuses the
// combine with the residual update and the next layer's RMSNorm).
int forward_impl(const moe_config* cfg, const void* x, const float* router_w, const float* router_bias,
                 const uint8_t* w13, const uint8_t* w13_scale, const uint8_t* w2, const uint8_t* w2_scale, float* out,
                 int32_t* topk_ids_out, float* topk_w_out, const moe_taps* taps, void* workspace,
                 size_t workspace_bytes, void* stream, bool combine, const int32_t* given_ids = nullptr,
                 const float* given_w = nullptr);
}  // namespace

int moe_forward_taps(const moe_config* cfg, const void* x, const float* router_w, const float* router_bias,
                     const uint8_t* w13, const uint8_t* w13_scale, const uint8_t* w2, const uint8_t* w2_scale,
                     float* out, int32_t* topk_ids_out, float* topk_w_out, const moe_taps* taps, void* workspace,
                     size_t workspace_bytes, void* stream) {
  return forward_impl(cfg, x, router_w, router_bias, w13, w13_scale, w2, w2_scale, out, topk_ids_out, topk_w_out,
                      taps, workspace, workspace_bytes, stream, true);
}

}  // extern "C"

namespace {
int forward_impl(const moe_config* cfg, const void* x, const float* router_w, const float* router_bias,
                 const uint8_t* w13, const uint8_t* w13_scale, const uint8_t* w2, const uint8_t* w2_scale, float* out,
                 int32_t* topk_ids_out, float* topk_w_out, const moe_taps* taps, void* workspace,
                 size_t workspace_bytes, void* stream, bool combine, const int32_t* given_ids,
                 const float* given_w) {
  int st = check_shape(cfg);
  if (st) return st;
  if (cfg->T == 0) return MOE_OK;
  const bool routed = given_ids != nullptr;
  if (!x || !w13 || !w13_scale || !w2 || !w2_scale || !out || !workspace) return MOE_ERR_INVALID_ARG;
  if (routed ? !given_w : !router_w) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || (!routed && !aligned16(router_w)) || !aligned16(w13) || !aligned16(w13_scale) ||
      !aligned16(w2) || !aligned16(w2_scale) || !aligned16(out) || ((uintptr_t)workspace & 255))
    return MOE_ERR_ALIGNMENT;
  const int T = cfg->T, H = cfg->H, I = cfg->I, E = cfg->E, k = cfg->top_k;
  const bool mx = cfg->act_mode == MOE_ACT_MXFP4;
  const size_t xbytes = (size_t)T * H * (cfg->x_dtype == MOE_X_F32 ? 4 : 2);
  if (overlaps(out, (size_t)T * H * 4, x, xbytes)) return MOE_ERR_ALIAS;
  Plan p = make_plan(cfg);
  if (workspace_bytes < p.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (overlaps(workspace, p.total, x, xbytes) || overlaps(workspace, p.total, out, (size_t)T * H * 4))
    return MOE_ERR_ALIAS;
  // int8 taps convert the FP8 hi/lo planes with the row scales: both or none
  if (taps && !mx && ((!taps->xq) != (!taps->xs) || (!taps->aq) != (!taps->as))) return MOE_ERR_INVALID_ARG;
  const int canon = cfg->weight_layout == MOE_LAYOUT_CANONICAL;

  hipStream_t s = (hipStream_t)stream;
  float* logits = at<float>(workspace, p.logits);
  int32_t* ids = topk_ids_out && !routed ? topk_ids_out : at<int32_t>(workspace, p.ids);
  float* w = topk_w_out && !routed ? topk_w_out : at<float>(workspace, p.w);
  uint8_t* xq = at<uint8_t>(workspace, p.xq);
  void* xs = at<void>(workspace, p.xs);
  int32_t* counts = at<int32_t>(workspace, p.counts);
  int32_t* offsets = at<int32_t>(workspace, p.offsets);
  int32_t* sorted = at<int32_t>(workspace, p.sorted);
  int32_t* pos = at<int32_t>(workspace, p.pos);
  int32_t* tiles = at<int32_t>(workspace, p.tiles);
  int32_t* ntiles = at<int32_t>(workspace, p.ntiles);
  int32_t* wide = mx ? at<int32_t>(workspace, p.wide) : nullptr;
  int32_t* nwide = mx ? at<int32_t>(workspace, p.nwide) : nullptr;
  void* sort_scratch = at<void>(workspace, p.sort_scratch);
  float* a = at<float>(workspace, p.a);
  uint8_t* aq = at<uint8_t>(workspace, p.aq);
  void* as = at<void>(workspace, p.as);
  float* y = at<float>(workspace, p.y);
  const int P = p.P;
  void* const* ev = taps ? taps->events : nullptr;
  auto mark = [&](int i) -> hipError_t { return ev && ev[i] ? hipEventRecord((hipEvent_t)ev[i], s) : hipSuccess; };


  // small batches whose routing and sort fit one workgroup run them in one
  // kernel (the top-k stage), and the sort stage is empty
  const bool route_sorts = !routed && moe_k_route_sort_fits(T, H, E, k);
  if (!routed) {
    // route: partial logits, then top-k with the quantization of x
    MOE_TRY(mark(2 * MOE_STAGE_ROUTER));
    // small batches quantize x in the router's launch (off the top-k
    // kernel's critical path), larger ones in the top-k kernel
    const bool qr = moe_k_router_quantizes_x(T, H, E, k);
    MOE_TRY(moe_k_router_partial(cfg->x_dtype, x, router_w, logits, T, H, E, k, mx, qr ? xq : nullptr,
                                 qr ? (uint8_t*)xs : nullptr, s));
    MOE_TRY(mark(2 * MOE_STAGE_ROUTER + 1));
    MOE_TRY(mark(2 * MOE_STAGE_TOPK));
    if (route_sorts)
      MOE_TRY(moe_k_route_sort_small(logits, router_bias, T, E, k, p.block_m, ids, w, counts, offsets, sorted, pos,
                                     tiles, ntiles, wide, nwide, s));
    else
      MOE_TRY(moe_k_topk_quant(cfg->x_dtype, logits, router_bias, x, T, H, E, k, qr ? 0 : 1, mx, ids, w, xq,
                               (uint8_t*)xs, s));
    MOE_TRY(mark(2 * MOE_STAGE_TOPK + 1));
    MOE_TRY(mark(2 * MOE_STAGE_QUANT_X));  // in the router launch or the top-k kernel
    MOE_TRY(mark(2 * MOE_STAGE_QUANT_X + 1));
  } else {
    // the caller's routing (ids clamped into [0, E) so that no id addresses
    // memory outside the per-expert arrays), then the quantization of x
    MOE_TRY(mark(2 * MOE_STAGE_ROUTER));
    MOE_TRY(mark(2 * MOE_STAGE_ROUTER + 1));
    MOE_TRY(mark(2 * MOE_STAGE_TOPK));
    MOE_TRY(moe_k_copy_routing(given_ids, given_w, P, E, ids, w, s));
    MOE_TRY(mark(2 * MOE_STAGE_TOPK + 1));
    MOE_TRY(mark(2 * MOE_STAGE_QUANT_X));
    if (mx)
      MOE_TRY(moe_k_quant_mxfp4(cfg->x_dtype, x, T, H, xq, (uint8_t*)xs, s));
    else
      MOE_TRY(moe_k_quant_int8(cfg->x_dtype, x, T, H, 1, xq, (float*)xs, nullptr, 0, nullptr, s));
    MOE_TRY(mark(2 * MOE_STAGE_QUANT_X + 1));
  }
  // sort
  MOE_TRY(mark(2 * MOE_STAGE_SORT));
  if (!route_sorts)
    MOE_TRY(moe_k_sort(ids, P, E, p.block_m, counts, offsets, sorted, pos, tiles, ntiles, wide, nwide, sort_scratch,
                       s));
  MOE_TRY(mark(2 * MOE_STAGE_SORT + 1));
  // expert GEMMs
  if (mx) {
    MOE_TRY(mark(2 * MOE_STAGE_GATE_UP));
    MOE_TRY(moe_k_prefill_gemm(1, canon, w13, w13_scale, xq, (const uint8_t*)xs, sorted, tiles, wide, nwide,
                               p.max_wide, H,
                               I / 32, k, P, 1, aq, (uint8_t*)as, nullptr, I, s));
    MOE_TRY(mark(2 * MOE_STAGE_GATE_UP + 1));
    MOE_TRY(mark(2 * MOE_STAGE_REQUANT));
    MOE_TRY(mark(2 * MOE_STAGE_REQUANT + 1));
    MOE_TRY(mark(2 * MOE_STAGE_DOWN));
    MOE_TRY(moe_k_prefill_gemm(0, canon, w2, w2_scale, aq, (const uint8_t*)as, sorted, tiles, wide, nwide,
                               p.max_wide, I,
                               H / 32, k, P, 0, nullptr, nullptr, y, H, s));
    MOE_TRY(mark(2 * MOE_STAGE_DOWN + 1));
    MOE_TRY(mark(2 * MOE_STAGE_COMBINE));
    if (combine) MOE_TRY(moe_k_combine(y, w, T, H, k, out, s));
    MOE_TRY(mark(2 * MOE_STAGE_COMBINE + 1));
  } else {
    MOE_TRY(mark(2 * MOE_STAGE_GATE_UP));
    MOE_TRY(moe_k_decode_gate_up(canon, w13, w13_scale, xq, (const float*)xs, sorted, tiles, ntiles, p.max_tiles, H, I, k,
                                 P, a, s));
    MOE_TRY(mark(2 * MOE_STAGE_GATE_UP + 1));
    MOE_TRY(mark(2 * MOE_STAGE_REQUANT));
    MOE_TRY(moe_k_requant_rows(a, I, pos, P, aq, (float*)as, s));
    MOE_TRY(mark(2 * MOE_STAGE_REQUANT + 1));
    MOE_TRY(mark(2 * MOE_STAGE_DOWN));
    MOE_TRY(moe_k_decode_down(canon, w2, w2_scale, aq, (const float*)as, sorted, tiles, ntiles, p.max_tiles, H, I, k, P, y,
                              s));
    MOE_TRY(mark(2 * MOE_STAGE_DOWN + 1));
    MOE_TRY(mark(2 * MOE_STAGE_COMBINE));
    if (combine) MOE_TRY(moe_k_combine(y, w, T, H, k, out, s));
    MOE_TRY(mark(2 * MOE_STAGE_COMBINE + 1));
  }

  if (taps) {
    if (taps->block_m) *taps->block_m = p.block_m;
    if (mx) {
      if (taps->xq) MOE_TRY(hipMemcpyAsync(taps->xq, xq, (size_t)T * H / 2, hipMemcpyDeviceToDevice, s));
      if (taps->xs) MOE_TRY(hipMemcpyAsync(taps->xs, xs, (size_t)T * H / 32, hipMemcpyDeviceToDevice, s));
      if (taps->aq) MOE_TRY(moe_k_gather_rows(aq, I / 2, pos, P, taps->aq, s));
      if (taps->as) MOE_TRY(moe_k_gather_rows(as, I / 32, pos, P, taps->as, s));
    } else {
      if (taps->xq) {
        MOE_TRY(moe_k_fp8pair_to_int8(xq, (const float*)xs, H, nullptr, T, (int8_t*)taps->xq, (float*)taps->xs, s));
      }
      if (taps->aq) {
        MOE_TRY(moe_k_fp8pair_to_int8(aq, (const float*)as, I, pos, P, (int8_t*)taps->aq, (float*)taps->as, s));
      }
    }
    if (taps->y) MOE_TRY(hipMemcpyAsync(taps->y, y, (size_t)P * H * 4, hipMemcpyDeviceToDevice, s));
    if (taps->counts) MOE_TRY(hipMemcpyAsync(taps->counts, counts, (size_t)E * 4, hipMemcpyDeviceToDevice, s));
    if (taps->offsets)
      MOE_TRY(hipMemcpyAsync(taps->offsets, offsets, (size_t)(E + 1) * 4, hipMemcpyDeviceToDevice, s));
    if (taps->sorted_pairs)
      MOE_TRY(hipMemcpyAsync(taps->sorted_pairs, sorted, (size_t)p.cap * 4, hipMemcpyDeviceToDevice, s));
    if (taps->pair_pos) MOE_TRY(hipMemcpyAsync(taps->pair_pos, pos, (size_t)P * 4, hipMemcpyDeviceToDevice, s));
  }
  return MOE_OK;
}
}  // namespace

extern "C" {

int moe_forward(const moe_config* cfg, const void* x, const float* router_w, const float* router_bias,
                const uint8_t* w13, const uint8_t* w13_scale, const uint8_t* w2, const uint8_t* w2_scale, float* out,
                int32_t* topk_ids_out, float* topk_w_out, void* workspace, size_t workspace_bytes, void* stream) {
  return moe_forward_taps(cfg, x, router_w, router_bias, w13, w13_scale, w2, w2_scale, out, topk_ids_out, topk_w_out,
                          nullptr, workspace, workspace_bytes, stream);
}

int moe_forward_routed(const moe_config* cfg, const void* x, const int32_t* topk_ids, const float* topk_w,
                       const uint8_t* w13, const uint8_t* w13_scale, const uint8_t* w2, const uint8_t* w2_scale,
                       float* out, const moe_taps* taps, void* workspace, size_t workspace_bytes, void* stream) {
  if (cfg && cfg->T > 0 && (!topk_ids || !topk_w)) return MOE_ERR_INVALID_ARG;
  return forward_impl(cfg, x, nullptr, nullptr, w13, w13_scale, w2, w2_scale, out, nullptr, nullptr, taps, workspace,
                      workspace_bytes, stream, true, topk_ids, topk_w);
}

namespace {
constexpr int kNoallocMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kNoallocMaxDevices];

// The device address of `scratch` on the current device, looked up once per
// device with that device current (each device holds its own copy).
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kNoallocMaxDevices) return hip_fail(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace

int moe_forward_noalloc(const moe_config* cfg, const void* x, const float* router_w, const float* router_bias,
                        const uint8_t* w13, const uint8_t* w13_scale, const uint8_t* w2, const uint8_t* w2_scale,
                        float* out, int32_t* topk_ids_out, float* topk_w_out, void* stream) {
  int st = check_shape(cfg);
  if (st) return st;
  if (make_plan(cfg).total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (cfg->T == 0) return MOE_OK;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st) return st;
  return forward_impl(cfg, x, router_w, router_bias, w13, w13_scale, w2, w2_scale, out, topk_ids_out, topk_w_out,
                      nullptr, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream, true);
}

int moe_stack_workspace_size(const moe_config* cfg, size_t* bytes) {
  int st = check_shape(cfg);
  if (st) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = make_plan(cfg).total + 2 * up256((size_t)cfg->T * cfg->H * 4);
  return MOE_OK;
}
int moe_forward_stack(const moe_config* cfg, int32_t L, float* x, const float* const* router_w,
                      const float* const* router_bias, const uint8_t* const* w13, const uint8_t* const* w13_scale,
                      const uint8_t* const* w2, const uint8_t* const* w2_scale, float* layer_out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return moe_forward_stack_taps(cfg, L, x, router_w, router_bias, w13, w13_scale, w2, w2_scale, layer_out, nullptr,
                                workspace, workspace_bytes, stream);
}
int moe_forward_stack_taps(const moe_config* cfg, int32_t L, float* x, const float* const* router_w,
                           const float* const* router_bias, const uint8_t* const* w13,
                           const uint8_t* const* w13_scale, const uint8_t* const* w2, const uint8_t* const* w2_scale,
                           float* layer_out, const moe_taps* taps, void* workspace, size_t workspace_bytes,
                           void* stream) {
  int st = check_shape(cfg);
  if (st) return st;
  if (cfg->x_dtype != MOE_X_F32) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (L < 0) return MOE_ERR_INVALID_ARG;
  if (L == 0 || cfg->T == 0) return MOE_OK;
  if (!x || !router_w || !w13 || !w13_scale || !w2 || !w2_scale || !workspace) return MOE_ERR_INVALID_ARG;
  const size_t fw = make_plan(cfg).total, nb = (size_t)cfg->T * cfg->H * 4;
  const size_t need = fw + 2 * up256(nb);
  if (workspace_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned16(x) || (layer_out && !aligned16(layer_out)) || ((uintptr_t)workspace & 255)) return MOE_ERR_ALIGNMENT;
  if (overlaps(workspace, need, x, nb) || (layer_out && overlaps(workspace, need, layer_out, nb * L)) ||
      (layer_out && overlaps(x, nb, layer_out, nb * L)))
    return MOE_ERR_ALIAS;
  for (int l = 0; l < L; ++l) {
    if (!router_w[l] || !w13[l] || !w13_scale[l] || !w2[l] || !w2_scale[l]) return MOE_ERR_INVALID_ARG;
    if (taps && cfg->act_mode == MOE_ACT_INT8 &&
        ((!taps[l].xq) != (!taps[l].xs) || (!taps[l].aq) != (!taps[l].as)))
      return MOE_ERR_INVALID_ARG;
  }
  hipStream_t s = (hipStream_t)stream;
  float* xn = at<float>(workspace, fw);
  float* ybuf = at<float>(workspace, fw + up256(nb));
  const Plan p = make_plan(cfg);
  const float* ypair = at<float>(workspace, p.y);
  const float* wts = at<float>(workspace, p.w);
  // x_{l+1} = x_l + moe_l(rmsnorm(x_l)): the first RMSNorm stands alone, each
  // layer's combine, residual update and the next layer's RMSNorm are fused
  MOE_TRY(moe_k_rmsnorm(x, cfg->T, cfg->H, xn, s));
  for (int l = 0; l < L; ++l) {
    float* yl = layer_out ? layer_out + (size_t)l * cfg->T * cfg->H : ybuf;
    st = forward_impl(cfg, xn, router_w[l], router_bias ? router_bias[l] : nullptr, w13[l], w13_scale[l], w2[l],
                      w2_scale[l], yl, nullptr, nullptr, taps ? &taps[l] : nullptr, workspace, fw, stream, false);
    if (st) return st;
    MOE_TRY(moe_k_combine_residual_norm(ypair, wts, cfg->T, cfg->H, cfg->top_k, x, layer_out ? yl : nullptr,
                                        l + 1 < L ? xn : nullptr, s));
  }
  return MOE_OK;
}
int moe_rmsnorm(int32_t T, int32_t H, const float* x, float* out, void* stream) {
  if (T < 0 || H < 64 || H % 64 || H > 65536) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (T == 0) return MOE_OK;
  if (!x || !out) return MOE_ERR_INVALID_ARG;
  if (overlaps(x, (size_t)T * H * 4, out, (size_t)T * H * 4)) return MOE_ERR_ALIAS;
  MOE_TRY(moe_k_rmsnorm(x, T, H, out, (hipStream_t)stream));
  return MOE_OK;
}

int moe_residual_add(int64_t n, float* x, const float* y, void* stream) {
  if (n < 0) return MOE_ERR_INVALID_ARG;
  if (n == 0) return MOE_OK;
  if (!x || !y) return MOE_ERR_INVALID_ARG;
  MOE_TRY(moe_k_residual(x, y, n, (hipStream_t)stream));
  return MOE_OK;
}

}  // extern "C"

// ------------------------------------------------------------ dense FP8 ----
namespace {

int check_dense(const moe_dense_config* c) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->x_dtype != MOE_X_F32 && c->x_dtype != MOE_X_BF16) return MOE_ERR_INVALID_ARG;
  if (c->weight_layout != MOE_LAYOUT_CANONICAL && c->weight_layout != MOE_LAYOUT_PREPACKED) return MOE_ERR_INVALID_ARG;
  if (c->M < 0 || c->M > (1 << 20)) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (c->K < 128 || c->K > 32768 || c->K % 128) return MOE_ERR_UNSUPPORTED_SHAPE;
  const int bn = moe_k_dense_block_n();
  if (c->N < bn || c->N > 65536 || c->N % bn) return MOE_ERR_UNSUPPORTED_SHAPE;
  // token rows are addressed with 32-bit byte offsets
  if ((uint64_t)c->M * c->K >= (1ull << 32)) return MOE_ERR_UNSUPPORTED_SHAPE;
  return MOE_OK;
}

bool dense_small(const moe_dense_config* c) { return c->M <= 32; }

// Workspace: the quantized token rows (M <= 32: one operand-packed 32-row
// tile), then the K-split partial sums of the small-batch kernel.
struct DensePlan {
  size_t xq, xs, part, total;
};

DensePlan dense_plan(const moe_dense_config* c) {
  DensePlan p;
  const bool sm = dense_small(c);
  p.xq = 0;
  p.xs = up256(sm ? (size_t)32 * c->K : (size_t)c->M * c->K);
  p.part = p.xs + up256(sm ? moe_k_dense_packed_scale_bytes(32, c->K) : (size_t)c->M * (c->K / 32));
  p.total = p.part + up256(moe_k_dense_partial_bytes(c->M, c->N, c->K));
  return p;
}

size_t dense_w_scale_bytes(const moe_dense_config* c) {
  return c->weight_layout == MOE_LAYOUT_PREPACKED ? moe_k_dense_packed_scale_bytes(c->N, c->K)
                                                  : (size_t)c->N * (c->K / 32);
}

int dense_check_pack_shape(int32_t N, int32_t K) {
  if (K < 128 || K > 32768 || K % 128 || N < 32 || N > 65536 || N % 32) return MOE_ERR_UNSUPPORTED_SHAPE;
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_dense_fp8_workspace_size(const moe_dense_config* cfg, size_t* bytes) {
  const int st = check_dense(cfg);
  if (st) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = dense_plan(cfg).total;
  return MOE_OK;
}

int moe_dense_fp8_quantize(int32_t rows, int32_t K, int32_t in_dtype, const void* v, uint8_t* codes,
                           uint8_t* scales, void* stream) {
  if (in_dtype != MOE_X_F32 && in_dtype != MOE_X_BF16) return MOE_ERR_INVALID_ARG;
  if (rows < 0 || K < 32 || K % 32 || K > 65536) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (rows == 0) return MOE_OK;
  if (!v || !codes || !scales) return MOE_ERR_INVALID_ARG;
  if (!aligned16(v) || !aligned16(codes)) return MOE_ERR_ALIGNMENT;
  MOE_TRY(moe_k_quant_mxfp8(in_dtype, v, rows, K, 0, codes, scales, (hipStream_t)stream));
  return MOE_OK;
}

int moe_dense_fp8_prepacked_size(int32_t N, int32_t K, size_t* code_bytes, size_t* scale_bytes) {
  const int st = dense_check_pack_shape(N, K);
  if (st) return st;
  if (!code_bytes || !scale_bytes) return MOE_ERR_INVALID_ARG;
  *code_bytes = (size_t)N * K;
  *scale_bytes = moe_k_dense_packed_scale_bytes(N, K);
  return MOE_OK;
}

static int dense_pack_entry(int to_packed, int32_t N, int32_t K, const uint8_t* src_c, const uint8_t* src_s,
                            uint8_t* dst_c, uint8_t* dst_s, void* stream) {
  const int st = dense_check_pack_shape(N, K);
  if (st) return st;
  if (!src_c || !src_s || !dst_c || !dst_s) return MOE_ERR_INVALID_ARG;
  if (!aligned16(src_c) || !aligned16(dst_c) || ((uintptr_t)(to_packed ? dst_s : src_s) & 3)) return MOE_ERR_ALIGNMENT;
  const size_t cb = (size_t)N * K, ps = moe_k_dense_packed_scale_bytes(N, K), cs = (size_t)N * (K / 32);
  const size_t sb_src = to_packed ? cs : ps, sb_dst = to_packed ? ps : cs;
  if (overlaps(dst_c, cb, src_c, cb) || overlaps(dst_c, cb, src_s, sb_src) || overlaps(dst_s, sb_dst, src_c, cb) ||
      overlaps(dst_s, sb_dst, src_s, sb_src) || overlaps(dst_c, cb, dst_s, sb_dst))
    return MOE_ERR_ALIAS;
  MOE_TRY(moe_k_dense_pack(to_packed, N, N, K, src_c, src_s, dst_c, dst_s, (hipStream_t)stream));
  return MOE_OK;
}

int moe_dense_fp8_prepack(int32_t N, int32_t K, const uint8_t* w, const uint8_t* w_scale, uint8_t* packed_w,
                          uint8_t* packed_scale, void* stream) {
  return dense_pack_entry(1, N, K, w, w_scale, packed_w, packed_scale, stream);
}

int moe_dense_fp8_unpack(int32_t N, int32_t K, const uint8_t* packed_w, const uint8_t* packed_scale, uint8_t* w,
                         uint8_t* w_scale, void* stream) {
  return dense_pack_entry(0, N, K, packed_w, packed_scale, w, w_scale, stream);
}

int moe_dense_fp8_gemm(const moe_dense_config* cfg, const uint8_t* xq, const uint8_t* xs, const uint8_t* w,
                       const uint8_t* w_scale, float* y, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_dense(cfg);
  if (st) return st;
  if (cfg->M == 0) return MOE_OK;
  if (!xq || !xs || !w || !w_scale || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned16(xq) || !aligned16(xs) || !aligned16(w) || !aligned16(w_scale) || !aligned16(y))
    return MOE_ERR_ALIGNMENT;
  const DensePlan p = dense_plan(cfg);
  const bool sm = dense_small(cfg);
  if (sm && (!workspace || workspace_bytes < p.total)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (sm && ((uintptr_t)workspace & 255)) return MOE_ERR_ALIGNMENT;
  const size_t ybytes = (size_t)cfg->M * cfg->N * 4, wsb = dense_w_scale_bytes(cfg);
  if (overlaps(y, ybytes, xq, (size_t)cfg->M * cfg->K) || overlaps(y, ybytes, xs, (size_t)cfg->M * cfg->K / 32) ||
      overlaps(y, ybytes, w, (size_t)cfg->N * cfg->K) || overlaps(y, ybytes, w_scale, wsb))
    return MOE_ERR_ALIAS;
  if (sm && overlaps(y, ybytes, workspace, p.total)) return MOE_ERR_ALIAS;
  hipStream_t s = (hipStream_t)stream;
  const int pw = cfg->weight_layout == MOE_LAYOUT_PREPACKED;
  if (sm) {  // the small-batch kernel reads the token tile operand-packed
    uint8_t* tq = at<uint8_t>(workspace, p.xq);
    uint8_t* ts = at<uint8_t>(workspace, p.xs);
    MOE_TRY(moe_k_dense_pack(1, 32, cfg->M, cfg->K, xq, xs, tq, ts, s));
    MOE_TRY(moe_k_dense_fp8_gemm(pw, tq, ts, w, w_scale, cfg->M, cfg->N, cfg->K, y, at<float>(workspace, p.part), s));
  } else {
    MOE_TRY(moe_k_dense_fp8_gemm(pw, xq, xs, w, w_scale, cfg->M, cfg->N, cfg->K, y, nullptr, s));
  }
  return MOE_OK;
}

int moe_dense_fp8_forward(const moe_dense_config* cfg, const void* x, const uint8_t* w, const uint8_t* w_scale,
                          float* y, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_dense(cfg);
  if (st) return st;
  if (cfg->M == 0) return MOE_OK;
  if (!x || !w || !w_scale || !y || !workspace) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w) || !aligned16(w_scale) || !aligned16(y) || ((uintptr_t)workspace & 255))
    return MOE_ERR_ALIGNMENT;
  const DensePlan p = dense_plan(cfg);
  if (workspace_bytes < p.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  const size_t ybytes = (size_t)cfg->M * cfg->N * 4, wsb = dense_w_scale_bytes(cfg);
  const size_t xbytes = (size_t)cfg->M * cfg->K * (cfg->x_dtype == MOE_X_F32 ? 4 : 2);
  if (overlaps(y, ybytes, x, xbytes) || overlaps(y, ybytes, w, (size_t)cfg->N * cfg->K) ||
      overlaps(y, ybytes, w_scale, wsb) || overlaps(workspace, p.total, x, xbytes) ||
      overlaps(workspace, p.total, y, ybytes))
    return MOE_ERR_ALIAS;
  hipStream_t s = (hipStream_t)stream;
  uint8_t* xq = at<uint8_t>(workspace, p.xq);
  uint8_t* xs = at<uint8_t>(workspace, p.xs);
  const bool sm = dense_small(cfg);
  MOE_TRY(moe_k_quant_mxfp8(cfg->x_dtype, x, cfg->M, cfg->K, sm ? 1 : 0, xq, xs, s));
  MOE_TRY(moe_k_dense_fp8_gemm(cfg->weight_layout == MOE_LAYOUT_PREPACKED, xq, xs, w, w_scale, cfg->M, cfg->N, cfg->K,
                               y, sm ? at<float>(workspace, p.part) : nullptr, s));
  return MOE_OK;
}

}  // extern "C"
