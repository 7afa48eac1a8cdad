/*
 * fp4moe.h -- C ABI of the routed mixture-of-experts layer with packed FP4
 * experts, written for AMD Instinct MI355X (gfx950, CDNA4).
 *
 * The layer is the routed mixture of experts with FP4 expert weights that
 * the DeepSeek-V4-Flash paper runs on MI250 (DeepSeek-V4-Flash on AMD gfx90a:
 * Correctness Recovery and Inference Performance Engineering, abstract): FP4
 * packed expert weights, int8-quantized activations for decode, a sort of the
 * tokens by expert, and a repair of the weight layout when the weights are
 * loaded. The model facts (256 routed experts, 6 active per token, 43 layers)
 * come from DeepSeek V4 Flash on 8x AMD gfx1201: packaged TP=8 deployment,
 * section What we set out to do.
 *
 * For one batch of T tokens it computes
 *   l[t,e]   = <x[t,:], Wr[e,:]> (+ b[e])               fp32, fixed order
 *   s        = sigmoid(l); the top_k largest per token, ties to the lower
 *              expert; w_j = s_j / sum_j s_j
 *   sort     : stable counting sort of the P = T*top_k (token, slot) pairs
 *   xq       = quant(x)      int8 per token, or MXFP4 (E2M1 + E8M0 per 32)
 *   h        = xq @ W13[e]^T with E2M1 weights, one E8M0 scale per 32 along K
 *   a        = silu(h[:I]) * h[I:],  aq = quant(a)
 *   y        = aq @ W2[e]^T
 *   out[t]   = sum_j w_j * y[t, j]
 *
 * Numerics (identical on every call and every run):
 *   - Router dot products: H is split into 64 contiguous chunks; each chunk is
 *     an fp32 fused-multiply-add chain over ascending k from 0; the 64 chunk
 *     sums are added as a perfect pairwise tree in index order; then the bias
 *     is added. sigmoid(z) = 1 / (1 + exp(-z)) with an exp built only from
 *     IEEE fp32 operations (Cody-Waite reduction by ln 2, degree-7 Taylor
 *     polynomial, exact power-of-two scaling).
 *   - int8 quantization of a row: s = amax / 127, q = clamp(rint(v / s), +-127).
 *   - MXFP4 quantization of 32 values (OCP Microscaling v1.0): scale exponent
 *     floor(log2 amax) - 2 biased by 127; values scaled by an exact power of
 *     two, rounded to nearest-even on the E2M1 grid, saturated at 6; the
 *     code's sign is the value's sign bit.
 *   - GEMM blocks of 32 along K are exact integer sums of code products; the
 *     scaled block sums are accumulated in fp32; an int8 row scale multiplies
 *     the finished sum.
 *   - a = (g * sigmoid(g)) * u; out = fma chain over slots j = 0..top_k-1.
 *
 * Conventions for every call below:
 *   - Array arguments are DEVICE pointers owned by the caller. The library
 *     never allocates or frees device memory in these calls and keeps no
 *     pointer after returning. Scratch memory comes from the caller's
 *     workspace, whose contents are undefined afterwards.
 *   - `stream` is a hipStream_t (NULL = the default stream). Calls only
 *     enqueue work; they never synchronize the stream. Results are ready when
 *     the stream's work has completed.
 *   - Arguments are checked on the host before anything is launched; on any
 *     error nothing is launched and the status says why. Launch failures
 *     return MOE_ERR_HIP with the HIP error code kept per thread
 *     (moe_last_hip_error). Faults inside kernels surface at the caller's
 *     next synchronization. No exception or abort crosses this interface.
 *   - Outputs are fully overwritten and bit-identical from run to run (no
 *     floating-point atomics anywhere).
 *   - Calls may run concurrently on different streams if they use different
 *     workspaces and outputs.
 *   - Shape limits: 1 <= T <= 1<<20, H % 256 == 0, 256 <= H <= 16384,
 *     I % 128 == 0, 128 <= I <= 16384, 1 <= E <= 1024, 1 <= top_k <= min(E, 16);
 *     with MOE_ACT_MXFP4 also T * H/2 < 2^32 and
 *     (T*top_k + min(E, T*top_k) * 63) * I/2 < 2^32 (the prefill GEMMs address
 *     activation rows with 32-bit offsets). T = 0 is accepted and does nothing.
 *   - Alignment: weights, x, out, quantized buffers: 16 bytes.
 */
#ifndef FP4MOE_H
#define FP4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP4MOE_ABI_VERSION 3

/* Status codes returned by every entry point. */
enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,         /* NULL where a pointer is required, bad enum value */
    MOE_ERR_UNSUPPORTED_SHAPE = 2,   /* outside the shape limits above */
    MOE_ERR_ALIGNMENT = 3,           /* a pointer is not 16-byte aligned */
    MOE_ERR_ALIAS = 4,               /* an output overlaps an input */
    MOE_ERR_WORKSPACE_TOO_SMALL = 5, /* workspace_bytes < moe_workspace_size() */
    MOE_ERR_HIP = 6                  /* a HIP call failed; see moe_last_hip_error() */
};

enum moe_x_dtype { MOE_X_F32 = 0, MOE_X_BF16 = 1 };       /* activation element type */
enum moe_act_mode { MOE_ACT_INT8 = 0, MOE_ACT_MXFP4 = 1 }; /* activation quantization */
enum moe_weight { MOE_W13 = 0, MOE_W2 = 1 };               /* which expert matrix */
/* Both layouts give identical results. The canonical rows are read by the
 * kernels 32 rows x 32 bytes a load; the prepacked tiles 1 KB contiguous a
 * load. On MI355X canonical weights ran the 4-token decode layer in about
 * 110 us against 72 us prepacked, the 64-token one in 572 against 298 us and
 * the 4,604-token prefill layer in 1.65 against 1.21 ms: prepack once when
 * the weights are loaded (moe_prepack). */
enum moe_weight_layout {
    MOE_LAYOUT_CANONICAL = 0, /* the interchange layout described under "weights" below */
    MOE_LAYOUT_PREPACKED = 1  /* the MFMA operand layout that moe_prepack writes (faster) */
};

/* Sort block sizes of the expert GEMMs: rows of one expert that one GEMM
 * tile covers (the expert segments of the sort are padded to a multiple). */
#define MOE_BLOCK_M_INT8 16
#define MOE_BLOCK_M_MXFP4 64

/* Layer shape and modes. act_mode selects the quantization of x and of the
 * intermediate activation (it changes the numbers, so it is never chosen
 * automatically): MOE_ACT_INT8 runs the low-M decode kernels, MOE_ACT_MXFP4
 * the scaled-FP4 MFMA grouped GEMM. A zero-initialized tail (block_m = 0,
 * weight_layout = MOE_LAYOUT_CANONICAL) selects the defaults. */
typedef struct moe_config {
    int32_t T;             /* tokens in the batch */
    int32_t H;             /* hidden size */
    int32_t I;             /* expert intermediate size */
    int32_t E;             /* routed experts */
    int32_t top_k;         /* experts per token */
    int32_t x_dtype;       /* enum moe_x_dtype */
    int32_t act_mode;      /* enum moe_act_mode */
    int32_t block_m;       /* 0 = the GEMMs' own (MOE_BLOCK_M_INT8 or MOE_BLOCK_M_MXFP4 for
                              act_mode); any other value must equal it, else
                              MOE_ERR_UNSUPPORTED_SHAPE */
    int32_t weight_layout; /* enum moe_weight_layout of w13/w2 in the forward calls */
} moe_config;

/* Optional copies of intermediate results of moe_forward_taps (any pointer
 * may be NULL). Pair p = t * top_k + j.
 *   xq, xs : quantized x. INT8: int8 [T][H] and fp32 [T]. MXFP4: codes
 *            [T][H/2] (low nibble = even k) and E8M0 bytes [T][H/32].
 *   aq, as : quantized activation per pair, like xq/xs with K = I, P rows.
 *   y      : fp32 [P][H], the down projection of each pair before weighting.
 *   counts, offsets, sorted_pairs, pair_pos : the expert sort used, as
 *            moe_sort returns them for the block size the kernels used
 *            (offsets [E+1]; sorted_pairs [offsets[E]]; pair_pos [P]).
 *   block_m: receives that block size (host int32, may be NULL).
 *   events : NULL, or 2 * MOE_N_STAGES hipEvent_t handles (host array); the
 *            library records events[2*i] on the stream before stage i and
 *            events[2*i+1] after it, so a caller can time each stage on the
 *            stream the kernels run on. A stage that launches nothing for
 *            this configuration records both events back to back. */
enum moe_stage {
    MOE_STAGE_ROUTER = 0,  /* router logits */
    MOE_STAGE_TOPK = 1,    /* sigmoid, top-k, renormalization */
    MOE_STAGE_QUANT_X = 2, /* activation quantization of x */
    MOE_STAGE_SORT = 3,    /* expert sort */
    MOE_STAGE_GATE_UP = 4, /* gate/up GEMM with SiLU*mul (and MXFP4 requant) */
    MOE_STAGE_REQUANT = 5, /* int8 requantization of the activation */
    MOE_STAGE_DOWN = 6,    /* down GEMM */
    MOE_STAGE_COMBINE = 7, /* weighted combine */
    MOE_N_STAGES = 8
};
typedef struct moe_taps {
    void* xq;
    void* xs;
    void* aq;
    void* as;
    float* y;
    int32_t* counts;
    int32_t* offsets;
    int32_t* sorted_pairs;
    int32_t* pair_pos;
    int32_t* block_m;
    void* const* events;
} moe_taps;

/* FP4MOE_ABI_VERSION of the built library. */
int moe_abi_version(void);

/* Static text for a status code (never NULL). */
const char* moe_status_string(int status);

/* The hipError_t of this thread's last MOE_ERR_HIP (0 if none). */
int moe_last_hip_error(void);

/* Bytes of device workspace that moe_route, moe_router_logits, moe_sort,
 * moe_forward, moe_forward_taps and moe_forward_routed need for this
 * configuration (the scratch of the layer of the gfx90a paper's abstract:
 * router partial sums, routing, the expert sort, the quantized activations
 * and the per-pair down projections). The caller allocates it (256-byte
 * aligned base) and may reuse it between calls on one stream.
 * Errors: MOE_ERR_INVALID_ARG (NULL cfg or bytes, bad enum), MOE_ERR_UNSUPPORTED_SHAPE. */
int moe_workspace_size(const moe_config* cfg, size_t* bytes);

/* ---------------------------------------------------------------- weights --
 * Expert weights are packed E2M1 codes with one E8M0 scale per 32 elements
 * along K (the FP4 expert weights of the gfx90a paper's abstract; element
 * and scale formats from OCP Microscaling v1.0).
 * Canonical layout (the interchange format):
 *   W13 (which = MOE_W13, N = 2I rows, K = H): codes [E][2I][H/2], scales
 *       [E][2I][H/32]; rows 0..I-1 are the gate projection, I..2I-1 the up
 *       projection.
 *   W2  (which = MOE_W2, N = H rows, K = I): codes [E][H][I/2], scales
 *       [E][H][I/32].
 *   In a code byte the low nibble is the even element along K.
 * The forward calls read either layout (cfg->weight_layout). The PREPACKED
 * layout that moe_prepack writes is the faster one: tiles of 32 rows x 64 K in
 * the operand order of the gfx950 32x32x64 scaled MFMA (each K-step of a tile
 * is one contiguous 1 KiB), gate and up tiles interleaved, scales grouped four
 * K-steps to a dword. It has the same byte count as the canonical layout (the
 * scales pad to a multiple of four K-steps); moe_unpack inverts the packing.
 *
 * The load-time layout repair of the gfx90a paper (abstract: the routed W2
 * rows were stored in another order than the kernels assumed, and the fix
 * repairs the layout when the weights are loaded) is row_perm: a device
 * int32 [N] permutation, or NULL for the identity, that makes packed row r
 * hold canonical row row_perm[r] of every expert, codes and scales together.
 * A matrix whose rows were stored in the permuted order pi is repaired by
 * passing the inverse permutation. Errors: MOE_ERR_UNSUPPORTED_SHAPE unless
 * K % 64 == 0 and N % 64 == 0 (W13) or N % 32 == 0 (W2); MOE_ERR_ALIGNMENT
 * for code pointers not 16-byte aligned; MOE_ERR_ALIAS when the packed and
 * canonical buffers overlap. row_perm must be a permutation of 0..N-1 (not
 * checked: an entry outside it reads outside the expert's rows). */
int moe_prepacked_size(int32_t which, int32_t E, int32_t N, int32_t K,
                       size_t* code_bytes, size_t* scale_bytes);
int moe_prepack(int32_t which, int32_t E, int32_t N, int32_t K,
                const uint8_t* codes, const uint8_t* scales, const int32_t* row_perm,
                uint8_t* packed_codes, uint8_t* packed_scales, void* stream);
int moe_unpack(int32_t which, int32_t E, int32_t N, int32_t K,
               const uint8_t* packed_codes, const uint8_t* packed_scales,
               uint8_t* codes, uint8_t* scales, void* stream);

/* ---------------------------------------------------------------- router --
 * Sigmoid-score top-k routing: each token picks top_k of the E routed experts
 * (DeepSeek V4 Flash on 8x AMD gfx1201, What we set out to do: 256 routed
 * experts, 6 active per token; the per-token expert selection whose hashes
 * the gfx90a paper checks, abstract).
 *   x          [T][H] fp32 or bf16 (cfg->x_dtype), row-major, 16-byte aligned
 *   router_w   fp32 [E][H], 16-byte aligned
 *   router_bias fp32 [E] or NULL: added to the logit before the sigmoid, so
 *              it moves selection and weights
 *   topk_ids   int32 [T][top_k] out: experts in selection order (highest
 *              score first; equal scores: lower expert first)
 *   topk_w     fp32 [T][top_k] out: S = ((s_0 + s_1) + s_2) + ..., w_j = s_j / S
 *              (1/top_k if S == 0)
 *   workspace  at least moe_workspace_size(cfg) bytes, 256-byte aligned
 * Errors: MOE_ERR_INVALID_ARG (NULL pointer, bad enum), MOE_ERR_UNSUPPORTED_SHAPE,
 * MOE_ERR_ALIGNMENT, MOE_ERR_WORKSPACE_TOO_SMALL, MOE_ERR_HIP. */
int moe_route(const moe_config* cfg, const void* x, const float* router_w, const float* router_bias,
              int32_t* topk_ids, float* topk_w, void* workspace, size_t workspace_bytes, void* stream);

/* The router logits alone (the scores of the routing of the gfx90a paper,
 * abstract, before the sigmoid), as moe_route computes them:
 * logits fp32 [T][E] (device, caller-owned, overwritten),
 * l[t][e] = pdot(x[t], router_w[e]) + router_bias[e], where pdot splits H
 * into 64 contiguous chunks, sums each chunk as a chain of fused
 * multiply-adds in ascending k and adds the 64 chunk sums as a perfect
 * pairwise tree in index order. Same shapes, workspace and errors as
 * moe_route (logits must not overlap the workspace: MOE_ERR_ALIAS). */
int moe_router_logits(const moe_config* cfg, const void* x, const float* router_w, const float* router_bias,
                      float* logits, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ sort --
 * Expert sort (the gfx90a paper retunes it for prefill, abstract): group the P pairs
 * (p = t * top_k + j) by expert, keeping ascending p within an expert, each
 * expert's segment padded up to a multiple of block_m (1 <= block_m <= 1024).
 *   counts [E]          pairs per expert
 *   offsets [E+1]       padded segment starts; offsets[E] = padded total
 *   sorted_pairs [cap]  pair index at each padded position, P in padding;
 *                       cap = P + min(E, P) * (block_m - 1)
 *   pair_pos [P]        padded position of each pair
 *   tile_expert [cap / block_m + 1]  expert of each block_m tile, in order
 *   n_tiles [1]         offsets[E] / block_m  (stays on the device)
 * Bit-exact: integers only. Only cfg->T, cfg->top_k and cfg->E are read.
 * All arrays are device memory owned by the caller; workspace as for
 * moe_workspace_size (its sort scratch). Errors: MOE_ERR_INVALID_ARG (NULL
 * pointer), MOE_ERR_UNSUPPORTED_SHAPE (block_m out of range),
 * MOE_ERR_ALIGNMENT, MOE_ERR_WORKSPACE_TOO_SMALL, MOE_ERR_HIP. ids outside
 * [0, E) are not allowed (not checked). */
int moe_sort(const moe_config* cfg, int32_t block_m, const int32_t* topk_ids,
             int32_t* counts, int32_t* offsets, int32_t* sorted_pairs, int32_t* pair_pos,
             int32_t* tile_expert, int32_t* n_tiles,
             void* workspace, size_t workspace_bytes, void* stream);

/* -------------------------------------------------------------- quantize --
 * Quantize rows of an activation matrix v [rows][K] (in_dtype: MOE_X_F32 or
 * MOE_X_BF16) with cfg->act_mode (int8 rows as the gfx90a paper quantizes
 * decode activations, abstract; MXFP4 per OCP Microscaling v1.0).
 *   INT8 : q int8 [rows][K], scales fp32 [rows]. K % 64 == 0.
 *   MXFP4: q codes [rows][K/2], scales E8M0 [rows][K/32]. K % 64 == 0.
 * Only cfg->act_mode is read. v, q: 16-byte aligned device memory owned by
 * the caller; scales: device memory. Errors: MOE_ERR_INVALID_ARG,
 * MOE_ERR_UNSUPPORTED_SHAPE (K outside 64..65536 or not a multiple of 64),
 * MOE_ERR_ALIGNMENT, MOE_ERR_HIP. */
int moe_quantize(const moe_config* cfg, int32_t rows, int32_t K, int32_t in_dtype,
                 const void* v, void* q, void* scales, void* stream);

/* --------------------------------------------------------------- forward --
 * The whole routed-MoE layer with FP4 packed expert weights and int8 or MXFP4
 * activations (the routed experts of the gfx90a paper, abstract: FP4 experts,
 * int8 decode activations, the expert sort, MFMA prefill): route, sort,
 * quantize x, gate/up GEMM with fused SiLU*mul and requantization, down
 * GEMM, weighted combine.
 *   x [T][H] (cfg->x_dtype), router_w fp32 [E][H], router_bias fp32 [E] or
 *   NULL, w13/w13_scale and w2/w2_scale in the layout cfg->weight_layout
 *   names (canonical or prepacked, see "weights"; all 16-byte aligned),
 *   out fp32 [T][H] (overwritten; must not overlap x),
 *   topk_ids_out int32 [T][top_k] and topk_w_out fp32 [T][top_k] or NULL,
 *   workspace of at least moe_workspace_size(cfg) bytes, 256-byte aligned.
 * Every pointer is device memory owned by the caller; nothing is kept.
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED_SHAPE (shape limits, or a
 * block_m other than the GEMMs'), MOE_ERR_ALIGNMENT, MOE_ERR_ALIAS (out over
 * x, or the workspace over x or out), MOE_ERR_WORKSPACE_TOO_SMALL,
 * MOE_ERR_HIP; nothing is launched on an error other than MOE_ERR_HIP. */
int moe_forward(const moe_config* cfg, const void* x, const float* router_w, const float* router_bias,
                const uint8_t* w13, const uint8_t* w13_scale, const uint8_t* w2, const uint8_t* w2_scale,
                float* out, int32_t* topk_ids_out, float* topk_w_out,
                void* workspace, size_t workspace_bytes, void* stream);

/* moe_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation):
 * the same layer, with the scratch taken from a fixed device array of
 * MOE_NOALLOC_SCRATCH_BYTES that the library holds on each device it runs on
 * (from the first call on that device until the process ends) instead of a
 * caller workspace. Nothing is allocated or freed in the call. The caller
 * still passes inputs and outputs as for moe_forward. A configuration whose
 * moe_workspace_size exceeds MOE_NOALLOC_SCRATCH_BYTES is refused with
 * MOE_ERR_WORKSPACE_TOO_SMALL before anything is launched (64 MiB holds a
 * decode batch of up to 64 tokens, or an MXFP4 batch of about 400 tokens, at
 * H 4096, I 2048, 256 experts, top-6). Every call on one device shares that
 * device's array: calls that overlap on one GPU (other streams, other host
 * threads) race and must be serialized by the caller. The array keeps the
 * last call's contents; no kernel depends on its initial contents. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int moe_forward_noalloc(const moe_config* cfg, const void* x, const float* router_w, const float* router_bias,
                        const uint8_t* w13, const uint8_t* w13_scale, const uint8_t* w2, const uint8_t* w2_scale,
                        float* out, int32_t* topk_ids_out, float* topk_w_out, void* stream);

/* moe_forward that also copies the intermediates named in taps and records
 * the stage events (NULL taps = moe_forward), for the fixed-token and hash
 * checks of the gfx90a paper (abstract). The copies are extra kernels after
 * the layer. sorted_pairs needs P + min(E, P) * (block_m - 1) entries with
 * block_m = MOE_BLOCK_M_INT8 (16) for MOE_ACT_INT8 and MOE_BLOCK_M_MXFP4 (64)
 * for MOE_ACT_MXFP4 (the value written to taps->block_m). xq and xs, and aq
 * and as, come in pairs: one without the other is MOE_ERR_INVALID_ARG,
 * reported before anything is launched. */
int moe_forward_taps(const moe_config* cfg, const void* x, const float* router_w, const float* router_bias,
                     const uint8_t* w13, const uint8_t* w13_scale, const uint8_t* w2, const uint8_t* w2_scale,
                     float* out, int32_t* topk_ids_out, float* topk_w_out, const moe_taps* taps,
                     void* workspace, size_t workspace_bytes, void* stream);

/* The layer without its router: the expert part of moe_forward (quantization
 * of x, sort, gate/up + SiLU-mul + requantization, down, combine) for routing
 * given by the caller -- as a rank of an expert-parallel deployment computes
 * the (token, expert) pairs dispatched to it, for instance one row per pair
 * with top_k = 1 and E = the rank's experts. The steps after the routing are
 * those of moe_forward (gfx90a paper, abstract: FP4 routed experts), so with
 * the router's own ids and weights the output equals moe_forward's bit for bit.
 *   topk_ids int32 [T][top_k]: expert of each slot, in [0, E); an id outside
 *     that range is clamped into it (memory-safe, result unspecified);
 *   topk_w fp32 [T][top_k]: the slot weights of the combine;
 *   router_w is not used; the other arguments and the workspace
 *   (moe_workspace_size(cfg) bytes) are as for moe_forward; taps as for
 *   moe_forward_taps (NULL for none). */
int moe_forward_routed(const moe_config* cfg, const void* x, const int32_t* topk_ids, const float* topk_w,
                       const uint8_t* w13, const uint8_t* w13_scale, const uint8_t* w2, const uint8_t* w2_scale,
                       float* out, const moe_taps* taps, void* workspace, size_t workspace_bytes, void* stream);

/* --------------------------------------------------- stacked-layer helpers --
 * Residual stream between stacked MoE layers, x_{l+1} = x_l + moe_l(rmsnorm(x_l)):
 * moe_rmsnorm: out[t] = x[t] / sqrt(ss / H + 1e-6), ss = the router's fixed-
 *   order dot product of x[t] with itself; IEEE sqrt and division; unit gain.
 *   x, out fp32 [T][H], H % 64 == 0; may not overlap.
 * moe_residual_add: x[i] += y[i] for i < n (fp32). */
int moe_rmsnorm(int32_t T, int32_t H, const float* x, float* out, void* stream);
int moe_residual_add(int64_t n, float* x, const float* y, void* stream);

/* ----------------------------------------------------------- layer stack --
 * A stack of MoE layers with the residual update between them, as in the
 * 43-layer routed stack of the model (DeepSeek V4 Flash on 8x AMD gfx1201:
 * packaged TP=8 deployment, What we set out to do: 43 layers of 256 routed
 * experts, 6 active per token). For l = 0 .. L-1:
 *     x <- x + moe_l(rmsnorm(x))
 * with x fp32 [T][H] updated in place (cfg->x_dtype must be MOE_X_F32; the
 * layer's input is the normalized stream, fp32). Per-layer device pointers
 * come in HOST arrays of length L: router_w[l], w13[l], w13_scale[l], w2[l],
 * w2_scale[l] (layout cfg->weight_layout), router_bias[l] (router_bias itself or any entry
 * may be NULL). layer_out (device fp32 [L][T][H], nullable) receives every
 * layer's moe output, for teacher-forced checks of one layer at a time.
 * workspace: at least moe_stack_workspace_size bytes, 256-byte aligned, not
 * overlapping x or layer_out. Returns the first failing layer's status;
 * layers before it have been applied to x. */
int moe_stack_workspace_size(const moe_config* cfg, size_t* bytes);
int moe_forward_stack(const moe_config* cfg, int32_t L, float* x, const float* const* router_w,
                      const float* const* router_bias, const uint8_t* const* w13, const uint8_t* const* w13_scale,
                      const uint8_t* const* w2, const uint8_t* const* w2_scale, float* layer_out,
                      void* workspace, size_t workspace_bytes, void* stream);

/* moe_forward_stack with per-layer taps: taps is NULL or a HOST array of L
 * moe_taps, and layer l's intermediates and stage events are handled as
 * moe_forward_taps handles them (the combine stage is fused into the
 * residual update and records its events around nothing; y, xq/xs, aq/as,
 * the sort arrays and block_m are those of layer l). Used to time one stage
 * of chosen layers on the stream the kernels run on. Same errors as
 * moe_forward_stack, plus MOE_ERR_INVALID_ARG for an unpaired int8 tap of
 * any layer (checked before anything is launched). */
int moe_forward_stack_taps(const moe_config* cfg, int32_t L, float* x, const float* const* router_w,
                           const float* const* router_bias, const uint8_t* const* w13,
                           const uint8_t* const* w13_scale, const uint8_t* const* w2, const uint8_t* const* w2_scale,
                           float* layer_out, const moe_taps* taps, void* workspace, size_t workspace_bytes,
                           void* stream);

/* ------------------------------------------------------ dense FP8 --------
 * Block-scaled FP8 dense projection y = x W^T, the format of the model's
 * dense (non-expert) projections: FP8 dense projections (DeepSeek-V4-Flash on
 * AMD gfx90a: Correctness Recovery and Inference Performance Engineering,
 * abstract) with FP8 block quantization (DeepSeek V4 Flash on 8x AMD gfx1201,
 * section What we set out to do). The pages fix neither the block shape nor
 * the scale format; this library takes OCP MX FP8 (Microscaling v1.0):
 *   - elements E4M3 (bias 7, no infinities, 0x7f / 0xff NaN, largest 448);
 *   - one E8M0 scale byte (2^(byte - 127)) per 32 consecutive elements along
 *     K, for every weight row and every activation row;
 *   - activation quantization per block of 32: scale exponent
 *     floor(log2 amax) - 8 biased by 127, clamped to [0, 254] (0 for an
 *     all-zero block); values scaled by the exact power of two, rounded to
 *     the nearest E4M3 value with ties to even, saturated at 448; the code's
 *     sign is the value's sign bit;
 *   - y[m][n] = sum over blocks b of 2^(sx[m][b] + sw[n][b] - 254) *
 *     sum_{k in b} x[m][k] w[n][k], summed by the matrix cores: in groups
 *     of 8 consecutive k, each product truncated toward zero at 2^(E - 13)
 *     (E the group's largest exponent sum, block scales included), the
 *     group sums added in fp32. So |y - exact| < sum over groups of
 *     2^(E - 10), plus the fp32 additions; exact when no product has bits
 *     below that point (e.g. operands of few binades).
 * Weights, in the layout cfg->weight_layout names:
 *   MOE_LAYOUT_CANONICAL: w codes uint8 [N][K] (row-major), w_scale uint8
 *     [N][K/32];
 *   MOE_LAYOUT_PREPACKED: the operand order of the matrix cores, made by
 *     moe_dense_fp8_prepack once when the weights are loaded: codes
 *     [N/32][K/64][2][64][16] (32-row tile, 64-K step, plane p, lane l, byte
 *     b: row 32 tile + l % 32, k = 64 step + 32 p + 16 (l / 32) + b), so
 *     every load is 1 KB contiguous; scales [N/32][ceil(K/256)][64] dwords,
 *     byte j of lane l = the E8M0 byte of block 2 (4 g + j) + l / 32 of row
 *     32 tile + l % 32 (127 past the last K-step).
 * A code 0x7f / 0xff (NaN) propagates NaN. Same conventions as the calls above
 * (device pointers owned by the caller, host-side checks, no allocation,
 * no floating-point atomics: bit-identical results from run to run).
 * Shape limits: 0 <= M <= 1<<20, K % 128 == 0 and 128 <= K <= 32768,
 * N % 256 == 0 and 256 <= N <= 65536, M * K < 2^32. M = 0 does nothing. */
typedef struct moe_dense_config {
    int32_t M;             /* tokens (rows of x and y) */
    int32_t N;             /* output features (rows of W) */
    int32_t K;             /* input features */
    int32_t x_dtype;       /* enum moe_x_dtype: element type of x for moe_dense_fp8_forward */
    int32_t weight_layout; /* enum moe_weight_layout of w and w_scale */
} moe_dense_config;

/* Workspace of moe_dense_fp8_forward (the quantized activations and, for
 * M <= 32, the partial sums of a K split) and of moe_dense_fp8_gemm (for
 * M <= 32: the activations repacked into the operand order, and the partial
 * sums). Errors: MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED_SHAPE. */
int moe_dense_fp8_workspace_size(const moe_dense_config* cfg, size_t* bytes);

/* Byte counts of the prepacked weight layout (codes: N * K; scales:
 * N/32 * ceil(K/256) * 256). Shapes: N % 32 == 0, 32 <= N <= 65536, K % 128
 * == 0, 128 <= K <= 32768. Errors: MOE_ERR_INVALID_ARG,
 * MOE_ERR_UNSUPPORTED_SHAPE. */
int moe_dense_fp8_prepacked_size(int32_t N, int32_t K, size_t* code_bytes, size_t* scale_bytes);

/* Canonical weights (w [N][K], w_scale [N][K/32]) to the prepacked layout
 * above, and back (a bijection on the codes; the scale padding is dropped
 * when unpacking). Code pointers 16-byte aligned, packed scales 4-byte
 * aligned; the four buffers must not overlap. Errors: MOE_ERR_INVALID_ARG,
 * MOE_ERR_UNSUPPORTED_SHAPE, MOE_ERR_ALIGNMENT, MOE_ERR_ALIAS, MOE_ERR_HIP. */
int moe_dense_fp8_prepack(int32_t N, int32_t K, const uint8_t* w, const uint8_t* w_scale, uint8_t* packed_w,
                          uint8_t* packed_scale, void* stream);
int moe_dense_fp8_unpack(int32_t N, int32_t K, const uint8_t* packed_w, const uint8_t* packed_scale, uint8_t* w,
                         uint8_t* w_scale, void* stream);

/* MXFP8 quantization of v [rows][K] (in_dtype MOE_X_F32 or MOE_X_BF16) into
 * codes uint8 [rows][K] and scales uint8 [rows][K/32], the rule above.
 * v and codes 16-byte aligned. Errors: MOE_ERR_INVALID_ARG,
 * MOE_ERR_UNSUPPORTED_SHAPE (K outside 32..65536 or not a multiple of 32),
 * MOE_ERR_ALIGNMENT, MOE_ERR_HIP. */
int moe_dense_fp8_quantize(int32_t rows, int32_t K, int32_t in_dtype, const void* v, uint8_t* codes,
                           uint8_t* scales, void* stream);

/* y fp32 [M][N] (overwritten) from quantized activations xq [M][K], xs
 * [M][K/32] and the weights. workspace (256-byte aligned, at least
 * moe_dense_fp8_workspace_size bytes) is used only when M <= 32 and may
 * be NULL otherwise. All pointers 16-byte aligned; y must not overlap an
 * input or the workspace. Errors: MOE_ERR_INVALID_ARG,
 * MOE_ERR_UNSUPPORTED_SHAPE, MOE_ERR_ALIGNMENT, MOE_ERR_ALIAS,
 * MOE_ERR_WORKSPACE_TOO_SMALL, MOE_ERR_HIP. */
int moe_dense_fp8_gemm(const moe_dense_config* cfg, const uint8_t* xq, const uint8_t* xs, const uint8_t* w,
                       const uint8_t* w_scale, float* y, void* workspace, size_t workspace_bytes, void* stream);

/* The projection from activations: quantize x [M][K] (cfg->x_dtype) into
 * the workspace, then the GEMM above into y fp32 [M][N]. Same errors. */
int moe_dense_fp8_forward(const moe_dense_config* cfg, const void* x, const uint8_t* w, const uint8_t* w_scale,
                          float* y, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP4MOE_H */
