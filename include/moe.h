/*
 * moe.h - C ABI of libmoe, a fused int4 / MXFP4 Mixture-of-Experts layer for
 * AMD Instinct MI355X (gfx950, CDNA4).
 *
 * The layer (sources: the colibri Vulkan-backend PR #418, the dasLLAMA vulkan
 * PR #3988 and the vllm.cpp warp-router PR #481):
 *   1. router logits L = x . W_router^T (fp32), unless the caller gives L;
 *   2. softmax over the E experts -> top-k (the lower index wins a tie) ->
 *      renormalise over the k picks, times route_scale (or a router variant:
 *      sigmoid scores, a selection bias; see moe_router_topk);
 *   3. token-to-expert permutation: per-expert buckets of slots, slot s = t*k+j;
 *   4. per expert, the SwiGLU MLP on its bucket's rows:
 *        h = silu(Wg x) * (Wu x),   o = Wd h,
 *      with int4 weights: nibble n stands for (n - 8), times an fp16 scale per
 *      32 consecutive inputs; or MXFP4 weights (the colibri PR's later fmt=7
 *      comment): nibble n is an e2m1 value, times 2^(e - 127) for a ue8m0
 *      byte e per 32 consecutive inputs;
 *   5. combine y[t] = sigma(x_t . g) * shared(x_t) + sum_j w[t][j] * o[t][j]
 *      (the shared expert optional; without a gate vector it adds at weight 1).
 *
 * Conventions for every entry point
 *   - All data pointers are DEVICE pointers (hipMalloc'd or torch CUDA tensors)
 *     unless stated otherwise; `shape` structs are HOST pointers.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     returns without a host synchronisation.  The library allocates nothing:
 *     the caller owns every buffer, scratch space included, and must keep it
 *     alive until the stream has run the work.
 *   - Arguments are checked on the host before anything is enqueued; a failed
 *     check returns an error code and enqueues nothing.  Faults inside kernels
 *     surface at the caller's next synchronisation, as for any HIP launch.
 *   - Entry points are thread-safe for distinct streams; two calls that share
 *     an output or workspace buffer must be ordered by the caller.
 *   - Logits must be finite; behaviour on NaN/Inf logits is unspecified.
 *
 * int4 planes (moe_q4): q = packed nibbles, uint8 [E][N][K/2]: element kk of
 * row n sits in byte kk/2, low nibble = even kk (the host byte layout, loaded
 * with a plain copy, no repacking).  s = fp16 scale bits, uint16 [E][N][K/32],
 * one scale per 32 consecutive inputs along K.  Gate and up planes have N = I,
 * K = H; down planes have N = H, K = I.  q and s must be 16-byte aligned.
 *
 * MXFP4 planes (moe_shape.format = MOE_FORMAT_MXFP4): q as above, each
 * nibble an OCP MX e2m1 code (bit 3 sign, bits 2..1 exponent with bias 1,
 * bit 0 mantissa: 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives); s = ue8m0
 * exponent bytes, uint8 [E][N][K/32], scale 2^(e - 127), e = 255 is NaN.  The
 * GEMV path dots the exact e2m1 values with fp16 activations and scales each
 * group's fp32 partial by 2^(e - 127) in fp32.  The MFMA path serves every
 * exponent too: per weight row it feeds the fp16 value e2m1 * 2^(e - 127 -
 * shift), with shift = (the row's largest finite exponent) - 140, and
 * multiplies the fp32 accumulator by 2^shift; groups within 36 of their
 * row's largest exponent are exact, a group 37 below rounds once to fp16's
 * subnormal grid, groups further below contribute zero (weights below 2^-34
 * of the row's largest), e = 255 gives NaN.
 *
 * Tiled planes (moe_shape.layout = MOE_LAYOUT_TILED, written by
 * moe_pack_weights): the same bytes regrouped so that the grouped MFMA GEMM
 * and the tiled GEMV read each weight block as one contiguous kilobyte.  Per
 * expert, the block
 * of rows 32*b .. 32*b+31 and inputs 64*c .. 64*c+63 is 1024 bytes at byte
 * ((b*(K/64) + c) * 1024); inside it, the 16 bytes of row 32*b+j for scale
 * group 2*c+h (inputs 64*c+32*h .. +31, same nibble order as above) sit at
 * byte (32*h + j) * 16.  The scales of that block are 64 scale elements
 * (fp16 for int4, ue8m0 bytes for MXFP4) at element ((b*(K/64) + c) * 64),
 * the one of row 32*b+j, group 2*c+h at index 32*h + j.  Expert e's plane
 * starts where it does in the row layout.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t. */
typedef struct ihipStream_t *moe_stream_t;

enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null/misaligned pointer, inconsistent sizes  */
  MOE_ERR_UNSUPPORTED = 2, /* outside the shapes the kernels serve         */
  MOE_ERR_WORKSPACE = 3,   /* ws_bytes smaller than moe_workspace_bytes()  */
  MOE_ERR_HIP = 4,         /* a HIP launch reported an error               */
  MOE_ERR_SCRATCH_LIMIT = 5, /* moe_layer_static: the shape needs more
                                scratch than MOE_STATIC_SCRATCH_BYTES      */
};

/* Expert MLP path.  AUTO picks the streaming GEMV when the expected rows per
 * expert are few (decode) and the grouped MFMA GEMM otherwise (prefill); see
 * moe_layout for the rule on each layout. */
enum moe_path { MOE_PATH_AUTO = 0, MOE_PATH_GEMV = 1, MOE_PATH_GEMM = 2 };

/* Weight plane layout (see above), served by both paths.  AUTO takes the
 * GEMV on TILED planes for up to 4 tokens (T*k <= 64), the MFMA GEMM beyond;
 * on ROWS planes it takes the GEMV while T*k < 8E. */
enum moe_layout { MOE_LAYOUT_ROWS = 0, MOE_LAYOUT_TILED = 1 };

/* Weight format (see above), for every plane of a call. */
enum moe_format { MOE_FORMAT_INT4 = 0, MOE_FORMAT_MXFP4 = 1 };

/* Router score function (see moe_router_topk): the softmax probability over
 * the E experts, or the sigmoid of each logit on its own. */
enum moe_score { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 };

/* One 4-bit plane set: q [E][N][K/2] packed nibbles, s [E][N][K/32] group
 * scales: fp16 bits (uint16) for int4, ue8m0 bytes (uint8) for MXFP4. */
typedef struct {
  const uint8_t *q;
  const void *s;
} moe_q4;

/* Layer shape.  T tokens, H hidden, E experts, k picks per token, I expert
 * intermediate, SI shared-expert intermediate (0 = none), group must be 32,
 * route_scale multiplies the renormalised weights, path is a moe_path,
 * layout a moe_layout and format a moe_format (both for every plane of the
 * call, shared ones included), top_p the expert top-p applied after the
 * top-k (see moe_router_topk; 0, the zero-initialised value, keeps all k),
 * score a moe_score and select_bias a DEVICE pointer to fp32 [E] or NULL,
 * n_group and topk_group the grouped routing (the router variant of
 * moe_router_topk; zero-initialised = the plain softmax router).
 * Served: 1 <= k <= min(E, 64), E <= 256, H % 64 == 0, I % 64 == 0,
 * SI % 64 == 0, T >= 1, T*k < 2^31, n_group <= 16. */
typedef struct {
  int32_t T, H, E, k, I, SI;
  int32_t group;
  float route_scale;
  int32_t path;
  int32_t layout;
  int32_t format;
  float top_p;
  int32_t score;
  const float *select_bias;
  int32_t n_group, topk_group;
} moe_shape;

/*
 * Softmax -> top-k -> renormalise, one 64-lane wave per token (the warp-per-
 * token router of vllm.cpp PR #481, re-shaped for wave64: expert e lives in
 * lane e % 64, register e / 64).
 *   logits : fp32 [T][E], row-major.
 *   idx    : int32 [T][k] out, expert ids in rank order (largest logit first,
 *            the lower index first among equal logits).
 *   w      : fp32 [T][k] out, w[t][j] = route_scale * exp(L_j - L_0) /
 *            sum_j' exp(L_j' - L_0), evaluated in fp64 and rounded once.
 *   top_p  : expert top-p after the top-k (the "expert-routing top-p" setting
 *            of the colibri PR's measured decode, which the page does not
 *            define; read as): with 0 < top_p < 1, pick j is kept while the
 *            full-softmax probability of the picks ranked above it,
 *            sum_{i<j} exp(L_i - L_0) / sum_e exp(L_e - L_0), is below top_p
 *            (the first pick is always kept); a dropped pick is written as
 *            idx -1, w 0, and the sums over j' above run over the kept picks.
 *            Any other value (0, >= 1, negative, NaN) keeps all k.  Dropped
 *            picks are skipped by moe_permute and by the layer.
 *   score, select_bias : router variant (the dasLLAMA PR's MoE seat lists a
 *            non-softmax gate and a router or selection bias among the shapes
 *            it declines, without defining them; read as the published
 *            DeepSeek-V3 routing without expert groups).  With score =
 *            MOE_SCORE_SOFTMAX and select_bias = NULL the plain router above
 *            runs.  Otherwise each expert gets a score s_e in fp64 -
 *            softmax(L)_e (MOE_SCORE_SOFTMAX) or 1 / (1 + exp(-L_e))
 *            (MOE_SCORE_SIGMOID) - the picks are the k largest keys s_e + b_e
 *            in rank order (b = select_bias, device fp32 [E], zero when NULL;
 *            the lower index wins a tie), and w[t][j] = route_scale * s_j /
 *            sum_j' s_j' over the picks (the bias steers the selection only).
 *            Top-p is not defined for variants: 0 < top_p < 1 with a variant
 *            is UNSUPPORTED.
 *   n_group, topk_group : grouped routing (the noaux_tc router the vllm.cpp
 *            PR's dispatch names without defining it; read as the published
 *            DeepSeek-V3 grouped top-k).  n_group 0 or 1: no grouping.  With
 *            n_group > 1 (dividing E, at most 16) the experts form n_group
 *            groups of E / n_group consecutive experts; a group's score is
 *            the sum of its two largest keys s_e + b_e (its one key for
 *            groups of one expert), in fp64; the topk_group groups with the
 *            largest scores are kept (the lower group index wins a tie) and
 *            the picks are the k largest keys among the kept groups' experts
 *            only, weighted as for the variants above.  A grouped router is
 *            a variant (for top-p).
 * Errors: INVALID_ARG (null pointer, T < 1, k < 1, k > E, unknown score,
 *         misaligned select_bias, n_group < 0, n_group > 1 not dividing E,
 *         topk_group outside 1..n_group, fewer than k experts in topk_group
 *         groups); UNSUPPORTED (E > 256, k > 64, top-p with a variant,
 *         n_group > 16).
 */
int moe_router_topk(const float *logits, int32_t T, int32_t E, int32_t k, float route_scale,
                    float top_p, int32_t score, const float *select_bias, int32_t n_group,
                    int32_t topk_group, int32_t *idx, float *w, moe_stream_t stream);

/*
 * Token-to-expert permutation (the bucket schedule of the dasLLAMA PR's routed
 * block: per-expert counts, exclusive scan, slots placed in slot order).  Up
 * to 4096 slots one workgroup does it all (LDS histogram, LDS scan, stable
 * scatter); beyond, three launches over blocks of 1024 slots (per-block
 * counts, one offsets pass, per-block scatters with the same in-slot-order
 * ranking), which need scratch.
 *   idx    : int32 [T][k] expert picks; slot s = t*k + j.
 *   off    : int32 [E+1] out, exclusive scan of the per-expert slot counts.
 *   sorted : int32 [T*k] out, slot ids grouped by expert, ascending within a
 *            bucket (sorted[off[e] .. off[e+1]) are expert e's slots).
 *   row_of : int32 [T*k] out, inverse map: sorted[row_of[s]] == s.
 *   ws     : device scratch of at least moe_permute_workspace_bytes(T, k, E)
 *            bytes, 256-byte aligned (may be NULL when that is 0); its
 *            contents on entry are ignored.
 * A pick outside [0, E) is dropped: it is counted nowhere, sorted holds only
 * valid slots (off[E] = their number) and row_of[s] = -1 for it.
 * Errors: INVALID_ARG (null pointer, T < 1, k < 1, misaligned ws);
 *         UNSUPPORTED (E > 256, T*k >= 2^31); WORKSPACE (ws_bytes short).
 */
int moe_permute(const int32_t *idx, int32_t T, int32_t k, int32_t E, int32_t *off,
                int32_t *sorted, int32_t *row_of, void *ws, size_t ws_bytes,
                moe_stream_t stream);

/* Scratch bytes moe_permute needs for these sizes: 0 up to 4096 slots,
 * 4 * ceil(T*k / 1024) * E beyond (0 also for sizes moe_permute rejects).
 * Host only. */
size_t moe_permute_workspace_bytes(int32_t T, int32_t k, int32_t E);

/*
 * The routed experts' SwiGLU MLPs with the weighted combine fused into the
 * down projection's epilogue (the colibri PR's fused expert group, its
 * Summary: gate and up products with the SiLU product formed on the device,
 * then down, the hidden row never leaving the device; the dasLLAMA PR's
 * routed block: each bucket's rows gathered through the slot map, and the
 * combine weighting each slot's down row by its routing weight onto the
 * token's output row):
 *   y[t][:] = sum over slots s = t*k+j in the buckets of w[s] * MLP_e(x[t]),
 *   MLP_e(x) = Wd_e (silu(Wg_e x) * (Wu_e x)),  silu(z) = z / (1 + exp(-z)).
 *   shape  : host pointer; T, H, E, k, I, group, path, layout, format are
 *            used (SI ignored).
 *   x      : bf16 bits [T][H], 16-byte aligned.
 *   off, sorted : as written by moe_permute.
 *   w      : fp32 [T][k] combine weights (from moe_router_topk).
 *   gate, up, down : 4-bit planes in shape->format and shape->layout.
 *   y      : fp32 [T][H] out, OVERWRITTEN (not accumulated), 16-byte aligned.
 * Value range: both paths keep the hidden row h = silu(g) * u in fp16, so a
 * hidden value beyond 65504 in magnitude becomes +-inf and its output row
 * non-finite (the call still returns MOE_OK); the MFMA path (path GEMM, or
 * AUTO at prefill sizes) also feeds x as fp16, so it serves |x| < 65520
 * (activations with |x| < 2^-14 keep fp16's subnormal spacing, 2^-24).
 *   ws     : device scratch of at least moe_workspace_bytes(shape) bytes,
 *            256-byte aligned; its contents on entry are ignored.
 * The order in which a token's k terms are added to y is not fixed (device
 * atomics); the result differs from an ordered sum only by fp32 rounding.
 * Errors: INVALID_ARG, UNSUPPORTED (also for path GEMV with TILED planes
 *         whose K/32 prepared activation groups exceed 48 KB of LDS, K >
 *         19648), WORKSPACE, HIP.
 */
int moe_expert_mlp(const moe_shape *shape, const uint16_t *x, const int32_t *off,
                   const int32_t *sorted, const float *w, moe_q4 gate, moe_q4 up, moe_q4 down,
                   float *y, void *ws, size_t ws_bytes, moe_stream_t stream);

/*
 * The whole layer: router (logits given, or x . W_router^T), top-k, weights,
 * permutation, expert MLPs, combine, and the optional sigmoid-gated shared
 * expert (the dasLLAMA PR's shared expert: one bucket over every token with an
 * identity map, weighted by sigmoid of one more router row).
 *   logits     : fp32 [T][E], or NULL when w_router is given (exactly one of
 *                the two must be non-NULL).
 *   w_router   : fp32 [E][H], or NULL.
 *   shared     : host array of 3 moe_q4 {gate, up, down} with E = 1 and
 *                I = shape->SI, or NULL (then shape->SI must be 0).
 *   shared_gate: fp32 [H] gate vector g, or NULL for an ungated shared expert
 *                (added at weight one).  Ignored without a shared expert.
 *   y          : fp32 [T][H] out, overwritten, 16-byte aligned.
 *   idx_out    : int32 [T][k] out, or NULL.
 *   w_out      : fp32 [T][k] out, or NULL.
 *   logits_out : fp32 [T][E] out (the logits used), or NULL.
 *   ws         : as for moe_expert_mlp.
 * Value range: as for moe_expert_mlp (the shared expert's hidden row too).
 * Errors: as moe_expert_mlp.
 */
int moe_layer(const moe_shape *shape, const uint16_t *x, const float *logits,
              const float *w_router, moe_q4 gate, moe_q4 up, moe_q4 down, const moe_q4 *shared,
              const float *shared_gate, float *y, int32_t *idx_out, float *w_out,
              float *logits_out, void *ws, size_t ws_bytes, moe_stream_t stream);

/*
 * moe_layer for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same work with
 * the same arguments except the workspace, which is a device array the
 * library owns, MOE_STATIC_SCRATCH_BYTES (16 MiB) per GPU, held from the
 * first call on that GPU until the process ends.  The call itself allocates
 * and frees nothing.
 *   Limit: shapes whose moe_workspace_bytes() exceeds the static scratch are
 *          rejected with MOE_ERR_SCRATCH_LIMIT before anything is enqueued
 *          (16 MiB serves decode and decode-batch sizes and prefill up to
 *          about 500 tokens at H = 2048, I = 1408 with a 5632-wide shared
 *          expert; not the 2048-token, 6144-wide prefill).
 *   Sharing: every call on one GPU uses that GPU's one scratch array, which
 *          keeps the last call's contents (nothing in it needs clearing: each
 *          call writes what it reads).  Calls that overlap on one GPU (two
 *          streams, or two host threads) race on it: the caller orders them.
 *   stream : must belong to the current device (whose scratch is used).
 * Errors: as moe_layer, plus SCRATCH_LIMIT; HIP if the scratch's device
 *         address cannot be obtained.
 */
#define MOE_STATIC_SCRATCH_BYTES (16u << 20)
int moe_layer_static(const moe_shape *shape, const uint16_t *x, const float *logits,
                     const float *w_router, moe_q4 gate, moe_q4 up, moe_q4 down,
                     const moe_q4 *shared, const float *shared_gate, float *y, int32_t *idx_out,
                     float *w_out, float *logits_out, moe_stream_t stream);

/*
 * The layer with its combine folded into the residual step (the dasLLAMA
 * PR's fold: the add+rms after the routed block adds the gated shared row and
 * the k weighted expert rows straight into the residual, then norms the row
 * for the next layer):
 *   residual[t] += sigma(x_t . g) * shared(x_t) + sum_j w[t][j] * o[t][j]
 *   x_next[t]    = bf16( residual[t] * norm_w / sqrt(mean_h residual[t][h]^2 + eps) )
 * The down pass adds into `residual` directly (no separate FFN output), and
 * one more launch writes the normed row in the layer's activation format, so
 * x_next can be the next layer's x.
 * With next_w_router, that launch also computes the next layer's router
 * logits from the bf16 normed rows (the vllm.cpp PR's closing hypothesis:
 * the router folded into the preceding kernel, fewer launches per step):
 *   next_logits[t][e] = sum_h x_next[t][h] * next_w_router[e][h]   (fp32)
 * so the next layer's call can take them as its given logits instead of
 * launching its own router GEMM.  Up to 32 tokens and H <= 6144 this is one
 * launch; beyond, the norm launch is followed by the router-logits kernel
 * over x_next (the same logits, up to fp32 summation order).
 *   residual : fp32 [T][H], in/out, 16-byte aligned; must not overlap any
 *              other argument.
 *   norm_w   : fp32 [H], the next layer's norm weight, 16-byte aligned.
 *   eps      : >= 0, added to the mean square inside the root.
 *   x_next   : bf16 bits [T][H] out, 16-byte aligned; may be x itself (x is
 *              no longer read when it is written).
 *   next_w_router : fp32 [next_E][H], 16-byte aligned, the next layer's
 *              router plane, or NULL (then next_logits must be NULL too and
 *              next_E is ignored).
 *   next_logits : fp32 [T][next_E] out, or NULL.
 *   the rest : as for moe_layer (no logits_out).
 * The order of the terms added into a residual element is not fixed (device
 * atomics); the result differs from an ordered sum by fp32 rounding only.
 * Errors: as moe_layer, plus INVALID_ARG for a null or misaligned residual,
 *         norm_w, x_next or next_w_router, a negative or NaN eps, exactly one
 *         of next_w_router / next_logits given, or next_E < 1 with them.
 */
int moe_layer_residual_rmsnorm(const moe_shape *shape, const uint16_t *x, const float *logits,
                               const float *w_router, moe_q4 gate, moe_q4 up, moe_q4 down,
                               const moe_q4 *shared, const float *shared_gate, float *residual,
                               const float *norm_w, float eps, uint16_t *x_next,
                               const float *next_w_router, int32_t next_E, float *next_logits,
                               int32_t *idx_out, float *w_out, void *ws, size_t ws_bytes,
                               moe_stream_t stream);

/*
 * Profiling twin of moe_layer: the same work, with stage i's kernel launched
 * through hipExtLaunchKernelGGL so that events[2i] and events[2i+1]
 * (hipEvent_t handles created by the caller) are recorded at that kernel's
 * start and end on `stream`; hipEventElapsedTime(events[2i], events[2i+1]) is
 * the kernel's device time (per-stage stamps in the spirit of the dasLLAMA
 * PR's per-role profile).  A stage the call does not run gets its two events
 * recorded back to back (an interval of no kernel, which measures only the
 * stream's gap there: it is not a stage time).
 *   events    : host array of n_events hipEvent_t, n_events >= 2*MOE_STAGE_COUNT.
 *   stage_ran : host int32 [MOE_STAGE_COUNT] out, or NULL: 1 for each stage
 *               whose kernel the call launched, 0 for the others (the fused
 *               small-batch routing runs inside the gate/up launch, so its
 *               top-k and permutation stages read 0).
 * Errors: as moe_layer, plus INVALID_ARG for a null or short event list.
 */
enum moe_stage {
  MOE_STAGE_START = 0,          /* before the first launch                   */
  MOE_STAGE_LOGITS = 1,         /* router logits (+ shared gate logit)       */
  MOE_STAGE_TOPK = 2,           /* softmax -> top-k -> renormalise           */
  MOE_STAGE_PERMUTE = 3,        /* permutation + expert schedule             */
  MOE_STAGE_ACTIVATIONS = 4,    /* fp16 activation copy (MFMA path only)     */
  MOE_STAGE_GATE_UP = 5,        /* routed gate/up + SiLU*mul (MFMA path: also
                                   the shared expert's, and clearing y)     */
  MOE_STAGE_SHARED_GATE_UP = 6, /* shared expert gate/up + SiLU*mul (GEMV
                                   path only)                               */
  MOE_STAGE_DOWN = 7,           /* routed down + weighted combine (MFMA path:
                                   and the shared expert's gated combine)   */
  MOE_STAGE_SHARED_DOWN = 8,    /* shared expert down + gated combine (GEMV
                                   path only)                               */
  MOE_STAGE_COUNT = 9
};
int moe_layer_profiled(const moe_shape *shape, const uint16_t *x, const float *logits,
                       const float *w_router, moe_q4 gate, moe_q4 up, moe_q4 down,
                       const moe_q4 *shared, const float *shared_gate, float *y,
                       int32_t *idx_out, float *w_out, float *logits_out, void *ws,
                       size_t ws_bytes, moe_stream_t stream, void *const *events,
                       int32_t n_events, int32_t *stage_ran);

/*
 * Regroup E experts' 4-bit planes from the row layout into the tiled layout
 * (see above), for the grouped MFMA GEMM's contiguous weight reads.  A pure
 * byte permutation of q and of s; the values are unchanged.  Meant to run once
 * when weights are loaded.
 *   src    : row-layout planes, q [E][N][K/2], s [E][N][K/32].
 *   format : a moe_format; it sets the scale element size (2 or 1 bytes).
 *   dst    : tiled planes of the same sizes (caller-allocated, 16-byte
 *            aligned, not overlapping src).
 * Errors: INVALID_ARG (null, E < 1, N < 1, N % 32 != 0, K % 64 != 0, bad
 *         format, misaligned, overlapping).
 */
int moe_pack_weights(moe_q4 src, int32_t E, int32_t N, int32_t K, int32_t format, moe_q4 dst,
                     moe_stream_t stream);

/* Scratch bytes moe_layer and moe_expert_mlp need for this shape (0 if the
 * shape is not served).  Host only; enqueues nothing. */
size_t moe_workspace_bytes(const moe_shape *shape);

/* Static description of a status code. */
const char *moe_status_string(int status);

/*
 * Test hook: runs one of the kernels' own device int4 decoders (the same
 * __device__ routine their main loops call) over one plane (q [N][K/2]
 * nibbles, s [N][K/32] fp16 bits) and writes what it stands for as fp32
 * [N][K] (device pointer `out`), in the plane's element order:
 *   mode 0: the gate/up GEMV's decoder (each nibble as the exact bf16 value
 *           128 + nibble), its offset and scale undone exactly in fp32: the
 *           exact weight (nibble - 8) * scale;
 *   mode 1: the MFMA GEMM's decoder for tiles of 2-4 row subtiles: its fp16
 *           operand, the exact weight rounded once to fp16 (nearest even);
 *   mode 2: the MFMA GEMM's decoder for one-subtile tiles: its fp16 operand,
 *           the same value as mode 1 for every scale with |s| <= 8188;
 *   mode 3: the down GEMV's decoder (each nibble as the exact fp16 value
 *           1024 + nibble), offset and scale undone exactly: the exact weight.
 * Errors: INVALID_ARG (null, N < 1, K % 32 != 0, misaligned, bad mode).
 */
int moe_debug_dequant_int4(moe_q4 plane, int32_t N, int32_t K, int32_t mode, float *out,
                           moe_stream_t stream);

/*
 * Test hook: the kernels' MXFP4 decoders over one plane (q [N][K/2] e2m1
 * nibbles, s [N][K/32] ue8m0 bytes), written as fp32 [N][K]:
 *   mode 0: the GEMVs' decoder (each byte's e2m1 pair by the packed fp4
 *           conversion) times the fp32 group scale 2^(e - 127): the exact
 *           weight for every e (NaN for e = 255);
 *   mode 1: the MFMA GEMM's decoder for tiles of 2-4 row subtiles: its fp16
 *           operand e2m1 * 2^(e - 127) rounded to nearest even;
 *   mode 2: the MFMA GEMM's decoder for one-subtile tiles: the same operand.
 * Errors: INVALID_ARG (null, N < 1, K % 32 != 0, misaligned, bad mode).
 */
int moe_debug_dequant_mxfp4(moe_q4 plane, int32_t N, int32_t K, int32_t mode, float *out,
                            moe_stream_t stream);

/*
 * Measurement hook: a streaming read of `bytes` (a multiple of 16) of device
 * memory at src (16-byte aligned) by `workgroups` workgroups of 256 threads,
 * each thread loading 16-byte words with the nontemporal hint of the GEMVs'
 * weight stream, in a grid-stride loop.  Nothing is written except, in a
 * case no real data produces (every word of a thread's xor fold all ones),
 * up to 256 words of sink (device, 4-byte aligned).  Timed by the caller, it
 * gives the practical HBM read rate the decode GEMVs are compared with.
 * Errors: INVALID_ARG (null, misaligned, bytes, workgroups outside
 *         1..2^20).
 */
int moe_debug_read_probe(const void *src, size_t bytes, int32_t workgroups, uint32_t *sink,
                         moe_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
