/*
 * moe.h -- C ABI of the MI355X (gfx950) quantised mixture-of-experts layer.
 *
 * What the layer computes (GeekNews #31297 "Show HN: running GLM 5.2 on a
 * slow computer", section "implemented features"; wpnews.pro "Colibri --
 * GLM-5.2 (744B MoE) on 25GB RAM in one pure C file", model spec table):
 *  - a DeepSeek-V3-style sigmoid router (noaux_tc: correction bias for
 *    selection, group-limited top-k, weights normalised and multiplied by
 *    routed_scaling_factor);
 *  - Q8_0-style int8 activations in blocks of 32 with one fp32 scale each;
 *  - routed and shared SwiGLU experts over int8 / packed int4 / packed int2
 *    weight codes with per-row fp32 scales, as integer dot products;
 *  - batch-union execution for multi-token batches (each selected expert
 *    read once per batch, applied to every token routed to it);
 *  - a weighted combine: 8 active + 1 shared expert per token.
 *
 * Conventions (all functions)
 *  - Every pointer argument that names a tensor is a DEVICE pointer; the
 *    moe_shape_t / moe_weights_t structs themselves live in host memory.
 *  - The caller owns every buffer.  The library never allocates or frees,
 *    never synchronises, and keeps no global state; calls are thread-safe
 *    as long as concurrent calls use distinct workspaces and outputs.  The
 *    one exception is the expert tier below: moe_tier_create allocates the
 *    tier's device memory (moe_tier_destroy frees it), and moe_tier_repin
 *    and moe_tier_counts synchronise the stream they are given.
 *  - Workspaces ("ws") are device scratch of at least the matching
 *    *_workspace_bytes size, 256-byte aligned.  They need no initial
 *    contents: a call writes every workspace byte it reads before reading
 *    it, and a later call depends on nothing left in it (except a MOE_STAGE
 *    call, which reads what the earlier stages of its sequence wrote).
 *  - Work is enqueued on `stream` (NULL = the default stream) and the call
 *    returns at once.  Inputs are never written.  Outputs are overwritten,
 *    except with MOE_ACCUMULATE, which adds into y.  y must not alias x.
 *  - Argument checks run before any launch: a call that returns an error
 *    has launched nothing.  T = 0 is a successful no-op.  A fault inside a
 *    kernel is asynchronous and surfaces on the caller's next synchronise.
 *  - Tensors are row-major and densely packed.
 *
 * Weight layout.  For an expert, gate and up are [I][H] (rows = I, in = H),
 * down is [H][I]; each row holds in*wbits/8 bytes of codes; scales are one
 * fp32 per row.  Codes are two's complement: wbits = 8 one int8 per byte;
 * wbits = 4 two per byte, element 2m in the low nibble of byte m; wbits = 2
 * four per byte, element 4m+i in bits 2i..2i+1.  A routed stack holds
 * n_experts experts back to back: expert e's gate codes start at
 * gate + e*I*(H*wbits/8) and its gate scales at gate_s + e*I.  Every row
 * must start 16-byte aligned, which holds when the base pointers are
 * 16-byte aligned (H*wbits/8 and I*wbits/8 are multiples of 16).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- types */
typedef struct {
    int32_t hidden;       /* H: multiple of 32; rows of H*wbits/8 bytes a multiple of 16 */
    int32_t inter;        /* I: expert intermediate size, same rules as H */
    int32_t n_experts;    /* E routed experts, 1..512 */
    int32_t n_group;      /* G groups of E/G consecutive experts, 1..64 */
    int32_t topk_group;   /* groups kept per token, 1..G */
    int32_t top_k;        /* experts per token, 1..min(32, topk_group*E/G) */
    int32_t n_shared;     /* 0 or 1 shared expert (weight 1, not scaled) */
    int32_t wbits;        /* 2, 4 or 8 */
    float   routed_scaling_factor;
    /* Adaptive expert top-p (GeekNews #31297, useful options: the --topp
     * knob).  In (0, 1): each token keeps the shortest prefix of its
     * selection (selection order, at least one expert) whose share of the
     * selection's summed sigmoid scores reaches routed_top_p (shares added in
     * slot order in fp64), and renormalises the kept weights to sum to
     * routed_scaling_factor; a dropped slot reports expert -1 and weight 0
     * and its expert is not read.  0 or >= 1: off (every selected expert is
     * kept).  Both paths take it: the grouped path's permutation gives a
     * dropped assignment no row. */
    float   routed_top_p;
} moe_shape_t;

typedef struct {
    const uint8_t *gate, *up, *down;        /* packed codes (device) */
    const float   *gate_s, *up_s, *down_s;  /* per-row fp32 scales (device) */
} moe_weights_t;

/* ---------------------------------------------------------------- errors */
enum {
    MOE_OK = 0,
    MOE_EINVAL = 1,        /* null pointer, negative size, inconsistent shape */
    MOE_EUNSUPPORTED = 2,  /* valid but outside what the kernels implement */
    MOE_EWORKSPACE = 3,    /* workspace smaller than the matching *_workspace_bytes */
    MOE_EHIP = 4,          /* a launch failed (hipGetLastError) */
    MOE_ESCRATCH = 5       /* the call needs more than the fixed scratch of
                              moe_layer_forward_noalloc */
};
const char *moe_strerror(int code);

/* ---------------------------------------------------------------- flags */
/* Paths.  GEMV: the batch-union plan of up to 8 tokens at a time, each
 * selected expert's rows streamed once per chunk and dotted against every
 * token of the chunk routed to it (HBM-bound decode and verify batches).
 * GROUPED: the T*k (token, expert) assignments are sorted by expert (as
 * moe_permute) and each expert's rows run as int8 MFMA GEMMs in tiles of
 * 128 assignments, with a separate fixed-order combine (prefill); it takes
 * shapes with H a multiple of 256 and I a multiple of 128 and returns
 * MOE_EUNSUPPORTED otherwise.  AUTO: GEMV up to 8 tokens, GROUPED above
 * when the shape allows it, else GEMV.  Both paths give the same routing
 * bit for bit; their float outputs differ only by rounding order. */
#define MOE_PATH_AUTO     0u
#define MOE_PATH_GEMV     1u
#define MOE_PATH_GROUPED  2u
#define MOE_ACCUMULATE    4u  /* y += layer(x) instead of y = layer(x) */
/* Stage selection, for timing one kernel of the path in isolation: when any
 * MOE_STAGE bit is set, only the selected launches of the path run, in
 * order.  Stage n is the n-th kernel launch of the chosen path (see
 * moe_layer_stage_count).  Stages exchange their intermediate results
 * through the workspace, so a caller running them one at a time must run
 * all of them, in order, with the same arguments and workspace. */
#define MOE_STAGE(n)      (1u << (8 + (n)))
#define MOE_STAGE_MASK    0xFF00u
/* moe_stack_forward only: router lookahead with n (1 .. 63) workgroups per
 * prefetched expert; 0 (the default) turns it off. */
#define MOE_LOOKAHEAD(n)  ((uint32_t)(n) << 16)
#define MOE_LOOKAHEAD_MASK 0x3F0000u

/* ---------------------------------------------------------------- router */
/* moe_route -- noaux_tc routing of T tokens (GeekNews #31297, implemented
 * features: DeepSeek-V3-style sigmoid router with noaux_tc and
 * routed_scaling_factor).
 *   x       [T][H] fp32      token hidden states (unquantised)
 *   gate_w  [E][H] fp32      router weights
 *   bias    [E]    fp32      correction bias, used for selection only
 *   topk_idx [T][k] int32    out: selected experts, ordered by biased score
 *                            descending, ties to the lower index
 *   topk_w   [T][k] fp32     out: sigmoid scores of the selected experts
 *                            normalised to sum 1, times routed_scaling_factor
 * Arithmetic: logits, sigmoid and all comparisons in fp64; group score =
 * sum of the two largest biased scores of the group; the topk_group best
 * groups are kept, the others excluded.
 * ws: device scratch of at least moe_route_workspace_bytes(shape, T) bytes. */
int moe_route(const moe_shape_t *shape, const float *x, int32_t T, const float *gate_w,
              const float *bias, int32_t *topk_idx, float *topk_w,
              void *ws, size_t ws_bytes, hipStream_t stream);
size_t moe_route_workspace_bytes(const moe_shape_t *shape, int32_t T);

/* ---------------------------------------------------------------- activations */
/* moe_quant_act -- Q8_0-style activation quantisation (GeekNews #31297,
 * implemented features: integer-dot kernels on Q8_0-style int8
 * activations).  Per row and per block of 32 consecutive elements:
 * d = max|x| / 127 (fp32 IEEE division), q = round-half-even(x / d)
 * (fp32 IEEE division), clamped to [-127, 127]; d = 0 gives q = 0.
 *   x [T][D] fp32, D a multiple of 32  ->  q [T][D] int8, d [T][D/32] fp32 */
int moe_quant_act(const float *x, int32_t T, int32_t D, int8_t *q, float *d, hipStream_t stream);

/* moe_block_dots -- the integer block sums the expert kernels build on
 * (exported for bit-exact testing):
 *   out[t][r][b] = sum_{j<32} code[r][32b+j] * q[t][32b+j]   (int32)
 *   codes [rows][D*wbits/8] packed as in the weight layout above (16-byte
 *   aligned rows), q [T][D] int8, out [T][rows][D/32] int32. */
int moe_block_dots(int32_t wbits, const uint8_t *codes, int32_t rows, int32_t D,
                   const int8_t *q, int32_t T, int32_t *out, hipStream_t stream);

/* moe_stream_read -- a measurement aid: the practical read bandwidth
 * that every HBM-bound kernel here is judged against.  Reads `bytes` bytes
 * at src (16-byte aligned, bytes a multiple of 16) once, as the weight
 * streams of the decode kernels do (16-byte non-temporal loads, 8 in flight
 * per thread, every load instruction of a workgroup reading one contiguous
 * window), in a grid of MOE_STREAM_SINK_WORDS threads; thread i writes the
 * XOR of the 32-bit words it read to sink[i], so the XOR of all of sink is
 * the XOR of all words of the buffer.  sink: MOE_STREAM_SINK_WORDS uint32
 * (device).  bytes = 0 is a no-op; other misuse gives MOE_EINVAL. */
#define MOE_STREAM_SINK_WORDS (2048u * 256u)
int moe_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream);

/* ---------------------------------------------------------------- experts */
/* moe_expert_ffn -- one SwiGLU expert on quantised activations, unweighted:
 *   g = W_gate x, u = W_up x, h = silu(g) * u, (qh, dh) = quant(h),
 *   y = W_down h,  each product an integer block dot scaled by the
 *   activation block scale and the weight row scale.
 *   w       weights stack; `expert` selects expert `expert` of it
 *   q, d    [T][H] int8 and [T][H/32] fp32 (as from moe_quant_act)
 *   y       [T][H] fp32 out
 * ws: at least moe_workspace_bytes(shape, T, MOE_PATH_GEMV) bytes. */
int moe_expert_ffn(const moe_shape_t *shape, const moe_weights_t *w, int32_t expert,
                   const int8_t *q, const float *d, int32_t T, float *y,
                   void *ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- layer */
/* moe_layer_forward -- the whole MoE layer for T tokens:
 *   y[t] = sum_{i<k} topk_w[t][i] * FFN_{topk_idx[t][i]}(q(x[t])) + FFN_shared(q(x[t]))
 *   x        [T][H] fp32
 *   routed   stack of E experts; shared: one expert (NULL iff n_shared = 0)
 *   y        [T][H] fp32 out (or accumulated into with MOE_ACCUMULATE)
 *   idx_out, w_out  [T][k] (nullable): the routing, as moe_route returns it
 *   flags    MOE_PATH_*, MOE_ACCUMULATE, MOE_STAGE(n)
 * ws: at least moe_workspace_bytes(shape, T, flags) bytes, 256-byte aligned;
 *   calls that share a workspace must not overlap in time. */
int moe_layer_forward(const moe_shape_t *shape, const float *x, int32_t T, const float *gate_w,
                      const float *bias, const moe_weights_t *routed, const moe_weights_t *shared,
                      float *y, int32_t *idx_out, float *w_out, uint32_t flags,
                      void *ws, size_t ws_bytes, hipStream_t stream);
size_t moe_workspace_bytes(const moe_shape_t *shape, int32_t T, uint32_t flags);

/* moe_layer_forward_noalloc -- moe_layer_forward without a workspace
 * argument, for callers that cannot allocate device memory: code under
 * stream capture, tight serving loops, hosts that forbid allocation on the
 * hot path.  It calls no allocator.  Its workspace is a fixed device buffer
 * of MOE_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs
 * on until the process ends; the first call on a device looks up that
 * device's copy (a one-time symbol lookup, no allocation).
 * Arguments, results and errors are those of moe_layer_forward on the same
 * inputs (bit for bit), plus MOE_ESCRATCH, returned before anything is
 * launched, when moe_workspace_bytes(shape, T, flags) exceeds the buffer:
 * at hidden 6144 / intermediate 2048 / 256 experts / top-8, the GEMV path
 * for up to 8 tokens needs under 1 MB, the grouped path about 0.3 MB per
 * token, so batches above about 100 tokens take moe_layer_forward.
 * All calls on one GPU share its buffer: calls that overlap in time on one
 * GPU (different streams, or threads without ordering) race; calls ordered
 * on one stream do not.  Nothing in the buffer needs clearing between
 * calls. */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
int moe_layer_forward_noalloc(const moe_shape_t *shape, const float *x, int32_t T, const float *gate_w,
                              const float *bias, const moe_weights_t *routed, const moe_weights_t *shared,
                              float *y, int32_t *idx_out, float *w_out, uint32_t flags, hipStream_t stream);

/* number of stages moe_layer_forward runs for these arguments (the n of
 * MOE_STAGE(n) runs from 0 to this minus 1); < 0 on bad arguments.
 * GEMV path: router + quantiser (one launch for T <= 8, else two), then
 * plan, gate/up, down per chunk of tokens; a single token (T = 1) of the
 * production row widths is routed by the gate/up launch itself, so its
 * stages are router + quantiser, gate/up, down.  GROUPED path: 7 stages -- router
 * logits, top-k, quantiser, permutation (three launches), gate/up, down,
 * combine. */
int moe_layer_stage_count(const moe_shape_t *shape, int32_t T, uint32_t flags);

/* ---------------------------------------------------------------- stack */
/* moe_rmsnorm -- out = x / sqrt(mean(x^2) + eps) * g per row, the sum of
 * squares and the scaling in fp64 (the norm before each MoE layer of the
 * decode stack x_{l+1} = x_l + MoE_l(RMSNorm(x_l))).
 *   x [T][H], g [H], out [T][H] fp32; out may alias x. */
int moe_rmsnorm(const float *x, const float *g, double eps, int32_t T, int32_t H, float *out,
                hipStream_t stream);

/* moe_stack_forward -- a decode stack of MoE layers (wpnews.pro spec table:
 * 75 MoE layers), each on its own weights and re-routed:
 *   for l in 0 .. n_layers-1:   x = x + MoE_l(RMSNorm_l(x))
 * RMSNorm as moe_rmsnorm with eps and the layer's norm weight; MoE_l as
 * moe_layer_forward with the layer's router, correction bias and experts;
 * the layer result is rounded to fp32 and added to x in fp32.  On the GEMV
 * path (T <= 8) with H <= 8192, H % 4 == 0 and 16-byte aligned x and norm
 * weights, the router launch forms RMSNorm_l(x) itself (the same fp32 values
 * as moe_rmsnorm) and no separate RMSNorm launch runs.
 *   x        [T][H] fp32 residual stream, updated in place
 *   layers   HOST array of n_layers descriptors (device pointers inside)
 *   idx_out, w_out  [n_layers][T][k] (nullable): every layer's routing
 *   flags    MOE_PATH_* (MOE_ACCUMULATE is implied); MOE_STAGE(n) selects
 *            stage n of every layer as moe_layer_stage_count counts them,
 *            with a separate RMSNorm launch (when there is one) run with
 *            stage 0; MOE_LOOKAHEAD(n) turns on the router lookahead
 *            (wpnews.pro Colibri page, paragraph "Router-lookahead prefetch
 *            (PILOT=1)"): for one token on the GEMV path, where the router
 *            launch normalises its input, layer l's router launch also runs
 *            layer l+1's router (its norm weight, router weights and
 *            correction bias) on layer l's input x, and layer l's gate/up
 *            launch gets n extra workgroups per expert that prediction
 *            selects (its top_k ranks by the noaux_tc selection, top-p not
 *            applied) and per shared expert of layer l+1; they read that
 *            expert's codes and scales with non-temporal loads so that they
 *            sit in the memory-side cache when layer l+1 reads them.  The
 *            results are identical with and without it; only the timing
 *            changes.  Elsewhere (T > 1, grouped path) it is ignored.
 * ws: at least moe_stack_workspace_bytes(shape, T, flags) bytes, 256-byte
 *   aligned (the lookahead adds the predicted logits and one word per
 *   wave of its workgroups).  The launches only read the layers array during the call, so a
 *   stream capture of one call replays with the same device pointers. */
typedef struct {
    const float *gate_w;        /* [E][H] router weights */
    const float *bias;          /* [E] correction bias */
    const float *norm_g;        /* [H] RMSNorm weight */
    moe_weights_t routed;       /* stack of E experts */
    moe_weights_t shared;       /* shared expert (ignored when n_shared = 0) */
} moe_layer_t;
int moe_stack_forward(const moe_shape_t *shape, float *x, int32_t T, const moe_layer_t *layers,
                      int32_t n_layers, double eps, int32_t *idx_out, float *w_out, uint32_t flags,
                      void *ws, size_t ws_bytes, hipStream_t stream);
size_t moe_stack_workspace_bytes(const moe_shape_t *shape, int32_t T, uint32_t flags);

/* ---------------------------------------------------------------- permute */
/* moe_permute -- the token permutation of the grouped path (batch-union
 * MoE, GeekNews #31297 implemented features), exported for testing.
 * Assignment a = t*k + i routes token t to expert idx[a].
 *   off  [E+1]  out: off[e] .. off[e+1]-1 are expert e's rows
 *   perm [T*k]  out: perm[row] = a, ascending a within each expert
 *   inv  [T*k]  out: inv[a] = row
 * ws: at least moe_permute_workspace_bytes(T, k, E) bytes, 256-byte aligned.
 * idx entries lie in [0, E), or are -1 for an assignment adaptive top-p
 * dropped: it gets no row and inv = -1, and rows 0 .. off[E]-1 hold the
 * kept assignments (any other value is treated as -1). */
int moe_permute(const int32_t *idx, int32_t T, int32_t k, int32_t E, int32_t *perm,
                int32_t *off, int32_t *inv, void *ws, size_t ws_bytes, hipStream_t stream);
size_t moe_permute_workspace_bytes(int32_t T, int32_t k, int32_t E);

/* ---------------------------------------------------------------- MTP draft verification */
/* moe_mtp_accept -- the acceptance step after a verify forward (GeekNews
 * #31297, implemented features: the multi-token-prediction head drafts
 * tokens, the main model verifies them in one batched forward whose MoE
 * layers run as moe_layer_forward with T = 1 + D, and rejection sampling
 * keeps sampled output lossless; useful options: --temp, 0 = greedy).
 * For each of B sequences with D drafts:
 *   tau > 0: p_i, q_i = softmax(logits_i / tau) in fp64; draft x_i is kept
 *     while u[i] * q_i(x_i) < p_i(x_i) (i ascending); at the first refusal
 *     (i = j) the emitted token is the inverse-CDF draw with u[D], in
 *     ascending token order, of max(0, p_j - q_j) (of p_j if that has no
 *     mass); after D kept drafts it is the draw of p_D.  This is speculative
 *     sampling (Leviathan et al. 2023; Chen et al. 2023); no nucleus filter.
 *   tau = 0: drafts are kept while they equal the target's argmax (lowest
 *     token on ties) and the emitted token is the argmax at the first
 *     mismatch, or of p_D.
 * All device pointers:
 *   draft    [B][D] int32, tokens in [0, V) (one outside is refused)
 *   p_logits [B][D+1][V] fp32: the target model's logits at the D+1
 *            verified positions (position i scores the token after draft i-1)
 *   q_logits [B][D][V] fp32: the draft model's logits each draft was drawn
 *            from (nullable when D = 0)
 *   u        [B][D+1] fp64 uniforms in [0, 1), the caller's random numbers:
 *            u[i] tests draft i, u[D] draws the emitted token
 *   n_acc    [B] out: drafts kept (0 .. D)
 *   next     [B] out: the token emitted after them
 * Sizes: D <= 16, V <= 1,048,576; V % 4 == 0 with 16-byte aligned rows
 * takes vector loads.  Logits must be finite.  Every token decision is made
 * in fp64; the probabilities come from per-4096-token chunk sums combined
 * in a fixed order, so results are run-to-run identical (and agree with a
 * sequential fp64 evaluation except where a decision lies within rounding
 * of its boundary).
 * ws: at least moe_mtp_accept_workspace_bytes(B, D, V) bytes, 256-byte
 *   aligned.  Four launches (two when tau = 0). */
int moe_mtp_accept(int32_t B, int32_t D, int32_t V, const int32_t *draft, const float *p_logits,
                   const float *q_logits, float tau, const double *u, int32_t *n_acc, int32_t *next,
                   void *ws, size_t ws_bytes, hipStream_t stream);
size_t moe_mtp_accept_workspace_bytes(int32_t B, int32_t D, int32_t V);

/* ---------------------------------------------------------------- expert tier
 * HBM / host expert tier (the pages' streaming design moved one tier up:
 * GeekNews #31297, implemented features, per-layer expert caches and the
 * pinned hot store; wpnews.pro feature list, "Live tier adaptation
 * (--repin N)").  A model whose routed experts exceed HBM keeps every
 * expert in pinned host memory and a fixed number of HBM slots per layer
 * for the hot ones.  The layer reads each routed expert where the expert
 * table says it is: from its HBM slot, or straight from pinned host memory
 * over PCIe (no copy in the forward, no host synchronisation).  The routing
 * counts every selection per expert on the device (the heat map).
 *
 * moe_tier_create -- one layer's tier.  host: that layer's routed stacks in
 *   pinned, device-mapped host memory (hipHostMalloc; [E][rows][bytes] as in
 *   moe_weights_t), owned by the caller and kept alive and unchanged until
 *   moe_tier_destroy.  slots: HBM slots, 0..E.  Allocates the slots, the
 *   table and the counts in device memory (synchronous); no expert is in
 *   HBM until the first repin.  The shape must be int4 at the production
 *   row widths (hidden and inter whose packed rows take the row-sweep
 *   kernels: 6144 and 2048); else MOE_EUNSUPPORTED.  A host pointer that is
 *   not device-mapped pinned memory: MOE_EINVAL.  *out = NULL on error.
 * moe_tier_repin -- the live repin: reads the counts (synchronises stream),
 *   applies moe_tier_plan with max_swaps = 4, copies each expert entering
 *   HBM into its slot (asynchronous host-to-device copies on stream), then
 *   updates the table and halves every count (the heat decays), all on
 *   stream after the work already queued there.  *copied (if not NULL) =
 *   experts copied.  Work queued on stream later sees the new table.
 * moe_tier_plan -- the repin decision alone (host only, no GPU): heat[E],
 *   slot_in[E] = current slot of each expert or -1; slot_out[E] = the slots
 *   after the repin.  Free slots first take the hottest streamed experts
 *   with heat > 0 (lowest slot first; hottest first, ties to the lower
 *   index).  Then at most max_swaps replacements: the next hottest streamed
 *   expert takes the slot of the coldest pinned one (ties: the higher
 *   index goes first) while its heat exceeds 1.25 times the other's (the
 *   25% hysteresis).  Returns the number of experts entering HBM, or minus
 *   MOE_EINVAL for bad arguments (an inconsistent slot_in).
 * moe_tier_prefetch -- the router lookahead's prefetch (wpnews.pro feature
 *   list, "Router-lookahead prefetch (PILOT=1)": layer L+1's router run on
 *   layer L's state predicts its experts, which a separate I/O thread
 *   fetches while layer L computes; here a side stream's copies): experts[n] (host) are
 *   one layer's predicted experts, in priority order.  Each one neither
 *   pinned nor already prefetched is copied into the tier's next prefetch
 *   slot (a ring of min(16, E) slots, apart from the pinned ones; the
 *   ring's oldest prefetch returns to the host stack) by asynchronous
 *   host-to-device copies on stream, then the table is updated on stream;
 *   at most one ring's worth per call, entries < 0 or >= E ignored.  The
 *   routing is unchanged wherever an expert is read from.  *copied (if not
 *   NULL) = experts copied.  The caller orders stream against every
 *   forward on the same tier (events): a forward that overlaps a prefetch or
 *   a repin of its tier races.  A repin frees the prefetch slot of an
 *   expert it pins.
 * moe_tier_resident -- slot_of[E] (host): each expert's pinned HBM slot,
 *   -2 for a prefetched expert, else -1.
 * moe_tier_counts -- counts[E] (host) = the current heat (synchronises
 *   stream).
 * moe_layer_forward_tiered -- moe_layer_forward on the GEMV path (T <= 8;
 *   MOE_PATH_GROUPED or T > 8: MOE_EUNSUPPORTED) with the routed experts
 *   read through the tier's table and counted.  Arguments and errors as
 *   moe_layer_forward, the workspace that of the GEMV path
 *   (moe_workspace_bytes with MOE_PATH_GEMV).  The results equal
 *   moe_layer_forward's on the same weights bit for bit, wherever each
 *   expert is.  The counts and the table are shared by every call on the
 *   tier: calls that overlap with a repin of the same tier race.
 * moe_tier_destroy -- frees the tier (no work using it may be in flight). */
typedef struct moe_tier moe_tier_t;
int moe_tier_create(const moe_shape_t *shape, const moe_weights_t *host, int32_t slots, moe_tier_t **out);
int moe_tier_repin(moe_tier_t *tier, int32_t *copied, hipStream_t stream);
int moe_tier_plan(const uint32_t *heat, int32_t E, int32_t C, const int32_t *slot_in, int32_t *slot_out,
                  int32_t max_swaps);
int moe_tier_prefetch(moe_tier_t *tier, const int32_t *experts, int32_t n, int32_t *copied, hipStream_t stream);
int moe_tier_resident(const moe_tier_t *tier, int32_t *slot_of);
int moe_tier_counts(const moe_tier_t *tier, uint32_t *counts, hipStream_t stream);
int moe_layer_forward_tiered(const moe_shape_t *shape, const float *x, int32_t T, const float *gate_w,
                             const float *bias, const moe_tier_t *tier, const moe_weights_t *shared, float *y,
                             int32_t *topk_idx, float *topk_w, uint32_t flags, void *workspace,
                             size_t workspace_bytes, hipStream_t stream);
void moe_tier_destroy(moe_tier_t *tier);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
