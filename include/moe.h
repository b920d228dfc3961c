/*
 * moe.h -- C ABI of the MI355X (gfx950) fused-MoE layer library, libmoe.so.
 *
 * The library computes one Mixture-of-Experts layer on one GPU with no data
 * or expert parallelism, as the modular "prepare -> experts -> finalize"
 * path with the no-op (no dispatch/combine) prepare/finalize of the pages:
 *
 *   "Fused MoE Kernel Features" (vLLM design doc): modular kernels split
 *     into a prepare/finalize object and an experts object; prepare takes
 *     "standard"-format activations and emits the quantised type, finalize
 *     returns standard format in the original dtype; quant formats G(128)
 *     (per-token group of 128), A (per token), T (per tensor); for top_k == 1
 *     some models apply the router weight to the input instead of the output.
 *   "[vLLM] MoE Oracle & Prepare/Finalize": the no-DP/EP prepare(a1,
 *     topk_weights, topk_ids, ..., apply_router_weight_on_input,
 *     quant_config) and finalize(output, fused_expert_output, topk_weights,
 *     topk_ids, ...) contracts.
 *   "[flashinfer] MoE Finalize + AllReduce fusion": finalize fused with the
 *     optional shared-expert row, residual add and RMSNorm (hidden 7168).
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is a DEVICE pointer unless marked (host).  The
 *     caller allocates and owns all memory; the library never allocates,
 *     frees or keeps a pointer after returning.
 *   - bf16 tensors are passed as uint16_t bit patterns, fp8 tensors as
 *     uint8_t OCP E4M3 codes (bias 7, no infinities, max finite 448);
 *     all tensors are dense row-major with the shapes given.
 *   - Work is enqueued asynchronously on `stream`; nothing synchronises the
 *     host.  Argument errors are detected on the host BEFORE anything is
 *     enqueued (no partial work) and returned as a moe_status; device-side
 *     faults surface at the caller's next synchronisation.  A launch failure
 *     reported by the HIP runtime is returned as MOE_ERR_HIP.
 *   - T == 0 is a valid no-op wherever T appears (moe_align still writes its
 *     zero counts/offsets).
 *   - moe_last_error() returns a thread-local message for the last failing
 *     call on the calling thread.
 *   - The library holds no state besides its compiled kernels; calls on
 *     different streams with disjoint outputs may overlap.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* null required pointer, bad size, top_k out of range, ... */
  MOE_ERR_UNSUPPORTED = 2,  /* a valid request outside what the kernels implement */
  MOE_ERR_WORKSPACE = 3,    /* workspace missing or smaller than the *_workspace_bytes query */
  MOE_ERR_HIP = 4           /* the HIP runtime reported a launch error */
} moe_status;

typedef enum moe_scoring {
  MOE_SCORING_SOFTMAX = 0,  /* softmax over all E logits */
  MOE_SCORING_SIGMOID = 1   /* elementwise sigmoid */
} moe_scoring;

/* Activation quant formats of the quant-format key ("Fused MoE Kernel
 * Features", table key): G(128) grouped by 128, A per activation token,
 * T per tensor.  Every fp8 format takes E4M3 weights with one fp32 scale
 * per 128x128 block of each matrix. */
typedef enum moe_quant {
  MOE_QUANT_NONE = 0,        /* bf16 activations and weights */
  MOE_QUANT_FP8_G128 = 1,    /* fp8 E4M3, one fp32 scale per (row, 128-column group): [T, H/128] */
  MOE_QUANT_FP8_TOKEN = 2,   /* fp8 E4M3, one fp32 scale per row ("A"): [T] */
  MOE_QUANT_FP8_TENSOR = 3   /* fp8 E4M3, one fp32 scale for the tensor ("T"): [1] */
} moe_quant;

/* The activation names of the fused-experts kernel table ("Fused MoE Kernel
 * Features", fused experts section): "silu", "silu_no_mul", "gelu",
 * "gelu_no_mul".  gelu is the exact form v * Phi(v) = v/2 (1 + erf(v/sqrt 2))
 * (the table lists the tanh approximation separately, as gelu_tanh). */
typedef enum moe_activation {
  MOE_ACT_SILU_MUL = 0,     /* z = silu(gate) * up, silu(v) = v / (1 + exp(-v)) ("silu") */
  MOE_ACT_SILU_NO_MUL = 1,  /* z = silu(W1 a), no up projection ("silu_no_mul") */
  MOE_ACT_GELU_MUL = 2,     /* z = gelu(gate) * up ("gelu") */
  MOE_ACT_GELU_NO_MUL = 3   /* z = gelu(W1 a), no up projection ("gelu_no_mul") */
} moe_activation;

/* Number of events moe_forward records when given a stage_events array. */
#define MOE_NUM_STAGE_EVENTS 8

/*
 * Expert weights (host struct holding device pointers).
 *   R = 2*inter for the gated activations MOE_ACT_SILU_MUL / MOE_ACT_GELU_MUL
 *       (rows [0, I) = gate W1, rows [I, 2I) = up W3),
 *       inter   for MOE_ACT_SILU_NO_MUL / MOE_ACT_GELU_NO_MUL (W1 only).
 *   w13        [E, R, H]   bf16 bits, or E4M3 codes (any fp8 quant)
 *   w13_scale  [E, R/128, H/128] fp32 block scales (fp8 only, else NULL)
 *   w2         [E, H, I]
 *   w2_scale   [E, H/128, I/128]
 *   shared_*   the always-on shared expert, same layouts without the E axis and
 *              with I_s = shared_inter; shared_inter == 0 means no shared expert.
 */
typedef struct moe_weights {
  int32_t num_experts;
  int32_t inter;
  int32_t quant;
  int32_t shared_inter;
  const void* w13;
  const float* w13_scale;
  const void* w2;
  const float* w2_scale;
  const void* shared_w13;
  const float* shared_w13_scale;
  const void* shared_w2;
  const float* shared_w2_scale;
} moe_weights;

/* Human-readable name of a status code (static string). */
const char* moe_status_str(int status);

/* Thread-local description of the last failed call on this thread ("" if none). */
const char* moe_last_error(void);

/*
 * moe_route -- top-k routing over router logits.
 * The pages consume topk_ids/topk_weights without defining them; the rule
 * implemented: per token, experts by descending logit, ties to the lower
 * expert index, first top_k kept (slot j = j-th largest).  Weights:
 *   SOFTMAX, renormalize=1: w_j = exp(l_j - l_0) / sum_{j'<k} exp(l_j' - l_0)
 *   SOFTMAX, renormalize=0: w_j = exp(l_j - max) / sum_{e<E} exp(l_e - max)
 *   SIGMOID, renormalize=1: w_j = sig(l_j) / sum_{j'<k} sig(l_j')
 *   SIGMOID, renormalize=0: w_j = sig(l_j)
 *   logits       [T, E] fp32, finite (precondition)
 *   topk_ids     [T, top_k] int32 out;  topk_weights [T, top_k] fp32 out
 * Limits: 1 <= E <= 1024, 1 <= top_k <= min(E, 64); else MOE_ERR_INVALID_ARG.
 */
int moe_route(const float* logits, int T, int E, int top_k, int scoring, int renormalize,
              int32_t* topk_ids, float* topk_weights, hipStream_t stream);

/*
 * The quant_config of the pages' prepare contract ("[vLLM] MoE Oracle &
 * Prepare/Finalize", no-DP/EP prepare code): which activation format
 * prepare emits and the weight block grid the experts expect with it.
 *   quant      a moe_quant
 *   act_group  activation channels per scale: 128 with MOE_QUANT_FP8_G128;
 *              0 with MOE_QUANT_FP8_TOKEN and MOE_QUANT_FP8_TENSOR (the
 *              group is the row, or the whole tensor); ignored with NONE
 *   w_block_n, w_block_k  weight-scale block (rows, columns): 128, 128 with
 *              every fp8 format; ignored with NONE
 * Any other group or block size is MOE_ERR_UNSUPPORTED.
 */
typedef struct moe_quant_config {
  int32_t quant;
  int32_t act_group;
  int32_t w_block_n;
  int32_t w_block_k;
} moe_quant_config;

/*
 * moe_prepare -- the no-DP/EP prepare ("[vLLM] MoE Oracle & Prepare/Finalize",
 * the no-DP/EP prepare code: prepare(a1, topk_weights, topk_ids, ...,
 * apply_router_weight_on_input, quant_config)): if apply_router_weight_on_input,
 * top_k must be 1 (else MOE_ERR_INVALID_ARG, the page's assert) and
 * a = bf16(a1 * bf16(topk_weights)); then quantise per qc->quant:
 *   MOE_QUANT_NONE:     a1q [T, H] bf16 = a        (a1q_scale unused, may be NULL)
 *   MOE_QUANT_FP8_G128: per (t, g): s = max(amax, 1e-10) / 448 (fp32),
 *                       q = E4M3_rne_sat(a / s);   a1q [T, H] E4M3, a1q_scale [T, H/128] fp32
 *   MOE_QUANT_FP8_TOKEN: the same rule with amax over the whole row; a1q_scale [T]
 *   MOE_QUANT_FP8_TENSOR: the same rule with amax over all of a; a1q_scale [1]
 *   a1             [T, H] bf16
 *   topk_weights   [T, top_k] fp32 (read only when apply_router_weight_on_input)
 *   topk_ids       [T, top_k] int32, accepted for the pages' signature and not
 *                  read: without expert parallelism there is no dispatch, so
 *                  the ids pass through unchanged (may be NULL)
 *   qc             (host) the quant config above; NULL is MOE_ERR_INVALID_ARG
 * Limits: H % 8 == 0; H % 128 == 0 for fp8; H <= 16384 per token.  a1q may
 * alias a1 only for MOE_QUANT_NONE.
 */
int moe_prepare(const uint16_t* a1, int T, int H, const float* topk_weights,
                const int32_t* topk_ids, int top_k, int apply_router_weight_on_input,
                const moe_quant_config* qc /* host */, void* a1q, float* a1q_scale,
                hipStream_t stream);

/*
 * moe_align -- sort the T*top_k flat rows i = t*top_k + j by expert into
 * block_m-padded groups.  Not a step the pages define: they hand topk_ids
 * to the experts and say only that each expert computes on its own tokens
 * ("Fused MoE Kernel Features", fused experts section); this is the plain
 * reading, a stable counting sort (deterministic; only one result is correct):
 *   expert_counts[e]   = #{i : ids[i] == e}                                  [E]
 *   expert_offsets[0]  = 0, [e+1] = [e] + ceil(counts[e] / block_m) * block_m  [E+1]
 *   sorted_token_ids   = per expert, its flat rows in ascending order, then
 *                        the pad sentinel T*top_k up to the next offset; the
 *                        sentinel also fills [offsets[E], sorted capacity)     [sorted cap]
 *   block_expert_ids[b]= expert owning slots [b*block_m, (b+1)*block_m), -1
 *                        for blocks at or past offsets[E]                     [block cap]
 *   num_tokens_post_padded[0] = offsets[E]                                    [1]
 * Capacities (moe_align_capacity): sorted cap = T*k + min(E, T*k)*(block_m-1),
 * block cap = ceil(sorted cap / block_m).  workspace: moe_align_workspace_bytes.
 * Limits: block_m in {16, 32, 64, 128, 256}; 1 <= E <= 1024; ids in [0, E)
 * (precondition; out-of-range ids are dropped from every output).
 * Paths: up to 32768 ids, one workgroup.  Above that, with E <= 256, at
 * most 65536 ids per CU the stream may use and topk_ids 16-byte aligned,
 * one launch that reads the ids once (not while the stream is capturing a
 * graph, nor with the environment variable MOE_ALIGN_RESIDENT=0); otherwise
 * three launches over tiles.  All paths give the same outputs.  The
 * one-launch path needs its grid resident at once (one workgroup per CU)
 * and waits on it for a bounded time: should a wait ever give up (another
 * kernel holding CUs for about a second), num_tokens_post_padded is -1 and
 * the other outputs are unspecified.  Calls that share a workspace must not
 * overlap.
 */
int moe_align(const int32_t* topk_ids, int T, int top_k, int E, int block_m,
              int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_token_ids,
              int32_t* block_expert_ids, int32_t* num_tokens_post_padded,
              void* workspace, size_t workspace_bytes, hipStream_t stream);
/* (host) capacities of sorted_token_ids and block_expert_ids. */
int moe_align_capacity(int T, int top_k, int E, int block_m,
                       int64_t* sorted_capacity, int64_t* block_capacity);
/* (host) workspace moe_align needs: 0 for T*top_k <= 32768 ids; above that,
 * the larger of the tiled path's 4*E*(9*tiles + 1) bytes (per-expert counts
 * of each eighth of a tile, the tiles' per-expert totals and the expert
 * totals), where tiles = ceil(T*top_k / tile) and tile is the smallest power
 * of two in [2048, 8192] with tile*1024 >= T*top_k (8192 above 2^23 ids),
 * and the one-launch path's 8*257 + 4*G*E bytes with G = min(256,
 * ceil(T*top_k / 4096)) (arrival flags and a go word; up to G tiles'
 * per-expert counts). */
size_t moe_align_workspace_bytes(int T, int top_k, int E, int block_m);

/*
 * moe_experts -- the modular experts stage ("Fused MoE Kernel Features":
 * modular experts take pre-quantised input and return the original dtype):
 * for every flat row i = t*k + j with e = topk_ids[t, j]
 *   h = W13[e] a[t] (fp32 accumulation), z = act(h),
 *   fused_expert_output[t, j, :] = bf16(W2[e] z)                  [T, top_k, H] bf16 out
 * z is held in bf16 (MOE_QUANT_NONE) or re-quantised to E4M3 G(128) along I
 * (every fp8 format) between the two grouped GEMMs.  With a shared expert, additionally
 *   shared_out[t, :] = bf16(W2s act(W13s s[t]))                    [T, H] bf16 out
 * where s = shared_in/shared_in_scale, the unweighted input in a1q's format
 * (pass a1q when the router weight was not applied on the input).
 *   a1q, a1q_scale      prepare's output ([T, H] + the format's scales for fp8)
 *   sorted_token_ids, block_expert_ids, num_tokens_post_padded: moe_align's
 *                       output for the same topk_ids and block_m
 *   workspace           moe_experts_workspace_bytes bytes
 * Limits: H % 128 == 0 (the second GEMM writes 128-column tiles); I % 64 == 0
 * for the gated bf16 activations, I % 128 == 0 otherwise; H, I <= 16384;
 * weights->quant must equal the activation format.
 */
int moe_experts(const void* a1q, const float* a1q_scale, const void* shared_in,
                const float* shared_in_scale, int T, int H, int top_k,
                const moe_weights* weights /* host */, int activation,
                const int32_t* sorted_token_ids, const int32_t* block_expert_ids,
                const int32_t* num_tokens_post_padded, int block_m,
                uint16_t* fused_expert_output, uint16_t* shared_out,
                void* workspace, size_t workspace_bytes, hipStream_t stream);
/* (host) workspace moe_experts needs. */
size_t moe_experts_workspace_bytes(int T, int H, int top_k, const moe_weights* weights,
                                   int activation, int block_m);
/*
 * (host) Where moe_experts keeps the intermediate activation z inside its
 * workspace.  z stays there after the call until the workspace is reused,
 * so a caller can inspect what the second GEMM consumed.  out[5] receives
 * byte offsets from the workspace start (SIZE_MAX when absent):
 *   out[0] z of the routed rows, [rows, I] bf16 (E4M3 codes for fp8); row r
 *          belongs to flat row sorted_token_ids[r] (pad rows hold no data)
 *   out[1] its G(128) scales [rows, I/128] fp32 (fp8 only)
 *   out[2] z of the shared expert [T, I_s]   out[3] its scales (fp8 only)
 *   out[4] rows = block capacity * block_m (a count, not an offset)
 */
int moe_experts_workspace_layout(int T, int H, int top_k, const moe_weights* weights,
                                 int activation, int block_m, size_t* out);

/*
 * moe_experts_batched -- the experts stage on the batched activation format
 * ("Fused MoE Kernel Features", backend and fused experts sections: prepare
 * emits either the standard or the batched format, and the batched experts
 * kernels take one batch of rows per expert).  With M = max_tokens, rows
 * [0, expert_num_tokens[e]) of batch e are expert e's input; for each such
 * row m
 *   out[e, m, :] = bf16(W2[e] act(W13[e] a[e, m]))           (fp32 accumulation)
 * exactly as moe_experts computes one routed row (z held in bf16, or E4M3
 * G(128) along I for every fp8 format).  Rows m >= expert_num_tokens[e] of
 * `out` are not written.
 *   a                  [E, M, H] bf16, or E4M3 codes for an fp8 format
 *   a_scale            fp8 only: G(128) [E, M, H/128]; per token [E, M];
 *                      per tensor [1] (fp32); the format is weights->quant
 *   expert_num_tokens  [E] int32 on the device; values are clamped to [0, M]
 *   out                [E, M, H] bf16
 *   block_m            GEMM row block, 0 = moe_pick_block_m(M, 1, 1, quant)
 *   workspace          moe_experts_batched_workspace_bytes bytes
 * The shared expert of `weights` (if any) is not run: it reads the
 * token-major input, which this format does not carry.  M == 0 is a no-op.
 * Limits: as moe_experts; E * (M + block_m) <= 2^30.
 */
int moe_experts_batched(const void* a, const float* a_scale, const int32_t* expert_num_tokens,
                        int max_tokens, int H, const moe_weights* weights /* host */,
                        int activation, int block_m, uint16_t* out, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);
/* (host) workspace moe_experts_batched needs (0 for invalid arguments). */
size_t moe_experts_batched_workspace_bytes(int max_tokens, int H, const moe_weights* weights,
                                           int activation, int block_m);
/*
 * (host) Where moe_experts_batched keeps its row schedule and the
 * intermediate z inside its workspace (readable after a call until the
 * workspace is reused).  out[4] receives byte offsets from the workspace
 * start (SIZE_MAX when absent):
 *   out[0] the schedule, int32 [rows]: row r of z is batch row
 *          sorted[r] = e*M + m, or the pad sentinel E*M (experts in index
 *          order, each padded to a multiple of block_m)
 *   out[1] z [rows, I] bf16 (E4M3 codes for fp8)
 *   out[2] its G(128) scales [rows, I/128] fp32 (fp8 only)
 *   out[3] rows = E * ceil(M / block_m) * block_m (a count, not an offset)
 */
int moe_experts_batched_workspace_layout(int max_tokens, int H, const moe_weights* weights,
                                         int activation, int block_m, size_t* out);

/*
 * moe_finalize -- the no-DP/EP finalize (weight-and-reduce over the top-k
 * expert rows) with the flashinfer finalize fusions:
 *   acc[t] = sum_j w'[t,j] * y[t,j,:]   (slot order; w' = 1 when the weight was
 *            applied on the input -- applied to the input instead of the output)
 *          + shared[t] + residual[t]    (each optional, NULL = absent)
 *   out[t] = acc[t] / sqrt(mean(acc[t]^2) + eps) * gamma    if gamma != NULL
 *          = acc[t]                                         otherwise
 *   output [T, H]: bf16 (out_quant NONE) or E4M3 + output_scale [T, H/128] fp32
 *   residual_out [T, H] bf16 = bf16(acc) when non-NULL
 *   fused_expert_output [T, top_k, H] bf16; topk_weights [T, top_k] fp32;
 *   topk_ids [T, top_k] is accepted for the pages' signature and not read
 *   (no expert map without EP); gamma [H] bf16.
 * Limits: H % 8 == 0, H <= 16384; H % 128 == 0 for fp8 output; 1 <= top_k <= 64.
 */
int moe_finalize(void* output, float* output_scale, int out_quant,
                 const uint16_t* fused_expert_output, const float* topk_weights,
                 const int32_t* topk_ids, int T, int top_k, int H,
                 int apply_router_weight_on_input, const uint16_t* shared,
                 const uint16_t* residual, uint16_t* residual_out, const uint16_t* gamma,
                 float eps, hipStream_t stream);

/*
 * moe_forward -- the whole layer, enqueued on one stream with no host sync:
 * route -> prepare -> align -> experts (routed GEMM-1, GEMM-2, shared expert)
 * -> finalize, intermediates in `workspace`.  The pages describe the stages
 * one by one ("[vLLM] MoE Oracle & Prepare/Finalize": the modular kernel runs
 * prepare, the experts and finalize in turn); this call is their composition
 * in that order, with routing (not on the pages) in front, and it takes the
 * same readings as the stage calls above.  The activation format is
 * weights->quant with the fixed 128 group and 128x128 weight blocks.
 *   x [T, H] bf16; logits [T, E] fp32; weights (host struct) as moe_experts;
 *   block_m 0 = choose (moe_pick_block_m); residual/gamma/residual_out as
 *   moe_finalize; output/output_scale per out_quant.
 *   stage_events (host array, may be NULL): MOE_NUM_STAGE_EVENTS caller-created
 *   hipEvents recorded on `stream` at: start, after route, prepare, align,
 *   routed GEMM-1, routed GEMM-2, shared expert, finalize.
 */
int moe_forward(const uint16_t* x, const float* logits, int T, int H, int top_k,
                int scoring, int renormalize, int apply_router_weight_on_input,
                const moe_weights* weights /* host */, int activation, int block_m,
                const uint16_t* residual, const uint16_t* gamma, float eps, int out_quant,
                void* output, float* output_scale, uint16_t* residual_out,
                void* workspace, size_t workspace_bytes,
                hipEvent_t* stage_events /* host, nullable */, hipStream_t stream);
/* (host) workspace moe_forward needs for these sizes (block_m 0 = chosen). */
size_t moe_forward_workspace_bytes(int T, int H, int top_k, const moe_weights* weights,
                                   int activation, int block_m,
                                   int apply_router_weight_on_input);
/*
 * moe_forward_graph_* -- the modular layer submitted as one graph launch (the
 * kernels of moe_forward; the fused single kernel of "[vLLM] MoE Oracle &
 * Prepare/Finalize"'s monolithic mode is moe_forward_monolithic below).
 * create captures moe_forward, for
 * exactly these sizes, weights and buffers, into an executable HIP graph;
 * launch replays it on any stream with one call, with no per-kernel host
 * work -- what a decode step needs, where the layer's kernels are shorter
 * than their submission.  The graph reads and writes the very buffers given
 * here, so the caller refreshes x and logits (and residual, gamma) in place
 * before each launch and reads output afterwards; replays on one stream
 * run in order, and two replays of one graph must not overlap.
 *   Arguments as moe_forward (no stage events); stream must be a created
 *   stream (capture is not allowed on the null stream), and nothing else may
 *   be enqueued on it from this thread while create runs.
 *   graph (host out): opaque handle; release it with moe_forward_graph_destroy.
 * Errors: moe_forward's checks (nothing captured, *graph = NULL) or
 * MOE_ERR_HIP from capture/instantiation.
 */
typedef struct moe_graph moe_graph;
int moe_forward_graph_create(const uint16_t* x, const float* logits, int T, int H, int top_k,
                             int scoring, int renormalize, int apply_router_weight_on_input,
                             const moe_weights* weights /* host */, int activation, int block_m,
                             const uint16_t* residual, const uint16_t* gamma, float eps,
                             int out_quant, void* output, float* output_scale,
                             uint16_t* residual_out, void* workspace, size_t workspace_bytes,
                             hipStream_t stream, moe_graph** graph /* host out */);
int moe_forward_graph_launch(moe_graph* graph, hipStream_t stream);
/* Releases the graph (NULL is a no-op); no replay of it may still be pending. */
int moe_forward_graph_destroy(moe_graph* graph);

/*
 * moe_forward_monolithic -- the whole layer as ONE kernel launch, for
 * decode-sized batches: the monolithic mode of "[vLLM] MoE Oracle &
 * Prepare/Finalize" (section on modular vs monolithic kernels: the monolithic
 * mode fuses routing, the experts and finalize into a single kernel instead
 * of the modular chain of stages).  One persistent launch runs routing, both
 * GEMMs of the routed and the shared experts and finalize, with grid-wide
 * barriers between the phases, so its workgroups must all be resident at
 * once: one per CU the stream may use.
 *   Arguments as moe_forward (no block_m, no stage events), with these
 *   limits: bf16 weights (quant MOE_QUANT_NONE), 1 <= T <= 512,
 *   T*top_k <= 512; out_quant MOE_QUANT_NONE or MOE_QUANT_FP8_G128.
 *   workspace (device): at least moe_forward_monolithic_workspace_bytes.
 *   The result equals moe_forward's up to the summation order of the GEMMs
 *   (fp32 sums of the same bf16 products, rounded once to bf16).
 * Errors: moe_forward's argument checks; MOE_ERR_UNSUPPORTED outside the
 * limits above, on a stream under graph capture (each launch carries a
 * fresh barrier epoch, which a replay would repeat), or when the kernel
 * cannot place a workgroup on the stream's CUs; MOE_ERR_WORKSPACE.  Nothing
 * is enqueued on an error.  The barriers' waits are bounded (about a second
 * each): if the grid cannot become resident (another process holding CUs),
 * the launch gives up and leaves output unwritten.
 */
int moe_forward_monolithic(const uint16_t* x, const float* logits, int T, int H, int top_k,
                           int scoring, int renormalize, int apply_router_weight_on_input,
                           const moe_weights* weights /* host */, int activation,
                           const uint16_t* residual, const uint16_t* gamma, float eps,
                           int out_quant, void* output, float* output_scale,
                           uint16_t* residual_out, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);
/* (host) workspace moe_forward_monolithic needs for these sizes. */
size_t moe_forward_monolithic_workspace_bytes(int T, int H, int top_k,
                                              const moe_weights* weights, int activation);

/*
 * moe_forward_noalloc -- moe_forward for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same layer, arguments and results as moe_forward,
 * with its workspace taken from a scratch array of MOE_NOALLOC_SCRATCH_BYTES
 * (64 MiB) compiled into the library, one per GPU, held from the first call
 * on that GPU until the process ends.  The call allocates nothing.  Sizes
 * whose moe_forward_workspace_bytes exceeds the scratch (beyond decode
 * sizes: e.g. T = 128 fits every layer shape of the workloads here) return
 * MOE_ERR_WORKSPACE before anything is enqueued.  Every call on one GPU
 * shares that GPU's scratch, so calls that overlap on one GPU (two streams,
 * or two host threads) race and must be serialised by the caller; calls in
 * one stream's order are fine.  The first call on a GPU looks up the
 * scratch's address there (MOE_ERR_HIP if that fails).
 */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int moe_forward_noalloc(const uint16_t* x, const float* logits, int T, int H, int top_k,
                        int scoring, int renormalize, int apply_router_weight_on_input,
                        const moe_weights* weights /* host */, int activation, int block_m,
                        const uint16_t* residual, const uint16_t* gamma, float eps, int out_quant,
                        void* output, float* output_scale, uint16_t* residual_out,
                        hipStream_t stream);

/* (host) the block_m moe_forward uses when given 0, by the average rows per
 * expert a = T*top_k/E: 16 (a <= 16), 32 (a <= 32), then bf16: 64 (a <= 64)
 * else 256; fp8: 64 (a <= 96), 128 (a <= 192) else 256.  quant is a moe_quant. */
int moe_pick_block_m(int T, int top_k, int num_experts, int quant);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
