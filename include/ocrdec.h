/*
 * ocrdec -- C ABI of the FastMTP speculative decode path of the jina-ocr-v1
 * decoder (DeepSeek-3B-MoE: 12 layers, d = 1280, 64 routed + 2 shared experts,
 * top-6, vocabulary 129,280, RoPE theta 1e6) on one AMD Instinct MI355X (gfx950).
 *
 * The four decode calls follow the method the jina-ocr-v1 blog describes in
 * "Model and training": one shared dense draft block proposes K tokens by
 * recursion, the verifier checks the K+1 rows greedily in one pass and keeps
 * the longest agreeing prefix plus its own next token, so the committed
 * sequence is exactly the verifier's greedy sequence.
 *
 * Conventions (all calls):
 *   - Every device buffer (weights, state, workspace, inputs, outputs) is
 *     allocated and owned by the caller and must outlive the model handle.
 *     The library never allocates device memory.
 *   - `stream` is a hipStream_t passed as void*.  Calls only enqueue work on
 *     it; outputs are valid once the stream has been synchronised.  No call
 *     synchronises the host.
 *   - Return 0 on success, or a negative OCRDEC_E* code; then nothing was
 *     enqueued and the state is unchanged.  ocrdec_last_error() returns a
 *     thread-local message describing the last failure.
 *   - `slots` (device int32 [B], or NULL for 0..B-1) maps the B sequences of a
 *     call to state slots < max_batch; slots in one call must be distinct.
 *   - Token ids read from device buffers are clamped to [0, vocab).
 *   - Calls on one model handle must be issued in order on one stream; they
 *     share the workspace.
 */
#ifndef OCRDEC_H
#define OCRDEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OCRDEC_OK 0
#define OCRDEC_EINVAL (-1)     /* null / misaligned pointer, bad B or K, unsupported shape */
#define OCRDEC_ECAPACITY (-2)  /* B > max_batch, K > max_k, positions past max_positions */
#define OCRDEC_EHIP (-3)       /* a HIP runtime call failed */

#define OCRDEC_F32 0           /* fp32 weights, fp32 KV cache */
#define OCRDEC_BF16 1          /* bf16 weights and embedding, bf16 KV cache */

/* Arithmetic path of the expert SwiGLU and the LM head, fixed per handle so
 * that a row's result never depends on how many rows share a call:
 *   OCRDEC_PATH_AUTO    matrix cores for bf16 handles with
 *                       max_batch * (max_k + 1) > 8 and vocab >= 64, else vector;
 *   OCRDEC_PATH_VECTOR  wavefront GEMV, fp32 activations (every dtype);
 *   OCRDEC_PATH_MATRIX  MFMA tiles with activations rounded to bf16
 *                       (bf16 handles with vocab >= 64 only, else OCRDEC_EINVAL). */
#define OCRDEC_PATH_AUTO 0
#define OCRDEC_PATH_VECTOR 1
#define OCRDEC_PATH_MATRIX 2

/* Model shape and capacity (plain data).  The kernels are built for the
 * decoder shape of the pages' spec table: d_model 1280, 10 heads x 128,
 * 64 routed + 2 shared experts of width 896, top-6, draft FFN 3584; other
 * values of those fields are rejected with OCRDEC_EINVAL.  n_layers >= 1,
 * vocab >= 2, max_positions <= 32768 (the pages' position limit),
 * max_batch in [1, 1024], max_k in [0, 7], max_batch * (max_k + 1) <= 1024
 * (rows of one verify call).
 *
 * KV cache: paged.  A page holds 64 consecutive positions of one sequence
 * (keys and values of every head, every verifier layer, and the draft
 * block's); a slot takes pages as its sequence grows and gives them back when
 * it is released or prefilled anew, so concurrent sequences share the pool by
 * their actual lengths (the French model card's concurrency-32 serving).
 * kv_pages = the pool's size in pages; 0 = max_batch * ceil(max_positions /
 * 64), enough for every slot at max_positions (never exhausted).  A call
 * whose sequences would need more pages than are free returns
 * OCRDEC_ECAPACITY with nothing enqueued. */
typedef struct {
  int n_layers, d_model, n_heads, head_dim, n_experts, n_shared, top_k, d_expert, d_draft_ffn, vocab;
  float rope_theta, norm_eps;
  int dtype;                                   /* OCRDEC_F32 | OCRDEC_BF16 */
  int max_batch, max_k, max_positions;
  int path;                                    /* OCRDEC_PATH_* */
  int kv_pages;                                /* KV page pool size; 0: the full size */
} ocrdec_config;

typedef struct ocrdec_model ocrdec_model;

/* Bytes of the per-sequence decode state (verifier and draft KV caches,
 * lengths, pending tokens, hidden-state feedback rows) and of the scratch
 * workspace.  Both buffers must be 256-byte aligned.  The state needs no
 * initialisation; ocrdec_prefill initialises a slot. */
size_t ocrdec_state_bytes(const ocrdec_config* cfg);
size_t ocrdec_workspace_bytes(const ocrdec_config* cfg);

/* Number of weight tensors and their canonical order (row-major, y = W x, W is
 * [out, in]); matrices in the model dtype, RMSNorm gains always fp32:
 *   0 embed [V,d]   1 lm_head [V,d]   2 final_norm [d]
 *   per layer l, base 3 + 8 l:
 *     attn_norm [d], wqkv [3*1280, d] (q, k, v rows, head-major), wo [d, 1280],
 *     ffn_norm [d], router [64, d], w_gate [66, 896, d], w_up [66, 896, d],
 *     w_down [66, d, 896]   (experts 0..63 routed, 64..65 shared)
 *   draft, base 3 + 8 L: norm_h [d], norm_e [d], fuse [d, 2d], attn_norm [d],
 *     wqkv [3*1280, d], wo [d, 1280], ffn_norm [d], w_gate [3584, d],
 *     w_up [3584, d], w_down [d, 3584], out_norm [d]
 * Every pointer must be 16-byte aligned. */
int ocrdec_num_weights(const ocrdec_config* cfg);

/* Create a handle over caller-owned device memory.  Zeroes the workspace's
 * counters on `stream` (pass the stream later calls use).  */
int ocrdec_create(const ocrdec_config* cfg, const void* const* weight_ptrs, int n_weights,
                  void* state, void* workspace, void* stream, ocrdec_model** out);
int ocrdec_destroy(ocrdec_model* m);

/* Prefill B sequences (host arrays slots_host, n_vision_host, n_prompt_host).
 * The blog's "Model and training" section (architecture figure caption and
 * spec table) puts a page's visual tokens -- 256 for the global 1024x1024
 * view plus 100 per local tile, at most 1,156 -- in front of the decoder; here
 * they are the rows of the prefix.  Rows 0..Nv-1 are the vision rows
 * vision[b] (device fp32 [B][nv_stride][d]), rows Nv..Nv+Np-1 the embeddings
 * of prompt[b] (device int32 [B][np_stride]), at positions 0..Nv+Np-1.
 * Runs the verifier over the prefix (filling its KV cache), the draft block over
 * the same rows (filling the draft KV cache; draft row p takes the verifier
 * hidden of p-1), and writes the greedy token of the last prefix row -- output
 * token 0 -- to pending_out[b] (device int32 [B]).  After the call the slot's
 * committed-output count is 1.  slots_host may be NULL (slots 0..B-1); slots
 * must be distinct and < max_batch.  Errors: OCRDEC_EINVAL for a null or
 * inconsistent argument or an empty prefix, OCRDEC_ECAPACITY if
 * Nv+Np+max_k+1 > max_positions (nothing is enqueued). */
int ocrdec_prefill(ocrdec_model* m, void* stream, int B, const int32_t* slots_host,
                   const float* vision, int nv_stride, const int32_t* n_vision_host,
                   const int32_t* prompt, int np_stride, const int32_t* n_prompt_host,
                   int32_t* pending_out);

/* FastMTP draft.  The blog's "Model and training" section (and the spec
 * table's MTP head row) describes one shared dense block applied recursively
 * for K steps, so draft parameters do not grow with depth; its "Getting
 * started" section says the head was trained with recursive hidden-state
 * feedback (an EAGLE-style proposer).  Pass 1 recomputes the rows accepted at
 * the last verify plus the pending token from the verifier's hidden states
 * (catch-up) and proposes d_1; passes 2..K feed the block's own output back.
 * draft_out: device int32 [B][K], written in full.  1 <= K <= max_k.
 * Errors: OCRDEC_EINVAL (null draft_out, K < 1), OCRDEC_ECAPACITY (B or K
 * above the handle's capacity, or -- without a slot map -- positions past
 * max_positions). */
int ocrdec_draft(ocrdec_model* m, void* stream, int B, const int32_t* slots, int K, int32_t* draft_out);

/* Greedy verification, as the blog's "Model and training" section describes
 * it: the verifier checks every proposal greedily in one pass.  Rows
 * [pending, d_1..d_K] of each sequence at positions kv_len..kv_len+K go
 * through all layers; their keys/values are written to the cache and the
 * greedy token (argmax, lowest id on ties) of every row to greedy_out (device
 * int32 [B][K+1]).  logits_out (nullable, device fp32 [B][K+1][vocab])
 * receives the final logits.  K = 0 is plain autoregressive decoding (draft
 * ignored, may be NULL).  A sequence whose rows would pass max_positions is
 * not computed: its overflow flag is set (reported by ocrdec_sync_positions)
 * and the accept that follows leaves it unchanged.  Errors: OCRDEC_EINVAL
 * (null greedy_out, null draft with K > 0), OCRDEC_ECAPACITY (B or K above
 * capacity; without a slot map, positions past max_positions). */
int ocrdec_verify(ocrdec_model* m, void* stream, int B, const int32_t* slots, int K,
                  const int32_t* draft, int32_t* greedy_out, float* logits_out);

/* Greedy longest-prefix acceptance (blog, "Model and training": the longest
 * prefix on which draft and verifier agree is kept, so the committed sequence
 * is the verifier's greedy sequence; the "Speculative decoding on L4" table
 * caption counts the verifier's bonus token in tau) with KV rollback: n = the
 * longest j <= K with d_i == g_{i-1} for all i <= j; commits d_1..d_n and the
 * bonus token g_n; the verifier cache keeps positions up to the last committed
 * token, rejected positions are dropped by a length update (no data moves).
 * Writes n to n_accepted_out[b] (device int32 [B]; -1 for a sequence the
 * verify did not compute because of max_positions, which is left unchanged)
 * and appends the n+1 tokens to out_tokens[b][out_len..] (device int32
 * [B][out_cap], tokens at index >= out_cap are dropped); out_len (device int32
 * [B], nullable) receives the new committed count (including output token 0
 * from the prefill).  It must directly follow the ocrdec_verify whose rows it
 * accepts, with the same B, K and slots pointer (else OCRDEC_EINVAL, nothing
 * enqueued); each verify is accepted at most once. */
int ocrdec_accept_rollback(ocrdec_model* m, void* stream, int B, const int32_t* slots, int K,
                           const int32_t* draft, const int32_t* greedy, int32_t* n_accepted_out,
                           int32_t* out_tokens, int32_t* out_len, int out_cap);

/* Controlled-draft parameters of ocrdec_decode_steps (benchmark harness;
 * defined in ocrdec_harness.h). */
typedef struct ocrdec_controlled_cfg ocrdec_controlled_cfg;

/* Whole speculative steps replayed as HIP graphs (the pages' CUDA-graph mode:
 * announcement and blog L4 tables, "Graph" rows).  n_steps steps of the B
 * sequences: per step ocrdec_draft (K >= 1), the controlled override when ctrl
 * is non-null (K >= 1; harness), ocrdec_verify and ocrdec_accept_rollback,
 * with the same results as issuing those calls one by one (K = 0: plain
 * autoregressive steps, draft may be NULL).  Each step is recorded once per
 * call shape as a HIP graph (on a library-private capture stream) and
 * replayed on `stream`; the graphs are cached in the handle.  draft (device
 * int32 [B][K]) and greedy ([B][K+1]) are caller scratch; n_accepted /
 * out_tokens / out_len as in ocrdec_accept_rollback (values of the last
 * step). */
int ocrdec_decode_steps(ocrdec_model* m, void* stream, int B, const int32_t* slots, int K, int n_steps,
                        const ocrdec_controlled_cfg* ctrl, int32_t* draft, int32_t* greedy,
                        int32_t* n_accepted_out, int32_t* out_tokens, int32_t* out_len, int out_cap);

/* For callers that cannot allocate memory -- code under HIP graph capture,
 * serving loops that forbid allocation, harnesses that refuse it.  The same
 * steps as ocrdec_decode_steps without a controlled override (draft, verify,
 * accept per step, with the same results bit for bit), issued as individual
 * launches on `stream` (no graphs are recorded or replayed), and with the
 * per-call scratch (activations, attention partials, routing tables, LM-head
 * partials) in a 32 MiB device array that the library holds on each GPU it
 * runs on until the process ends, instead of the handle's workspace.  The
 * call allocates nothing and needs its scratch to fit: OCRDEC_ECAPACITY,
 * nothing enqueued, if B*(max_k+1) rows at the handle's max_positions need
 * more than 32 MiB (4 rows need about 1.3 MiB at 2,048 positions, 3.3 MiB at
 * 32,768; 1,024 rows do not fit).  Every call on one GPU -- from any handle --
 * shares that array and leaves its contents behind: calls that overlap on one
 * GPU (other streams, other threads, other handles) race and must not be
 * issued.  The handle's workspace is untouched.  Under capture the call's host
 * work -- the KV pages it takes, the attention grids sized for the positions
 * it can reach, the position bookkeeping -- happens once, at capture: record
 * the call anew for each use rather than replaying one recording. */
int ocrdec_decode_steps_noalloc(ocrdec_model* m, void* stream, int B, const int32_t* slots, int K, int n_steps,
                                int32_t* draft, int32_t* greedy, int32_t* n_accepted_out,
                                int32_t* out_tokens, int32_t* out_len, int out_cap);

/* Position bookkeeping: between synchronisations the host assumes that every
 * step commits K + 1 tokens (an upper bound that sizes the attention grids and
 * the OCRDEC_ECAPACITY checks).  This call synchronises `stream` and resets the
 * bound of every slot to its true cache length, so long generations are not
 * refused early.  It returns OCRDEC_ECAPACITY (naming the slots) if, since the
 * last call, a step of some sequence was not taken because it would have
 * passed max_positions (the flags are then cleared; the bounds are still
 * updated), and OCRDEC_EHIP if the read fails. */
int ocrdec_sync_positions(ocrdec_model* m, void* stream);

/* KV pages.  ocrdec_release_slot returns the pages of `slot` to the pool (the
 * table update is enqueued on `stream`; issue every call of a handle on one
 * stream, so that earlier work on the pages finishes first); the slot must be
 * prefilled again before its next decode call.  Decode calls give pages to
 * the slots they touch -- slots 0..B-1, or, with a device slot map, every slot
 * that holds pages -- for their positions up to the host's bound (see
 * ocrdec_sync_positions) plus what the call adds, so release finished
 * sequences.  A slot without pages writes no cache rows.  ocrdec_kv_pages
 * reports the pool's size and its free pages (host pointers, nullable). */
int ocrdec_release_slot(ocrdec_model* m, void* stream, int slot);
int ocrdec_kv_pages(ocrdec_model* m, int* total, int* free_pages);

const char* ocrdec_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* OCRDEC_H */
