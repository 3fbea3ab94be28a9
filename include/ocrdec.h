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
 * (rows of one verify call). */
typedef struct {
  int n_layers, d_model, n_heads, head_dim, n_experts, n_shared, top_k, d_expert, d_draft_ffn, vocab;
  float rope_theta, norm_eps;
  int dtype;                                   /* OCRDEC_F32 | OCRDEC_BF16 */
  int max_batch, max_k, max_positions;
  int path;                                    /* OCRDEC_PATH_* */
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

/* Prefill B sequences (host arrays slots_host, n_vision_host, n_prompt_host):
 * rows 0..Nv-1 are the vision rows vision[b] (device fp32 [B][nv_stride][d]),
 * rows Nv..Nv+Np-1 the embeddings of prompt[b] (device int32 [B][np_stride]).
 * Runs the verifier over the prefix (filling its KV cache), the draft block over
 * the same rows (filling the draft KV cache; draft row p takes the verifier
 * hidden of p-1), and writes the greedy token of the last prefix row -- output
 * token 0 -- to pending_out[b] (device int32 [B]).  After the call the slot's
 * committed-output count is 1.  OCRDEC_ECAPACITY if Nv+Np+max_k+1 > max_positions. */
int ocrdec_prefill(ocrdec_model* m, void* stream, int B, const int32_t* slots_host,
                   const float* vision, int nv_stride, const int32_t* n_vision_host,
                   const int32_t* prompt, int np_stride, const int32_t* n_prompt_host,
                   int32_t* pending_out);

/* FastMTP draft (the pages' "one shared dense block applied recursively for K
 * steps"): pass 1 recomputes the rows accepted at the last verify plus the
 * pending token from the verifier's hidden states (catch-up) and proposes d_1;
 * passes 2..K feed the block's own output back.  draft_out: device int32 [B][K]. */
int ocrdec_draft(ocrdec_model* m, void* stream, int B, const int32_t* slots, int K, int32_t* draft_out);

/* Verifier pass over rows [pending, d_1..d_K] of each sequence at positions
 * kv_len..kv_len+K through all layers; writes their keys/values to the cache and
 * the greedy token of every row to greedy_out (device int32 [B][K+1]).
 * logits_out (nullable, device fp32 [B][K+1][vocab]) receives the final logits.
 * K = 0 is plain autoregressive decoding (draft ignored, may be NULL). */
int ocrdec_verify(ocrdec_model* m, void* stream, int B, const int32_t* slots, int K,
                  const int32_t* draft, int32_t* greedy_out, float* logits_out);

/* Greedy longest-prefix acceptance (blog, "Model and training") with KV
 * rollback: n = the longest j <= K with d_i == g_{i-1} for all i <= j; commits
 * d_1..d_n and the bonus token g_n; the verifier cache keeps positions up to the
 * last committed token, rejected positions are dropped by a length update (no
 * data moves).  Writes n to n_accepted_out[b] (device int32 [B]) and appends the
 * n+1 tokens to out_tokens[b][out_len..] (device int32 [B][out_cap], tokens at
 * index >= out_cap are dropped); out_len (device int32 [B], nullable) receives
 * the new committed count (including output token 0 from the prefill). */
int ocrdec_accept_rollback(ocrdec_model* m, void* stream, int B, const int32_t* slots, int K,
                           const int32_t* draft, const int32_t* greedy, int32_t* n_accepted_out,
                           int32_t* out_tokens, int32_t* out_len, int out_cap);

/* Benchmark harness (not part of the method): overwrite draft[b][j-1] with the
 * token a lossless run commits at that place, trace[b][out_len-1+j] (device
 * int32 [B][trace_stride], ids past trace_len read as 0), replaced -- when the
 * top 53 bits of H = SplitMix64-chain(seed, b_index, step, j) fall below
 * `threshold` -- by (true + 1 + (H mod 2^32) mod (vocab-1)) mod vocab, which is
 * never the true token.  b_index is the sequence's slot. */
int ocrdec_controlled_drafts(ocrdec_model* m, void* stream, int B, const int32_t* slots, int K,
                             const int32_t* trace, int trace_stride, int trace_len,
                             uint64_t seed, uint64_t threshold, int32_t* draft_inout);

/* Controlled-draft parameters for ocrdec_decode_steps (see
 * ocrdec_controlled_drafts). */
typedef struct {
  const int32_t* trace;
  int trace_stride, trace_len;
  uint64_t seed, threshold;
} ocrdec_controlled_cfg;

/* n_steps speculative steps of the B sequences: per step ocrdec_draft (K >= 1),
 * the controlled override when ctrl is non-null (K >= 1), ocrdec_verify and
 * ocrdec_accept_rollback, with the same results as issuing those calls one by
 * one (K = 0: plain autoregressive steps, draft may be NULL).  Each step is recorded once per call shape as a HIP graph (on a
 * library-private capture stream) and replayed on `stream`; the graphs are
 * cached in the handle.  draft (device int32 [B][K]) and greedy ([B][K+1]) are
 * caller scratch; n_accepted / out_tokens / out_len as in
 * ocrdec_accept_rollback (values of the last step). */
int ocrdec_decode_steps(ocrdec_model* m, void* stream, int B, const int32_t* slots, int K, int n_steps,
                        const ocrdec_controlled_cfg* ctrl, int32_t* draft, int32_t* greedy,
                        int32_t* n_accepted_out, int32_t* out_tokens, int32_t* out_len, int out_cap);

/* Position bookkeeping: between synchronisations the host assumes that every
 * step commits K + 1 tokens (an upper bound that sizes the attention grids and
 * the OCRDEC_ECAPACITY checks).  This call synchronises `stream` and resets the
 * bound of every slot to its true cache length, so long generations are not
 * refused early.  Returns OCRDEC_EHIP if the read fails. */
int ocrdec_sync_positions(ocrdec_model* m, void* stream);

/* Long-context benchmark harness (not part of the method).
 * ocrdec_load_sequence: fill slot `slot` with a caller-made verifier cache of
 * n_pos positions -- kv: device, model dtype, [n_layers][K|V][head][n_pos][128]
 * (keys already rotated) -- and make pending_token the token at position
 * n_pos, as a prefill would (the draft cache is not filled).  Errors:
 * OCRDEC_EINVAL for a bad slot / token / null pointer, OCRDEC_ECAPACITY if
 * n_pos + max_k + 1 > max_positions.
 * ocrdec_set_router_logits: later verify calls take each layer's router logits
 * from logits (device fp32 [n_layers][rows][64], rows = B*(K+1) of the call;
 * the caller keeps it alive) instead of the router weights; NULL restores the
 * router. */
int ocrdec_load_sequence(ocrdec_model* m, void* stream, int slot, int n_pos, int pending_token, const void* kv);
int ocrdec_set_router_logits(ocrdec_model* m, const float* logits);

/* Parity taps (nullable device pointers, used by later verify/prefill calls):
 * route_idx int32 [n_layers][rows][8] receives each layer's routing (6 routed
 * experts by decreasing score, then the shared experts 64, 65); hidden fp32
 * [rows][d] receives the final pre-norm hidden rows of the last verify. */
int ocrdec_set_taps(ocrdec_model* m, int32_t* route_idx, float* hidden);

/* Kernel timing of the grouped expert GEMV (gate/up and down launches):
 * enable != 0 records HIP events around each launch from now on (clears the
 * totals).  ocrdec_expert_stats synchronises those events and returns the
 * total milliseconds and launch count of each of the two kernels, and the
 * number of (layer, expert) weight sets they streamed since timing was enabled,
 * counted on the device. */
int ocrdec_expert_timing(ocrdec_model* m, int enable);  /* synchronises the device */
int ocrdec_expert_stats(ocrdec_model* m, double* ms_gate_up, long long* n_gate_up, double* ms_down,
                        long long* n_down, long long* expert_sets);

/* Benchmark harness: replay the grouped expert gate/up GEMV n_rounds times over
 * the weights of every layer in turn (n_rounds * n_layers back-to-back launches
 * on `stream`), with the routing of the last verify call, so that a pair of
 * events around the call times the kernel alone.  If expert_sets_per_launch
 * (host, nullable) is given, the call first synchronises the stream and stores
 * that routing's active-expert count there. */
int ocrdec_replay_expert_gate_up(ocrdec_model* m, void* stream, int n_rounds, int* expert_sets_per_launch);

/* Calibration (not part of the method): n_launches back-to-back launches on
 * `stream` of a kernel that only reads `bytes` bytes (16-byte loads, 4,096
 * workgroups) and writes nothing but, in practice never, one word to sink
 * (device, >= 4 bytes).  Launch i reads region i mod n_regions of the device
 * buffer buf, which holds n_regions consecutive regions of `bytes` bytes: with
 * as many regions as a replay has layers, the reads do not hit the GPU's
 * last-level cache any more than the replayed kernel's do.  A pair of events
 * around the call gives the rate a plain streaming kernel reaches at that size,
 * the practical ceiling for the bandwidth-bound kernels above.  OCRDEC_EINVAL
 * if buf or sink is null, bytes < 16 or not a multiple of 256, n_regions < 1 or
 * n_launches < 0. */
int ocrdec_read_probe(void* stream, const void* buf, size_t bytes, int n_regions, int n_launches, uint32_t* sink);

const char* ocrdec_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* OCRDEC_H */
