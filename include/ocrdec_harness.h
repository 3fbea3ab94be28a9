/*
 * ocrdec harness calls -- not part of the decode method.  These serve the
 * benchmark (controlled acceptance, kernel timing and replays, a plain-read
 * calibration, a loaded long-context cache, given router logits) and the
 * parity tests (taps that copy out routing decisions, hidden rows and the
 * history of the decode steps).  Conventions as in ocrdec.h.
 */
#ifndef OCRDEC_HARNESS_H
#define OCRDEC_HARNESS_H

#include "ocrdec.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Controlled acceptance: overwrite draft[b][j-1] with the token a lossless run
 * commits at that place, trace[b][out_len-1+j] (device int32 [B][trace_stride],
 * ids past trace_len read as 0), replaced -- when the top 53 bits of
 * H = SplitMix64-chain(seed, slot, step, j) fall below `threshold` -- by
 * (true + 1 + (H mod 2^32) mod (vocab-1)) mod vocab, which is never the true
 * token.  step is the slot's count of accepted steps. */
int ocrdec_controlled_drafts(ocrdec_model* m, void* stream, int B, const int32_t* slots, int K,
                             const int32_t* trace, int trace_stride, int trace_len,
                             uint64_t seed, uint64_t threshold, int32_t* draft_inout);

/* The same override inside ocrdec_decode_steps. */
struct ocrdec_controlled_cfg {
  const int32_t* trace;
  int trace_stride, trace_len;
  uint64_t seed, threshold;
};

/* Long-context benchmark.  ocrdec_load_sequence: fill slot `slot` with a
 * caller-made verifier cache of n_pos positions -- kv: device, model dtype,
 * [n_layers][K|V][head][n_pos][128] (keys already rotated) -- and make
 * pending_token the token at position n_pos, as a prefill would (the draft
 * cache is not filled).  Errors: OCRDEC_EINVAL for a bad slot / token / null
 * pointer, OCRDEC_ECAPACITY if n_pos + max_k + 1 > max_positions.
 * ocrdec_set_router_logits: later verify calls take each layer's router
 * logits from logits (device fp32 [n_layers][rows][64], rows = B*(K+1) of the
 * call; the caller keeps it alive) instead of the router weights; NULL
 * restores the router. */
int ocrdec_load_sequence(ocrdec_model* m, void* stream, int slot, int n_pos, int pending_token, const void* kv);
int ocrdec_set_router_logits(ocrdec_model* m, const float* logits);

/* The MoE half of each vector-path verifier layer (at most 8 rows per call)
 * runs as the router-logits launch and one persistent launch for routing,
 * expert gate/up, down and combine (fused != 0), or as the five launches
 * router logits, routing, gate/up, down, combine (fused = 0, the default: the
 * faster on MI355X); both give the same bits.  ocrdec_moe_grid returns the persistent launch's
 * workgroup count on this GPU (0: it is not used). */
int ocrdec_set_moe_launches(ocrdec_model* m, int fused);
int ocrdec_moe_grid(ocrdec_model* m);

/* Parity taps: nullable device buffers that later calls fill.
 *   route_idx  int32 [n_layers][rows][8]: each verify call's routing (6 routed
 *              experts by decreasing score, then the shared experts 64, 65);
 *   hidden     fp32 [rows][d]: the final pre-norm hidden rows of the last verify;
 *   route_pos  int32 [n_layers][route_pos_cap][8]: the routing of every row of
 *              state slot route_pos_slot -- prefill and verify rows -- by
 *              position (< route_pos_cap); after a decode, the rows of the
 *              committed positions, since a committed row is the last row
 *              computed at its position;
 *   accepted   int32 [max_batch][step_cap]: n of each accepted step, by slot
 *              and the slot's step number (< step_cap);
 *   drafts     int32 [max_batch][step_cap][8]: the K proposals the draft
 *              block made at each step (before any controlled override).
 * Decode-step graphs are recorded per tap set.  NULL clears every tap. */
typedef struct {
  int32_t* route_idx;
  float* hidden;
  int32_t* route_pos;
  int route_pos_slot, route_pos_cap;
  int32_t* accepted;
  int32_t* drafts;
  int step_cap;
} ocrdec_taps;
int ocrdec_set_taps(ocrdec_model* m, const ocrdec_taps* taps);

/* Kernel timing of the grouped expert GEMV (gate/up and down launches):
 * enable != 0 records HIP events around each launch from now on (clears the
 * totals).  ocrdec_expert_stats synchronises those events and returns the
 * total milliseconds and launch count of each of the two kernels, and the
 * number of (layer, expert) weight sets they streamed since timing was enabled,
 * counted on the device. */
int ocrdec_expert_timing(ocrdec_model* m, int enable);  /* synchronises the device */
int ocrdec_expert_stats(ocrdec_model* m, double* ms_gate_up, long long* n_gate_up, double* ms_down,
                        long long* n_down, long long* expert_sets);

/* Replay the dominant expert kernel n_rounds times over the weights of every
 * layer in turn (n_rounds * n_layers back-to-back launches on `stream`), with
 * the routing of the last layer of the last verify call, so that a pair of
 * events around the call times the kernel alone.  The kernel is the grouped
 * expert gate/up GEMV, or -- where the persistent MoE launch is in use -- that
 * launch, which then routes from the last router logits and writes its output
 * rows to scratch (the residual rows are left as they are).  If
 * expert_sets_per_launch (host, nullable) is given, the call first
 * synchronises the stream and stores that routing's active-expert count
 * there. */
int ocrdec_replay_expert_gate_up(ocrdec_model* m, void* stream, int n_rounds, int* expert_sets_per_launch);

/* Calibration: n_launches back-to-back launches on `stream` of a kernel that
 * only reads `bytes` bytes (16-byte loads, 4,096 workgroups) and writes
 * nothing but, in practice never, one word to sink (device, >= 4 bytes).
 * Launch i reads region i mod n_regions of the device buffer buf, which holds
 * n_regions consecutive regions of `bytes` bytes: with as many regions as a
 * replay has layers, the reads do not hit the GPU's last-level cache any more
 * than the replayed kernel's do.  A pair of events around the call gives the
 * rate a plain streaming kernel reaches at that size, the practical ceiling
 * for the bandwidth-bound kernels.  OCRDEC_EINVAL if buf or sink is null,
 * bytes < 16 or not a multiple of 256, n_regions < 1 or n_launches < 0. */
int ocrdec_read_probe(void* stream, const void* buf, size_t bytes, int n_regions, int n_launches, uint32_t* sink);

#ifdef __cplusplus
}
#endif
#endif /* OCRDEC_HARNESS_H */
