// Host-side launchers of the ocrdec kernels (one per kernel family).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "common.h"

namespace ocr {

enum Epi { EPI_STORE = 0, EPI_ADD = 1, EPI_SWIGLU = 2 };

// x: [M][D] residual rows; gain: RMSNorm gain (never null here).
// Writes q (RoPE'd, fp32 [M][QD]) and, for valid rows, k / v into the paged
// cache kv (the page of each row's position must exist).
template <typename T>
void launch_qkv_rope(hipStream_t s, const float* x, const float* gain, float eps, const T* wqkv, int M,
                     RowPlan plan, float* q, KvView<T> kv, const float2* rope);
// tab[pos][i] = (cos, sin)(pos * theta^(-2i/128)), i < 64, for pos < max_pos.
void launch_rope_table(hipStream_t s, int max_pos, float theta, float2* tab);

// out[m][n] (op)= sum_k W[n][k] * a[m][k] for n < N; a optionally RMSNorm'ed
// (gain != null).  EPI_SWIGLU: out[m][j] = silu(W0[j].a) * (W1[j].a), j < N.
template <typename T>
void launch_gemv(hipStream_t s, int K, Epi epi, const float* a, long lda, const float* gain, float eps,
                 const T* W0, const T* W1, int N, int M, float* out, long ldo);

// LM head fused with argmax (two launches: per-block bests, then the final
// reduction).  Output row m reads activation row (last_valid ? m*Q + cnt[m]-1
// : m) of x, RMSNorms it with gain, forms the vocab logits (optionally stored to
// logits[m][V]) and writes the argmax (lowest id on ties) to tok[m * tok_stride].
template <typename T>
void launch_lmhead(hipStream_t s, const float* x, const int* cnt, int Q, bool last_valid, const float* gain,
                   float eps, const T* W, int V, int M, float* part_val, int* part_idx, float* logits, int* tok,
                   int tok_stride);
int lmhead_blocks(int V);
// Stage 2 of the argmax: tok[m * tok_stride] = best of part[m][0 .. nblk).
void launch_argmax_final(hipStream_t s, const float* part_val, const int* part_idx, int nblk, int M, int* tok,
                         int tok_stride);

// Split-KV decode attention (partials per chunk) and the merge of the chunks
// into out, in two launches.
template <typename T>
void launch_attention(hipStream_t s, const float* q, KvView<T> kv, RowPlan plan, int B, int n_chunks,
                      int tiles_per_chunk, float* part, float* out);

// Prefill attention: n entries of plan.Q = PREFILL_CHUNK rows; row i of entry
// b (i < cnt[b]) is the query at position base[b] + i of slot slot[b] and sees
// keys 0 .. base[b] + i of the cache, all of them written before the call.
// out[b * Q + i] = the head outputs (rows past cnt: zero).  bf16 caches on the
// matrix cores, fp32 caches on the vector units.
// bf16: the entry's key tiles are split into at most PF_SPLITS runs of equal
// length (the last one shorter), one block each, whose partials (o, m, l per
// row, [entry][head][split][row][130] in part) are merged in split order; the
// split depends only on the entry's own last position, so a row's result
// never depends on the other entries of the pass.
constexpr int PF_SPLITS = 4;
// Split s of an entry with n_tiles key tiles: tiles [t0, t1); false if empty.
__host__ __device__ inline bool prefill_split(int n_tiles, int s, int& t0, int& t1) {
  const int per = (n_tiles + PF_SPLITS - 1) / PF_SPLITS;
  t0 = s * per;
  t1 = t0 + per < n_tiles ? t0 + per : n_tiles;
  return per > 0 && t0 < t1;
}
template <typename T>
void launch_attention_prefill(hipStream_t s, const float* q, KvView<T> kv, RowPlan plan, int n, float* part,
                              float* out);

struct MoeBufs {
  float* bnorm;   // [M][D] normalised rows
  int* ridx;      // [M][8]
  float* rgate;   // [M][8]
  int* perm;      // [8M] pair id by sorted position
  int* inv;       // [8M] sorted position of pair id
  int* off;       // [NX + 1]
  int* act;       // [NX] active experts in increasing id
  int* n_act;     // [1]
  int4* slot_info;  // [NX] (expert, first pair, end pair, n_act); expert -1 past n_act
  int4* items;    // [expert_item_cap(M)] matrix-core work items: (expert, first pair, end pair, 0),
                  // at most ITEM_PAIRS pairs each, experts in slot order; expert -1 past the last
  long long* stats;  // [0] += active experts per layer
  float* rlogit;  // [M][64] router logits
  float* hx;      // [8M][DI]
  float* y;       // [8M][D]
};

// Work item of row y of an expert kernel's grid (M rows in the call): rows 0
// and 1 are the shared experts, always active, with pairs (TOPK + y) M ..
// (TOPK + y + 1) M - 1 (the sort puts them after the 6M routed pairs; .w = the
// mask of all rows), so their weight loads wait for no routing read; rows
// y >= 2 take routed slot y - 2 of the routing table (expert -1 past the routed
// ones).  The grid is expert_slot_cap(M) rows.
__device__ __forceinline__ int4 expert_work(const MoeBufs& mb, int y, int M) {
  if (y < NSH) return make_int4(NE + y, (TOPK + y) * M, (TOPK + y + 1) * M, M < 31 ? (1 << M) - 1 : -1);
  int4 info = mb.slot_info[y - NSH];
  if (info.x >= NE) info.x = -1;
  return info;
}

// Routing taps of one layer (parity harness): call (nullable) receives the
// routing of the call's rows, [M][8]; pos (nullable) receives, for the rows of
// state slot pos_slot only, the routing by position, [pos_cap][8] (valid rows
// at positions < pos_cap), so that a whole page's routing -- prefix and every
// committed decode row, which is always the last row computed at its position
// -- can be read after a run.
struct RouteTap {
  int* call;
  int* pos;
  int pos_slot, pos_cap;
  RowPlan plan;
};

// Router logits (rlogit) and the routing tables; logit_override (nullable,
// [M][64]) replaces the computed logits before the top-6.  With cnt (one zero
// word, left at zero) and M <= MRG, one launch does both.
template <typename T>
void launch_router(hipStream_t s, const float* x, const float* gain, float eps, const T* wr, int M,
                   const MoeBufs& mb, const RouteTap& tap, const float* logit_override, unsigned* cnt);
// The first half of launch_router: the normalised rows into mb.bnorm and the
// router logits (or a copy of logit_override) into mb.rlogit.
template <typename T>
void launch_router_logits(hipStream_t s, const float* x, const float* gain, float eps, const T* wr, int M,
                          const MoeBufs& mb, const float* logit_override);
// Grouped expert GEMVs after launch_router (M <= MRG: every pair of an
// expert at once; beyond, MRG pairs at a time) and the combine into the
// residual rows x.
template <typename T>
void launch_expert_gate_up(hipStream_t s, const T* wg, const T* wu, int M, const MoeBufs& mb);
template <typename T>
void launch_expert_down(hipStream_t s, const T* wd, int M, const MoeBufs& mb);
void launch_moe_combine(hipStream_t s, float* x, int M, const MoeBufs& mb);
int expert_slot_cap(int M);
// Matrix-core work items of prefill passes: at most ITEM_PAIRS pairs of one
// expert, so a shared expert's rows of a long prefix spread over many
// workgroups (their re-reads of the expert's weights come from the caches:
// prefill passes load weights with ordinary, not non-temporal, loads).  Upper
// bound on the items of a call: sum over experts of ceil(pairs / ITEM_PAIRS).
constexpr int ITEM_PAIRS = 64;
__host__ __device__ inline int expert_item_cap(int M) { return NX + (NSLOT * M + ITEM_PAIRS - 1) / ITEM_PAIRS; }
// M <= MRG rows: the down GEMV whose last workgroup per output column adds
// the combine to x -- the same bits as launch_expert_down + launch_moe_combine.
// cnt: DOWN_CNT_WORDS zero words (left at zero).
constexpr int DOWN_CNT_WORDS = (D / 16) * 32;
// The routing counter of launch_router sits after them, in the same buffer:
// every user of those words leaves them at zero, in stream order.
constexpr int ROUTE_CNT_WORD = DOWN_CNT_WORDS;
template <typename T>
void launch_expert_down_combine(hipStream_t s, const T* wd, int M, const MoeBufs& mb, float* x, unsigned* cnt);

// The rest of the MoE half of a layer for M <= 8 rows, after
// launch_router_logits, in one persistent launch of `grid` workgroups
// (routing, gate/up, down and the combine, with the arithmetic and results of
// the launches above): x_out = x_in + MoE(x_in).  sync: MOE_SYNC_WORDS zero
// words (left at zero by every launch), word MOE_SYNC_ERR set if a bounded
// wait timed out.  moe_fused_grid: the largest grid the GPU holds at once (0
// if unknown).
constexpr int MOE_SYNC_WORDS = 209 * 32;
constexpr int MOE_SYNC_ERR = 3;
template <typename T>
int moe_fused_grid(int n_cu);
template <typename T>
void launch_moe_experts(hipStream_t s, int grid, const float* x_in, float* x_out, const T* wg, const T* wu,
                        const T* wd, int M, const MoeBufs& mb, const RouteTap& tap, unsigned* sync);

// Matrix-core variants (bf16 weights): the same outputs as the vector
// launchers above, with the activations rounded to bf16 for the MFMA inputs.
// deep: prefill passes (weights three chunks ahead, activations two; more
// registers), else decode calls (one chunk ahead, more workgroups in flight).
void launch_expert_gate_up_mfma(hipStream_t s, const bf16* wg, const bf16* wu, int M, const MoeBufs& mb, bool deep);
void launch_expert_down_mfma(hipStream_t s, const bf16* wd, int M, const MoeBufs& mb, bool deep);
// Dense layers on the matrix cores (bf16 weights): the outputs of launch_gemv
// (K, epi) in {(1280, add / store / SwiGLU), (2560, store), (3584, add)}, N a
// multiple of 64, and of launch_qkv_rope, with the inputs as bf16 hi + lo parts.
// The gemv launchers return false, launching nothing, for any other (K, epi)
// (a gain only with K = 1280).  rscale: scratch of M floats (the rows' RMSNorm
// scales, computed by a launch of their own when a gain is given).
bool launch_gemv_mfma(hipStream_t s, int K, Epi epi, const float* a, long lda, const float* gain, float eps,
                      const bf16* W0, const bf16* W1, int N, int M, float* out, long ldo, float* rscale);
void launch_qkv_rope_mfma(hipStream_t s, const float* x, const float* gain, float eps, const bf16* wqkv, int M,
                          RowPlan plan, float* q, KvView<bf16> kv, const float2* rope, float* rscale);
// The same with k split over the four wavefronts of 16-row blocks (decode-sized
// calls: many blocks, no LDS staging).
bool launch_gemv_ks(hipStream_t s, int K, Epi epi, const float* a, long lda, const float* gain, float eps,
                    const bf16* W0, const bf16* W1, int N, int M, float* out, long ldo);
void launch_qkv_rope_ks(hipStream_t s, const float* x, const float* gain, float eps, const bf16* wqkv, int M,
                        RowPlan plan, float* q, KvView<bf16> kv, const float2* rope);
// LM head + argmax: xn ([M][D] scratch) receives the normalised rows; V >= 16.
void launch_lmhead_mfma(hipStream_t s, const float* x, const int* cnt, int Q, bool last_valid, const float* gain,
                        float eps, const bf16* W, int V, int M, float* xn, float* part_val, int* part_idx,
                        float* logits, int* tok, int tok_stride);

// ---- row plans, embeddings, acceptance --------------------------------------
struct StateView {
  int* kv_len; int* draft_len; int* pending; int* n_prev; int* out_len; int* step; int* prefix_len;
  int* ovf;        // [max_batch] set when a step would pass max_pos (the step is not taken)
  int* cu_tok;     // [max_batch][cu_stride]
  int cu_stride;
  float* hbuf;     // [max_batch][cu_stride][D]
  int n_slots;     // max_batch
  int max_pos;     // cache positions per slot
};

// Step-history taps of the decode calls (parity harness; nullable): acc[slot]
// [cap] receives n of the slot's step number t (t < cap) and drafts[slot][cap]
// [8] the K proposals of that step as the draft block made them.
struct StepTap {
  int* acc;
  int* drafts;
  int cap;
};

template <typename T>
void launch_plan_verify(hipStream_t s, int B, int K, const int* slots_in, StateView sv, const int* draft,
                        const T* embed, int V, int* plan_base, int* plan_cnt, int* plan_slot, float* x);
template <typename T>
void launch_plan_draft_catchup(hipStream_t s, int B, int Q, const int* slots_in, StateView sv,
                               const T* embed, int V, const float* g_h, const float* g_e, float eps,
                               int* plan_base, int* plan_cnt, int* plan_slot, float* cat);
// Draft pass input + fusion projection in one launch (vector path): step = 0
// is the catch-up pass (M = B Q rows), step = 1 pass j >= 2 (M = B rows,
// d_{j-1} from the LM-head partials part_val / part_idx of the previous pass,
// written to draft_out).  out = W_fuse . cat, [M][D]; out must not alias u_prev.
// Plain read of n16 16-byte words at buf (calibration; see k_read_probe).
void launch_read_probe(hipStream_t s, const void* buf, long n16, uint32_t* sink);
template <typename T>
void launch_draft_fuse(hipStream_t s, int step, int j, int Q, int Qprev, int K, const int* slots_in, StateView sv,
                       const T* embed, int V, const float* g_h, const float* g_e, float eps, const float* u_prev,
                       const float* part_val, const int* part_idx, int nblk, int* draft_out, int* plan_base,
                       int* plan_cnt, int* plan_slot, const T* w_fuse, int M, float* out);
template <typename T>
void launch_plan_draft_step(hipStream_t s, int B, int j, int Qprev, int K, StateView sv, const int* draft_out,
                            const T* embed, int V, const float* g_h, const float* g_e, float eps,
                            const float* u_prev, int* plan_base, int* plan_cnt, const int* plan_slot,
                            float* cat);
// One prefill pass of up to PREFILL_GROUP entries; entry j is the rows p0[j]
// .. p0[j] + cnt[j] - 1 (cnt <= PREFILL_CHUNK) of sequence seq[j] (slot
// slot[j], n_vision nvis[j], prefix length plen[j]), in activation rows
// j * PREFILL_CHUNK + i.  Entries of one sequence are consecutive and in
// position order, so a long prefix fills several entries of one pass.
constexpr int PREFILL_GROUP = 64;
struct PrefillGroup {
  int n;
  int seq[PREFILL_GROUP], slot[PREFILL_GROUP], p0[PREFILL_GROUP], cnt[PREFILL_GROUP], nvis[PREFILL_GROUP],
      plen[PREFILL_GROUP];
};
template <typename T>
void launch_plan_prefill(hipStream_t s, const PrefillGroup& g, const float* vision, int nv_stride,
                         const int* prompt, int np_stride, const T* embed, int V, int* plan_base, int* plan_cnt,
                         int* plan_slot, float* x, float* esave);
// hprev / hnext: [max_batch][D] per-slot last verifier hidden of the previous /
// this pass (two buffers, alternating by pass).
void launch_draft_prefill_cat(hipStream_t s, const PrefillGroup& g, const float* xfinal, const float* esave,
                              const float* hprev, float* hnext, const float* g_h, const float* g_e, float eps,
                              float* cat);
// dst[f] = the last prefix row of the f-th entry (in entry order) that ends its
// sequence in this pass.
void launch_prefill_last_rows(hipStream_t s, const PrefillGroup& g, const float* xfinal, float* dst);
// tok: greedy tokens of those rows, by the same rank; pending_out: [B] of the call.
void launch_prefill_finish(hipStream_t s, const PrefillGroup& g, const float* xfinal, const int* tok, StateView sv,
                           int* pending_out);
void launch_set_sequence(hipStream_t s, int slot, int P, int tok, StateView sv);
// KV page-table entries set by value (at most PAGESET_N per launch, each
// entry once: the launch's threads store in no set order).
constexpr int PAGESET_N = 240;
struct PageSet {
  int n;
  int idx[PAGESET_N], page[PAGESET_N];
};
void launch_set_pages(hipStream_t s, int* table, const PageSet& ps);
// Copy a caller's cache of one layer ([K|V][head][n_pos][128]) into a slot's pages.
template <typename T>
void launch_load_kv(hipStream_t s, const T* src, int n_pos, KvView<T> kv, int slot);
// Acceptance; with part_val non-null the greedy tokens are first reduced from
// the LM head's per-block bests (part_val / part_idx, nblk per row) and
// written to greedy_w (the verify then skips its argmax stage 2).
// A sequence whose step would pass the cache (kv_len + K + 1 > max_pos; the
// verify plan has set its overflow flag and computed no rows for it) commits
// nothing and keeps its state; n_acc[b] = -1.
void launch_accept(hipStream_t s, int B, int K, const int* plan_slot, const int* draft, const int* greedy,
                   const float* xfinal, StateView sv, int* n_acc, int* out_tokens, int* out_len_out,
                   int out_cap, const StepTap& tap, const float* part_val = nullptr, const int* part_idx = nullptr,
                   int nblk = 0, int* greedy_w = nullptr);
// drafts tap: the K proposals of each sequence of the call (draft[b][K]) at
// the slot's current step number.
void launch_draft_tap(hipStream_t s, int B, int K, const int* plan_slot, StateView sv, const int* draft,
                      const StepTap& tap);
void launch_controlled(hipStream_t s, int B, int K, const int* slots_in, StateView sv, const int* trace,
                       int trace_stride, int trace_len, uint64_t seed, uint64_t thr, int V, int* draft);
void launch_copy_rows(hipStream_t s, const float* src, float* dst, long n);
// p[0 .. n) = v, by a kernel (graph-capture safe, unlike a memset node).
void launch_fill_i32(hipStream_t s, int* p, long n, int v);

}  // namespace ocr
