// Host-side launchers of the ocrdec kernels (one per kernel family).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "common.h"

namespace ocr {

enum Epi { EPI_STORE = 0, EPI_ADD = 1, EPI_SWIGLU = 2 };

// x: [M][D] residual rows; gain: RMSNorm gain (never null here).
// Writes q (RoPE'd, fp32 [M][QD]) and, for valid rows, k / v into the cache
// kv[slot][0|1][head][pos][HD] (slot stride = 2*NH*max_pos*HD elements).
template <typename T>
void launch_qkv_rope(hipStream_t s, const float* x, const float* gain, float eps, const T* wqkv, int M,
                     RowPlan plan, float* q, T* kv, int max_pos, const float2* rope);
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

template <typename T>
void launch_attention(hipStream_t s, const float* q, const T* kv, int max_pos, RowPlan plan, int B,
                      int n_chunks, int tiles_per_chunk, float* part, float* out);

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

// Router logits (rlogit) and the routing tables; logit_override (nullable,
// [M][64]) replaces the computed logits before the top-6.
template <typename T>
void launch_router(hipStream_t s, const float* x, const float* gain, float eps, const T* wr, int M,
                   const MoeBufs& mb, int* tap, const float* logit_override);
template <typename T>
void launch_expert_gate_up(hipStream_t s, const T* wg, const T* wu, int M, const MoeBufs& mb, int* tap);
template <typename T>
void launch_expert_down(hipStream_t s, const T* wd, int M, const MoeBufs& mb);
void launch_moe_combine(hipStream_t s, float* x, int M, const MoeBufs& mb);
int expert_slot_cap(int M);

// Matrix-core variants (bf16 weights): the same outputs as the vector
// launchers above, with the activations rounded to bf16 for the MFMA inputs.
void launch_expert_gate_up_mfma(hipStream_t s, const bf16* wg, const bf16* wu, int M, const MoeBufs& mb);
void launch_expert_down_mfma(hipStream_t s, const bf16* wd, int M, const MoeBufs& mb);
// Dense layers on the matrix cores (bf16 weights): the outputs of launch_gemv
// (K, epi) in {(1280, add / store / SwiGLU), (2560, store), (3584, add)}, N a
// multiple of 64, and of launch_qkv_rope, with the inputs as bf16 hi + lo parts.
void launch_gemv_mfma(hipStream_t s, int K, Epi epi, const float* a, long lda, const float* gain, float eps,
                      const bf16* W0, const bf16* W1, int N, int M, float* out, long ldo);
void launch_qkv_rope_mfma(hipStream_t s, const float* x, const float* gain, float eps, const bf16* wqkv, int M,
                          RowPlan plan, float* q, bf16* kv, int max_pos, const float2* rope);
// The same with k split over the four wavefronts of 16-row blocks (decode-sized
// calls: many blocks, no LDS staging).
void launch_gemv_ks(hipStream_t s, int K, Epi epi, const float* a, long lda, const float* gain, float eps,
                    const bf16* W0, const bf16* W1, int N, int M, float* out, long ldo);
void launch_qkv_rope_ks(hipStream_t s, const float* x, const float* gain, float eps, const bf16* wqkv, int M,
                        RowPlan plan, float* q, bf16* kv, int max_pos, const float2* rope);
// LM head + argmax: xn ([M][D] scratch) receives the normalised rows; V >= 16.
void launch_lmhead_mfma(hipStream_t s, const float* x, const int* cnt, int Q, bool last_valid, const float* gain,
                        float eps, const bf16* W, int V, int M, float* xn, float* part_val, int* part_idx,
                        float* logits, int* tok, int tok_stride);

// ---- row plans, embeddings, acceptance --------------------------------------
struct StateView {
  int* kv_len; int* draft_len; int* pending; int* n_prev; int* out_len; int* step; int* prefix_len;
  int* cu_tok;     // [max_batch][cu_stride]
  int cu_stride;
  float* hbuf;     // [max_batch][cu_stride][D]
  int n_slots;     // max_batch
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
constexpr int PREFILL_GROUP = 32;
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
// tok: [n] greedy tokens of the group's last valid rows; pending_out: [B] of the call.
void launch_prefill_finish(hipStream_t s, const PrefillGroup& g, const float* xfinal, const int* tok, StateView sv,
                           int* pending_out);
void launch_set_sequence(hipStream_t s, int slot, int P, int tok, StateView sv);
// Acceptance; with part_val non-null the greedy tokens are first reduced from
// the LM head's per-block bests (part_val / part_idx, nblk per row) and
// written to greedy_w (the verify then skips its argmax stage 2).
void launch_accept(hipStream_t s, int B, int K, const int* plan_slot, const int* draft, const int* greedy,
                   const float* xfinal, StateView sv, int* n_acc, int* out_tokens, int* out_len_out,
                   int out_cap, const float* part_val = nullptr, const int* part_idx = nullptr, int nblk = 0,
                   int* greedy_w = nullptr);
void launch_controlled(hipStream_t s, int B, int K, const int* slots_in, StateView sv, const int* trace,
                       int trace_stride, int trace_len, uint64_t seed, uint64_t thr, int V, int* draft);
void launch_copy_rows(hipStream_t s, const float* src, float* dst, long n);

}  // namespace ocr
