// Host side of the ocrdec C ABI: buffer layout inside the caller's state and
// workspace, argument checks, and the launch sequence of each call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <map>
#include <string>
#include <tuple>
#include <type_traits>
#include <vector>

#include "launch.h"
#include "ocrdec.h"

using namespace ocr;

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Offsets of every sub-buffer inside the state and the workspace.
struct Plan {
  // derived sizes
  int Qmax, M_max, prefill_group, cu_stride, tiles_per_chunk, chunk_keys, n_chunks_cap, lm_nblk;
  size_t esz, kv_layer_elems;
  // state
  size_t s_kv, s_dkv, s_ints, s_cu, s_hbuf, s_rope, s_total;
  // workspace
  size_t w_x, w_q, w_attn, w_part, w_bnorm, w_ridx, w_rgate, w_perm, w_inv, w_off, w_act, w_slot, w_rlogit, w_misc, w_stats, w_hx,
      w_y, w_cat, w_u, w_u2, w_dffn, w_esave, w_hsave, w_lmv, w_lmi, w_plan, w_total;
};

bool shape_ok(const ocrdec_config* c, std::string* why) {
  if (!c) { *why = "config is null"; return false; }
  if (c->d_model != D || c->n_heads != NH || c->head_dim != HD || c->n_experts != NE || c->n_shared != NSH ||
      c->top_k != TOPK || c->d_expert != DI || c->d_draft_ffn != DF) {
    *why = "unsupported shape: the kernels are built for d=1280, 10x128 heads, 64+2 experts of 896, top-6, "
           "draft FFN 3584";
    return false;
  }
  if (c->n_layers < 1 || c->vocab < 2) { *why = "n_layers must be >= 1 and vocab >= 2"; return false; }
  if (c->dtype != OCRDEC_F32 && c->dtype != OCRDEC_BF16) { *why = "dtype must be OCRDEC_F32 or OCRDEC_BF16"; return false; }
  if (c->max_batch < 1 || c->max_batch > 1024) { *why = "max_batch must be in [1, 1024]"; return false; }
  if (c->max_k < 0 || c->max_k > 7) { *why = "max_k must be in [0, 7]"; return false; }
  if (c->max_batch * (c->max_k + 1) > 1024) { *why = "max_batch * (max_k + 1) must be <= 1024"; return false; }
  if (c->max_positions < 16 || c->max_positions > 32768) { *why = "max_positions must be in [16, 32768]"; return false; }
  if (!(c->norm_eps > 0.f) || !(c->rope_theta > 1.f)) { *why = "norm_eps must be > 0 and rope_theta > 1"; return false; }
  if (c->path < OCRDEC_PATH_AUTO || c->path > OCRDEC_PATH_MATRIX) { *why = "path must be OCRDEC_PATH_*"; return false; }
  if (c->path == OCRDEC_PATH_MATRIX && (c->dtype != OCRDEC_BF16 || c->vocab < 64)) {
    *why = "the matrix-core path needs bf16 weights and vocab >= 64";
    return false;
  }
  return true;
}

// Matrix cores for the experts and the LM head: fixed per handle.
bool use_matrix_path(const ocrdec_config* c) {
  if (c->path == OCRDEC_PATH_MATRIX) return true;
  if (c->path == OCRDEC_PATH_VECTOR) return false;
  return c->dtype == OCRDEC_BF16 && c->vocab >= 64 && c->max_batch * (c->max_k + 1) > MRG;
}

Plan make_plan(const ocrdec_config* c) {
  Plan p{};
  p.Qmax = std::max(c->max_k + 1, PREFILL_CHUNK);
  // prefill passes take up to prefill_group entries of PREFILL_CHUNK rows
  p.prefill_group = PREFILL_GROUP;
  p.M_max = std::max(c->max_batch * (c->max_k + 1), PREFILL_CHUNK * p.prefill_group);
  p.cu_stride = c->max_k + 1;
  p.tiles_per_chunk = c->max_positions > 4096 ? 4 : 1;
  p.chunk_keys = p.tiles_per_chunk * ATT_TILE;
  p.n_chunks_cap = (c->max_positions + p.chunk_keys - 1) / p.chunk_keys;
  p.lm_nblk = lmhead_blocks(c->vocab);
  p.esz = c->dtype == OCRDEC_BF16 ? 2 : 4;
  p.kv_layer_elems = (size_t)c->max_batch * 2 * NH * (size_t)c->max_positions * HD;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = align256(o + bytes); return r; };
  p.s_kv = take(p.kv_layer_elems * c->n_layers * p.esz);
  p.s_dkv = take(p.kv_layer_elems * p.esz);
  p.s_ints = take((size_t)7 * c->max_batch * 4);
  p.s_cu = take((size_t)c->max_batch * p.cu_stride * 4);
  p.s_hbuf = take((size_t)c->max_batch * p.cu_stride * D * 4);
  p.s_rope = take((size_t)c->max_positions * (HD / 2) * 8);
  p.s_total = o;
  o = 0;
  const size_t M = p.M_max;
  p.w_x = take(M * D * 4);
  p.w_q = take(M * QD * 4);
  p.w_attn = take(M * QD * 4);
  p.w_part = take(M * NH * (size_t)p.n_chunks_cap * (HD + 2) * 4);
  p.w_bnorm = take(M * D * 4);
  p.w_ridx = take(M * NSLOT * 4);
  p.w_rgate = take(M * NSLOT * 4);
  p.w_perm = take(M * NSLOT * 4);
  p.w_inv = take(M * NSLOT * 4);
  p.w_off = take((NX + 1) * 4);
  p.w_act = take(NX * 4);
  p.w_slot = take(NX * 16);
  p.w_rlogit = take(M * NE * 4);
  p.w_misc = take(64 * 4);       // [0] n_act, [16..] prefill tokens
  p.w_stats = take(8 * 8);
  p.w_hx = take(M * NSLOT * DI * 4);
  p.w_y = take(M * NSLOT * D * 4);
  p.w_cat = take(M * 2 * D * 4);
  p.w_u = take(M * D * 4);
  p.w_u2 = take((size_t)c->max_batch * D * 4);  // second output buffer of the recursive draft passes
  p.w_dffn = take(M * DF * 4);
  p.w_esave = take(M * D * 4);
  p.w_hsave = take((size_t)2 * c->max_batch * D * 4);
  p.w_lmv = take(M * (size_t)p.lm_nblk * 4);
  p.w_lmi = take(M * (size_t)p.lm_nblk * 4);
  p.w_plan = take((size_t)3 * std::max(c->max_batch, PREFILL_GROUP) * 4);
  p.w_total = o;
  return p;
}

}  // namespace

struct ocrdec_model {
  ocrdec_config cfg;
  Plan p;
  std::vector<const void*> w;
  char* state;
  char* ws;
  StateView sv;
  float *x, *q, *attn, *part, *cat, *u, *u2, *dffn, *esave, *hsave[2], *lm_val;
  int *lm_idx, *plan_base, *plan_cnt, *plan_slot, *tok_tmp;
  MoeBufs mb;
  const float2* rope;
  // Host-side upper bound on (last position + 1) of every slot: set by prefill,
  // raised by K + 1 per accept.  It sizes the attention grids and the capacity
  // checks; the device clamps positions to the cache in any case.
  std::vector<int> slot_bound;
  int32_t* tap_route;
  float* tap_hidden;
  bool timing;
  std::vector<hipEvent_t> ev;  // triplets: before gate/up, between, after down
  size_t ev_used;
  long long stats_base;        // device expert counter when timing was enabled
  int last_verify_rows;        // M of the last verify call (0 before any)
  bool matrix;                 // experts and LM head on the matrix cores
  const float* router_override;  // [n_layers][M][64] router logits for verify calls, or null
  hipStream_t capture_stream;  // private stream the decode-step graphs are recorded on
  std::map<std::vector<uintptr_t>, hipGraphExec_t> graphs;  // by call shape
};

namespace {

enum WIdx { W_EMBED = 0, W_LM = 1, W_FNORM = 2, W_LAYER0 = 3 };
enum LIdx { L_ANORM = 0, L_QKV, L_WO, L_FNORM, L_ROUTER, L_GATE, L_UP, L_DOWN, L_N };
enum DIdx { D_NH = 0, D_NE, D_FUSE, D_ANORM, D_QKV, D_WO, D_FNORM, D_GATE, D_UP, D_DOWN, D_ONORM, D_N };

int num_weights(const ocrdec_config* c) { return W_LAYER0 + L_N * c->n_layers + D_N; }

template <typename T> const T* wmat(const ocrdec_model* m, int i) { return static_cast<const T*>(m->w[i]); }
const float* wvec(const ocrdec_model* m, int i) { return static_cast<const float*>(m->w[i]); }
int lw(const ocrdec_model* m, int l, int k) { (void)m; return W_LAYER0 + L_N * l + k; }
int dw(const ocrdec_model* m, int k) { return W_LAYER0 + L_N * m->cfg.n_layers + k; }

int hip_check(const char* where) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(OCRDEC_EHIP, std::string(where) + ": " + hipGetErrorString(e));
  return OCRDEC_OK;
}

int chunks_for(const ocrdec_model* m, int max_pos_touched) {
  return std::min(m->p.n_chunks_cap, max_pos_touched / m->p.chunk_keys + 1);
}

// Bound for the sequences of a call: slots 0..B-1 when `slots` is null, else every slot.
int call_bound(const ocrdec_model* m, int B, const int32_t* slots) {
  const int n = slots ? (int)m->slot_bound.size() : B;
  int b = 0;
  for (int i = 0; i < n; ++i) b = std::max(b, m->slot_bound[i]);
  return b;
}

void timing_mark(ocrdec_model* m, hipStream_t s) {
  if (!m->timing) return;
  if (m->ev_used >= m->ev.size()) {
    if (m->ev.size() >= (size_t)3 * 65536) return;
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) { m->timing = false; return; }
    m->ev.push_back(e);
  }
  if (hipEventRecord(m->ev[m->ev_used], s) == hipSuccess) ++m->ev_used;
}

// Arithmetic of a pass.  Decode calls of a matrix-path handle run the experts,
// the LM head and the dense layers on the matrix cores for every row count (so
// a row's result never depends on the call; the dense layers in 16-row blocks
// with k split over the wavefronts); a prefill pass of a bf16 model runs the
// experts and the dense layers on the matrix cores whatever the handle (64-row
// strips; the prefix is computed once and shared by every decode that follows).
enum DensePath { DENSE_VECTOR = 0, DENSE_KSPLIT = 1, DENSE_STRIP = 2 };
struct PassPath {
  bool experts;  // grouped experts on the matrix cores
  int dense;     // DensePath of the QKV / O / draft GEMVs
};

template <typename T>
PassPath decode_path(const ocrdec_model* m) {
  const bool mx = std::is_same<T, bf16>::value && m->matrix;
  return PassPath{mx, mx ? DENSE_KSPLIT : DENSE_VECTOR};
}

template <typename T>
PassPath prefill_path(const ocrdec_model* m) {
  (void)m;
  const bool bf = std::is_same<T, bf16>::value;
  return PassPath{bf, bf ? DENSE_STRIP : DENSE_VECTOR};
}

template <typename T>
void expert_gate_up(ocrdec_model* m, hipStream_t s, int l, int M, int* tap, bool mx) {
  if constexpr (std::is_same<T, bf16>::value) {
    if (mx) {
      launch_expert_gate_up_mfma(s, wmat<T>(m, lw(m, l, L_GATE)), wmat<T>(m, lw(m, l, L_UP)), M, m->mb);
      return;
    }
  }
  launch_expert_gate_up<T>(s, wmat<T>(m, lw(m, l, L_GATE)), wmat<T>(m, lw(m, l, L_UP)), M, m->mb, tap);
}

template <typename T>
void expert_down(ocrdec_model* m, hipStream_t s, int l, int M, bool mx) {
  if constexpr (std::is_same<T, bf16>::value) {
    if (mx) {
      launch_expert_down_mfma(s, wmat<T>(m, lw(m, l, L_DOWN)), M, m->mb);
      return;
    }
  }
  launch_expert_down<T>(s, wmat<T>(m, lw(m, l, L_DOWN)), M, m->mb);
}

// LM head + argmax over M output rows (see launch_lmhead).
template <typename T>
void lm_head(ocrdec_model* m, hipStream_t s, const float* x, int Q, bool last_valid, const float* gain, int M,
             float* logits, int* tok, int tok_stride) {
  const ocrdec_config& c = m->cfg;
  if constexpr (std::is_same<T, bf16>::value) {
    if (m->matrix) {
      launch_lmhead_mfma(s, x, m->plan_cnt, Q, last_valid, gain, c.norm_eps, wmat<T>(m, W_LM), c.vocab, M,
                         m->mb.bnorm, m->lm_val, m->lm_idx, logits, tok, tok_stride);
      return;
    }
  }
  launch_lmhead<T>(s, x, m->plan_cnt, Q, last_valid, gain, c.norm_eps, wmat<T>(m, W_LM), c.vocab, M, m->lm_val,
                   m->lm_idx, logits, tok, tok_stride);
}

// Dense layers on the path dp (DensePath).
template <typename T>
void dense_gemv(ocrdec_model* m, hipStream_t s, int dp, int K, Epi epi, const float* a, long lda,
                const float* gain, const T* W0, const T* W1, int N, int M, float* out, long ldo) {
  if constexpr (std::is_same<T, bf16>::value) {
    if (dp == DENSE_STRIP) {
      launch_gemv_mfma(s, K, epi, a, lda, gain, m->cfg.norm_eps, W0, W1, N, M, out, ldo);
      return;
    }
    if (dp == DENSE_KSPLIT) {
      launch_gemv_ks(s, K, epi, a, lda, gain, m->cfg.norm_eps, W0, W1, N, M, out, ldo);
      return;
    }
  }
  launch_gemv<T>(s, K, epi, a, lda, gain, m->cfg.norm_eps, W0, W1, N, M, out, ldo);
}

template <typename T>
void dense_qkv(ocrdec_model* m, hipStream_t s, int dp, const float* x, const float* gain, const T* W, int M,
               RowPlan plan, T* kv) {
  if constexpr (std::is_same<T, bf16>::value) {
    if (dp == DENSE_STRIP) {
      launch_qkv_rope_mfma(s, x, gain, m->cfg.norm_eps, W, M, plan, m->q, kv, m->cfg.max_positions, m->rope);
      return;
    }
    if (dp == DENSE_KSPLIT) {
      launch_qkv_rope_ks(s, x, gain, m->cfg.norm_eps, W, M, plan, m->q, kv, m->cfg.max_positions, m->rope);
      return;
    }
  }
  launch_qkv_rope<T>(s, x, gain, m->cfg.norm_eps, W, M, plan, m->q, kv, m->cfg.max_positions, m->rope);
}

template <typename T>
void verifier_layers(ocrdec_model* m, hipStream_t s, PassPath pp, int M, int B, RowPlan plan, int nch, bool taps,
                     const float* rlog) {
  const ocrdec_config& c = m->cfg;
  for (int l = 0; l < c.n_layers; ++l) {
    T* kvl = static_cast<T*>((void*)(m->state + m->p.s_kv)) + (size_t)l * m->p.kv_layer_elems;
    dense_qkv<T>(m, s, pp.dense, m->x, wvec(m, lw(m, l, L_ANORM)), wmat<T>(m, lw(m, l, L_QKV)), M, plan, kvl);
    launch_attention<T>(s, m->q, kvl, c.max_positions, plan, B, nch, m->p.tiles_per_chunk, m->part, m->attn);
    dense_gemv<T>(m, s, pp.dense, QD, EPI_ADD, m->attn, QD, nullptr, wmat<T>(m, lw(m, l, L_WO)), nullptr, D, M,
                  m->x, D);
    int* tap = (taps && m->tap_route) ? m->tap_route + (size_t)l * M * NSLOT : nullptr;
    launch_router<T>(s, m->x, wvec(m, lw(m, l, L_FNORM)), c.norm_eps, wmat<T>(m, lw(m, l, L_ROUTER)), M, m->mb,
                     tap, rlog ? rlog + (size_t)l * M * NE : nullptr);
    timing_mark(m, s);
    expert_gate_up<T>(m, s, l, M, tap, pp.experts);
    timing_mark(m, s);
    expert_down<T>(m, s, l, M, pp.experts);
    timing_mark(m, s);
    launch_moe_combine(s, m->x, M, m->mb);
  }
}

// The draft block on rows u (M of them): the fusion projection of cat into
// u (skipped when a fused launch has already written u), attention, SwiGLU FFN.
template <typename T>
void draft_layer(ocrdec_model* m, hipStream_t s, PassPath pp, int M, int B, RowPlan plan, int nch, float* u,
                 bool fused_in) {
  const ocrdec_config& c = m->cfg;
  const int mx = pp.dense;
  T* dkv = static_cast<T*>((void*)(m->state + m->p.s_dkv));
  if (!fused_in)
    dense_gemv<T>(m, s, mx, 2 * D, EPI_STORE, m->cat, 2 * D, nullptr, wmat<T>(m, dw(m, D_FUSE)), nullptr, D, M, u,
                  D);
  dense_qkv<T>(m, s, mx, u, wvec(m, dw(m, D_ANORM)), wmat<T>(m, dw(m, D_QKV)), M, plan, dkv);
  launch_attention<T>(s, m->q, dkv, c.max_positions, plan, B, nch, m->p.tiles_per_chunk, m->part, m->attn);
  dense_gemv<T>(m, s, mx, QD, EPI_ADD, m->attn, QD, nullptr, wmat<T>(m, dw(m, D_WO)), nullptr, D, M, u, D);
  dense_gemv<T>(m, s, mx, D, EPI_SWIGLU, u, D, wvec(m, dw(m, D_FNORM)), wmat<T>(m, dw(m, D_GATE)),
                wmat<T>(m, dw(m, D_UP)), DF, M, m->dffn, DF);
  dense_gemv<T>(m, s, mx, DF, EPI_ADD, m->dffn, DF, nullptr, wmat<T>(m, dw(m, D_DOWN)), nullptr, D, M, u, D);
}

// Prefill in passes of up to prefill_group entries of PREFILL_CHUNK rows: the
// (sequence, chunk) pairs in sequence order, cut into passes, so a long prefix
// spreads over several entries of one pass and short ones share passes.  All
// rows' keys / values are written before the pass's attention reads them, and
// each row's arithmetic is the same whatever its pass.
template <typename T>
int do_prefill(ocrdec_model* m, hipStream_t s, int B, const int32_t* slots_host, const float* vision, int nv_stride,
               const int32_t* nv_host, const int32_t* prompt, int np_stride, const int32_t* np_host,
               int32_t* pending_out) {
  const ocrdec_config& c = m->cfg;
  std::vector<std::pair<int, int>> ent;  // (sequence, first position)
  for (int b = 0; b < B; ++b)
    for (int p0 = 0; p0 < nv_host[b] + np_host[b]; p0 += PREFILL_CHUNK) ent.emplace_back(b, p0);
  int t = 0;
  for (size_t e0 = 0; e0 < ent.size(); e0 += m->p.prefill_group, ++t) {
    const float* hprev = m->hsave[t & 1];
    float* hnext = m->hsave[(t + 1) & 1];
    PrefillGroup g{};
    g.n = (int)std::min(ent.size() - e0, (size_t)m->p.prefill_group);
    bool finish = false;
    int max_pos = 0;
    for (int j = 0; j < g.n; ++j) {
      const int b = ent[e0 + j].first, p0 = ent[e0 + j].second;
      const int P = nv_host[b] + np_host[b];
      g.seq[j] = b;
      g.slot[j] = slots_host ? slots_host[b] : b;
      g.p0[j] = p0;
      g.cnt[j] = std::min(PREFILL_CHUNK, P - p0);
      g.nvis[j] = nv_host[b];
      g.plen[j] = P;
      finish = finish || (p0 + g.cnt[j] == P);
      max_pos = std::max(max_pos, p0 + g.cnt[j] - 1);
    }
    launch_plan_prefill<T>(s, g, vision, nv_stride, prompt, np_stride, wmat<T>(m, W_EMBED), c.vocab, m->plan_base,
                           m->plan_cnt, m->plan_slot, m->x, m->esave);
    const int M = g.n * PREFILL_CHUNK;
    RowPlan plan{m->plan_base, m->plan_cnt, m->plan_slot, PREFILL_CHUNK, 0};
    const int nch = chunks_for(m, std::min(c.max_positions - 1, max_pos));
    verifier_layers<T>(m, s, prefill_path<T>(m), M, g.n, plan, nch, false, nullptr);
    if (finish) lm_head<T>(m, s, m->x, PREFILL_CHUNK, true, wvec(m, W_FNORM), g.n, nullptr, m->tok_tmp, 1);
    launch_draft_prefill_cat(s, g, m->x, m->esave, hprev, hnext, wvec(m, dw(m, D_NH)), wvec(m, dw(m, D_NE)),
                             c.norm_eps, m->cat);
    draft_layer<T>(m, s, prefill_path<T>(m), M, g.n, plan, nch, m->u, false);
    if (finish) launch_prefill_finish(s, g, m->x, m->tok_tmp, m->sv, pending_out);
  }
  for (int b = 0; b < B; ++b) m->slot_bound[slots_host ? slots_host[b] : b] = nv_host[b] + np_host[b];
  return hip_check("ocrdec_prefill");
}

template <typename T>
int do_draft(ocrdec_model* m, hipStream_t s, int B, const int32_t* slots, int K, int32_t* draft_out) {
  const ocrdec_config& c = m->cfg;
  const int Q = K + 1;
  // same chunk count as the verify of this step (a decode-step graph is keyed on it)
  const int nch = chunks_for(m, std::min(c.max_positions - 1, call_bound(m, B, slots) + K));
  const PassPath pp = decode_path<T>(m);
  const int ident = slots == nullptr;
  const RowPlan plan{m->plan_base, m->plan_cnt, m->plan_slot, Q, ident};
  const RowPlan p1{m->plan_base, m->plan_cnt, m->plan_slot, 1, ident};
  if (pp.dense == DENSE_VECTOR) {
    // each pass's plan, input rows and fusion projection in one launch (pass j
    // >= 2 also takes d_{j-1} from the previous LM head's partials, so only the
    // last pass runs the argmax stage 2); passes alternate between two output
    // buffers since a pass reads the previous one's rows
    const int nblk = lmhead_blocks(c.vocab);
    const T* wf = wmat<T>(m, dw(m, D_FUSE));
    launch_draft_fuse<T>(s, 0, 1, Q, Q, K, slots, m->sv, wmat<T>(m, W_EMBED), c.vocab, wvec(m, dw(m, D_NH)),
                         wvec(m, dw(m, D_NE)), c.norm_eps, nullptr, nullptr, nullptr, nblk, draft_out, m->plan_base,
                         m->plan_cnt, m->plan_slot, wf, B * Q, m->u);
    draft_layer<T>(m, s, pp, B * Q, B, plan, nch, m->u, true);
    lm_head<T>(m, s, m->u, Q, true, wvec(m, dw(m, D_ONORM)), B, nullptr, K == 1 ? draft_out : nullptr, K);
    float* uprev = m->u;
    for (int j = 2; j <= K; ++j) {
      float* u = (uprev == m->u) ? m->u2 : m->u;
      launch_draft_fuse<T>(s, 1, j, Q, (j == 2) ? Q : 1, K, nullptr, m->sv, wmat<T>(m, W_EMBED), c.vocab,
                           wvec(m, dw(m, D_NH)), wvec(m, dw(m, D_NE)), c.norm_eps, uprev, m->lm_val, m->lm_idx, nblk,
                           draft_out, m->plan_base, m->plan_cnt, m->plan_slot, wf, B, u);
      draft_layer<T>(m, s, pp, B, B, p1, nch, u, true);
      lm_head<T>(m, s, u, 1, true, wvec(m, dw(m, D_ONORM)), B, nullptr, j == K ? draft_out + (j - 1) : nullptr, K);
      uprev = u;
    }
    return hip_check("ocrdec_draft");
  }
  launch_plan_draft_catchup<T>(s, B, Q, slots, m->sv, wmat<T>(m, W_EMBED), c.vocab, wvec(m, dw(m, D_NH)),
                               wvec(m, dw(m, D_NE)), c.norm_eps, m->plan_base, m->plan_cnt, m->plan_slot, m->cat);
  draft_layer<T>(m, s, pp, B * Q, B, plan, nch, m->u, false);
  lm_head<T>(m, s, m->u, Q, true, wvec(m, dw(m, D_ONORM)), B, nullptr, draft_out, K);
  for (int j = 2; j <= K; ++j) {
    const int Qprev = (j == 2) ? Q : 1;
    launch_plan_draft_step<T>(s, B, j, Qprev, K, m->sv, draft_out, wmat<T>(m, W_EMBED), c.vocab,
                              wvec(m, dw(m, D_NH)), wvec(m, dw(m, D_NE)), c.norm_eps, m->u, m->plan_base, m->plan_cnt,
                              m->plan_slot, m->cat);
    draft_layer<T>(m, s, pp, B, B, p1, nch, m->u, false);
    lm_head<T>(m, s, m->u, 1, true, wvec(m, dw(m, D_ONORM)), B, nullptr, draft_out + (j - 1), K);
  }
  return hip_check("ocrdec_draft");
}

template <typename T>
int do_verify(ocrdec_model* m, hipStream_t s, int B, const int32_t* slots, int K, const int32_t* draft,
              int32_t* greedy_out, float* logits_out, bool greedy_in_accept = false) {
  const ocrdec_config& c = m->cfg;
  const int Q = K + 1, M = B * Q;
  const int nch = chunks_for(m, std::min(c.max_positions - 1, call_bound(m, B, slots) + K));
  launch_plan_verify<T>(s, B, K, slots, m->sv, draft, wmat<T>(m, W_EMBED), c.vocab, m->plan_base, m->plan_cnt,
                        m->plan_slot, m->x);
  RowPlan plan{m->plan_base, m->plan_cnt, m->plan_slot, Q, slots == nullptr};
  verifier_layers<T>(m, s, decode_path<T>(m), M, B, plan, nch, true, m->router_override);
  m->last_verify_rows = M;
  // greedy_in_accept: the accept launch that follows reduces the greedy tokens
  lm_head<T>(m, s, m->x, Q, false, wvec(m, W_FNORM), M, logits_out, greedy_in_accept ? nullptr : greedy_out, 1);
  if (m->tap_hidden) launch_copy_rows(s, m->x, m->tap_hidden, (long)M * D);
  return hip_check("ocrdec_verify");
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_call(ocrdec_model* m, int B, int K) {
  (void)hipGetLastError();  // launch errors are checked after this call's launches
  if (!m) return fail(OCRDEC_EINVAL, "model is null");
  if (B < 1) return fail(OCRDEC_EINVAL, "B must be >= 1");
  if (K < 0) return fail(OCRDEC_EINVAL, "K must be >= 0");
  if (B > m->cfg.max_batch) return fail(OCRDEC_ECAPACITY, "B exceeds max_batch");
  if (K > m->cfg.max_k) return fail(OCRDEC_ECAPACITY, "K exceeds max_k");
  return OCRDEC_OK;
}

}  // namespace

extern "C" {

const char* ocrdec_last_error(void) { return g_err.c_str(); }

size_t ocrdec_state_bytes(const ocrdec_config* cfg) {
  std::string why;
  if (!shape_ok(cfg, &why)) { fail(OCRDEC_EINVAL, why); return 0; }
  return make_plan(cfg).s_total;
}

size_t ocrdec_workspace_bytes(const ocrdec_config* cfg) {
  std::string why;
  if (!shape_ok(cfg, &why)) { fail(OCRDEC_EINVAL, why); return 0; }
  return make_plan(cfg).w_total;
}

int ocrdec_num_weights(const ocrdec_config* cfg) {
  std::string why;
  if (!shape_ok(cfg, &why)) return fail(OCRDEC_EINVAL, why);
  return num_weights(cfg);
}

int ocrdec_create(const ocrdec_config* cfg, const void* const* weight_ptrs, int n_weights, void* state,
                  void* workspace, void* stream, ocrdec_model** out) {
  std::string why;
  if (!out) return fail(OCRDEC_EINVAL, "out is null");
  *out = nullptr;
  if (!shape_ok(cfg, &why)) return fail(OCRDEC_EINVAL, why);
  if (!weight_ptrs || n_weights != num_weights(cfg))
    return fail(OCRDEC_EINVAL, "weight_ptrs is null or n_weights != ocrdec_num_weights()");
  for (int i = 0; i < n_weights; ++i)
    if (!weight_ptrs[i] || !aligned(weight_ptrs[i], 16))
      return fail(OCRDEC_EINVAL, "weight pointer " + std::to_string(i) + " is null or not 16-byte aligned");
  if (!state || !workspace || !aligned(state, 256) || !aligned(workspace, 256))
    return fail(OCRDEC_EINVAL, "state / workspace must be non-null and 256-byte aligned");
  ocrdec_model* m = new ocrdec_model();
  m->cfg = *cfg;
  m->p = make_plan(cfg);
  m->w.assign(weight_ptrs, weight_ptrs + n_weights);
  m->state = static_cast<char*>(state);
  m->ws = static_cast<char*>(workspace);
  const Plan& p = m->p;
  const int mb = cfg->max_batch;
  int* ints = reinterpret_cast<int*>(m->state + p.s_ints);
  m->sv.kv_len = ints;
  m->sv.draft_len = ints + mb;
  m->sv.pending = ints + 2 * mb;
  m->sv.n_prev = ints + 3 * mb;
  m->sv.out_len = ints + 4 * mb;
  m->sv.step = ints + 5 * mb;
  m->sv.prefix_len = ints + 6 * mb;
  m->sv.cu_tok = reinterpret_cast<int*>(m->state + p.s_cu);
  m->sv.cu_stride = p.cu_stride;
  m->sv.hbuf = reinterpret_cast<float*>(m->state + p.s_hbuf);
  m->sv.n_slots = mb;
  m->rope = reinterpret_cast<const float2*>(m->state + p.s_rope);
  auto wf = [&](size_t off) { return reinterpret_cast<float*>(m->ws + off); };
  auto wi = [&](size_t off) { return reinterpret_cast<int*>(m->ws + off); };
  m->x = wf(p.w_x);
  m->q = wf(p.w_q);
  m->attn = wf(p.w_attn);
  m->part = wf(p.w_part);
  m->cat = wf(p.w_cat);
  m->u = wf(p.w_u);
  m->u2 = wf(p.w_u2);
  m->dffn = wf(p.w_dffn);
  m->esave = wf(p.w_esave);
  m->hsave[0] = wf(p.w_hsave);
  m->hsave[1] = wf(p.w_hsave) + (size_t)cfg->max_batch * D;
  m->lm_val = wf(p.w_lmv);
  m->lm_idx = wi(p.w_lmi);
  const int pm = std::max(mb, PREFILL_GROUP);
  m->plan_base = wi(p.w_plan);
  m->plan_cnt = wi(p.w_plan) + pm;
  m->plan_slot = wi(p.w_plan) + 2 * pm;
  int* misc = wi(p.w_misc);
  m->mb.n_act = misc;
  m->tok_tmp = misc + 16;
  m->mb.bnorm = wf(p.w_bnorm);
  m->mb.ridx = wi(p.w_ridx);
  m->mb.rgate = wf(p.w_rgate);
  m->mb.perm = wi(p.w_perm);
  m->mb.inv = wi(p.w_inv);
  m->mb.off = wi(p.w_off);
  m->mb.act = wi(p.w_act);
  m->mb.slot_info = reinterpret_cast<int4*>(m->ws + p.w_slot);
  m->mb.rlogit = wf(p.w_rlogit);
  m->mb.stats = reinterpret_cast<long long*>(m->ws + p.w_stats);
  m->mb.hx = wf(p.w_hx);
  m->mb.y = wf(p.w_y);
  m->slot_bound.assign(cfg->max_batch, 0);
  m->tap_route = nullptr;
  m->tap_hidden = nullptr;
  m->timing = false;
  m->ev_used = 0;
  m->stats_base = 0;
  m->last_verify_rows = 0;
  m->matrix = use_matrix_path(cfg);
  m->router_override = nullptr;
  m->capture_stream = nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // clear an error left by earlier, unrelated runtime calls
  hipError_t err = hipMemsetAsync(misc, 0, 64 * 4, s);
  if (err == hipSuccess) err = hipMemsetAsync(m->mb.stats, 0, 64, s);
  if (err == hipSuccess) err = hipMemsetAsync(m->state + p.s_ints, 0, p.s_hbuf - p.s_ints, s);
  if (err == hipSuccess) {
    launch_rope_table(s, cfg->max_positions, cfg->rope_theta, reinterpret_cast<float2*>(m->state + p.s_rope));
    err = hipGetLastError();
  }
  if (err != hipSuccess) {
    delete m;
    return fail(OCRDEC_EHIP, std::string("initialising the state / workspace failed: ") + hipGetErrorString(err));
  }
  *out = m;
  return OCRDEC_OK;
}

int ocrdec_destroy(ocrdec_model* m) {
  if (!m) return fail(OCRDEC_EINVAL, "model is null");
  for (hipEvent_t e : m->ev) (void)hipEventDestroy(e);
  for (auto& kv : m->graphs) (void)hipGraphExecDestroy(kv.second);
  if (m->capture_stream) (void)hipStreamDestroy(m->capture_stream);
  delete m;
  return OCRDEC_OK;
}

int ocrdec_prefill(ocrdec_model* m, void* stream, int B, const int32_t* slots_host, const float* vision, int nv_stride,
                   const int32_t* n_vision_host, const int32_t* prompt, int np_stride, const int32_t* n_prompt_host,
                   int32_t* pending_out) {
  int rc = check_call(m, B, 0);
  if (rc) return rc;
  if (!n_vision_host || !n_prompt_host || !pending_out) return fail(OCRDEC_EINVAL, "null length / output pointer");
  std::vector<int> seen;
  for (int b = 0; b < B; ++b) {
    const int slot = slots_host ? slots_host[b] : b;
    if (slot < 0 || slot >= m->cfg.max_batch) return fail(OCRDEC_EINVAL, "slot out of range");
    if (std::find(seen.begin(), seen.end(), slot) != seen.end()) return fail(OCRDEC_EINVAL, "duplicate slot");
    seen.push_back(slot);
    const int Nv = n_vision_host[b], Np = n_prompt_host[b];
    if (Nv < 0 || Np < 0 || Nv + Np < 1) return fail(OCRDEC_EINVAL, "prefix must hold at least one row");
    if (Nv > 0 && (!vision || nv_stride < Nv)) return fail(OCRDEC_EINVAL, "vision is null or nv_stride < n_vision");
    if (Np > 0 && (!prompt || np_stride < Np)) return fail(OCRDEC_EINVAL, "prompt is null or np_stride < n_prompt");
    if (Nv + Np + m->cfg.max_k + 1 > m->cfg.max_positions)
      return fail(OCRDEC_ECAPACITY, "prefix + max_k + 1 exceeds max_positions");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (m->cfg.dtype == OCRDEC_BF16)
    return do_prefill<bf16>(m, s, B, slots_host, vision, nv_stride, n_vision_host, prompt, np_stride, n_prompt_host,
                            pending_out);
  return do_prefill<float>(m, s, B, slots_host, vision, nv_stride, n_vision_host, prompt, np_stride, n_prompt_host,
                           pending_out);
}

int ocrdec_draft(ocrdec_model* m, void* stream, int B, const int32_t* slots, int K, int32_t* draft_out) {
  int rc = check_call(m, B, K);
  if (rc) return rc;
  if (K < 1) return fail(OCRDEC_EINVAL, "draft needs K >= 1");
  if (!draft_out) return fail(OCRDEC_EINVAL, "draft_out is null");
  if (!slots && call_bound(m, B, slots) + K > m->cfg.max_positions)
    return fail(OCRDEC_ECAPACITY, "positions would exceed max_positions");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (m->cfg.dtype == OCRDEC_BF16) return do_draft<bf16>(m, s, B, slots, K, draft_out);
  return do_draft<float>(m, s, B, slots, K, draft_out);
}

int ocrdec_verify(ocrdec_model* m, void* stream, int B, const int32_t* slots, int K, const int32_t* draft,
                  int32_t* greedy_out, float* logits_out) {
  int rc = check_call(m, B, K);
  if (rc) return rc;
  if (!greedy_out || (K > 0 && !draft)) return fail(OCRDEC_EINVAL, "greedy_out is null, or draft is null with K > 0");
  if (!slots && call_bound(m, B, slots) + K + 1 > m->cfg.max_positions)
    return fail(OCRDEC_ECAPACITY, "positions would exceed max_positions");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (m->cfg.dtype == OCRDEC_BF16) return do_verify<bf16>(m, s, B, slots, K, draft, greedy_out, logits_out);
  return do_verify<float>(m, s, B, slots, K, draft, greedy_out, logits_out);
}

int ocrdec_accept_rollback(ocrdec_model* m, void* stream, int B, const int32_t* slots, int K, const int32_t* draft,
                           const int32_t* greedy, int32_t* n_accepted_out, int32_t* out_tokens, int32_t* out_len,
                           int out_cap) {
  int rc = check_call(m, B, K);
  if (rc) return rc;
  if (!greedy || (K > 0 && !draft)) return fail(OCRDEC_EINVAL, "greedy is null, or draft is null with K > 0");
  if (out_tokens && out_cap < 1) return fail(OCRDEC_EINVAL, "out_cap must be >= 1 with out_tokens");
  hipStream_t s = static_cast<hipStream_t>(stream);
  launch_accept(s, B, K, m->plan_slot, draft, greedy, m->x, m->sv, n_accepted_out, out_tokens, out_len, out_cap);
  const int n = slots ? (int)m->slot_bound.size() : B;
  for (int i = 0; i < n; ++i) m->slot_bound[i] = std::min(m->cfg.max_positions, m->slot_bound[i] + K + 1);
  return hip_check("ocrdec_accept_rollback");
}

int ocrdec_controlled_drafts(ocrdec_model* m, void* stream, int B, const int32_t* slots, int K, const int32_t* trace,
                             int trace_stride, int trace_len, uint64_t seed, uint64_t threshold, int32_t* draft_inout) {
  int rc = check_call(m, B, K);
  if (rc) return rc;
  if (K < 1 || !trace || !draft_inout || trace_len < 0 || trace_stride < trace_len)
    return fail(OCRDEC_EINVAL, "bad controlled-draft arguments");
  hipStream_t s = static_cast<hipStream_t>(stream);
  launch_controlled(s, B, K, slots, m->sv, trace, trace_stride, trace_len, seed, threshold, m->cfg.vocab, draft_inout);
  return hip_check("ocrdec_controlled_drafts");
}

int ocrdec_replay_expert_gate_up(ocrdec_model* m, void* stream, int n_rounds, int* expert_sets_per_launch) {
  if (!m || n_rounds < 0) return fail(OCRDEC_EINVAL, "bad replay arguments");
  if (m->last_verify_rows < 1) return fail(OCRDEC_EINVAL, "no verify call to replay");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (expert_sets_per_launch) {
    int na = 0;
    if (hipStreamSynchronize(s) != hipSuccess ||
        hipMemcpy(&na, m->mb.n_act, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess)
      return fail(OCRDEC_EHIP, "reading the active-expert count failed");
    *expert_sets_per_launch = na;
  }
  const int M = m->last_verify_rows;
  for (int r = 0; r < n_rounds; ++r) {
    for (int l = 0; l < m->cfg.n_layers; ++l) {
      if (m->cfg.dtype == OCRDEC_BF16) expert_gate_up<bf16>(m, s, l, M, nullptr, decode_path<bf16>(m).experts);
      else expert_gate_up<float>(m, s, l, M, nullptr, false);
    }
  }
  return hip_check("ocrdec_replay_expert_gate_up");
}

int ocrdec_read_probe(void* stream, const void* buf, size_t bytes, int n_regions, int n_launches, uint32_t* sink) {
  if (!buf || !sink || bytes < 16 || bytes % 256 != 0 || n_regions < 1 || n_launches < 0)
    return fail(OCRDEC_EINVAL, "bad read-probe arguments");
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int i = 0; i < n_launches; ++i)
    launch_read_probe(s, static_cast<const char*>(buf) + (size_t)(i % n_regions) * bytes, (long)(bytes / 16), sink);
  return hip_check("ocrdec_read_probe");
}

int ocrdec_decode_steps(ocrdec_model* m, void* stream, int B, const int32_t* slots, int K, int n_steps,
                        const ocrdec_controlled_cfg* ctrl, int32_t* draft, int32_t* greedy,
                        int32_t* n_accepted_out, int32_t* out_tokens, int32_t* out_len, int out_cap) {
  int rc = check_call(m, B, K);
  if (rc) return rc;
  if (n_steps < 0 || !greedy || (K > 0 && !draft)) return fail(OCRDEC_EINVAL, "bad decode-step arguments");
  if (out_tokens && out_cap < 1) return fail(OCRDEC_EINVAL, "out_cap must be >= 1 with out_tokens");
  if (ctrl && (!ctrl->trace || ctrl->trace_len < 0 || ctrl->trace_stride < ctrl->trace_len))
    return fail(OCRDEC_EINVAL, "bad controlled-draft arguments");
  if (m->timing) return fail(OCRDEC_EINVAL, "expert timing is on; use the individual calls");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!m->capture_stream && hipStreamCreateWithFlags(&m->capture_stream, hipStreamNonBlocking) != hipSuccess)
    return fail(OCRDEC_EHIP, "creating the capture stream failed");
  for (int step = 0; step < n_steps; ++step) {
    const int bound = call_bound(m, B, slots);
    if (!slots && bound + K + 1 > m->cfg.max_positions)
      return fail(OCRDEC_ECAPACITY, "positions would exceed max_positions");
    const int nch = chunks_for(m, std::min(m->cfg.max_positions - 1, bound + K));
    std::vector<uintptr_t> key = {(uintptr_t)B, (uintptr_t)K, (uintptr_t)nch, (uintptr_t)slots,
                                  (uintptr_t)draft, (uintptr_t)greedy, (uintptr_t)n_accepted_out,
                                  (uintptr_t)out_tokens, (uintptr_t)out_len, (uintptr_t)out_cap,
                                  (uintptr_t)m->tap_route, (uintptr_t)m->tap_hidden};
    if (ctrl) {
      key.push_back((uintptr_t)ctrl->trace);
      key.push_back((uintptr_t)ctrl->trace_stride);
      key.push_back((uintptr_t)ctrl->trace_len);
      key.push_back((uintptr_t)ctrl->seed);
      key.push_back((uintptr_t)ctrl->threshold);
    }
    auto it = m->graphs.find(key);
    if (it == m->graphs.end()) {
      if (m->graphs.size() >= 256) {
        for (auto& kv : m->graphs) (void)hipGraphExecDestroy(kv.second);
        m->graphs.clear();
      }
      hipStream_t cs = m->capture_stream;
      if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess)
        return fail(OCRDEC_EHIP, "hipStreamBeginCapture failed");
      int r1 = OCRDEC_OK;
      if (K > 0)
        r1 = m->cfg.dtype == OCRDEC_BF16 ? do_draft<bf16>(m, cs, B, slots, K, draft)
                                         : do_draft<float>(m, cs, B, slots, K, draft);
      if (r1 == OCRDEC_OK && ctrl && K > 0)
        launch_controlled(cs, B, K, slots, m->sv, ctrl->trace, ctrl->trace_stride, ctrl->trace_len, ctrl->seed,
                          ctrl->threshold, m->cfg.vocab, draft);
      // the verify's argmax stage 2 runs inside the accept launch
      if (r1 == OCRDEC_OK)
        r1 = m->cfg.dtype == OCRDEC_BF16 ? do_verify<bf16>(m, cs, B, slots, K, draft, greedy, nullptr, true)
                                         : do_verify<float>(m, cs, B, slots, K, draft, greedy, nullptr, true);
      if (r1 == OCRDEC_OK)
        launch_accept(cs, B, K, m->plan_slot, draft, greedy, m->x, m->sv, n_accepted_out, out_tokens, out_len,
                      out_cap, m->lm_val, m->lm_idx, lmhead_blocks(m->cfg.vocab), greedy);
      hipGraph_t graph = nullptr;
      const hipError_t ec = hipStreamEndCapture(cs, &graph);
      if (r1 != OCRDEC_OK || ec != hipSuccess) {
        if (graph) (void)hipGraphDestroy(graph);
        return r1 != OCRDEC_OK ? r1 : fail(OCRDEC_EHIP, std::string("hipStreamEndCapture: ") + hipGetErrorString(ec));
      }
      hipGraphExec_t exec = nullptr;
      const hipError_t ei = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
      (void)hipGraphDestroy(graph);
      if (ei != hipSuccess) return fail(OCRDEC_EHIP, std::string("hipGraphInstantiate: ") + hipGetErrorString(ei));
      it = m->graphs.emplace(key, exec).first;
    }
    const hipError_t el = hipGraphLaunch(it->second, s);
    if (el != hipSuccess) return fail(OCRDEC_EHIP, std::string("hipGraphLaunch: ") + hipGetErrorString(el));
    const int n = slots ? (int)m->slot_bound.size() : B;
    for (int i = 0; i < n; ++i) m->slot_bound[i] = std::min(m->cfg.max_positions, m->slot_bound[i] + K + 1);
    m->last_verify_rows = B * (K + 1);
  }
  return OCRDEC_OK;
}

int ocrdec_sync_positions(ocrdec_model* m, void* stream) {
  if (!m) return fail(OCRDEC_EINVAL, "model is null");
  const int n = m->cfg.max_batch;
  std::vector<int> kv(n);
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess ||
      hipMemcpy(kv.data(), m->sv.kv_len, (size_t)n * sizeof(int), hipMemcpyDeviceToHost) != hipSuccess)
    return fail(OCRDEC_EHIP, "reading the cache lengths failed");
  for (int i = 0; i < n; ++i) m->slot_bound[i] = std::max(0, std::min(kv[i], m->cfg.max_positions));
  return OCRDEC_OK;
}

int ocrdec_set_router_logits(ocrdec_model* m, const float* logits) {
  if (!m) return fail(OCRDEC_EINVAL, "model is null");
  m->router_override = logits;
  return OCRDEC_OK;
}

int ocrdec_load_sequence(ocrdec_model* m, void* stream, int slot, int n_pos, int pending_token, const void* kv) {
  (void)hipGetLastError();
  if (!m || !kv) return fail(OCRDEC_EINVAL, "model or kv is null");
  if (slot < 0 || slot >= m->cfg.max_batch) return fail(OCRDEC_EINVAL, "slot out of range");
  if (n_pos < 1 || n_pos + m->cfg.max_k + 1 > m->cfg.max_positions)
    return fail(OCRDEC_ECAPACITY, "n_pos + max_k + 1 exceeds max_positions");
  if (pending_token < 0 || pending_token >= m->cfg.vocab) return fail(OCRDEC_EINVAL, "pending_token out of range");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t esz = m->p.esz, mp = (size_t)m->cfg.max_positions;
  const char* src = static_cast<const char*>(kv);
  for (int l = 0; l < m->cfg.n_layers; ++l) {
    char* dst = m->state + m->p.s_kv + ((size_t)l * m->p.kv_layer_elems + (size_t)slot * 2 * NH * mp * HD) * esz;
    // [K|V][head] planes: n_pos rows of HD in the source, max_positions rows in the cache
    for (int j = 0; j < 2 * NH; ++j) {
      const hipError_t e = hipMemcpyAsync(dst + (size_t)j * mp * HD * esz,
                                          src + (((size_t)l * 2 * NH + j) * n_pos) * HD * esz,
                                          (size_t)n_pos * HD * esz, hipMemcpyDeviceToDevice, s);
      if (e != hipSuccess) return fail(OCRDEC_EHIP, std::string("hipMemcpyAsync: ") + hipGetErrorString(e));
    }
  }
  launch_set_sequence(s, slot, n_pos, pending_token, m->sv);
  m->slot_bound[slot] = n_pos;
  return hip_check("ocrdec_load_sequence");
}

int ocrdec_set_taps(ocrdec_model* m, int32_t* route_idx, float* hidden) {
  if (!m) return fail(OCRDEC_EINVAL, "model is null");
  m->tap_route = route_idx;
  m->tap_hidden = hidden;
  return OCRDEC_OK;
}

int ocrdec_expert_timing(ocrdec_model* m, int enable) {
  if (!m) return fail(OCRDEC_EINVAL, "model is null");
  m->timing = enable != 0;
  m->ev_used = 0;
  m->stats_base = 0;
  if (hipDeviceSynchronize() != hipSuccess ||
      hipMemcpy(&m->stats_base, m->mb.stats, sizeof(long long), hipMemcpyDeviceToHost) != hipSuccess)
    return fail(OCRDEC_EHIP, "reading the expert counter failed");
  return OCRDEC_OK;
}

int ocrdec_expert_stats(ocrdec_model* m, double* ms_gate_up, long long* n_gate_up, double* ms_down, long long* n_down,
                        long long* expert_sets) {
  if (!m) return fail(OCRDEC_EINVAL, "model is null");
  double a = 0, b = 0;
  long long na = 0, nb = 0;
  const size_t n = (m->ev_used / 3) * 3;
  if (n > 0 && hipEventSynchronize(m->ev[n - 1]) != hipSuccess) return fail(OCRDEC_EHIP, "hipEventSynchronize failed");
  for (size_t i = 0; i + 2 < n; i += 3) {
    float t1 = 0, t2 = 0;
    if (hipEventElapsedTime(&t1, m->ev[i], m->ev[i + 1]) != hipSuccess ||
        hipEventElapsedTime(&t2, m->ev[i + 1], m->ev[i + 2]) != hipSuccess)
      return fail(OCRDEC_EHIP, "hipEventElapsedTime failed");
    a += t1;
    b += t2;
    ++na;
    ++nb;
  }
  long long sets = 0;
  if (hipMemcpy(&sets, m->mb.stats, sizeof(long long), hipMemcpyDeviceToHost) != hipSuccess)
    return fail(OCRDEC_EHIP, "hipMemcpy of the expert counter failed");
  if (ms_gate_up) *ms_gate_up = a;
  if (n_gate_up) *n_gate_up = na;
  if (ms_down) *ms_down = b;
  if (n_down) *n_down = nb;
  if (expert_sets) *expert_sets = sets - m->stats_base;
  return OCRDEC_OK;
}

}  // extern "C"
