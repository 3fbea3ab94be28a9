// Host side of the ocrdec C ABI: buffer layout inside the caller's state and
// workspace, argument checks, and the launch sequence of each call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <type_traits>
#include <unordered_map>
#include <vector>

#include "launch.h"
#include "ocrdec.h"
#include "ocrdec_harness.h"

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
  int max_blocks, n_pages, M_max, prefill_group, cu_stride, tiles_per_chunk, chunk_keys, n_chunks_cap, lm_nblk, plan_n;
  size_t esz, kv_layer_elems;
  // state
  size_t s_kv, s_dkv, s_table, s_ints, s_cu, s_hbuf, s_rope, s_total;
  // workspace
  size_t w_x, w_rscale, w_q, w_attn, w_part, w_bnorm, w_ridx, w_rgate, w_perm, w_inv, w_off, w_act, w_slot, w_items, w_rlogit, w_misc, w_stats, w_sync, w_hx,
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
  if (c->kv_pages < 0) { *why = "kv_pages must be >= 0 (0: one page per 64 positions of every slot)"; return false; }
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

// decode_only: the scratch of decode calls alone (draft, verify, accept) of up
// to max_batch sequences at depth max_k, without the prefill's buffers.
Plan make_plan(const ocrdec_config* c, bool decode_only = false) {
  Plan p{};
  // prefill passes take up to prefill_group entries of PREFILL_CHUNK rows
  p.prefill_group = decode_only ? 0 : PREFILL_GROUP;
  p.M_max = std::max(c->max_batch * (c->max_k + 1), PREFILL_CHUNK * p.prefill_group);
  p.plan_n = std::max(c->max_batch, p.prefill_group);
  p.cu_stride = c->max_k + 1;
  p.tiles_per_chunk = c->max_positions > 4096 ? 4 : 1;
  p.chunk_keys = p.tiles_per_chunk * ATT_TILE;
  p.n_chunks_cap = (c->max_positions + p.chunk_keys - 1) / p.chunk_keys;
  p.lm_nblk = lmhead_blocks(c->vocab);
  p.esz = c->dtype == OCRDEC_BF16 ? 2 : 4;
  // KV pages: KV_PAGE positions of one sequence each, for every head, keys
  // and values; one table row of max_blocks pages per slot
  p.max_blocks = (c->max_positions + KV_PAGE - 1) / KV_PAGE;
  p.n_pages = c->kv_pages > 0 ? std::min(c->kv_pages, c->max_batch * p.max_blocks) : c->max_batch * p.max_blocks;
  p.kv_layer_elems = (size_t)p.n_pages * 2 * NH * KV_PAGE * HD;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = align256(o + bytes); return r; };
  p.s_kv = take(p.kv_layer_elems * c->n_layers * p.esz);
  p.s_dkv = take(p.kv_layer_elems * p.esz);
  p.s_table = take((size_t)c->max_batch * p.max_blocks * 4);
  p.s_ints = take((size_t)8 * c->max_batch * 4);
  p.s_cu = take((size_t)c->max_batch * p.cu_stride * 4);
  p.s_hbuf = take((size_t)c->max_batch * p.cu_stride * D * 4);
  p.s_rope = take((size_t)c->max_positions * (HD / 2) * 8);
  p.s_total = o;
  o = 0;
  const size_t M = p.M_max;
  p.w_x = take(M * D * 4);
  p.w_rscale = take(M * 4);
  p.w_q = take(M * QD * 4);
  p.w_attn = take(M * QD * 4);
  // split-KV partials of the decode calls, or of a prefill pass's key splits
  p.w_part = take(std::max((size_t)c->max_batch * (c->max_k + 1) * NH * (size_t)p.n_chunks_cap,
                           (size_t)p.prefill_group * NH * PF_SPLITS * PREFILL_CHUNK) *
                  (HD + 2) * 4);
  p.w_bnorm = take(M * D * 4);
  p.w_ridx = take(M * NSLOT * 4);
  p.w_rgate = take(M * NSLOT * 4);
  p.w_perm = take(M * NSLOT * 4);
  p.w_inv = take(M * NSLOT * 4);
  p.w_off = take((NX + 1) * 4);
  p.w_act = take(NX * 4);
  p.w_slot = take(NX * 16);
  p.w_items = take((size_t)expert_item_cap(p.M_max) * 16);
  p.w_rlogit = take(M * NE * 4);
  p.w_misc = take(64 * 4);       // [0] n_act, [16..] prefill tokens
  p.w_stats = take(8 * 8);
  static_assert(ROUTE_CNT_WORD < MOE_SYNC_WORDS, "the down-combine and routing counters share the MoE sync words");
  p.w_sync = take((size_t)MOE_SYNC_WORDS * 4);
  p.w_hx = take(M * NSLOT * DI * 4);
  p.w_y = take(M * NSLOT * D * 4);
  p.w_cat = take(M * 2 * D * 4);
  p.w_u = take(M * D * 4);
  p.w_u2 = take((size_t)c->max_batch * D * 4);  // second output buffer of the recursive draft passes
  p.w_dffn = take(M * DF * 4);
  p.w_esave = take(decode_only ? 0 : M * D * 4);
  p.w_hsave = take(decode_only ? 0 : (size_t)2 * c->max_batch * D * 4);
  p.w_lmv = take(M * (size_t)p.lm_nblk * 4);
  p.w_lmi = take(M * (size_t)p.lm_nblk * 4);
  p.w_plan = take((size_t)3 * p.plan_n * 4);
  p.w_total = o;
  return p;
}

// The per-call scratch buffers of the decode calls, laid out by a Plan inside
// one region (the caller's workspace, or the library's no-allocation scratch).
struct WsPtrs {
  float *x, *rscale, *q, *attn, *part, *cat, *u, *u2, *dffn, *esave, *hsave[2], *lm_val;
  int *lm_idx, *plan_base, *plan_cnt, *plan_slot, *tok_tmp;
  unsigned* sync;   // the persistent MoE launch's counters (zero between launches)
  MoeBufs mb;
};

// Scratch of ocrdec_decode_steps_noalloc: a file-scope device array, one copy
// per GPU the library runs on, held until the process ends.  Host code uses
// the device address returned by hipGetSymbolAddress (kept per device at
// handle creation), never the array's name.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::vector<char*> g_scratch_ptr;     // by device ordinal
std::vector<std::string> g_scratch_err;

// The scratch address on device `dev` (the current device), looked up once.
char* scratch_for_device(int dev, std::string* why) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (dev < 0) { *why = "no current device"; return nullptr; }
  if ((size_t)dev >= g_scratch_ptr.size()) {
    g_scratch_ptr.resize(dev + 1, nullptr);
    g_scratch_err.resize(dev + 1);
  }
  if (g_scratch_ptr[dev] == nullptr && g_scratch_err[dev].empty()) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      g_scratch_err[dev] = std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e);
    } else {
      g_scratch_ptr[dev] = static_cast<char*>(ptr);
    }
  }
  *why = g_scratch_err[dev];
  return g_scratch_ptr[dev];
}

WsPtrs bind_workspace(char* ws, const Plan& p, int max_batch) {
  WsPtrs b{};
  auto wf = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  auto wi = [&](size_t off) { return reinterpret_cast<int*>(ws + off); };
  b.x = wf(p.w_x);
  b.rscale = wf(p.w_rscale);
  b.q = wf(p.w_q);
  b.attn = wf(p.w_attn);
  b.part = wf(p.w_part);
  b.cat = wf(p.w_cat);
  b.u = wf(p.w_u);
  b.u2 = wf(p.w_u2);
  b.dffn = wf(p.w_dffn);
  b.esave = wf(p.w_esave);
  b.hsave[0] = wf(p.w_hsave);
  b.hsave[1] = wf(p.w_hsave) + (size_t)max_batch * D;
  b.lm_val = wf(p.w_lmv);
  b.lm_idx = wi(p.w_lmi);
  b.plan_base = wi(p.w_plan);
  b.plan_cnt = wi(p.w_plan) + p.plan_n;
  b.plan_slot = wi(p.w_plan) + 2 * p.plan_n;
  int* misc = wi(p.w_misc);
  b.mb.n_act = misc;
  b.tok_tmp = misc + 16;
  b.mb.bnorm = wf(p.w_bnorm);
  b.mb.ridx = wi(p.w_ridx);
  b.mb.rgate = wf(p.w_rgate);
  b.mb.perm = wi(p.w_perm);
  b.mb.inv = wi(p.w_inv);
  b.mb.off = wi(p.w_off);
  b.mb.act = wi(p.w_act);
  b.mb.slot_info = reinterpret_cast<int4*>(ws + p.w_slot);
  b.mb.items = reinterpret_cast<int4*>(ws + p.w_items);
  b.mb.rlogit = wf(p.w_rlogit);
  b.mb.stats = reinterpret_cast<long long*>(ws + p.w_stats);
  b.sync = reinterpret_cast<unsigned*>(ws + p.w_sync);
  b.mb.hx = wf(p.w_hx);
  b.mb.y = wf(p.w_y);
  return b;
}

}  // namespace

struct ocrdec_model {
  ocrdec_config cfg;
  Plan p;
  std::vector<const void*> w;
  char* state;
  char* ws;
  StateView sv;
  WsPtrs b;                    // per-call scratch inside the workspace (or the no-allocation scratch)
  const float2* rope;
  // Host-side upper bound on (last position + 1) of every slot: set by prefill,
  // raised by K + 1 per accept.  It sizes the attention grids and the capacity
  // checks; the device clamps positions to the cache in any case.
  std::vector<int> slot_bound;
  ocrdec_taps taps;            // parity harness taps (all null when unused)
  StepTap step_tap;
  const char* launch_fail;     // set when a launcher met an unsupported shape (checked by hip_check)
  // the last verify call (for the accept that must follow it): rows per
  // sequence, sequences and slot map; B = 0 once an accept has consumed it
  int lv_B, lv_K;
  const int32_t* lv_slots;
  bool timing;
  std::vector<hipEvent_t> ev;  // triplets: before gate/up, between, after down
  size_t ev_used;
  long long stats_base;        // device expert counter when timing was enabled
  int last_verify_rows;        // M of the last verify call (0 before any)
  bool matrix;                 // experts and LM head on the matrix cores
  const float* router_override;  // [n_layers][M][64] router logits for verify calls, or null
  hipStream_t capture_stream;  // private stream the decode-step graphs are recorded on
  std::map<std::vector<uintptr_t>, hipGraphExec_t> graphs;  // by call shape
  char* scratch;               // this device's no-allocation scratch (null if unavailable)
  std::string scratch_err;
  int moe_grid;                // workgroups of the persistent MoE launch (0: not available)
  bool fused_moe;              // vector-path MoE halves in one persistent launch (else five launches)
  // KV page pool: free pages (a stack) and each slot's pages by block
  std::vector<int> free_pages;
  std::vector<std::vector<int>> slot_pages;
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

int hip_check(ocrdec_model* m, const char* where) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(OCRDEC_EHIP, std::string(where) + ": " + hipGetErrorString(e));
  if (m != nullptr && m->launch_fail != nullptr) {
    const char* what = m->launch_fail;
    m->launch_fail = nullptr;
    return fail(OCRDEC_EINVAL, std::string(where) + ": unsupported launch shape (" + what + ")");
  }
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

// ---- KV page pool --------------------------------------------------------
// A slot holds pages for its blocks 0 .. n-1 (positions 0 .. 64 n - 1); pages
// come from a free stack and return to it when the slot is released or
// prefilled anew.  Table updates are queued and written by small kernels on
// the call's stream before its work.
struct PageUpdates {
  std::vector<std::pair<int, int>> v;  // (table index, page)
};

int pages_for(const ocrdec_model* m, int n_pos) {
  return (std::min(n_pos, m->cfg.max_positions) + KV_PAGE - 1) / KV_PAGE;
}

void flush_pages(ocrdec_model* m, hipStream_t s, PageUpdates& u) {
  // an entry updated twice (a slot released, then given pages again) keeps
  // its last value: one launch writes each entry once, since its threads
  // store in no set order
  std::vector<std::pair<int, int>> last;
  std::unordered_map<int, size_t> at;
  last.reserve(u.v.size());
  for (const auto& e : u.v) {
    auto it = at.find(e.first);
    if (it != at.end()) {
      last[it->second].second = e.second;
    } else {
      at.emplace(e.first, last.size());
      last.push_back(e);
    }
  }
  int* table = reinterpret_cast<int*>(m->state + m->p.s_table);
  for (size_t i = 0; i < last.size(); i += PAGESET_N) {
    PageSet ps{};
    ps.n = (int)std::min<size_t>(PAGESET_N, last.size() - i);
    for (int j = 0; j < ps.n; ++j) {
      ps.idx[j] = last[i + j].first;
      ps.page[j] = last[i + j].second;
    }
    launch_set_pages(s, table, ps);
  }
  u.v.clear();
}

void release_pages(ocrdec_model* m, int slot, PageUpdates& u) {
  std::vector<int>& own = m->slot_pages[slot];
  for (size_t j = 0; j < own.size(); ++j) {
    m->free_pages.push_back(own[j]);
    u.v.emplace_back(slot * m->p.max_blocks + (int)j, -1);
  }
  own.clear();
}

// Pages for positions 0 .. n_pos - 1 of slot; false (nothing taken) if the
// pool cannot supply them.
bool grow_pages(ocrdec_model* m, int slot, int n_pos, PageUpdates& u) {
  std::vector<int>& own = m->slot_pages[slot];
  const int need = pages_for(m, n_pos);
  if (need <= (int)own.size()) return true;
  if ((size_t)(need - (int)own.size()) > m->free_pages.size()) return false;
  while ((int)own.size() < need) {
    const int pg = m->free_pages.back();
    m->free_pages.pop_back();
    u.v.emplace_back(slot * m->p.max_blocks + (int)own.size(), pg);
    own.push_back(pg);
  }
  return true;
}

// Every slot a decode call may touch (0 .. B-1, or every slot that holds
// pages when the call maps slots on the device) gets pages through its bound
// + extra positions; if the pool cannot supply all of them, nothing is taken.
int ensure_pages(ocrdec_model* m, hipStream_t s, int B, const int32_t* slots, int extra) {
  const int n = slots ? m->cfg.max_batch : B;
  long need = 0;
  for (int i = 0; i < n; ++i) {
    if (slots && m->slot_pages[i].empty()) continue;
    need += std::max(0, pages_for(m, m->slot_bound[i] + extra) - (int)m->slot_pages[i].size());
  }
  if (need == 0) return OCRDEC_OK;
  if (need > (long)m->free_pages.size())
    return fail(OCRDEC_ECAPACITY, "KV page pool exhausted: the call needs " + std::to_string(need) + " more pages, " +
                                      std::to_string(m->free_pages.size()) +
                                      " are free (release finished slots with ocrdec_release_slot)");
  PageUpdates u;
  for (int i = 0; i < n; ++i)
    if (!(slots && m->slot_pages[i].empty())) grow_pages(m, i, m->slot_bound[i] + extra, u);
  flush_pages(m, s, u);
  return OCRDEC_OK;
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
  bool prefill;  // prefix entries: the prefill attention
};

template <typename T>
PassPath decode_path(const ocrdec_model* m) {
  const bool mx = std::is_same<T, bf16>::value && m->matrix;
  return PassPath{mx, mx ? DENSE_KSPLIT : DENSE_VECTOR, false};
}

template <typename T>
PassPath prefill_path(const ocrdec_model* m) {
  (void)m;
  const bool bf = std::is_same<T, bf16>::value;
  return PassPath{bf, bf ? DENSE_STRIP : DENSE_VECTOR, true};
}

template <typename T>
void expert_gate_up(ocrdec_model* m, hipStream_t s, int l, int M, bool mx, bool deep = false) {
  if constexpr (std::is_same<T, bf16>::value) {
    if (mx) {
      launch_expert_gate_up_mfma(s, wmat<T>(m, lw(m, l, L_GATE)), wmat<T>(m, lw(m, l, L_UP)), M, m->b.mb, deep);
      return;
    }
  }
  launch_expert_gate_up<T>(s, wmat<T>(m, lw(m, l, L_GATE)), wmat<T>(m, lw(m, l, L_UP)), M, m->b.mb);
}

template <typename T>
void expert_down(ocrdec_model* m, hipStream_t s, int l, int M, bool mx, bool deep = false) {
  if constexpr (std::is_same<T, bf16>::value) {
    if (mx) {
      launch_expert_down_mfma(s, wmat<T>(m, lw(m, l, L_DOWN)), M, m->b.mb, deep);
      return;
    }
  }
  launch_expert_down<T>(s, wmat<T>(m, lw(m, l, L_DOWN)), M, m->b.mb);
}

// LM head + argmax over M output rows (see launch_lmhead).
template <typename T>
void lm_head(ocrdec_model* m, hipStream_t s, const float* x, int Q, bool last_valid, const float* gain, int M,
             float* logits, int* tok, int tok_stride) {
  const ocrdec_config& c = m->cfg;
  if constexpr (std::is_same<T, bf16>::value) {
    if (m->matrix) {
      launch_lmhead_mfma(s, x, m->b.plan_cnt, Q, last_valid, gain, c.norm_eps, wmat<T>(m, W_LM), c.vocab, M,
                         m->b.mb.bnorm, m->b.lm_val, m->b.lm_idx, logits, tok, tok_stride);
      return;
    }
  }
  launch_lmhead<T>(s, x, m->b.plan_cnt, Q, last_valid, gain, c.norm_eps, wmat<T>(m, W_LM), c.vocab, M, m->b.lm_val,
                   m->b.lm_idx, logits, tok, tok_stride);
}

// Dense layers on the path dp (DensePath).
template <typename T>
void dense_gemv(ocrdec_model* m, hipStream_t s, int dp, int K, Epi epi, const float* a, long lda,
                const float* gain, const T* W0, const T* W1, int N, int M, float* out, long ldo) {
  if constexpr (std::is_same<T, bf16>::value) {
    if (dp == DENSE_STRIP) {
      if (!launch_gemv_mfma(s, K, epi, a, lda, gain, m->cfg.norm_eps, W0, W1, N, M, out, ldo, m->b.rscale))
        m->launch_fail = "matrix-core dense layer: no kernel for this (K, epilogue)";
      return;
    }
    if (dp == DENSE_KSPLIT) {
      if (!launch_gemv_ks(s, K, epi, a, lda, gain, m->cfg.norm_eps, W0, W1, N, M, out, ldo))
        m->launch_fail = "k-split dense layer: no kernel for this (K, epilogue)";
      return;
    }
  }
  launch_gemv<T>(s, K, epi, a, lda, gain, m->cfg.norm_eps, W0, W1, N, M, out, ldo);
}

// The paged KV cache of verifier layer l (l < 0: the draft block's).
template <typename T>
KvView<T> kv_view(const ocrdec_model* m, int l) {
  char* base = m->state + (l < 0 ? m->p.s_dkv : m->p.s_kv + (size_t)l * m->p.kv_layer_elems * m->p.esz);
  return KvView<T>{reinterpret_cast<T*>(base), reinterpret_cast<const int*>(m->state + m->p.s_table),
                   m->p.max_blocks, m->cfg.max_positions};
}

template <typename T>
void dense_qkv(ocrdec_model* m, hipStream_t s, int dp, const float* x, const float* gain, const T* W, int M,
               RowPlan plan, KvView<T> kv) {
  if constexpr (std::is_same<T, bf16>::value) {
    if (dp == DENSE_STRIP) {
      launch_qkv_rope_mfma(s, x, gain, m->cfg.norm_eps, W, M, plan, m->b.q, kv, m->rope, m->b.rscale);
      return;
    }
    if (dp == DENSE_KSPLIT) {
      launch_qkv_rope_ks(s, x, gain, m->cfg.norm_eps, W, M, plan, m->b.q, kv, m->rope);
      return;
    }
  }
  launch_qkv_rope<T>(s, x, gain, m->cfg.norm_eps, W, M, plan, m->b.q, kv, m->rope);
}

// The rest of the MoE half of layer l (vector path, M <= 8), after the router
// logits, in one persistent launch: x_out = x + MoE(x), x = the layer's
// residual rows.
template <typename T>
void moe_experts(ocrdec_model* m, hipStream_t s, int l, int M, const RouteTap& tap, float* x_out) {
  launch_moe_experts<T>(s, m->moe_grid, m->b.x, x_out, wmat<T>(m, lw(m, l, L_GATE)), wmat<T>(m, lw(m, l, L_UP)),
                        wmat<T>(m, lw(m, l, L_DOWN)), M, m->b.mb, tap, m->b.sync);
}

// Attention of the pass's rows into b.attn: the prefill attention for prefix
// entries, else split-KV decode attention.
template <typename T>
void attention(ocrdec_model* m, hipStream_t s, PassPath pp, const float* q, KvView<T> kv, RowPlan plan, int B,
               int nch) {
  if (pp.prefill) {
    launch_attention_prefill<T>(s, q, kv, plan, B, m->b.part, m->b.attn);
    return;
  }
  launch_attention<T>(s, q, kv, plan, B, nch, m->p.tiles_per_chunk, m->b.part, m->b.attn);
}

template <typename T>
void verifier_layers(ocrdec_model* m, hipStream_t s, PassPath pp, int M, int B, RowPlan plan, int nch, bool taps,
                     const float* rlog) {
  const ocrdec_config& c = m->cfg;
  for (int l = 0; l < c.n_layers; ++l) {
    const KvView<T> kvl = kv_view<T>(m, l);
    dense_qkv<T>(m, s, pp.dense, m->b.x, wvec(m, lw(m, l, L_ANORM)), wmat<T>(m, lw(m, l, L_QKV)), M, plan, kvl);
    attention<T>(m, s, pp, m->b.q, kvl, plan, B, nch);
    dense_gemv<T>(m, s, pp.dense, QD, EPI_ADD, m->b.attn, QD, nullptr, wmat<T>(m, lw(m, l, L_WO)), nullptr, D, M,
                  m->b.x, D);
    RouteTap tap{};
    tap.call = (taps && m->taps.route_idx) ? m->taps.route_idx + (size_t)l * M * NSLOT : nullptr;
    if (m->taps.route_pos != nullptr) {
      tap.pos = m->taps.route_pos + (size_t)l * m->taps.route_pos_cap * NSLOT;
      tap.pos_slot = m->taps.route_pos_slot;
      tap.pos_cap = m->taps.route_pos_cap;
    }
    tap.plan = plan;
    if (!pp.experts && M <= MRG && m->fused_moe && m->moe_grid > 0) {
      launch_router_logits<T>(s, m->b.x, wvec(m, lw(m, l, L_FNORM)), c.norm_eps, wmat<T>(m, lw(m, l, L_ROUTER)),
                              M, m->b.mb, rlog ? rlog + (size_t)l * M * NE : nullptr);
      timing_mark(m, s);
      moe_experts<T>(m, s, l, M, tap, m->b.x);
      timing_mark(m, s);
      timing_mark(m, s);
      continue;
    }
    launch_router<T>(s, m->b.x, wvec(m, lw(m, l, L_FNORM)), c.norm_eps, wmat<T>(m, lw(m, l, L_ROUTER)), M, m->b.mb,
                     tap, rlog ? rlog + (size_t)l * M * NE : nullptr, m->b.sync + ROUTE_CNT_WORD);
    timing_mark(m, s);
    expert_gate_up<T>(m, s, l, M, pp.experts, pp.prefill);
    timing_mark(m, s);
    if (!pp.experts && M <= MRG) {  // the combine inside the down launch
      launch_expert_down_combine<T>(s, wmat<T>(m, lw(m, l, L_DOWN)), M, m->b.mb, m->b.x, m->b.sync);
      timing_mark(m, s);
      continue;
    }
    expert_down<T>(m, s, l, M, pp.experts, pp.prefill);
    timing_mark(m, s);
    launch_moe_combine(s, m->b.x, M, m->b.mb);
  }
}

// The draft block on rows u (M of them): the fusion projection of cat into
// u (skipped when a fused launch has already written u), attention, SwiGLU FFN.
template <typename T>
void draft_layer(ocrdec_model* m, hipStream_t s, PassPath pp, int M, int B, RowPlan plan, int nch, float* u,
                 bool fused_in) {
  const ocrdec_config& c = m->cfg;
  const int mx = pp.dense;
  const KvView<T> dkv = kv_view<T>(m, -1);
  if (!fused_in)
    dense_gemv<T>(m, s, mx, 2 * D, EPI_STORE, m->b.cat, 2 * D, nullptr, wmat<T>(m, dw(m, D_FUSE)), nullptr, D, M, u,
                  D);
  dense_qkv<T>(m, s, mx, u, wvec(m, dw(m, D_ANORM)), wmat<T>(m, dw(m, D_QKV)), M, plan, dkv);
  attention<T>(m, s, pp, m->b.q, dkv, plan, B, nch);
  dense_gemv<T>(m, s, mx, QD, EPI_ADD, m->b.attn, QD, nullptr, wmat<T>(m, dw(m, D_WO)), nullptr, D, M, u, D);
  dense_gemv<T>(m, s, mx, D, EPI_SWIGLU, u, D, wvec(m, dw(m, D_FNORM)), wmat<T>(m, dw(m, D_GATE)),
                wmat<T>(m, dw(m, D_UP)), DF, M, m->b.dffn, DF);
  dense_gemv<T>(m, s, mx, DF, EPI_ADD, m->b.dffn, DF, nullptr, wmat<T>(m, dw(m, D_DOWN)), nullptr, D, M, u, D);
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
    const float* hprev = m->b.hsave[t & 1];
    float* hnext = m->b.hsave[(t + 1) & 1];
    PrefillGroup g{};
    g.n = (int)std::min(ent.size() - e0, (size_t)m->p.prefill_group);
    int n_finish = 0;
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
      n_finish += (p0 + g.cnt[j] == P) ? 1 : 0;
      max_pos = std::max(max_pos, p0 + g.cnt[j] - 1);
    }
    launch_plan_prefill<T>(s, g, vision, nv_stride, prompt, np_stride, wmat<T>(m, W_EMBED), c.vocab, m->b.plan_base,
                           m->b.plan_cnt, m->b.plan_slot, m->b.x, m->b.esave);
    const int M = g.n * PREFILL_CHUNK;
    RowPlan plan{m->b.plan_base, m->b.plan_cnt, m->b.plan_slot, PREFILL_CHUNK, 0};
    const int nch = chunks_for(m, std::min(c.max_positions - 1, max_pos));
    verifier_layers<T>(m, s, prefill_path<T>(m), M, g.n, plan, nch, false, nullptr);
    if (n_finish > 0) {  // the LM head on each finishing sequence's last row only
      launch_prefill_last_rows(s, g, m->b.x, m->b.u);
      lm_head<T>(m, s, m->b.u, 1, false, wvec(m, W_FNORM), n_finish, nullptr, m->b.tok_tmp, 1);
    }
    launch_draft_prefill_cat(s, g, m->b.x, m->b.esave, hprev, hnext, wvec(m, dw(m, D_NH)), wvec(m, dw(m, D_NE)),
                             c.norm_eps, m->b.cat);
    draft_layer<T>(m, s, prefill_path<T>(m), M, g.n, plan, nch, m->b.u, false);
    if (n_finish > 0) launch_prefill_finish(s, g, m->b.x, m->b.tok_tmp, m->sv, pending_out);
  }
  for (int b = 0; b < B; ++b) m->slot_bound[slots_host ? slots_host[b] : b] = nv_host[b] + np_host[b];
  m->lv_B = 0;
  return hip_check(m, "ocrdec_prefill");
}

template <typename T>
int do_draft(ocrdec_model* m, hipStream_t s, int B, const int32_t* slots, int K, int32_t* draft_out) {
  const ocrdec_config& c = m->cfg;
  // The catch-up pass carries the rows accepted at the last verify plus the
  // pending token: up to (that verify's K) + 1 rows, so it is laid out for the
  // handle's deepest draft, max_k + 1 rows per sequence, and K may change from
  // one step to the next.
  const int Q = m->p.cu_stride;
  // same chunk count as the verify of this step (a decode-step graph is keyed on it)
  const int nch = chunks_for(m, std::min(c.max_positions - 1, call_bound(m, B, slots) + K));
  const PassPath pp = decode_path<T>(m);
  const int ident = slots == nullptr;
  const RowPlan plan{m->b.plan_base, m->b.plan_cnt, m->b.plan_slot, Q, ident};
  const RowPlan p1{m->b.plan_base, m->b.plan_cnt, m->b.plan_slot, 1, ident};
  if (pp.dense == DENSE_VECTOR) {
    // each pass's plan, input rows and fusion projection in one launch (pass j
    // >= 2 also takes d_{j-1} from the previous LM head's partials, so only the
    // last pass runs the argmax stage 2); passes alternate between two output
    // buffers since a pass reads the previous one's rows
    const int nblk = lmhead_blocks(c.vocab);
    const T* wf = wmat<T>(m, dw(m, D_FUSE));
    launch_draft_fuse<T>(s, 0, 1, Q, Q, K, slots, m->sv, wmat<T>(m, W_EMBED), c.vocab, wvec(m, dw(m, D_NH)),
                         wvec(m, dw(m, D_NE)), c.norm_eps, nullptr, nullptr, nullptr, nblk, draft_out, m->b.plan_base,
                         m->b.plan_cnt, m->b.plan_slot, wf, B * Q, m->b.u);
    draft_layer<T>(m, s, pp, B * Q, B, plan, nch, m->b.u, true);
    lm_head<T>(m, s, m->b.u, Q, true, wvec(m, dw(m, D_ONORM)), B, nullptr, K == 1 ? draft_out : nullptr, K);
    float* uprev = m->b.u;
    for (int j = 2; j <= K; ++j) {
      float* u = (uprev == m->b.u) ? m->b.u2 : m->b.u;
      launch_draft_fuse<T>(s, 1, j, Q, (j == 2) ? Q : 1, K, nullptr, m->sv, wmat<T>(m, W_EMBED), c.vocab,
                           wvec(m, dw(m, D_NH)), wvec(m, dw(m, D_NE)), c.norm_eps, uprev, m->b.lm_val, m->b.lm_idx, nblk,
                           draft_out, m->b.plan_base, m->b.plan_cnt, m->b.plan_slot, wf, B, u);
      draft_layer<T>(m, s, pp, B, B, p1, nch, u, true);
      lm_head<T>(m, s, u, 1, true, wvec(m, dw(m, D_ONORM)), B, nullptr, j == K ? draft_out + (j - 1) : nullptr, K);
      uprev = u;
    }
    if (m->step_tap.drafts != nullptr) launch_draft_tap(s, B, K, m->b.plan_slot, m->sv, draft_out, m->step_tap);
    return hip_check(m, "ocrdec_draft");
  }
  launch_plan_draft_catchup<T>(s, B, Q, slots, m->sv, wmat<T>(m, W_EMBED), c.vocab, wvec(m, dw(m, D_NH)),
                               wvec(m, dw(m, D_NE)), c.norm_eps, m->b.plan_base, m->b.plan_cnt, m->b.plan_slot, m->b.cat);
  draft_layer<T>(m, s, pp, B * Q, B, plan, nch, m->b.u, false);
  lm_head<T>(m, s, m->b.u, Q, true, wvec(m, dw(m, D_ONORM)), B, nullptr, draft_out, K);
  for (int j = 2; j <= K; ++j) {
    const int Qprev = (j == 2) ? Q : 1;
    launch_plan_draft_step<T>(s, B, j, Qprev, K, m->sv, draft_out, wmat<T>(m, W_EMBED), c.vocab,
                              wvec(m, dw(m, D_NH)), wvec(m, dw(m, D_NE)), c.norm_eps, m->b.u, m->b.plan_base, m->b.plan_cnt,
                              m->b.plan_slot, m->b.cat);
    draft_layer<T>(m, s, pp, B, B, p1, nch, m->b.u, false);
    lm_head<T>(m, s, m->b.u, 1, true, wvec(m, dw(m, D_ONORM)), B, nullptr, draft_out + (j - 1), K);
  }
  if (m->step_tap.drafts != nullptr) launch_draft_tap(s, B, K, m->b.plan_slot, m->sv, draft_out, m->step_tap);
  return hip_check(m, "ocrdec_draft");
}

template <typename T>
int do_verify(ocrdec_model* m, hipStream_t s, int B, const int32_t* slots, int K, const int32_t* draft,
              int32_t* greedy_out, float* logits_out, bool greedy_in_accept = false) {
  const ocrdec_config& c = m->cfg;
  const int Q = K + 1, M = B * Q;
  const int nch = chunks_for(m, std::min(c.max_positions - 1, call_bound(m, B, slots) + K));
  launch_plan_verify<T>(s, B, K, slots, m->sv, draft, wmat<T>(m, W_EMBED), c.vocab, m->b.plan_base, m->b.plan_cnt,
                        m->b.plan_slot, m->b.x);
  RowPlan plan{m->b.plan_base, m->b.plan_cnt, m->b.plan_slot, Q, slots == nullptr};
  verifier_layers<T>(m, s, decode_path<T>(m), M, B, plan, nch, true, m->router_override);
  m->last_verify_rows = M;
  // greedy_in_accept: the accept launch that follows reduces the greedy tokens
  lm_head<T>(m, s, m->b.x, Q, false, wvec(m, W_FNORM), M, logits_out, greedy_in_accept ? nullptr : greedy_out, 1);
  if (m->taps.hidden) launch_copy_rows(s, m->b.x, m->taps.hidden, (long)M * D);
  m->lv_B = B;
  m->lv_K = K;
  m->lv_slots = slots;
  return hip_check(m, "ocrdec_verify");
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
  m->sv.ovf = ints + 7 * mb;
  m->sv.max_pos = cfg->max_positions;
  m->sv.cu_tok = reinterpret_cast<int*>(m->state + p.s_cu);
  m->sv.cu_stride = p.cu_stride;
  m->sv.hbuf = reinterpret_cast<float*>(m->state + p.s_hbuf);
  m->sv.n_slots = mb;
  m->rope = reinterpret_cast<const float2*>(m->state + p.s_rope);
  m->b = bind_workspace(m->ws, p, mb);
  int* misc = m->b.mb.n_act;
  m->slot_bound.assign(cfg->max_batch, 0);
  m->slot_pages.assign(cfg->max_batch, {});
  m->free_pages.reserve(p.n_pages);
  m->free_pages.resize(p.n_pages);
  for (int i = 0; i < p.n_pages; ++i) m->free_pages[i] = p.n_pages - 1 - i;  // page 0 is taken first
  m->taps = ocrdec_taps{};
  m->step_tap = StepTap{};
  m->launch_fail = nullptr;
  m->lv_B = 0;
  m->lv_K = 0;
  m->lv_slots = nullptr;
  m->timing = false;
  m->ev_used = 0;
  m->stats_base = 0;
  m->last_verify_rows = 0;
  m->matrix = use_matrix_path(cfg);
  m->router_override = nullptr;
  m->capture_stream = nullptr;
  {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    m->scratch = scratch_for_device(dev, &m->scratch_err);
    int n_cu = 0;
    if (dev < 0 || hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n_cu = 0;
    m->moe_grid = n_cu > 0 ? (cfg->dtype == OCRDEC_BF16 ? moe_fused_grid<bf16>(n_cu) : moe_fused_grid<float>(n_cu)) : 0;
    if (m->moe_grid < NE / 4) m->moe_grid = 0;
    (void)hipGetLastError();
    m->fused_moe = false;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // clear an error left by earlier, unrelated runtime calls
  hipError_t err = hipMemsetAsync(misc, 0, 64 * 4, s);
  if (err == hipSuccess) err = hipMemsetAsync(m->b.mb.stats, 0, 64, s);
  if (err == hipSuccess) err = hipMemsetAsync(m->b.sync, 0, (size_t)MOE_SYNC_WORDS * 4, s);
  if (err == hipSuccess) err = hipMemsetAsync(m->state + p.s_ints, 0, p.s_hbuf - p.s_ints, s);
  if (err == hipSuccess)  // every table entry -1: no page
    err = hipMemsetAsync(m->state + p.s_table, 0xff, (size_t)cfg->max_batch * p.max_blocks * 4, s);
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
  {  // the slots' old pages go back to the pool, then pages for the prefixes
    long need = 0, have = (long)m->free_pages.size();
    for (int b = 0; b < B; ++b) {
      need += pages_for(m, n_vision_host[b] + n_prompt_host[b]);
      have += (long)m->slot_pages[slots_host ? slots_host[b] : b].size();
    }
    if (need > have)
      return fail(OCRDEC_ECAPACITY, "KV page pool exhausted: the prefixes need " + std::to_string(need) +
                                        " pages, " + std::to_string(have) + " are free or held by these slots");
    PageUpdates u;
    for (int b = 0; b < B; ++b) release_pages(m, slots_host ? slots_host[b] : b, u);
    for (int b = 0; b < B; ++b) {
      const int slot = slots_host ? slots_host[b] : b;
      m->slot_bound[slot] = 0;
      grow_pages(m, slot, n_vision_host[b] + n_prompt_host[b], u);
    }
    flush_pages(m, s, u);
  }
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
  if ((rc = ensure_pages(m, s, B, slots, K + 1)) != OCRDEC_OK) return rc;
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
  if ((rc = ensure_pages(m, s, B, slots, K + 1)) != OCRDEC_OK) return rc;
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
  if (m->lv_B == 0) return fail(OCRDEC_EINVAL, "ocrdec_accept_rollback must follow an ocrdec_verify call");
  if (B != m->lv_B || K != m->lv_K || slots != m->lv_slots)
    return fail(OCRDEC_EINVAL, "ocrdec_accept_rollback must take the B, K and slots of the verify it follows");
  hipStream_t s = static_cast<hipStream_t>(stream);
  launch_accept(s, B, K, m->b.plan_slot, draft, greedy, m->b.x, m->sv, n_accepted_out, out_tokens, out_len, out_cap,
                m->step_tap);
  m->lv_B = 0;
  const int n = slots ? (int)m->slot_bound.size() : B;
  for (int i = 0; i < n; ++i) m->slot_bound[i] = std::min(m->cfg.max_positions, m->slot_bound[i] + K + 1);
  return hip_check(m, "ocrdec_accept_rollback");
}

int ocrdec_controlled_drafts(ocrdec_model* m, void* stream, int B, const int32_t* slots, int K, const int32_t* trace,
                             int trace_stride, int trace_len, uint64_t seed, uint64_t threshold, int32_t* draft_inout) {
  int rc = check_call(m, B, K);
  if (rc) return rc;
  if (K < 1 || !trace || !draft_inout || trace_len < 0 || trace_stride < trace_len)
    return fail(OCRDEC_EINVAL, "bad controlled-draft arguments");
  hipStream_t s = static_cast<hipStream_t>(stream);
  launch_controlled(s, B, K, slots, m->sv, trace, trace_stride, trace_len, seed, threshold, m->cfg.vocab, draft_inout);
  return hip_check(m, "ocrdec_controlled_drafts");
}

int ocrdec_replay_expert_gate_up(ocrdec_model* m, void* stream, int n_rounds, int* expert_sets_per_launch) {
  if (!m || n_rounds < 0) return fail(OCRDEC_EINVAL, "bad replay arguments");
  if (m->last_verify_rows < 1) return fail(OCRDEC_EINVAL, "no verify call to replay");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (expert_sets_per_launch) {
    int na = 0;
    if (hipStreamSynchronize(s) != hipSuccess ||
        hipMemcpy(&na, m->b.mb.n_act, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess)
      return fail(OCRDEC_EHIP, "reading the active-expert count failed");
    *expert_sets_per_launch = na;
  }
  const int M = m->last_verify_rows;
  const bool fused = !m->matrix && M <= MRG && m->fused_moe && m->moe_grid > 0;
  for (int r = 0; r < n_rounds; ++r) {
    for (int l = 0; l < m->cfg.n_layers; ++l) {
      if (fused) {  // the persistent expert launch, its output to scratch (the residual rows stay as they are)
        const RouteTap none{};
        if (m->cfg.dtype == OCRDEC_BF16) moe_experts<bf16>(m, s, l, M, none, m->b.u);
        else moe_experts<float>(m, s, l, M, none, m->b.u);
        continue;
      }
      if (m->cfg.dtype == OCRDEC_BF16) expert_gate_up<bf16>(m, s, l, M, decode_path<bf16>(m).experts);
      else expert_gate_up<float>(m, s, l, M, false);
    }
  }
  return hip_check(m, "ocrdec_replay_expert_gate_up");
}

int ocrdec_read_probe(void* stream, const void* buf, size_t bytes, int n_regions, int n_launches, uint32_t* sink) {
  if (!buf || !sink || bytes < 16 || bytes % 256 != 0 || n_regions < 1 || n_launches < 0)
    return fail(OCRDEC_EINVAL, "bad read-probe arguments");
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int i = 0; i < n_launches; ++i)
    launch_read_probe(s, static_cast<const char*>(buf) + (size_t)(i % n_regions) * bytes, (long)(bytes / 16), sink);
  return hip_check(nullptr, "ocrdec_read_probe");
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
  // pages for every step of the call, before any of them runs
  if ((rc = ensure_pages(m, s, B, slots, std::min(n_steps, m->cfg.max_positions) * (K + 1))) != OCRDEC_OK) return rc;
  for (int step = 0; step < n_steps; ++step) {
    const int bound = call_bound(m, B, slots);
    if (!slots && bound + K + 1 > m->cfg.max_positions)
      return fail(OCRDEC_ECAPACITY, "positions would exceed max_positions");
    const int nch = chunks_for(m, std::min(m->cfg.max_positions - 1, bound + K));
    // everything a recorded step bakes in: the call's shape and pointers, the
    // router override and the taps
    std::vector<uintptr_t> key = {(uintptr_t)B, (uintptr_t)K, (uintptr_t)nch, (uintptr_t)slots,
                                  (uintptr_t)draft, (uintptr_t)greedy, (uintptr_t)n_accepted_out,
                                  (uintptr_t)out_tokens, (uintptr_t)out_len, (uintptr_t)out_cap,
                                  (uintptr_t)m->router_override, (uintptr_t)m->taps.route_idx,
                                  (uintptr_t)m->taps.hidden, (uintptr_t)m->taps.route_pos,
                                  (uintptr_t)m->taps.route_pos_slot, (uintptr_t)m->taps.route_pos_cap,
                                  (uintptr_t)m->step_tap.acc, (uintptr_t)m->step_tap.drafts,
                                  (uintptr_t)m->step_tap.cap, (uintptr_t)m->fused_moe};
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
        launch_accept(cs, B, K, m->b.plan_slot, draft, greedy, m->b.x, m->sv, n_accepted_out, out_tokens, out_len,
                      out_cap, m->step_tap, m->b.lm_val, m->b.lm_idx, lmhead_blocks(m->cfg.vocab), greedy);
      m->lv_B = 0;
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

int ocrdec_decode_steps_noalloc(ocrdec_model* m, void* stream, int B, const int32_t* slots, int K, int n_steps,
                                int32_t* draft, int32_t* greedy, int32_t* n_accepted_out, int32_t* out_tokens,
                                int32_t* out_len, int out_cap) {
  int rc = check_call(m, B, K);
  if (rc) return rc;
  if (n_steps < 0 || !greedy || (K > 0 && !draft)) return fail(OCRDEC_EINVAL, "bad decode-step arguments");
  if (out_tokens && out_cap < 1) return fail(OCRDEC_EINVAL, "out_cap must be >= 1 with out_tokens");
  if (m->timing) return fail(OCRDEC_EINVAL, "expert timing is on; use the individual calls");
  if (m->scratch == nullptr)
    return fail(OCRDEC_EHIP, "the no-allocation scratch is not available on this device: " + m->scratch_err);
  // the decode calls' scratch for this call's rows, laid out in the static array
  ocrdec_config c = m->cfg;
  c.max_batch = B;                 // the draft's catch-up pass keeps the handle's max_k + 1 rows
  const Plan dp = make_plan(&c, true);
  if (dp.w_total > kScratchBytes)
    return fail(OCRDEC_ECAPACITY, "the call needs " + std::to_string(dp.w_total) +
                                      " bytes of scratch; the no-allocation limit is " +
                                      std::to_string(kScratchBytes) + " (fewer rows B*(K+1) or max_positions)");
  hipStream_t s = static_cast<hipStream_t>(stream);
  struct Swap {  // the handle's workspace pointers are restored on every return
    ocrdec_model* m;
    WsPtrs saved;
    ~Swap() { m->b = saved; }
  } swap{m, m->b};
  m->b = bind_workspace(m->scratch, dp, B);
  launch_fill_i32(s, reinterpret_cast<int*>(m->b.mb.stats), 2, 0);  // the expert counter starts at zero
  launch_fill_i32(s, reinterpret_cast<int*>(m->b.sync), MOE_SYNC_WORDS, 0);  // and the MoE counters
  // pages for every step of the call (the pool is host-side: no device allocation)
  if ((rc = ensure_pages(m, s, B, slots, std::min(n_steps, m->cfg.max_positions) * (K + 1))) != OCRDEC_OK) return rc;
  for (int step = 0; step < n_steps; ++step) {
    if (!slots && call_bound(m, B, slots) + K + 1 > m->cfg.max_positions)
      return fail(OCRDEC_ECAPACITY, "positions would exceed max_positions");
    int r1 = OCRDEC_OK;
    if (K > 0)
      r1 = m->cfg.dtype == OCRDEC_BF16 ? do_draft<bf16>(m, s, B, slots, K, draft)
                                       : do_draft<float>(m, s, B, slots, K, draft);
    if (r1 == OCRDEC_OK)
      r1 = m->cfg.dtype == OCRDEC_BF16 ? do_verify<bf16>(m, s, B, slots, K, draft, greedy, nullptr)
                                       : do_verify<float>(m, s, B, slots, K, draft, greedy, nullptr);
    if (r1 != OCRDEC_OK) return r1;
    launch_accept(s, B, K, m->b.plan_slot, draft, greedy, m->b.x, m->sv, n_accepted_out, out_tokens, out_len,
                  out_cap, m->step_tap);
    m->lv_B = 0;
    const int n = slots ? (int)m->slot_bound.size() : B;
    for (int i = 0; i < n; ++i) m->slot_bound[i] = std::min(m->cfg.max_positions, m->slot_bound[i] + K + 1);
    m->last_verify_rows = B * (K + 1);
  }
  return hip_check(m, "ocrdec_decode_steps_noalloc");
}

int ocrdec_sync_positions(ocrdec_model* m, void* stream) {
  if (!m) return fail(OCRDEC_EINVAL, "model is null");
  const int n = m->cfg.max_batch;
  std::vector<int> kv(n), ovf(n);
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess ||
      hipMemcpy(kv.data(), m->sv.kv_len, (size_t)n * sizeof(int), hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(ovf.data(), m->sv.ovf, (size_t)n * sizeof(int), hipMemcpyDeviceToHost) != hipSuccess)
    return fail(OCRDEC_EHIP, "reading the cache lengths failed");
  for (int i = 0; i < n; ++i) m->slot_bound[i] = std::max(0, std::min(kv[i], m->cfg.max_positions));
  unsigned werr = 0;
  if (hipMemcpy(&werr, m->b.sync + MOE_SYNC_ERR, sizeof(unsigned), hipMemcpyDeviceToHost) != hipSuccess)
    return fail(OCRDEC_EHIP, "reading the wait-error word failed");
  if (werr != 0) {
    const unsigned zero = 0;
    (void)hipMemcpy(m->b.sync + MOE_SYNC_ERR, &zero, sizeof(unsigned), hipMemcpyHostToDevice);
    return fail(OCRDEC_EHIP, "a wait inside the persistent MoE launch timed out (its workgroups were not all "
                             "resident on the GPU); results since the last check are not valid");
  }
  std::string over;
  for (int i = 0; i < n; ++i)
    if (ovf[i]) over += (over.empty() ? "" : ", ") + std::to_string(i);
  if (!over.empty()) {
    const std::vector<int> zero(n, 0);
    if (hipMemcpy(m->sv.ovf, zero.data(), (size_t)n * sizeof(int), hipMemcpyHostToDevice) != hipSuccess)
      return fail(OCRDEC_EHIP, "clearing the overflow flags failed");
    return fail(OCRDEC_ECAPACITY, "slot(s) " + over + ": a step would pass max_positions and was not taken");
  }
  return OCRDEC_OK;
}

int ocrdec_set_moe_launches(ocrdec_model* m, int fused) {
  if (!m) return fail(OCRDEC_EINVAL, "model is null");
  m->fused_moe = fused != 0;
  return OCRDEC_OK;
}

int ocrdec_moe_grid(ocrdec_model* m) {
  if (!m) return fail(OCRDEC_EINVAL, "model is null");
  return m->moe_grid;
}

int ocrdec_set_router_logits(ocrdec_model* m, const float* logits) {
  if (!m) return fail(OCRDEC_EINVAL, "model is null");
  m->router_override = logits;
  return OCRDEC_OK;
}

int ocrdec_release_slot(ocrdec_model* m, void* stream, int slot) {
  if (!m) return fail(OCRDEC_EINVAL, "model is null");
  if (slot < 0 || slot >= m->cfg.max_batch) return fail(OCRDEC_EINVAL, "slot out of range");
  PageUpdates u;
  release_pages(m, slot, u);
  m->slot_bound[slot] = 0;
  flush_pages(m, static_cast<hipStream_t>(stream), u);
  return hip_check(m, "ocrdec_release_slot");
}

int ocrdec_kv_pages(ocrdec_model* m, int* total, int* free_pages) {
  if (!m) return fail(OCRDEC_EINVAL, "model is null");
  if (total) *total = m->p.n_pages;
  if (free_pages) *free_pages = (int)m->free_pages.size();
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
  {
    if (pages_for(m, n_pos) > (int)(m->free_pages.size() + m->slot_pages[slot].size()))
      return fail(OCRDEC_ECAPACITY, "KV page pool exhausted: the sequence needs more pages than are free");
    PageUpdates u;
    release_pages(m, slot, u);
    m->slot_bound[slot] = 0;
    grow_pages(m, slot, n_pos, u);
    flush_pages(m, s, u);
  }
  const size_t layer_src = (size_t)2 * NH * n_pos * HD;  // elements of one layer in the source
  for (int l = 0; l < m->cfg.n_layers; ++l) {
    if (m->cfg.dtype == OCRDEC_BF16)
      launch_load_kv<bf16>(s, static_cast<const bf16*>(kv) + l * layer_src, n_pos, kv_view<bf16>(m, l), slot);
    else
      launch_load_kv<float>(s, static_cast<const float*>(kv) + l * layer_src, n_pos, kv_view<float>(m, l), slot);
  }
  launch_set_sequence(s, slot, n_pos, pending_token, m->sv);
  m->slot_bound[slot] = n_pos;
  m->lv_B = 0;
  return hip_check(m, "ocrdec_load_sequence");
}

int ocrdec_set_taps(ocrdec_model* m, const ocrdec_taps* taps) {
  if (!m) return fail(OCRDEC_EINVAL, "model is null");
  if (taps == nullptr) {
    m->taps = ocrdec_taps{};
    m->step_tap = StepTap{};
    return OCRDEC_OK;
  }
  if (taps->route_pos != nullptr &&
      (taps->route_pos_slot < 0 || taps->route_pos_slot >= m->cfg.max_batch || taps->route_pos_cap < 1))
    return fail(OCRDEC_EINVAL, "route_pos needs a slot in [0, max_batch) and route_pos_cap >= 1");
  if ((taps->accepted != nullptr || taps->drafts != nullptr) && taps->step_cap < 1)
    return fail(OCRDEC_EINVAL, "step taps need step_cap >= 1");
  m->taps = *taps;
  m->step_tap = StepTap{taps->accepted, taps->drafts, taps->step_cap};
  return OCRDEC_OK;
}

int ocrdec_expert_timing(ocrdec_model* m, int enable) {
  if (!m) return fail(OCRDEC_EINVAL, "model is null");
  m->timing = enable != 0;
  m->ev_used = 0;
  m->stats_base = 0;
  if (hipDeviceSynchronize() != hipSuccess ||
      hipMemcpy(&m->stats_base, m->b.mb.stats, sizeof(long long), hipMemcpyDeviceToHost) != hipSuccess)
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
  if (hipMemcpy(&sets, m->b.mb.stats, sizeof(long long), hipMemcpyDeviceToHost) != hipSuccess)
    return fail(OCRDEC_EHIP, "hipMemcpy of the expert counter failed");
  if (ms_gate_up) *ms_gate_up = a;
  if (n_gate_up) *n_gate_up = na;
  if (ms_down) *ms_down = b;
  if (n_down) *n_down = nb;
  if (expert_sets) *expert_sets = sets - m->stats_base;
  return OCRDEC_OK;
}

}  // extern "C"
