// Row plans and embedding gathers of each call, greedy longest-prefix
// acceptance with KV rollback, prefill bookkeeping, and the controlled-draft
// override used by the benchmark harness.
#include "launch.h"

namespace ocr {

__device__ __forceinline__ int clamp_tok(int t, int V) { return t < 0 ? 0 : (t >= V ? V - 1 : t); }
__device__ __forceinline__ int clamp_slot(int s, int n) { return s < 0 ? 0 : (s >= n ? n - 1 : s); }

template <typename T>
__device__ __forceinline__ void embed_row(const T* __restrict__ E, int tok, float* __restrict__ dst) {
  const T* src = E + (long)tok * D;
  for (int k = threadIdx.x; k < D; k += 256) dst[k] = WT<T>::load1(src + k);
}

// Block b: sequence b of a verify call.  Rows b*(K+1) + i hold
// [pending, d_1 .. d_K] at positions kv_len .. kv_len + K.  The draft tokens
// are read with the slot, then every row's embedding loads go out at once
// (row indices clamped to K, rows past K not stored).  A sequence whose rows
// would pass the cache (kv_len + K + 1 > max_pos) gets no valid rows (nothing
// is written to its cache) and its overflow flag is set; the accept then
// leaves it unchanged.
constexpr int QV = 8;  // rows per sequence of a verify call: K + 1 <= 8
template <typename T>
__global__ __launch_bounds__(256) void k_plan_verify(int K, const int* __restrict__ slots_in, StateView sv,
                                                     const int* __restrict__ draft, const T* __restrict__ E,
                                                     int V, int* plan_base, int* plan_cnt, int* plan_slot,
                                                     float* __restrict__ x) {
  constexpr int J = D / 256;
  const int b = blockIdx.x;
  int dt[QV - 1];
#pragma unroll
  for (int i = 0; i < QV - 1; ++i) dt[i] = (K > 0) ? draft[b * K + min(i, K - 1)] : 0;
  const int slot = clamp_slot(slots_in ? slots_in[b] : b, sv.n_slots);
  if (threadIdx.x == 0) {
    const int kl = sv.kv_len[slot];
    const bool over = kl + K + 1 > sv.max_pos;
    plan_slot[b] = slot;
    plan_base[b] = kl;
    plan_cnt[b] = over ? 0 : K + 1;
    if (over) sv.ovf[slot] = 1;
  }
  const int pend = sv.pending[slot];
  float v[QV][J];
#pragma unroll
  for (int i = 0; i < QV; ++i) {
    const int r = min(i, K);
    const int tok = clamp_tok(r == 0 ? pend : dt[max(r - 1, 0)], V);
    const T* src = E + (long)tok * D;
#pragma unroll
    for (int j = 0; j < J; ++j) v[i][j] = WT<T>::load1(src + threadIdx.x + 256 * j);
  }
#pragma unroll
  for (int i = 0; i < QV; ++i)
    if (i <= K) {
      float* dst = x + (long)(b * (K + 1) + i) * D;
#pragma unroll
      for (int j = 0; j < J; ++j) dst[threadIdx.x + 256 * j] = v[i][j];
    }
}

// RMSNorm of one D-row into dst (256 threads).
__device__ __forceinline__ void norm_row(const float* __restrict__ src, const float* __restrict__ g, float eps,
                                         float* __restrict__ dst, float* red) {
  float v[D / 256];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < D / 256; ++j) {
    v[j] = src[threadIdx.x + 256 * j];
    ss = fmaf(v[j], v[j], ss);
  }
  ss = block_sum256(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)D + eps);
#pragma unroll
  for (int j = 0; j < D / 256; ++j) dst[threadIdx.x + 256 * j] = (v[j] * r) * g[threadIdx.x + 256 * j];
}

// Draft fusion input of one row: [RMSNorm(h; g_h), RMSNorm(e; g_e)], e = E[tok]
// (the arithmetic of norm_row; both rows' loads issued together).
// cat from the two rows' values already in registers (vh[j], ve[j]: element
// threadIdx.x + 256 j)
__device__ __forceinline__ void draft_cat_regs(const float (&vh)[D / 256], const float (&ve)[D / 256],
                                               const float* __restrict__ g_h, const float* __restrict__ g_e,
                                               float eps, float* __restrict__ cat, float* red) {
  constexpr int J = D / 256;
  float sh = 0.f, se = 0.f;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    sh = fmaf(vh[j], vh[j], sh);
    se = fmaf(ve[j], ve[j], se);
  }
  sh = block_sum256(sh, red);
  se = block_sum256(se, red);
  const float rh = 1.0f / sqrtf(sh / (float)D + eps), re = 1.0f / sqrtf(se / (float)D + eps);
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int k = threadIdx.x + 256 * j;
    cat[k] = (vh[j] * rh) * g_h[k];
    cat[D + k] = (ve[j] * re) * g_e[k];
  }
}
template <typename T>
__device__ __forceinline__ void draft_cat_row(const float* __restrict__ h, int tok, const T* __restrict__ E,
                                              const float* __restrict__ g_h, const float* __restrict__ g_e,
                                              float eps, float* __restrict__ cat, float* red) {
  constexpr int J = D / 256;
  const T* er = E + (long)tok * D;
  float vh[J], ve[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    vh[j] = h[threadIdx.x + 256 * j];
    ve[j] = WT<T>::load1(er + threadIdx.x + 256 * j);
  }
  draft_cat_regs(vh, ve, g_h, g_e, eps, cat, red);
}

// Catch-up pass: sequence b has cnt = n_prev + 1 valid rows at positions
// draft_len .. kv_len; row i takes the verifier hidden hbuf[i] (of position
// draft_len - 1 + i) and the committed token cu_tok[i] (at draft_len + i).
// Block (i, b) builds row i of sequence b; grid (Q, B).
template <typename T>
__global__ __launch_bounds__(256) void k_plan_draft_catchup(int Q, const int* __restrict__ slots_in,
                                                            StateView sv, const T* __restrict__ E, int V,
                                                            const float* __restrict__ g_h,
                                                            const float* __restrict__ g_e, float eps,
                                                            int* plan_base, int* plan_cnt, int* plan_slot,
                                                            float* __restrict__ cat) {
  __shared__ float red[4];
  const int i = blockIdx.x, b = blockIdx.y;
  const int slot = clamp_slot(slots_in ? slots_in[b] : b, sv.n_slots);
  const int cnt = max(1, min(sv.n_prev[slot] + 1, Q));
  if (i == 0 && threadIdx.x == 0) {
    plan_slot[b] = slot;
    plan_base[b] = sv.draft_len[slot];
    plan_cnt[b] = cnt;
  }
  float* c = cat + (long)(b * Q + i) * 2 * D;
  if (i < cnt) {
    const float* h = sv.hbuf + ((long)slot * sv.cu_stride + i) * D;
    const int tok = clamp_tok(sv.cu_tok[slot * sv.cu_stride + i], V);
    draft_cat_row(h, tok, E, g_h, g_e, eps, c, red);
  } else {
    for (int k = threadIdx.x; k < 2 * D; k += 256) c[k] = 0.f;
  }
}

// Pass j >= 2: one row per sequence at position kv_len + j - 1 taking the
// previous pass's block output (its last valid row) and the embedding of d_{j-1}.
template <typename T>
__global__ __launch_bounds__(256) void k_plan_draft_step(int j, int Qprev, int K, StateView sv,
                                                         const int* __restrict__ draft_out, const T* __restrict__ E,
                                                         int V, const float* __restrict__ g_h,
                                                         const float* __restrict__ g_e, float eps,
                                                         const float* __restrict__ u_prev, int* plan_base,
                                                         int* plan_cnt, const int* __restrict__ plan_slot,
                                                         float* __restrict__ cat) {
  __shared__ float red[4];
  __shared__ int prev_cnt;
  const int b = blockIdx.x;
  const int slot = plan_slot[b];
  if (threadIdx.x == 0) prev_cnt = max(1, min(plan_cnt[b], Qprev));
  __syncthreads();
  const float* h = u_prev + (long)(b * Qprev + prev_cnt - 1) * D;
  const int tok = clamp_tok(draft_out[b * K + j - 2], V);
  draft_cat_row(h, tok, E, g_h, g_e, eps, cat + (long)b * 2 * D, red);
  __syncthreads();
  if (threadIdx.x == 0) {
    plan_base[b] = sv.kv_len[slot] + j - 1;
    plan_cnt[b] = 1;
  }
}

// Draft pass input and fusion projection in one launch (the vector path's
// replacement for a plan kernel above, the argmax stage 2 before it and the
// fusion GEMV after it; same arithmetic, so the same bits).  Output row r of
// the pass gets out[r] = W_fuse . cat_r with cat_r = [RMSNorm(h) g_h,
// RMSNorm(E[tok]) g_e] built in LDS by every block for its rows:
//  - catch-up (j = 1): r = b Q + i, h = hbuf[slot][i], tok = cu_tok[slot][i]
//    for i < cnt_b = max(1, min(n_prev + 1, Q)), zero rows past cnt_b;
//  - step (j >= 2): r = b, tok = d_{j-1} = the argmax of the previous pass's
//    LM-head partials (also written to draft_out), h = the previous pass's
//    output row b Qprev + pc_b - 1, pc_b = 1 past the catch-up, else cnt_b.
// Blocks with blockIdx.x = 0 write the plan entries of their rows (no block
// reads them).  Each wavefront owns 2 output rows, as the generic GEMV with
// K = 2 D; grid (D / 8, ceil(M / MR)).  out must not alias u_prev.
template <typename T>
struct DraftIn {
  int step, j, Q, Qprev, K, V;
  const int* slots_in;  // catch-up: sequence -> slot (nullable: identity)
  StateView sv;
  const T* E;
  const float* g_h;
  const float* g_e;
  float eps;
  const float* u_prev;     // step: previous pass's output rows
  const float* part_val;   // step: LM-head per-block bests of the previous pass, [B][nblk]
  const int* part_idx;
  int nblk;
  int* draft_out;          // step: [B][K], d_{j-1} at column j - 2
  int* plan_base;
  int* plan_cnt;
  int* plan_slot;
};

template <typename T, int MR>
__global__ __launch_bounds__(256) void k_draft_fuse(DraftIn<T> a, const T* __restrict__ W, int M,
                                                    float* __restrict__ out) {
  extern __shared__ float smem[];
  float* xs = smem;  // [MR][2 D]
  __shared__ float red[4];
  __shared__ float amv[4];
  __shared__ int ami[4];
  constexpr int K2 = 2 * D, R = 2;
  const int wave = wave_id();
  const int n0 = (blockIdx.x * 4 + wave) * R;
  const int m0 = blockIdx.y * MR;
  const int m_act = min(MR, M - m0);
  const T* rows[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rows[r] = W + (long)min(n0 + r, D - 1) * K2;
  WaveGemv<T, K2, R, MR> g;
  g.load(rows);
  const bool writer = blockIdx.x == 0 && threadIdx.x == 0;
  if (a.step) {
    for (int m = 0; m < m_act; ++m) {
      const int b = m0 + m;
      const int slot = a.plan_slot[b];
      const int pc = (a.Qprev == 1) ? 1 : max(1, min(a.sv.n_prev[slot] + 1, a.Qprev));
      const float* h = a.u_prev + (long)(b * a.Qprev + pc - 1) * D;
      const int id = argmax_block(a.part_val + (long)b * a.nblk, a.part_idx + (long)b * a.nblk, a.nblk, amv, ami);
      if (writer) {
        a.draft_out[b * a.K + a.j - 2] = id;
        a.plan_base[b] = a.sv.kv_len[slot] + a.j - 1;
        a.plan_cnt[b] = 1;
      }
      draft_cat_row(h, clamp_tok(id, a.V), a.E, a.g_h, a.g_e, a.eps, xs + m * K2, red);
    }
  } else {
    // catch-up: every row's plan reads, then its token and hidden row, then its
    // embedding row go out for all rows before the first reduction (row
    // indices clamped into range; rows past cnt are zeroed, not built)
    constexpr int J = D / 256;
    int sl[MR], ii[MR], cn[MR], tk[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const int r = m0 + min(m, m_act - 1);
      const int b = r / a.Q;
      ii[m] = r - b * a.Q;
      sl[m] = clamp_slot(a.slots_in ? a.slots_in[b] : b, a.sv.n_slots);
      cn[m] = max(1, min(a.sv.n_prev[sl[m]] + 1, a.Q));
      if (writer && m < m_act && ii[m] == 0) {
        a.plan_slot[b] = sl[m];
        a.plan_base[b] = a.sv.draft_len[sl[m]];
        a.plan_cnt[b] = cn[m];
      }
    }
    float vh[MR][J], ve[MR][J];
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const long e = (long)sl[m] * a.sv.cu_stride + min(ii[m], cn[m] - 1);
      tk[m] = clamp_tok(a.sv.cu_tok[e], a.V);
      const float* h = a.sv.hbuf + e * D;
#pragma unroll
      for (int j = 0; j < J; ++j) vh[m][j] = h[threadIdx.x + 256 * j];
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const T* er = a.E + (long)tk[m] * D;
#pragma unroll
      for (int j = 0; j < J; ++j) ve[m][j] = WT<T>::load1(er + threadIdx.x + 256 * j);
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      if (m >= m_act) break;
      float* c = xs + m * K2;
      if (ii[m] < cn[m]) {
        draft_cat_regs(vh[m], ve[m], a.g_h, a.g_e, a.eps, c, red);
      } else {
        for (int k = threadIdx.x; k < K2; k += 256) c[k] = 0.f;
      }
    }
  }
  __syncthreads();
  float acc[R][MR];
  g.fma(xs, m_act, acc);
  const WaveTotals<R, MR> t(acc);
  const int n = n0 + t.r;
  if (t.lead && t.m < m_act && n < D) out[(long)(m0 + t.m) * D + n] = t.val;
}

// Prefill pass: rows j * PREFILL_CHUNK + i (entry j, i < cnt[j]) hold
// positions p0[j] + i of sequence seq[j] -- vision rows, then prompt ids; rows
// past cnt[j] are zero.  esave keeps the input rows for the draft prefill.
// Grid (PREFILL_CHUNK, n).
template <typename T>
__global__ __launch_bounds__(256) void k_plan_prefill(PrefillGroup g, const float* __restrict__ vision,
                                                      int nv_stride, const int* __restrict__ prompt, int np_stride,
                                                      const T* __restrict__ E, int V, int* plan_base,
                                                      int* plan_cnt, int* plan_slot, float* __restrict__ x,
                                                      float* __restrict__ esave) {
  const int i = blockIdx.x, j = blockIdx.y;
  const int p = g.p0[j] + i;
  const int b = g.seq[j];
  if (i == 0 && threadIdx.x == 0) {
    plan_slot[j] = g.slot[j];
    plan_base[j] = g.p0[j];
    plan_cnt[j] = g.cnt[j];
  }
  const long row = (long)j * PREFILL_CHUNK + i;
  float* dst = x + row * D;
  if (i >= g.cnt[j]) {
    for (int k = threadIdx.x; k < D; k += 256) dst[k] = 0.f;
  } else if (p < g.nvis[j]) {
    const float* src = vision + ((long)b * nv_stride + p) * D;
    for (int k = threadIdx.x; k < D; k += 256) dst[k] = src[k];
  } else {
    embed_row(E, clamp_tok(prompt[(long)b * np_stride + p - g.nvis[j]], V), dst);
  }
  __syncthreads();
  for (int k = threadIdx.x; k < D; k += 256) esave[row * D + k] = dst[k];
}

// Draft prefill rows of a pass: row (j, i) at position p = p0[j] + i takes
// (h_{p-1}, e_p); h of an entry's first row is the last verifier hidden of
// the entry before it when that is the same sequence, else of the sequence's
// previous pass (hprev[slot]; a zero row at p = 0).  The last verifier hidden
// of a sequence's last entry in the pass goes to hnext[slot].  Grid
// (PREFILL_CHUNK, n).
__global__ __launch_bounds__(256) void k_draft_prefill_cat(PrefillGroup g, const float* __restrict__ xfinal,
                                                           const float* __restrict__ esave,
                                                           const float* __restrict__ hprev,
                                                           float* __restrict__ hnext, const float* __restrict__ g_h,
                                                           const float* __restrict__ g_e, float eps,
                                                           float* __restrict__ cat) {
  __shared__ float red[4];
  __shared__ float zero[D];
  const int i = blockIdx.x, j = blockIdx.y;
  const long row = (long)j * PREFILL_CHUNK + i;
  const int slot = g.slot[j];
  const float* h;
  if (i > 0) {
    h = xfinal + (row - 1) * D;
  } else if (j > 0 && g.seq[j - 1] == g.seq[j]) {
    h = xfinal + ((long)(j - 1) * PREFILL_CHUNK + g.cnt[j - 1] - 1) * D;
  } else if (g.p0[j] > 0) {
    h = hprev + (long)slot * D;
  } else {
    for (int k = threadIdx.x; k < D; k += 256) zero[k] = 0.f;
    __syncthreads();
    h = zero;
  }
  float* dst = cat + row * 2 * D;
  norm_row(h, g_h, eps, dst, red);
  norm_row(esave + row * D, g_e, eps, dst + D, red);
  if (i == g.cnt[j] - 1 && (j + 1 == g.n || g.seq[j + 1] != g.seq[j]))
    for (int k = threadIdx.x; k < D; k += 256) hnext[(long)slot * D + k] = xfinal[row * D + k];
}

// Entry j ends its sequence's prefix in this pass.
__device__ __forceinline__ bool prefill_ends(const PrefillGroup& g, int j) { return g.p0[j] + g.cnt[j] == g.plen[j]; }
// Finishing entries before entry j.
__device__ __forceinline__ int prefill_rank(const PrefillGroup& g, int j) {
  int f = 0;
  for (int i = 0; i < j; ++i) f += prefill_ends(g, i) ? 1 : 0;
  return f;
}

// The last prefix row of each sequence that ends in this pass, compacted:
// dst[f] = xfinal[row of entry j's last row], f = j's rank among the
// finishing entries (the LM head then runs on these rows only).  Grid n.
__global__ __launch_bounds__(256) void k_prefill_last_rows(PrefillGroup g, const float* __restrict__ xfinal,
                                                           float* __restrict__ dst) {
  const int j = blockIdx.x;
  if (!prefill_ends(g, j)) return;
  const int f = prefill_rank(g, j);
  const float* src = xfinal + ((long)j * PREFILL_CHUNK + g.cnt[j] - 1) * D;
  for (int k = threadIdx.x; k < D; k += 256) dst[(long)f * D + k] = src[k];
}

// Entries that end their sequence's prefix: state of the slot, and output
// token 0 (the greedy token of the last prefix row, tok[f], f the entry's
// rank among the finishing entries) to pending_out[seq].  Grid n.
__global__ __launch_bounds__(256) void k_prefill_finish(PrefillGroup g, const float* __restrict__ xfinal,
                                                        const int* __restrict__ tok, StateView sv,
                                                        int* __restrict__ pending_out) {
  const int j = blockIdx.x;
  const int P = g.plen[j];
  if (!prefill_ends(g, j)) return;
  const int slot = g.slot[j];
  const int y0 = tok[prefill_rank(g, j)];
  if (threadIdx.x == 0) {
    sv.kv_len[slot] = P;
    sv.draft_len[slot] = P;
    sv.pending[slot] = y0;
    sv.n_prev[slot] = 0;
    sv.out_len[slot] = 1;
    sv.step[slot] = 0;
    sv.prefix_len[slot] = P;
    sv.ovf[slot] = 0;
    sv.cu_tok[slot * sv.cu_stride] = y0;
    pending_out[g.seq[j]] = y0;
  }
  const float* xl = xfinal + ((long)j * PREFILL_CHUNK + g.cnt[j] - 1) * D;
  float* hb = sv.hbuf + (long)slot * sv.cu_stride * D;
  for (int k = threadIdx.x; k < D; k += 256) hb[k] = xl[k];
}

// A slot whose verifier cache was loaded by the caller: P cached positions,
// pending token tok, no draft history (its hidden-state feedback row is zero).
__global__ void k_set_sequence(int slot, int P, int tok, StateView sv) {
  if (threadIdx.x == 0) {
    sv.kv_len[slot] = P;
    sv.draft_len[slot] = P;
    sv.pending[slot] = tok;
    sv.n_prev[slot] = 0;
    sv.out_len[slot] = 1;
    sv.step[slot] = 0;
    sv.prefix_len[slot] = P;
    sv.ovf[slot] = 0;
    sv.cu_tok[slot * sv.cu_stride] = tok;
  }
  float* hb = sv.hbuf + (long)slot * sv.cu_stride * D;
  for (int k = threadIdx.x; k < D; k += 256) hb[k] = 0.f;
}

// Greedy longest-prefix acceptance (one block per sequence).
// Argmax stage 2 of one row by one wavefront (the block-wide version's rule:
// largest value, lowest id among equal ones), all of a lane's loads issued
// together (indices clamped to the last block); every lane gets the id.
__device__ __forceinline__ int argmax_wave(const float* __restrict__ rv, const int* __restrict__ ri, int nblk) {
  constexpr int AW = 32;
  const int lane = lane_id();
  float v = -INFINITY;
  int id = 0x7fffffff;
  for (int b0 = 0; b0 < nblk; b0 += 64 * AW) {
    float pv[AW];
    int pi[AW];
#pragma unroll
    for (int j = 0; j < AW; ++j) {
      const int k = min(b0 + lane + 64 * j, nblk - 1);
      pv[j] = rv[k];
      pi[j] = ri[k];
    }
#pragma unroll
    for (int j = 0; j < AW; ++j)
      if (pv[j] > v || (pv[j] == v && pi[j] < id)) { v = pv[j]; id = pi[j]; }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {  // any pairing gives the same result
    const float ov = xchg(v, off);
    const int oi = xchg_i(id, off);
    if (ov > v || (ov == v && oi < id)) { v = ov; id = oi; }
  }
  return id;
}

// Acceptance of sequence b (block b).  With AM the verify rows' greedy tokens
// are first reduced here from the LM head's per-block bests (part_val /
// part_idx, [B (K+1)][nblk]) and written to greedy_w; otherwise they are read
// from greedy.
template <bool AM>
__global__ __launch_bounds__(256) void k_accept(int K, const int* __restrict__ plan_slot,
                                                const int* __restrict__ draft, const int* __restrict__ greedy,
                                                const float* __restrict__ xfinal, StateView sv,
                                                int* __restrict__ n_acc, int* __restrict__ out_tokens,
                                                int* __restrict__ out_len_out, int out_cap, StepTap tap,
                                                const float* __restrict__ part_val, const int* __restrict__ part_idx,
                                                int nblk, int* __restrict__ greedy_w) {
  constexpr int J = D / 256;
  __shared__ int sn;
  __shared__ int gs[QV];
  const int b = blockIdx.x;
  const int lane = lane_id(), wave = wave_id();
  // the verify rows' final hidden states (rows past K clamped, not stored)
  // are fetched before the acceptance is known
  float hv[QV][J];
#pragma unroll
  for (int i = 0; i < QV; ++i) {
    const float* src = xfinal + (long)(b * (K + 1) + min(i, K)) * D;
#pragma unroll
    for (int j = 0; j < J; ++j) hv[i][j] = src[threadIdx.x + 256 * j];
  }
  const int slot = plan_slot[b];
  if constexpr (AM) {
    for (int i = wave; i <= K; i += 4) {
      const long r = (long)b * (K + 1) + i;
      const int id = argmax_wave(part_val + r * nblk, part_idx + r * nblk, nblk);
      if (lane == 0) {
        gs[i] = id;
        greedy_w[r] = id;
      }
    }
    __syncthreads();
  }
  if (wave == 0) {
    // lane i < K compares d_i with the verifier's g_i; n = the first mismatch
    const int dv = (lane < K) ? draft[b * K + lane] : 0;
    const int gv = (lane <= K) ? (AM ? gs[lane] : greedy[b * (K + 1) + lane]) : 0;
    const int old = sv.kv_len[slot];
    const int ol0 = sv.out_len[slot];
    const int st = sv.step[slot];
    const bool over = old + K + 1 > sv.max_pos;  // the verify computed no rows for it
    const uint64_t miss = __ballot(!(lane < K && dv == gv));
    const int n = __builtin_ctzll(miss);  // <= K
    const int gn = __builtin_amdgcn_readlane(gv, n);  // n is the same on every lane
    if (!over && lane <= n) {
      const int t = (lane < n) ? dv : gn;
      sv.cu_tok[slot * sv.cu_stride + lane] = t;
      if (out_tokens != nullptr && ol0 + lane < out_cap) out_tokens[(long)b * out_cap + ol0 + lane] = t;
    }
    if (lane == 0) {
      if (over) {
        if (n_acc != nullptr) n_acc[b] = -1;
        if (out_len_out != nullptr) out_len_out[b] = ol0;
        sn = -1;
      } else {
        const int ol = ol0 + n + 1;
        sv.out_len[slot] = ol;
        sv.kv_len[slot] = old + n + 1;
        sv.draft_len[slot] = old + 1;
        sv.pending[slot] = gn;
        sv.n_prev[slot] = n;
        sv.step[slot] = st + 1;
        if (n_acc != nullptr) n_acc[b] = n;
        if (out_len_out != nullptr) out_len_out[b] = ol;
        if (tap.acc != nullptr && st < tap.cap) tap.acc[(long)slot * tap.cap + st] = n;
        sn = n;
      }
    }
  }
  __syncthreads();
  const int n = sn;
#pragma unroll
  for (int i = 0; i < QV; ++i)
    if (i <= n) {
      float* dst = sv.hbuf + ((long)slot * sv.cu_stride + i) * D;
#pragma unroll
      for (int j = 0; j < J; ++j) dst[threadIdx.x + 256 * j] = hv[i][j];
    }
}

// SplitMix64 output function (Steele, Lea & Flood 2014).
__device__ __forceinline__ uint64_t splitmix64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__global__ void k_controlled(int B, int K, const int* __restrict__ slots_in, StateView sv,
                             const int* __restrict__ trace, int trace_stride, int trace_len, uint64_t seed,
                             uint64_t thr, int V, int* __restrict__ draft) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= B * K) return;
  const int b = t / K, j = t % K + 1;
  const int slot = clamp_slot(slots_in ? slots_in[b] : b, sv.n_slots);
  const int c = sv.out_len[slot];
  const int idx = c - 1 + j;
  const int true_tok = (idx < trace_len) ? trace[(long)b * trace_stride + idx] : 0;
  uint64_t h = splitmix64(seed);
  h = splitmix64(h ^ (uint64_t)(uint32_t)slot);
  h = splitmix64(h ^ (uint64_t)(uint32_t)sv.step[slot]);
  h = splitmix64(h ^ (uint64_t)(uint32_t)j);
  int tok = true_tok;
  if ((h >> 11) < thr) tok = (int)(((uint64_t)true_tok + 1 + (h & 0xFFFFFFFFull) % (uint64_t)(V - 1)) % (uint64_t)V);
  draft[b * K + j - 1] = tok;
}

// Drafts tap: the K proposals of sequence b at its slot's step number.
__global__ void k_draft_tap(int B, int K, const int* __restrict__ plan_slot, StateView sv,
                            const int* __restrict__ draft, StepTap tap) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= B * K) return;
  const int b = t / K, j = t % K;
  const int slot = plan_slot[b];
  const int st = sv.step[slot];
  if (st < tap.cap) tap.drafts[((long)slot * tap.cap + st) * QV + j] = draft[b * K + j];
}

__global__ void k_copy(const float* __restrict__ src, float* __restrict__ dst, long n) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) dst[i] = src[i];
}

// ---------------------------------------------------------------- launchers
template <typename T>
void launch_plan_verify(hipStream_t s, int B, int K, const int* slots_in, StateView sv, const int* draft,
                        const T* embed, int V, int* plan_base, int* plan_cnt, int* plan_slot, float* x) {
  hipLaunchKernelGGL((k_plan_verify<T>), dim3(B), dim3(256), 0, s, K, slots_in, sv, draft, embed, V, plan_base,
                     plan_cnt, plan_slot, x);
}
template <typename T>
void launch_plan_draft_catchup(hipStream_t s, int B, int Q, const int* slots_in, StateView sv, const T* embed,
                               int V, const float* g_h, const float* g_e, float eps, int* plan_base, int* plan_cnt,
                               int* plan_slot, float* cat) {
  hipLaunchKernelGGL((k_plan_draft_catchup<T>), dim3(Q, B), dim3(256), 0, s, Q, slots_in, sv, embed, V, g_h, g_e, eps,
                     plan_base, plan_cnt, plan_slot, cat);
}
template <typename T>
void launch_plan_draft_step(hipStream_t s, int B, int j, int Qprev, int K, StateView sv, const int* draft_out,
                            const T* embed, int V, const float* g_h, const float* g_e, float eps,
                            const float* u_prev, int* plan_base, int* plan_cnt, const int* plan_slot, float* cat) {
  hipLaunchKernelGGL((k_plan_draft_step<T>), dim3(B), dim3(256), 0, s, j, Qprev, K, sv, draft_out, embed, V, g_h,
                     g_e, eps, u_prev, plan_base, plan_cnt, plan_slot, cat);
}
template <typename T>
void launch_draft_fuse(hipStream_t s, int step, int j, int Q, int Qprev, int K, const int* slots_in, StateView sv,
                       const T* embed, int V, const float* g_h, const float* g_e, float eps, const float* u_prev,
                       const float* part_val, const int* part_idx, int nblk, int* draft_out, int* plan_base,
                       int* plan_cnt, int* plan_slot, const T* w_fuse, int M, float* out) {
  const DraftIn<T> a{step, j, Q, Qprev, K, V, slots_in, sv, embed, g_h, g_e, eps, u_prev, part_val, part_idx,
                     nblk, draft_out, plan_base, plan_cnt, plan_slot};
#define OCR_DF_CASE(MRV)                                                                               \
  {                                                                                                    \
    const size_t lds = (size_t)MRV * 2 * D * 4;                                                        \
    static const bool attr_set = (allow_lds(k_draft_fuse<T, MRV>, lds), true);                         \
    (void)attr_set;                                                                                    \
    hipLaunchKernelGGL((k_draft_fuse<T, MRV>), dim3(D / 8, (M + MRV - 1) / MRV), dim3(256), lds, s, a, \
                       w_fuse, M, out);                                                                \
  }
  if (M <= 1) OCR_DF_CASE(1)
  else if (M <= 2) OCR_DF_CASE(2)
  else if (M <= 4) OCR_DF_CASE(4)
  else OCR_DF_CASE(MRG)
#undef OCR_DF_CASE
}
template <typename T>
void launch_plan_prefill(hipStream_t s, const PrefillGroup& g, const float* vision, int nv_stride,
                         const int* prompt, int np_stride, const T* embed, int V, int* plan_base, int* plan_cnt,
                         int* plan_slot, float* x, float* esave) {
  hipLaunchKernelGGL((k_plan_prefill<T>), dim3(PREFILL_CHUNK, g.n), dim3(256), 0, s, g, vision, nv_stride, prompt,
                     np_stride, embed, V, plan_base, plan_cnt, plan_slot, x, esave);
}
void launch_draft_prefill_cat(hipStream_t s, const PrefillGroup& g, const float* xfinal, const float* esave,
                              const float* hprev, float* hnext, const float* g_h, const float* g_e, float eps,
                              float* cat) {
  hipLaunchKernelGGL(k_draft_prefill_cat, dim3(PREFILL_CHUNK, g.n), dim3(256), 0, s, g, xfinal, esave, hprev, hnext,
                     g_h, g_e, eps, cat);
}
void launch_prefill_last_rows(hipStream_t s, const PrefillGroup& g, const float* xfinal, float* dst) {
  hipLaunchKernelGGL(k_prefill_last_rows, dim3(g.n), dim3(256), 0, s, g, xfinal, dst);
}
void launch_prefill_finish(hipStream_t s, const PrefillGroup& g, const float* xfinal, const int* tok, StateView sv,
                           int* pending_out) {
  hipLaunchKernelGGL(k_prefill_finish, dim3(g.n), dim3(256), 0, s, g, xfinal, tok, sv, pending_out);
}
// Page-table updates: table[ps.idx[i]] = ps.page[i], i < ps.n.
__global__ void k_set_pages(int* __restrict__ table, PageSet ps) {
  const int i = threadIdx.x;
  if (i < ps.n) table[ps.idx[i]] = ps.page[i];
}
void launch_set_pages(hipStream_t s, int* table, const PageSet& ps) {
  hipLaunchKernelGGL(k_set_pages, dim3(1), dim3(256), 0, s, table, ps);
}

// A caller's cache of one layer, [K|V][head][n_pos][HD], into the pages of
// `slot`: block (block j of positions, plane K|V x head) copies its rows.
template <typename T>
__global__ __launch_bounds__(256) void k_load_kv(const T* __restrict__ src, int n_pos, KvView<T> kv, int slot) {
  const int j = blockIdx.x, plane = blockIdx.y;
  const int rows = min(KV_PAGE, n_pos - j * KV_PAGE);
  const int pg = kv.raw_page(slot, j * KV_PAGE);
  if (pg < 0) return;
  T* dst = kv.rows(pg, plane / NH, plane % NH);
  const T* from = src + ((long)plane * n_pos + (long)j * KV_PAGE) * HD;
  for (int e = threadIdx.x; e < rows * HD; e += 256) dst[e] = from[e];
}
template <typename T>
void launch_load_kv(hipStream_t s, const T* src, int n_pos, KvView<T> kv, int slot) {
  hipLaunchKernelGGL((k_load_kv<T>), dim3((n_pos + KV_PAGE - 1) / KV_PAGE, 2 * NH), dim3(256), 0, s, src, n_pos, kv,
                     slot);
}
template void launch_load_kv<float>(hipStream_t, const float*, int, KvView<float>, int);
template void launch_load_kv<bf16>(hipStream_t, const bf16*, int, KvView<bf16>, int);

void launch_set_sequence(hipStream_t s, int slot, int P, int tok, StateView sv) {
  hipLaunchKernelGGL(k_set_sequence, dim3(1), dim3(256), 0, s, slot, P, tok, sv);
}
void launch_accept(hipStream_t s, int B, int K, const int* plan_slot, const int* draft, const int* greedy,
                   const float* xfinal, StateView sv, int* n_acc, int* out_tokens, int* out_len_out, int out_cap,
                   const StepTap& tap, const float* part_val, const int* part_idx, int nblk, int* greedy_w) {
  if (part_val != nullptr)
    hipLaunchKernelGGL((k_accept<true>), dim3(B), dim3(256), 0, s, K, plan_slot, draft, greedy, xfinal, sv, n_acc,
                       out_tokens, out_len_out, out_cap, tap, part_val, part_idx, nblk, greedy_w);
  else
    hipLaunchKernelGGL((k_accept<false>), dim3(B), dim3(256), 0, s, K, plan_slot, draft, greedy, xfinal, sv, n_acc,
                       out_tokens, out_len_out, out_cap, tap, part_val, part_idx, nblk, greedy_w);
}
void launch_draft_tap(hipStream_t s, int B, int K, const int* plan_slot, StateView sv, const int* draft,
                      const StepTap& tap) {
  const int n = B * K;
  hipLaunchKernelGGL(k_draft_tap, dim3((n + 255) / 256), dim3(256), 0, s, B, K, plan_slot, sv, draft, tap);
}
void launch_controlled(hipStream_t s, int B, int K, const int* slots_in, StateView sv, const int* trace,
                       int trace_stride, int trace_len, uint64_t seed, uint64_t thr, int V, int* draft) {
  const int n = B * K;
  hipLaunchKernelGGL(k_controlled, dim3((n + 255) / 256), dim3(256), 0, s, B, K, slots_in, sv, trace,
                     trace_stride, trace_len, seed, thr, V, draft);
}
__global__ void k_fill_i32(int* __restrict__ p, long n, int v) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) p[i] = v;
}
void launch_fill_i32(hipStream_t s, int* p, long n, int v) {
  hipLaunchKernelGGL(k_fill_i32, dim3(1), dim3(256), 0, s, p, n, v);
}
void launch_copy_rows(hipStream_t s, const float* src, float* dst, long n) {
  hipLaunchKernelGGL(k_copy, dim3(64), dim3(256), 0, s, src, dst, n);
}

// Plain read of n16 16-byte words (grid-stride, 8 loads in flight per
// thread), folded by xor; sink[0] is written only if the fold hits a fixed
// value, which keeps the loads from being dropped.  Calibration only: it
// shows what a kernel that does nothing but read reaches at a given size.
__global__ __launch_bounds__(256) void k_read_probe(const uint4* __restrict__ p, long n16, uint32_t* sink) {
  constexpr int U = 8;
  uint32_t acc = 0;
  const long stride = (long)gridDim.x * 256 * U;
  for (long base = (long)blockIdx.x * 256 * U + threadIdx.x; base < n16; base += stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long i = min(base + (long)u * 256, n16 - 1);
      v[u] = p[i];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}
void launch_read_probe(hipStream_t s, const void* buf, long n16, uint32_t* sink) {
  hipLaunchKernelGGL(k_read_probe, dim3(4096), dim3(256), 0, s, static_cast<const uint4*>(buf), n16, sink);
}

#define OCR_INST_MISC(T)                                                                                          \
  template void launch_plan_verify<T>(hipStream_t, int, int, const int*, StateView, const int*, const T*, int,   \
                                      int*, int*, int*, float*);                                                 \
  template void launch_plan_draft_catchup<T>(hipStream_t, int, int, const int*, StateView, const T*, int,        \
                                             const float*, const float*, float, int*, int*, int*, float*);       \
  template void launch_draft_fuse<T>(hipStream_t, int, int, int, int, int, const int*, StateView, const T*, int,   \
                                     const float*, const float*, float, const float*, const float*, const int*, int,  \
                                     int*, int*, int*, int*, const T*, int, float*);                                  \
  template void launch_plan_draft_step<T>(hipStream_t, int, int, int, int, StateView, const int*, const T*, int, \
                                          const float*, const float*, float, const float*, int*, int*,           \
                                          const int*, float*);                                                   \
  template void launch_plan_prefill<T>(hipStream_t, const PrefillGroup&, const float*, int, const int*, int,     \
                                       const T*, int, int*, int*, int*, float*, float*);
OCR_INST_MISC(float)
OCR_INST_MISC(bf16)

}  // namespace ocr
