// Mixture-of-experts decode kernels: fused RMSNorm -> router -> softmax top-6
// with a stable counting sort of the (row, slot) pairs by expert, the grouped
// expert SwiGLU GEMV (gate/up, then down) over the union of active experts,
// and the fixed-order combine into the residual stream.
//
// Routing slots per row: 0..5 = routed experts by decreasing score (gate =
// softmax probability over the 64 routed experts, not renormalised), 6..7 =
// the two shared experts (ids 64, 65, gate 1).  Pair id = row * 8 + slot.
#include "launch.h"

namespace ocr {

// Routing of up to 8 rows held in LDS.
struct RouteLds {
  int pe[64];        // expert of pair p = row * 8 + slot
  float pg[64];      // gate of pair p
  int perm[64];      // pair id by sorted position
  int inv[64];       // sorted position of pair id
  int cnt[NX + 1], off[NX + 1], act[NX + 1];
  int na;
};

// Inclusive prefix sum over the 64 lanes of a wavefront: within each 16-lane
// row by DPP row shifts (lanes past the row's start read 0), then the row
// totals as scalars.
__device__ __forceinline__ int wave_incl_scan(int c) {
  const int lane = lane_id();
  int incl = c;
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x111, 0xF, 0xF, false);  // row_shr:1
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x112, 0xF, 0xF, false);  // row_shr:2
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x114, 0xF, 0xF, false);  // row_shr:4
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x118, 0xF, 0xF, false);  // row_shr:8
  const int t0 = __builtin_amdgcn_readlane(incl, 15), t1 = __builtin_amdgcn_readlane(incl, 31);
  const int t2 = __builtin_amdgcn_readlane(incl, 47);
  return incl + (lane >= 16 ? t0 : 0) + (lane >= 32 ? t1 : 0) + (lane >= 48 ? t2 : 0);
}

// Stable counting sort of P <= 64 pairs by one wavefront (lane = pair): the
// lanes holding the same expert found from one ballot per bit of the id (7
// bits cover 0..65), rank = those below this lane, count written by the
// lowest; offsets by a wavefront scan (routed experts 0..63 in id order, then
// the shared experts 64, 65).
__device__ __forceinline__ void sort_pairs_wave(int P, RouteLds& r) {
  static_assert(NX <= 128, "expert ids must fit in 7 bits");
  const int lane = lane_id();
  const bool valid = lane < P;
  const int e = valid ? r.pe[lane] : 0;
  const uint64_t lt = (1ull << lane) - 1ull;
  for (int x = lane; x <= NX; x += 64) r.cnt[x] = 0;
  uint64_t same = __ballot(valid);
#pragma unroll
  for (int bit = 0; bit < 7; ++bit) {
    const uint64_t set = __ballot(valid && ((e >> bit) & 1));
    same &= ((e >> bit) & 1) ? set : ~set;
  }
  const int rank = valid ? __popcll(same & lt) : 0;
  if (valid && rank == 0) r.cnt[e] = __popcll(same);
  const int c = r.cnt[lane];
  const int incl = wave_incl_scan(c);
  r.off[lane] = incl - c;
  const int routed = __builtin_amdgcn_readlane(incl, 63);
  const uint64_t amask = __ballot(c > 0);
  if (c > 0) r.act[__popcll(amask & lt)] = lane;
  int na = __popcll(amask);
  const int c64 = r.cnt[NE], c65 = r.cnt[NE + 1];
  if (lane == 0) {
    r.off[NE] = routed;
    r.off[NE + 1] = routed + c64;
    r.off[NX] = routed + c64 + c65;
    if (c64 > 0) r.act[na] = NE;
    if (c65 > 0) r.act[na + (c64 > 0)] = NE + 1;
    r.na = na + (c64 > 0) + (c65 > 0);
  }
  if (valid) {
    const int pos = r.off[e] + rank;
    r.perm[pos] = lane;
    r.inv[lane] = pos;
  }
}

// Lane e of a wavefront, holding logit v of a row whose 64 logits are in lg
// (LDS): rank = the number of experts that beat it (a larger logit, or an
// equal one and a lower id), so ranks 0..5 are the routed slots in decreasing
// order; gate = its softmax probability over the 64 (max = the largest logit,
// sum by the xor butterfly).
__device__ __forceinline__ void rank_and_gate(const float* lg, float v, int& rank, float& gate) {
  const int lane = lane_id();
  int rk = 0;
  float mx = v;
#pragma unroll 16
  for (int o = 0; o < NE; ++o) {
    const float u = lg[o];
    rk += (u > v || (u == v && o < lane)) ? 1 : 0;
    mx = fmaxf(mx, u);
  }
  const float ex = expf(v - mx);
  rank = rk;
  gate = ex / wave_sum(ex);
}

// Route M <= 8 rows from their logits (rlogit[m][64]) into LDS; all 256
// threads of the block call it (two barriers inside).  Wavefront w handles rows
// w, w+4 with rank_and_gate, then wavefront 0 sorts the pairs.  AGENT: the
// logits were written by other workgroups of the same launch.
template <bool AGENT = false>
__device__ __forceinline__ void route_rows(const float* __restrict__ rlogit, int M, RouteLds& r) {
  __shared__ float lg[4][NE];
  const int wave = wave_id(), lane = lane_id();
  for (int m = wave; m < M; m += 4) {
    const float v = AGENT ? ld_agent(rlogit + m * NE + lane) : rlogit[m * NE + lane];
    lg[wave][lane] = v;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    int rank;
    float gate;
    rank_and_gate(lg[wave], v, rank, gate);
    if (rank < TOPK) {
      r.pe[m * NSLOT + rank] = lane;
      r.pg[m * NSLOT + rank] = gate;
    }
    if (lane < NSH) {
      r.pe[m * NSLOT + TOPK + lane] = NE + lane;
      r.pg[m * NSLOT + TOPK + lane] = 1.0f;
    }
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  if (wave == 0) sort_pairs_wave(M * NSLOT, r);
  __syncthreads();
}

// Routing taps of pair p = row m * 8 + k (expert e): the call's table, and the
// table by position for the rows of the tapped slot.
__device__ __forceinline__ void tap_pair(const RouteTap& tap, int m, int k, int e) {
  if (tap.call != nullptr) tap.call[m * NSLOT + k] = e;
  if (tap.pos != nullptr) {
    const int b = m / tap.plan.Q, i = m - b * tap.plan.Q;
    if (tap.plan.slot[b] == tap.pos_slot && i < tap.plan.cnt[b]) {
      const int pos = tap.plan.base[b] + i;
      if (pos >= 0 && pos < tap.pos_cap) tap.pos[(long)pos * NSLOT + k] = e;
    }
  }
}

// Publish the routing of the LDS copy for the kernels that follow (down,
// combine) and the taps; stats[0] = st0 (its value at kernel start, read by
// thread 0) + the active experts.
__device__ __forceinline__ void publish_route(const RouteLds& r, int M, const MoeBufs& mb, const RouteTap& tap,
                                              long long st0) {
  const int tid = threadIdx.x;
  const int P = M * NSLOT;
  for (int p = tid; p < P; p += 256) {
    mb.ridx[p] = r.pe[p];
    mb.rgate[p] = r.pg[p];
    mb.perm[p] = r.perm[p];
    mb.inv[p] = r.inv[p];
    tap_pair(tap, p / NSLOT, p % NSLOT, r.pe[p]);
  }
  for (int e = tid; e <= NX; e += 256) mb.off[e] = r.off[e];
  for (int sl = tid; sl < expert_item_cap(M); sl += 256) {  // M <= 8: one item per active expert
    if (sl < r.na) {
      const int e = r.act[sl];
      int rows = 0;  // bit m: row m has a pair routed to e (pairs sort by row)
      for (int p = r.off[e]; p < r.off[e + 1]; ++p) rows |= 1 << (r.perm[p] / NSLOT);
      mb.act[sl] = e;
      mb.slot_info[sl] = make_int4(e, r.off[e], r.off[e + 1], rows);
      mb.items[sl] = make_int4(e, r.off[e], r.off[e + 1], 0);
    } else {
      if (sl < NX) mb.slot_info[sl] = make_int4(-1, 0, 0, 0);
      mb.items[sl] = make_int4(-1, 0, 0, 0);
    }
  }
  if (tid == 0) {
    *mb.n_act = r.na;
    mb.stats[0] = st0 + r.na;
  }
}

// Router logits: wavefront w of block x computes expert 4x + w for every row
// (RMSNorm'ed with the FFN gain in the prologue; block 0 also stores the
// normalised rows for the experts).  rlogit[m][e] fp32.  ROUTE (M <= MR, one
// block row): the last of the NE / 4 blocks to finish (a counter, *cnt, left
// at zero) routes the rows -- from logit_override instead when it is given,
// which it also copies into rlogit -- and publishes the tables and the taps,
// as k_route_small does after this kernel.  The logits cross blocks through
// agent-scope stores and loads.
template <typename T, int MR, bool ROUTE>
__global__ __launch_bounds__(256) void k_router_logits(const float* __restrict__ x, const float* __restrict__ gain,
                                                       float eps, const T* __restrict__ wr, int M,
                                                       float* __restrict__ bnorm, float* __restrict__ rlogit,
                                                       MoeBufs mb, RouteTap tap,
                                                       const float* __restrict__ logit_override,
                                                       unsigned* __restrict__ cnt) {
  extern __shared__ float xs[];  // [MR][D]
  const int wave = wave_id();
  const int e = blockIdx.x * 4 + wave;
  const int m0 = blockIdx.y * MR;
  const int m_act = min(MR, M - m0);
  const T* rows[1] = {wr + (long)e * D};
  WaveGemv<T, D, 1, MR> g;
  g.load(rows);
  norm_rows_wave<D, MR>(x, D, RowIdentity{m0}, m_act, gain, eps, xs);
  __syncthreads();
  if (blockIdx.x == 0)
    for (int k = threadIdx.x; k < m_act * D; k += 256) bnorm[(long)m0 * D + k] = xs[k];
  float acc[1][MR];
  g.fma(xs, m_act, acc);
  const WaveTotals<1, MR> t(acc);
  if constexpr (!ROUTE) {
    if (t.lead && t.m < m_act) rlogit[(long)(m0 + t.m) * NE + e] = t.val;
  } else {
    __shared__ int s_last;
    __shared__ RouteLds r;
    if (t.lead && t.m < m_act) st_agent(rlogit + (long)(m0 + t.m) * NE + e, t.val);
    stores_done();
    __syncthreads();
    if (threadIdx.x == 0) s_last = atomic_add_agent(cnt, 1u) + 1 == gridDim.x;
    __syncthreads();
    if (!s_last) return;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const long long st0 = (threadIdx.x == 0) ? mb.stats[0] : 0;
    if (logit_override != nullptr) {
      route_rows<false>(logit_override, M, r);
      for (int k = threadIdx.x; k < M * NE; k += 256) rlogit[k] = logit_override[k];
    } else {
      route_rows<true>(rlogit, M, r);
    }
    publish_route(r, M, mb, tap, st0);
    if (threadIdx.x == 0) st_agent_u(cnt, 0u);
  }
}

// M <= 8 without a counter: top-6 per row and the sort by one block,
// published to global.
__global__ __launch_bounds__(256) void k_route_small(const float* __restrict__ rlogit, int M, MoeBufs mb,
                                                     RouteTap tap) {
  __shared__ RouteLds r;
  const long long st0 = (threadIdx.x == 0) ? mb.stats[0] : 0;  // read early: off the kernel's tail
  route_rows<false>(rlogit, M, r);
  publish_route(r, M, mb, tap, st0);
}

// Larger batches (8 < M <= 2048): top-6 per row, one wavefront per row
// (rank_and_gate; lg: the wavefront's 64-float LDS row), published to the
// routing tables and taps; pe (optional, LDS): the row's 8 experts by slot.
__device__ __forceinline__ void topk_row(float v, int m, float* lg, const MoeBufs& mb, const RouteTap& tap,
                                         int* pe) {
  const int lane = lane_id();
  lg[lane] = v;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  int rank;
  float gate;
  rank_and_gate(lg, v, rank, gate);
  if (rank < TOPK) {
    mb.ridx[m * NSLOT + rank] = lane;
    mb.rgate[m * NSLOT + rank] = gate;
    tap_pair(tap, m, rank, lane);
    if (pe != nullptr) pe[rank] = lane;
  }
  if (lane < NSH) {
    mb.ridx[m * NSLOT + TOPK + lane] = NE + lane;
    mb.rgate[m * NSLOT + TOPK + lane] = 1.0f;
    tap_pair(tap, m, TOPK + lane, NE + lane);
    if (pe != nullptr) pe[TOPK + lane] = NE + lane;
  }
  __builtin_amdgcn_wave_barrier();  // lg is read by every lane before the next row overwrites it
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
}

__global__ __launch_bounds__(256) void k_topk_rows(const float* __restrict__ rlogit, int M, MoeBufs mb,
                                                   RouteTap tap) {
  __shared__ float lg[4][NE];
  const int wave = wave_id(), lane = lane_id();
  const int m = blockIdx.x * 4 + wave;
  if (m >= M) return;
  topk_row(rlogit[(long)m * NE + lane], m, lg[wave], mb, tap, nullptr);
}

// ... then a stable counting sort of the 8M pairs by expert in one 1024-thread
// block.  Wavefront w owns rows [w M / 16, (w + 1) M / 16), i.e. a contiguous
// pair range, read in segments of 64 pairs (lane = pair; all segments' loads
// issued together).  Seven ballots over a segment's expert-id bits give each
// pair its rank among the range's earlier pairs of the same expert (the
// range's running counts in LDS).  The per-range counts give per-expert offsets (experts in id
// order) and per-range bases; pair p lands at off[e] + base[w][e] + rank --
// the permutation of any stable sort by expert id.  TOPK_IN (M <= RL_TOPK_ROWS):
// each wavefront first takes the top-6 of its own rows (as k_topk_rows does),
// keeping the pairs' experts in LDS -- one launch instead of two.
constexpr int RL_WAVES = 16;
constexpr int RL_SEGS = 16;  // segments per wavefront: M <= RL_WAVES * RL_SEGS * 8 = 2048
constexpr int RL_TOPK_ROWS = 128;
constexpr int RL_TOPK_RPW = RL_TOPK_ROWS / RL_WAVES;  // rows per wavefront at most
template <bool TOPK_IN>
__global__ __launch_bounds__(1024) void k_sort_pairs(int M, MoeBufs mb, RouteTap tap) {
  __shared__ int wcnt[RL_WAVES][NX + 1];  // per range: counts, then exclusive bases
  __shared__ int tot[NX + 1], off[NX + 1], act[NX + 1], ioff[NX + 1];
  __shared__ int na_s;
  const int wave = threadIdx.x >> 6, lane = lane_id(), tid = threadIdx.x;
  const int r_lo = M * wave / RL_WAVES, r_hi = M * (wave + 1) / RL_WAVES;
  const int p_lo = NSLOT * r_lo, p_hi = NSLOT * r_hi;
  const uint64_t lt = (1ull << lane) - 1ull;
  int seg_e[RL_SEGS], seg_rank[RL_SEGS];
  if constexpr (TOPK_IN) {
    __shared__ float lg[RL_WAVES][NE];
    __shared__ int pe[RL_WAVES][RL_TOPK_RPW * NSLOT];
    float v[RL_TOPK_RPW];
#pragma unroll
    for (int j = 0; j < RL_TOPK_RPW; ++j) v[j] = (r_lo + j < r_hi) ? mb.rlogit[(long)(r_lo + j) * NE + lane] : 0.f;
#pragma unroll
    for (int j = 0; j < RL_TOPK_RPW; ++j)
      if (r_lo + j < r_hi) topk_row(v[j], r_lo + j, lg[wave], mb, tap, &pe[wave][j * NSLOT]);
    static_assert(RL_TOPK_RPW * NSLOT <= 64, "one segment per wavefront");
    seg_e[0] = (p_lo + lane < p_hi) ? pe[wave][lane] : -1;
    seg_rank[0] = 0;
#pragma unroll
    for (int sg = 1; sg < RL_SEGS; ++sg) {
      seg_e[sg] = -1;
      seg_rank[sg] = 0;
    }
  } else {
#pragma unroll
    for (int sg = 0; sg < RL_SEGS; ++sg) {
      const int p = p_lo + 64 * sg + lane;
      seg_e[sg] = (p < p_hi) ? mb.ridx[p] : -1;
      seg_rank[sg] = 0;
    }
  }
  // running count of each expert in this range (LDS, one row per wavefront):
  // a segment's equal experts are found from seven ballots over the id bits;
  // a pair's rank = the expert's count before the segment + the equal lanes
  // below it; the lowest of them then adds the segment's count
  int* cnt = wcnt[wave];
  for (int x = lane; x <= NX; x += 64) cnt[x] = 0;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
#pragma unroll
  for (int sg = 0; sg < RL_SEGS; ++sg) {
    if (p_lo + 64 * sg >= p_hi) break;
    const int e = seg_e[sg];
    const bool valid = e >= 0;
    uint64_t same = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 7; ++bit) {
      const uint64_t set = __ballot(valid && ((e >> bit) & 1));
      same &= (valid && ((e >> bit) & 1)) ? set : ~set;
    }
    const int below = __popcll(same & lt);
    const int before = valid ? cnt[e] : 0;
    seg_rank[sg] = before + below;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
    if (valid && below == 0) cnt[e] = before + __popcll(same);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
  }
  __syncthreads();
  // per-expert totals; per-range exclusive bases
  if (tid < NX) {
    int acc = 0;
    for (int w = 0; w < RL_WAVES; ++w) {
      const int c = wcnt[w][tid];
      wcnt[w][tid] = acc;
      acc += c;
    }
    tot[tid] = acc;
  }
  __syncthreads();
  // offsets (experts in id order), the active list (routed experts in id
  // order, then the shared ones) and each active expert's first work item
  // (ITEM_PAIRS pairs per item), by wavefront scans in wavefront 0
  if (wave == 0) {
    const int c = tot[lane];  // routed expert `lane`
    const int c64 = tot[NE], c65 = tot[NE + 1];
    const int incl = wave_incl_scan(c);
    const int routed = __builtin_amdgcn_readlane(incl, 63);
    off[lane] = incl - c;
    const uint64_t am = __ballot(c > 0);
    const int nr = __popcll(am);
    const int nit = (c + ITEM_PAIRS - 1) / ITEM_PAIRS;  // 0 for an idle expert
    const int iincl = wave_incl_scan(nit);
    if (c > 0) {
      const int sl = __popcll(am & lt);
      act[sl] = lane;
      ioff[sl] = iincl - nit;
    }
    if (lane == 0) {
      off[NE] = routed;
      off[NE + 1] = routed + c64;
      off[NX] = routed + c64 + c65;
      int na = nr, it = __builtin_amdgcn_readlane(iincl, 63);
      if (c64 > 0) {
        act[na] = NE;
        ioff[na++] = it;
        it += (c64 + ITEM_PAIRS - 1) / ITEM_PAIRS;
      }
      if (c65 > 0) {
        act[na] = NE + 1;
        ioff[na++] = it;
        it += (c65 + ITEM_PAIRS - 1) / ITEM_PAIRS;
      }
      ioff[na] = it;
      na_s = na;
      *mb.n_act = na;
      mb.stats[0] += na;
    }
  }
  __syncthreads();
  const int na = na_s;
  for (int sl = tid; sl < na; sl += 1024) {
    const int e = act[sl];
    for (int i = ioff[sl], k = off[e]; i < ioff[sl + 1]; ++i, k += ITEM_PAIRS)
      mb.items[i] = make_int4(e, k, min(k + ITEM_PAIRS, off[e + 1]), 0);
  }
  for (int i = ioff[na] + tid; i < expert_item_cap(M); i += 1024) mb.items[i] = make_int4(-1, 0, 0, 0);
  for (int e = tid; e <= NX; e += 1024) mb.off[e] = off[e];
  for (int sl = tid; sl < NX; sl += 1024) {
    if (sl < na) {
      mb.act[sl] = act[sl];
      mb.slot_info[sl] = make_int4(act[sl], off[act[sl]], off[act[sl] + 1], na);
    } else {
      mb.slot_info[sl] = make_int4(-1, 0, 0, na);
    }
  }
  // final positions
#pragma unroll
  for (int sg = 0; sg < RL_SEGS; ++sg) {
    const int e = seg_e[sg];
    if (e >= 0) {
      const int p = p_lo + 64 * sg + lane;
      const int pos = off[e] + wcnt[wave][e] + seg_rank[sg];
      mb.perm[pos] = p;
      mb.inv[p] = pos;
    }
  }
}

int expert_slot_cap(int M) { return min(NE, TOPK * M) + NSH; }

// Router: logits in a 16-block kernel, then the top-6 and the sort (one
// block for M <= 8; a per-row top-6 kernel and a one-block sort beyond).
// Router logits into mb.rlogit (or a copy of logit_override) and the
// normalised rows into mb.bnorm.
template <typename T>
void launch_router_logits(hipStream_t s, const float* x, const float* gain, float eps, const T* wr, int M,
                          const MoeBufs& mb, const float* logit_override) {
#define OCR_RL_CASE(MRV)                                                                                   \
  hipLaunchKernelGGL((k_router_logits<T, MRV, false>), dim3(NE / 4, (M + MRV - 1) / MRV), dim3(256),       \
                     (size_t)MRV * D * 4, s, x, gain, eps, wr, M, mb.bnorm, mb.rlogit, mb, RouteTap{}, nullptr,  \
                     nullptr);
  if (M <= 1) OCR_RL_CASE(1)
  else if (M <= 2) OCR_RL_CASE(2)
  else if (M <= 4) OCR_RL_CASE(4)
  else OCR_RL_CASE(MRG)
#undef OCR_RL_CASE
  if (logit_override != nullptr) launch_copy_rows(s, logit_override, mb.rlogit, (long)M * NE);
}

template <typename T>
void launch_router(hipStream_t s, const float* x, const float* gain, float eps, const T* wr, int M,
                   const MoeBufs& mb, const RouteTap& tap, const float* logit_override, unsigned* cnt) {
  if (M <= MRG && cnt != nullptr) {  // one launch: the last logits block routes
#define OCR_RR_CASE(MRV)                                                                                 \
  hipLaunchKernelGGL((k_router_logits<T, MRV, true>), dim3(NE / 4, 1), dim3(256), (size_t)MRV * D * 4, s, x, \
                     gain, eps, wr, M, mb.bnorm, mb.rlogit, mb, tap, logit_override, cnt);
    if (M <= 1) OCR_RR_CASE(1)
    else if (M <= 2) OCR_RR_CASE(2)
    else if (M <= 4) OCR_RR_CASE(4)
    else OCR_RR_CASE(MRG)
#undef OCR_RR_CASE
    return;
  }
  launch_router_logits<T>(s, x, gain, eps, wr, M, mb, logit_override);
  if (M <= MRG) {
    hipLaunchKernelGGL(k_route_small, dim3(1), dim3(256), 0, s, mb.rlogit, M, mb, tap);
  } else if (M <= RL_TOPK_ROWS) {
    hipLaunchKernelGGL(k_sort_pairs<true>, dim3(1), dim3(1024), 0, s, M, mb, tap);
  } else {
    hipLaunchKernelGGL(k_topk_rows, dim3((M + 3) / 4), dim3(256), 0, s, mb.rlogit, M, mb, tap);
    hipLaunchKernelGGL(k_sort_pairs<false>, dim3(1), dim3(1024), 0, s, M, mb, RouteTap{});
  }
}

// Gather the activation rows m < m_act <= MR (row_of(m) into src) into LDS;
// 256 threads, 16-byte loads (rows are whole multiples of 16 bytes), the loads
// of every row issued before any LDS store.
template <int K, int MR, typename SrcRow>
__device__ __forceinline__ void gather_rows(const float* __restrict__ src, SrcRow row_of, int m_act, float* xs) {
  static_assert(K % 4 == 0, "row length");
  constexpr int K4 = K / 4;
  constexpr int J = (K4 + 255) / 256;
  float4 v[MR][J];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    if (m < m_act) {
      const float4* r = reinterpret_cast<const float4*>(src + (long)row_of(m) * K);
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int k = threadIdx.x + 256 * j;
        v[m][j] = (k < K4) ? r[k] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    if (m < m_act) {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int k = threadIdx.x + 256 * j;
        if (k < K4) reinterpret_cast<float4*>(xs + m * K)[k] = v[m][j];
      }
    }
  }
}

// Gate/up (M <= 8): block (x, slot s) handles active expert s; wavefront w
// owns units j0 .. j0+UPW-1, j0 = UPW (4x + w): rows gate[j] then up[j], all
// loads issued at once.  The (at most MR) pairs routed to the expert get
// hx[pair][j] = silu(gate . b) * (up . b).  expert_work gives the expert, its
// pair range and a bit mask of its rows: the shared experts' blocks need no
// read for it, the routed ones fetch weights and normalised rows after one
// dependent read of the routing table.
template <typename T, int MR, int UPW>
__global__ __launch_bounds__(256) void k_expert_gate_up(const T* __restrict__ wg, const T* __restrict__ wu, int M,
                                                        MoeBufs mb) {
  extern __shared__ float xs[];
  const int wave = wave_id();
  const int4 info = expert_work(mb, blockIdx.y, M);
  const int e = info.x;
  if (e < 0) return;
  const int k0 = info.y;
  const int m_act = min(MR, info.z - k0);
  const int j0 = (blockIdx.x * 4 + wave) * UPW;
  const T* gbase = wg + ((long)e * DI + j0) * D;
  const T* ubase = wu + ((long)e * DI + j0) * D;
  const T* rows[2 * UPW];
#pragma unroll
  for (int u = 0; u < UPW; ++u) {
    rows[u] = gbase + (long)u * D;
    rows[UPW + u] = ubase + (long)u * D;
  }
  WaveGemv<T, D, 2 * UPW, MR> g;
  g.load(rows);
  const int mask = info.w;
  gather_rows<D, MR>(mb.bnorm, [=](int m) {  // the m-th set bit of the row mask
    int mk = mask;
    for (int i = 0; i < m; ++i) mk &= mk - 1;
    return __builtin_ctz(mk);
  }, m_act, xs);
  __syncthreads();
  float acc[2 * UPW][MR];
  g.fma(xs, m_act, acc);
  const WaveTotals<2 * UPW, MR> t(acc);
  const float up = t.partner(UPW);  // gate unit u pairs with up unit u (r = u, UPW + u)
  if (t.lead && t.r < UPW && t.m < m_act) mb.hx[(long)(k0 + t.m) * DI + j0 + t.r] = silu(t.val) * up;
}

// Down (M <= 8) and the combine: block (x, slot s); wavefront w owns output
// rows n0 .. n0+RPW-1, n0 = RPW (4x + w): y[pair][n] = W_d[n] . hx[pair].  The
// last block of column x to finish (a counter per column, cnt[x * 32], left
// at zero) adds the column's 4 RPW outputs of every row to the residual:
// x[m][n] += y_shared0 + y_shared1 + sum_j gate_j * y_routed_j, in this
// order, the arithmetic of k_moe_combine.  y crosses blocks through
// agent-scope stores and loads.
constexpr int DN_CNT_STRIDE = 32;
template <typename T, int MR, int RPW>
__global__ __launch_bounds__(256) void k_expert_down(const T* __restrict__ wd, int M, MoeBufs mb,
                                                     float* __restrict__ x, unsigned* __restrict__ cnt) {
  extern __shared__ float xs[];
  __shared__ int s_last;
  const int4 info = expert_work(mb, blockIdx.y, M);
  const int e = info.x;
  const int wave = wave_id(), tid = threadIdx.x;
  if (e >= 0) {
    const int k0 = info.y;
    const int m_act = min(MR, info.z - k0);
    const int n0 = (blockIdx.x * 4 + wave) * RPW;
    const T* base = wd + ((long)e * D + n0) * DI;
    const T* rows[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) rows[r] = base + (long)r * DI;
    WaveGemv<T, DI, RPW, MR> g;
    g.load(rows);
    gather_rows<DI, MR>(mb.hx, [&](int m) { return k0 + m; }, m_act, xs);
    __syncthreads();
    float acc[RPW][MR];
    g.fma(xs, m_act, acc);
    const WaveTotals<RPW, MR> t(acc);
    if (t.lead && t.m < m_act) st_agent(mb.y + (long)(k0 + t.m) * D + n0 + t.r, t.val);
  }
  stores_done();
  __syncthreads();
  unsigned* c = cnt + blockIdx.x * DN_CNT_STRIDE;
  if (tid == 0) s_last = atomic_add_agent(c, 1u) + 1 == gridDim.y;
  __syncthreads();
  if (!s_last) return;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  constexpr int W = 4 * RPW;  // outputs of the column
  if (tid < W * M) {
    const int m = tid / W, n = blockIdx.x * W + tid % W;
    const int* inv = mb.inv + m * NSLOT;
    const float* gt = mb.rgate + m * NSLOT;
    float a = ld_agent(mb.y + (long)inv[TOPK] * D + n);
    a += ld_agent(mb.y + (long)inv[TOPK + 1] * D + n);
#pragma unroll
    for (int j = 0; j < TOPK; ++j) a = fmaf(gt[j], ld_agent(mb.y + (long)inv[j] * D + n), a);
    x[(long)m * D + n] += a;
  }
  if (tid == 0) st_agent_u(c, 0u);
}

// Batches with more than MRG rows: the same per-row arithmetic, MRG pairs at a
// time, one tile per wavefront, the tile re-read for every group of pairs.
template <typename T>
__global__ __launch_bounds__(256) void k_expert_gate_up_groups(const T* __restrict__ wg, const T* __restrict__ wu,
                                                               int M, MoeBufs mb) {
  extern __shared__ float xs[];
  const int4 info = expert_work(mb, blockIdx.y, M);
  const int e = info.x;
  if (e < 0) return;
  const int wave = wave_id();
  const int j = (blockIdx.x * 4 + wave) * 2;
  for (int kb = info.y; kb < info.z; kb += MRG) {
    const int m_act = min(MRG, info.z - kb);
    const T* gb = wg + ((long)e * DI + j) * D;
    const T* ub = wu + ((long)e * DI + j) * D;
    asm volatile("" : "+v"(gb), "+v"(ub));  // the weights are re-read per group, not hoisted
    const T* rows[4] = {gb, gb + D, ub, ub + D};
    WaveGemv<T, D, 4, MRG> g;
    g.load(rows);
    gather_rows<D, MRG>(mb.bnorm, [&](int m) { return mb.perm[kb + m] / NSLOT; }, m_act, xs);
    __syncthreads();
    float acc[4][MRG];
    g.fma(xs, m_act, acc);
    const WaveTotals<4, MRG> t(acc);
    const float up = t.partner(2);  // rows gate j, j+1, up j, j+1
    if (t.lead && t.r < 2 && t.m < m_act) mb.hx[(long)(kb + t.m) * DI + j + t.r] = silu(t.val) * up;
    __syncthreads();
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_expert_down_groups(const T* __restrict__ wd, int M, MoeBufs mb) {
  extern __shared__ float xs[];
  const int4 info = expert_work(mb, blockIdx.y, M);
  const int e = info.x;
  if (e < 0) return;
  const int wave = wave_id();
  const int n0 = (blockIdx.x * 4 + wave) * 4;
  for (int kb = info.y; kb < info.z; kb += MRG) {
    const int m_act = min(MRG, info.z - kb);
    const T* b = wd + ((long)e * D + n0) * DI;
    asm volatile("" : "+v"(b));
    const T* rows[4] = {b, b + DI, b + 2 * DI, b + 3 * DI};
    WaveGemv<T, DI, 4, MRG> g;
    g.load(rows);
    gather_rows<DI, MRG>(mb.hx, [&](int m) { return kb + m; }, m_act, xs);
    __syncthreads();
    float acc[4][MRG];
    g.fma(xs, m_act, acc);
    const WaveTotals<4, MRG> t(acc);
    if (t.lead && t.m < m_act) mb.y[(long)(kb + t.m) * D + n0 + t.r] = t.val;
    __syncthreads();
  }
}

#ifndef OCR_GU_UPW
#define OCR_GU_UPW 1
#endif
#ifndef OCR_DN_RPW
#define OCR_DN_RPW 4
#endif
constexpr int GU_UPW = OCR_GU_UPW;   // gate/up units per wavefront
constexpr int DN_RPW = OCR_DN_RPW;   // down rows per wavefront
static_assert((D / (4 * DN_RPW)) * DN_CNT_STRIDE <= DOWN_CNT_WORDS, "down-combine counters");

template <typename T>
void launch_expert_gate_up(hipStream_t s, const T* wg, const T* wu, int M, const MoeBufs& mb) {
  const dim3 grid(DI / (4 * GU_UPW), expert_slot_cap(M));
#define OCR_GU_CASE(MRV) \
  hipLaunchKernelGGL((k_expert_gate_up<T, MRV, GU_UPW>), grid, dim3(256), (size_t)MRV * D * 4, s, wg, wu, M, mb);
  if (M <= 1) OCR_GU_CASE(1)
  else if (M <= 2) OCR_GU_CASE(2)
  else if (M <= 4) OCR_GU_CASE(4)
  else if (M <= MRG) OCR_GU_CASE(MRG)
  else
    hipLaunchKernelGGL((k_expert_gate_up_groups<T>), dim3(DI / 8, expert_slot_cap(M)), dim3(256),
                       (size_t)MRG * D * 4, s, wg, wu, M, mb);
#undef OCR_GU_CASE
}

template <typename T>
void launch_expert_down(hipStream_t s, const T* wd, int M, const MoeBufs& mb) {
  hipLaunchKernelGGL((k_expert_down_groups<T>), dim3(D / 16, expert_slot_cap(M)), dim3(256),
                     (size_t)MRG * DI * 4, s, wd, M, mb);
}

template <typename T>
void launch_expert_down_combine(hipStream_t s, const T* wd, int M, const MoeBufs& mb, float* x, unsigned* cnt) {
  const dim3 grid(D / (4 * DN_RPW), expert_slot_cap(M));
#define OCR_DN_CASE(MRV)                                                                                     \
  hipLaunchKernelGGL((k_expert_down<T, MRV, DN_RPW>), grid, dim3(256), (size_t)MRV * DI * 4, s, wd, M, mb, x, \
                     cnt);
  if (M <= 1) OCR_DN_CASE(1)
  else if (M <= 2) OCR_DN_CASE(2)
  else if (M <= 4) OCR_DN_CASE(4)
  else OCR_DN_CASE(MRG)
#undef OCR_DN_CASE
}

// x[r] += y_shared0 + y_shared1 + sum_j gate_j * y_routed_j, in this order.
__global__ __launch_bounds__(256) void k_moe_combine(float* __restrict__ x, MoeBufs mb) {
  const int r = blockIdx.x;
  const int* inv = mb.inv + r * NSLOT;
  const float* gt = mb.rgate + r * NSLOT;
  static_assert(D % 256 == 0, "row length");
#pragma unroll
  for (int t = 0; t < D / 256; ++t) {  // unrolled: every load of the row goes out at once
    const int n = threadIdx.x + 256 * t;
    float acc = mb.y[(long)inv[TOPK] * D + n];
    acc += mb.y[(long)inv[TOPK + 1] * D + n];
#pragma unroll
    for (int j = 0; j < TOPK; ++j) acc = fmaf(gt[j], mb.y[(long)inv[j] * D + n], acc);
    x[(long)r * D + n] += acc;
  }
}

void launch_moe_combine(hipStream_t s, float* x, int M, const MoeBufs& mb) {
  hipLaunchKernelGGL(k_moe_combine, dim3(M), dim3(256), 0, s, x, mb);
}

#define OCR_INST_MOE(T)                                                                                  \
  template void launch_router<T>(hipStream_t, const float*, const float*, float, const T*, int,          \
                                 const MoeBufs&, const RouteTap&, const float*, unsigned*);              \
  template void launch_router_logits<T>(hipStream_t, const float*, const float*, float, const T*, int,   \
                                        const MoeBufs&, const float*);                                   \
  template void launch_expert_gate_up<T>(hipStream_t, const T*, const T*, int, const MoeBufs&);                \
  template void launch_expert_down<T>(hipStream_t, const T*, int, const MoeBufs&);                           \
  template void launch_expert_down_combine<T>(hipStream_t, const T*, int, const MoeBufs&, float*, unsigned*);
OCR_INST_MOE(float)
OCR_INST_MOE(bf16)

}  // namespace ocr

namespace ocr {

// ---- the experts of a decoder layer in one persistent launch (M <= 8) -------
//
// After the router-logits launch (which also stores the normalised rows), one
// launch does what the routing, gate/up, down and combine launches do, with
// the same arithmetic (so the same bits), waiting inside the launch only where
// the data requires it: every workgroup routes the rows itself from the
// logits (a few hundred cycles); the gate/up items of the two shared experts
// need no routing and their weights go out first; the down items wait until
// every gate/up item is done, with their weights already in flight; per slice
// of 16 outputs, the workgroup that finishes the last expert of the slice adds
// the slice to the residual in the fixed order.  Data that crosses workgroups
// goes through agent-scope stores and loads (no L2 write-back or invalidate
// is needed); the counters are agent-scope atomics.  The wait polls a ready
// flag that the last arriver writes to 32 cache lines, each polled by one
// lane of the workgroups of one stripe, so that the polls do not crowd one
// line while other workgroups still stream their weights.  Every wait is
// bounded: a timeout (a grid that is not all resident) sets the error word,
// which the host reports, and the launch runs to its end.  The grid is at
// most the number of workgroups the GPU holds at once; each launch leaves
// every counter at zero for the next.
constexpr int FZ_STRIPES = 32;
constexpr int FZ_SLICES = D / 16;     // down slices of 16 outputs (4 wavefronts x 4 rows)
constexpr int FZ_GU = DI / 4;         // gate/up items per expert (one unit per wavefront)
// Sync words, one cache line (32 words) apart where several workgroups meet:
// line 0: (unused), gate/up top count, done top count, error word;
// lines 1+s: gate/up count of stripe s; 33+s: done count of stripe s;
// 97+s: gate/up-done flag copy s; 129+x: done count of down slice x.
constexpr int FZ_LINE = 32;
constexpr int FZ_S_GUTOP = 1, FZ_S_TOP = 2, FZ_S_ERR = MOE_SYNC_ERR;
constexpr int FZ_S_GU = 1 * FZ_LINE, FZ_S_DONE = 33 * FZ_LINE, FZ_S_GFLAG = 97 * FZ_LINE,
              FZ_S_SLICE = 129 * FZ_LINE;
static_assert(FZ_S_ERR > FZ_S_TOP && FZ_S_ERR < FZ_LINE && FZ_S_SLICE + FZ_SLICES * FZ_LINE <= MOE_SYNC_WORDS,
              "sync word layout");

// One thread: wait until the flag is set, bounded; on timeout (or an earlier
// one) set / see the error word and give up.
__device__ __forceinline__ void wait_flag(const unsigned* flag, unsigned* err) {
  for (int n = 0; n < (1 << 20); ++n) {
    if (ld_agent_u(flag) != 0u) { __atomic_signal_fence(__ATOMIC_SEQ_CST); return; }
    if ((n & 15) == 15 && ld_agent_u(err) != 0) return;
    __builtin_amdgcn_s_sleep(4);
  }
  st_agent_u(err, 1u);
}

// Set the 32 copies of a ready flag (one cache line apart).
__device__ __forceinline__ void raise_flag(unsigned* flags) {
  for (int s = 0; s < FZ_STRIPES; ++s) st_agent_u(flags + s * FZ_LINE, 1u);
}

// Workgroups b < G with b % FZ_STRIPES == s.
__device__ __forceinline__ unsigned stripe_count(int G, int s) {
  return s < G ? (unsigned)((G - s + FZ_STRIPES - 1) / FZ_STRIPES) : 0u;
}

// x_out = x_in + the experts' combine; the normalised rows come from
// mb.bnorm and the router logits from mb.rlogit (the router-logits launch).
template <typename T, int MR>
__global__ __launch_bounds__(256) void k_moe_fused(const float* __restrict__ x_in, float* __restrict__ x_out,
                                                   const T* __restrict__ wg, const T* __restrict__ wu,
                                                   const T* __restrict__ wd, int M, MoeBufs mb, RouteTap tap,
                                                   unsigned* __restrict__ sync) {
  extern __shared__ float xs[];  // [MR][D] normalised rows; in the down phase [MR][DI] expert hidden rows
  __shared__ RouteLds r;
  __shared__ int s_flag;
  const int G = gridDim.x, b = blockIdx.x, wave = wave_id(), tid = threadIdx.x;
  unsigned* err = sync + FZ_S_ERR;
  const long long st0 = (b == 0 && tid == 0) ? mb.stats[0] : 0;

  // gate/up item i: expert slot i / FZ_GU (0, 1: the shared experts, then the
  // routed ones in increasing id), unit 4 (i % FZ_GU) + wave
  auto item_expert = [&](int slot, int& e, int& k0, int& m_act, int (&rows)[MR]) {
    if (slot < NSH) {  // known without the routing: all rows, after the 6M routed pairs
      e = NE + slot;
      k0 = (TOPK + slot) * M;
      m_act = M;
#pragma unroll
      for (int m = 0; m < MR; ++m) rows[m] = m;
    } else {
      e = r.act[slot - NSH];
      k0 = r.off[e];
      m_act = r.off[e + 1] - k0;
#pragma unroll
      for (int m = 0; m < MR; ++m) rows[m] = r.perm[k0 + min(m, max(m_act - 1, 0))] / NSLOT;
    }
  };
  // the first gate/up item's weights go out before anything else
  int i = b;
  bool have = i < NSH * FZ_GU;
  WaveGemv<T, D, 2, MR> g0, g1;
  if (have) {
    const int e = NE + i / FZ_GU, j = (i % FZ_GU) * 4 + wave;
    const T* rows[2] = {wg + ((long)e * DI + j) * D, wu + ((long)e * DI + j) * D};
    g0.load(rows);
  }
  // the normalised rows (all M of them) into LDS, then the routing
  for (int q = tid; q < M * D; q += 256) xs[q] = mb.bnorm[q];
  route_rows(mb.rlogit, M, r);
  if (b == 0) publish_route(r, M, mb, tap, st0);
  __syncthreads();
  const int n_gu = r.na * FZ_GU;
  if (!have) {
    have = i < n_gu;
    if (have) {
      int e, k0, m_act, rows_i[MR];
      item_expert(i / FZ_GU, e, k0, m_act, rows_i);
      const int j = (i % FZ_GU) * 4 + wave;
      const T* rows[2] = {wg + ((long)e * DI + j) * D, wu + ((long)e * DI + j) * D};
      g0.load(rows);
    }
  }
  // gate/up items, two in flight per wavefront
  auto gate_up = [&](const WaveGemv<T, D, 2, MR>& g, int it) {
    int e, k0, m_act, rows_i[MR];
    item_expert(it / FZ_GU, e, k0, m_act, rows_i);
    const int j = (it % FZ_GU) * 4 + wave;
    float acc[2][MR];
    g.fma_rows(xs, rows_i, m_act, acc);
    const WaveTotals<2, MR> t(acc);
    const float up = t.partner(1);
    if (t.lead && t.r < 1 && t.m < m_act) st_agent(mb.hx + (long)(k0 + t.m) * DI + j, silu(t.val) * up);
  };
  for (int par = 0; have; par ^= 1) {
    const int inext = i + G;
    const bool hnext = inext < n_gu;
    if (hnext) {
      int e, k0, m_act, rows_i[MR];
      item_expert(inext / FZ_GU, e, k0, m_act, rows_i);
      const int j = (inext % FZ_GU) * 4 + wave;
      const T* rows[2] = {wg + ((long)e * DI + j) * D, wu + ((long)e * DI + j) * D};
      if (par) g0.load(rows); else g1.load(rows);
    }
    if (par) gate_up(g1, i); else gate_up(g0, i);
    i = inext;
    have = hnext;
  }
  stores_done();
  __syncthreads();
  if (tid == 0) {  // the last workgroup of a stripe counts the stripe; the last stripe raises the flag
    const int st = b % FZ_STRIPES;
    if (atomic_add_agent(sync + FZ_S_GU + st * FZ_LINE, 1u) + 1 == stripe_count(G, st) &&
        atomic_add_agent(sync + FZ_S_GUTOP, 1u) + 1 == (unsigned)min(G, FZ_STRIPES)) {
      stores_done();
      raise_flag(sync + FZ_S_GFLAG);
    }
  }

  // down items: a contiguous range per workgroup (consecutive slices of one expert share the gather)
  const int n_dn = r.na * FZ_SLICES;
  const int lo = (int)((long)b * n_dn / G), hi = (int)((long)(b + 1) * n_dn / G);
  WaveGemv<T, DI, 4, MR> gd;
  auto dn_rows = [&](int it, const T* (&rows)[4]) {
    int e, k0, m_act, rows_i[MR];
    item_expert(it / FZ_SLICES, e, k0, m_act, rows_i);
    const int n0 = ((it % FZ_SLICES) * 4 + wave) * 4;
#pragma unroll
    for (int q = 0; q < 4; ++q) rows[q] = wd + ((long)e * D + n0 + q) * DI;
  };
  if (lo < hi) {
    const T* rows[4];
    dn_rows(lo, rows);
    gd.load(rows);
  }
  // every gate/up item of the grid is done
  if (tid == 0) wait_flag(sync + FZ_S_GFLAG + (b % FZ_STRIPES) * FZ_LINE, err);
  __syncthreads();
  int cur_slot = -1;
  for (int it = lo; it < hi; ++it) {
    const int slot = it / FZ_SLICES, xsl = it % FZ_SLICES;
    int e, k0, m_act, rows_i[MR];
    item_expert(slot, e, k0, m_act, rows_i);
    if (slot != cur_slot) {  // the expert's hidden rows k0 .. k0 + m_act - 1 into LDS
      if (cur_slot >= 0) __syncthreads();
      for (int q = tid; q < m_act * DI; q += 256) xs[q] = ld_agent(mb.hx + (long)k0 * DI + q);
      __syncthreads();
      cur_slot = slot;
    }
    float acc[4][MR];
    gd.fma(xs, m_act, acc);
    if (it + 1 < hi) {
      const T* rows[4];
      dn_rows(it + 1, rows);
      gd.load(rows);
    }
    const WaveTotals<4, MR> t(acc);
    const int n0 = (xsl * 4 + wave) * 4;
    if (t.lead && t.m < m_act) st_agent(mb.y + (long)(k0 + t.m) * D + n0 + t.r, t.val);
    stores_done();
    __syncthreads();
    if (tid == 0) {
      const unsigned old = atomic_add_agent(sync + FZ_S_SLICE + xsl * FZ_LINE, 1u);
      s_flag = old + 1 == (unsigned)r.na;
    }
    __syncthreads();
    if (s_flag) {  // the last expert of this slice: x += shared 0 + shared 1 + sum gate_j y_j, in this order
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      if (tid < 16 * M) {
        const int m = tid / 16, n = xsl * 16 + tid % 16;
        const int* inv = r.inv + m * NSLOT;
        const float* gt = r.pg + m * NSLOT;
        float acc2 = ld_agent(mb.y + (long)inv[TOPK] * D + n);
        acc2 += ld_agent(mb.y + (long)inv[TOPK + 1] * D + n);
#pragma unroll
        for (int jj = 0; jj < TOPK; ++jj) acc2 = fmaf(gt[jj], ld_agent(mb.y + (long)inv[jj] * D + n), acc2);
        x_out[(long)m * D + n] = x_in[(long)m * D + n] + acc2;
      }
      if (tid == 0) st_agent_u(sync + FZ_S_SLICE + xsl * FZ_LINE, 0u);  // its last user this launch
    }
  }
  // leave the counters at zero: the last workgroup to finish resets them
  stores_done();
  __syncthreads();
  if (tid == 0) {
    const int st = b % FZ_STRIPES;
    if (atomic_add_agent(sync + FZ_S_DONE + st * FZ_LINE, 1u) + 1 == stripe_count(G, st)) {
      if (atomic_add_agent(sync + FZ_S_TOP, 1u) + 1 == (unsigned)min(G, FZ_STRIPES)) {
        st_agent_u(sync + FZ_S_GUTOP, 0u);
        for (int q = 0; q < FZ_STRIPES; ++q) {
          st_agent_u(sync + FZ_S_GU + q * FZ_LINE, 0u);
          st_agent_u(sync + FZ_S_DONE + q * FZ_LINE, 0u);
          st_agent_u(sync + FZ_S_GFLAG + q * FZ_LINE, 0u);
        }
        st_agent_u(sync + FZ_S_TOP, 0u);
      }
    }
  }
}

template <typename T, int MR>
static size_t moe_fused_lds() {
  return (size_t)MR * D * 4;
}

template <typename T>
int moe_fused_grid(int n_cu) {
  // the grid must be resident all at once: workgroups per CU for the largest
  // variant (8 rows, the most LDS), at most 4
  int occ = 0;
  const size_t lds = moe_fused_lds<T, MRG>();
  allow_lds(k_moe_fused<T, MRG>, lds);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k_moe_fused<T, MRG>, 256, lds) != hipSuccess || occ < 1)
    return 0;
  return std::min(occ, 4) * n_cu;
}

template <typename T>
void launch_moe_experts(hipStream_t s, int grid, const float* x_in, float* x_out, const T* wg, const T* wu,
                        const T* wd, int M, const MoeBufs& mb, const RouteTap& tap, unsigned* sync) {
#define OCR_FZ_CASE(MRV)                                                                                      \
  {                                                                                                           \
    const size_t lds = moe_fused_lds<T, MRV>();                                                               \
    static const bool attr_set = (allow_lds(k_moe_fused<T, MRV>, lds), true);                                 \
    (void)attr_set;                                                                                           \
    hipLaunchKernelGGL((k_moe_fused<T, MRV>), dim3(grid), dim3(256), lds, s, x_in, x_out, wg, wu, wd, M, mb,  \
                       tap, sync);                                                                            \
  }
  if (M <= 1) OCR_FZ_CASE(1)
  else if (M <= 2) OCR_FZ_CASE(2)
  else if (M <= 4) OCR_FZ_CASE(4)
  else OCR_FZ_CASE(MRG)
#undef OCR_FZ_CASE
}

template int moe_fused_grid<float>(int);
template int moe_fused_grid<bf16>(int);
template void launch_moe_experts<float>(hipStream_t, int, const float*, float*, const float*, const float*,
                                        const float*, int, const MoeBufs&, const RouteTap&, unsigned*);
template void launch_moe_experts<bf16>(hipStream_t, int, const float*, float*, const bf16*, const bf16*,
                                       const bf16*, int, const MoeBufs&, const RouteTap&, unsigned*);

}  // namespace ocr
