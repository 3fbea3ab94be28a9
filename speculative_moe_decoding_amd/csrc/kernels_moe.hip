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
  // inclusive scan of the counts: within each 16-lane row by DPP row shifts
  // (lanes past the row's start read 0), then the row totals as scalars
  int incl = c;
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x111, 0xF, 0xF, false);  // row_shr:1
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x112, 0xF, 0xF, false);  // row_shr:2
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x114, 0xF, 0xF, false);  // row_shr:4
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x118, 0xF, 0xF, false);  // row_shr:8
  const int t0 = __builtin_amdgcn_readlane(incl, 15), t1 = __builtin_amdgcn_readlane(incl, 31);
  const int t2 = __builtin_amdgcn_readlane(incl, 47), t3 = __builtin_amdgcn_readlane(incl, 63);
  incl += (lane >= 16 ? t0 : 0) + (lane >= 32 ? t1 : 0) + (lane >= 48 ? t2 : 0);
  r.off[lane] = incl - c;
  const int routed = t0 + t1 + t2 + t3;
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
// w, w+4 with rank_and_gate, then wavefront 0 sorts the pairs.
__device__ __forceinline__ void route_rows(const float* __restrict__ rlogit, int M, RouteLds& r) {
  __shared__ float lg[4][NE];
  const int wave = wave_id(), lane = lane_id();
  for (int m = wave; m < M; m += 4) {
    const float v = rlogit[m * NE + lane];
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
  for (int sl = tid; sl < NX; sl += 256) {
    if (sl < r.na) {
      const int e = r.act[sl];
      int rows = 0;  // bit m: row m has a pair routed to e (pairs sort by row)
      for (int p = r.off[e]; p < r.off[e + 1]; ++p) rows |= 1 << (r.perm[p] / NSLOT);
      mb.act[sl] = e;
      mb.slot_info[sl] = make_int4(e, r.off[e], r.off[e + 1], rows);
    } else {
      mb.slot_info[sl] = make_int4(-1, 0, 0, 0);
    }
  }
  if (tid == 0) {
    *mb.n_act = r.na;
    mb.stats[0] = st0 + r.na;
  }
}

// Router logits: wavefront w of block x computes expert 4x + w for every row
// (RMSNorm'ed with the FFN gain in the prologue; block 0 also stores the
// normalised rows for the experts).  rlogit[m][e] fp32.
template <typename T, int MR>
__global__ __launch_bounds__(256) void k_router_logits(const float* __restrict__ x, const float* __restrict__ gain,
                                                       float eps, const T* __restrict__ wr, int M,
                                                       float* __restrict__ bnorm, float* __restrict__ rlogit) {
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
  if (t.lead && t.m < m_act) rlogit[(long)(m0 + t.m) * NE + e] = t.val;
}

// M <= 8: top-6 per row and the sort by one block, published to global.
__global__ __launch_bounds__(256) void k_route_small(const float* __restrict__ rlogit, int M, MoeBufs mb,
                                                     RouteTap tap) {
  __shared__ RouteLds r;
  const long long st0 = (threadIdx.x == 0) ? mb.stats[0] : 0;  // read early: off the kernel's tail
  route_rows(rlogit, M, r);
  publish_route(r, M, mb, tap, st0);
}

// Larger batches (8 < M <= 1024): top-6 per row, one wavefront per row
// (rank_and_gate) ...
__global__ __launch_bounds__(256) void k_topk_rows(const float* __restrict__ rlogit, int M, MoeBufs mb,
                                                   RouteTap tap) {
  __shared__ float lg[4][NE];
  const int wave = wave_id(), lane = lane_id();
  const int m = blockIdx.x * 4 + wave;
  if (m >= M) return;
  const float v = rlogit[(long)m * NE + lane];
  lg[wave][lane] = v;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  int rank;
  float gate;
  rank_and_gate(lg[wave], v, rank, gate);
  if (rank < TOPK) {
    mb.ridx[m * NSLOT + rank] = lane;
    mb.rgate[m * NSLOT + rank] = gate;
    tap_pair(tap, m, rank, lane);
  }
  if (lane < NSH) {
    mb.ridx[m * NSLOT + TOPK + lane] = NE + lane;
    mb.rgate[m * NSLOT + TOPK + lane] = 1.0f;
    tap_pair(tap, m, TOPK + lane, NE + lane);
  }
}

// ... then a stable counting sort of the 8M pairs by expert in one 1024-thread
// block.  Wavefront w owns rows [w M / 16, (w + 1) M / 16), i.e. a contiguous
// pair range, read in segments of 64 pairs (lane = pair; all segments' loads
// issued together).  Ballots over a segment's distinct experts give each pair
// its rank among the range's earlier pairs of the same expert (the range's
// running count of expert e sits in lane e, or lane e - 64 for the shared
// experts).  The per-range counts give per-expert offsets (experts in id
// order) and per-range bases; pair p lands at off[e] + base[w][e] + rank --
// the permutation of any stable sort by expert id.
constexpr int RL_WAVES = 16;
constexpr int RL_SEGS = 8;  // segments per wavefront: M <= RL_WAVES * RL_SEGS * 8 = 1024
__global__ __launch_bounds__(1024) void k_sort_pairs(int M, MoeBufs mb) {
  __shared__ int wcnt[RL_WAVES][NX + 1];  // per range: counts, then exclusive bases
  __shared__ int off[NX + 1], act[NX + 1];
  __shared__ int na_s;
  const int wave = threadIdx.x >> 6, lane = lane_id(), tid = threadIdx.x;
  const int p_lo = NSLOT * (M * wave / RL_WAVES), p_hi = NSLOT * (M * (wave + 1) / RL_WAVES);
  const uint64_t lt = (1ull << lane) - 1ull;
  int seg_e[RL_SEGS], seg_rank[RL_SEGS];
#pragma unroll
  for (int sg = 0; sg < RL_SEGS; ++sg) {
    const int p = p_lo + 64 * sg + lane;
    seg_e[sg] = (p < p_hi) ? mb.ridx[p] : -1;
    seg_rank[sg] = 0;
  }
  int c_lo = 0, c_hi = 0;
#pragma unroll
  for (int sg = 0; sg < RL_SEGS; ++sg) {
    if (p_lo + 64 * sg >= p_hi) break;
    const int e = seg_e[sg];
    const bool valid = e >= 0;
    uint64_t todo = __ballot(valid);
    int rank = 0;
    while (todo) {
      const int leader = __builtin_ctzll(todo);
      const int el = __builtin_amdgcn_readlane(e, leader);
      const uint64_t same = __ballot(e == el);
      const int n = __popcll(same);
      const int before = (el < NE) ? __builtin_amdgcn_readlane(c_lo, el) : __builtin_amdgcn_readlane(c_hi, el - NE);
      if (e == el) rank = before + __popcll(same & lt);
      if (el < NE) {
        if (lane == el) c_lo += n;
      } else if (lane == el - NE) {
        c_hi += n;
      }
      todo &= ~same;
    }
    seg_rank[sg] = rank;
  }
  wcnt[wave][lane] = c_lo;
  if (lane < NSH) wcnt[wave][NE + lane] = c_hi;
  __syncthreads();
  // per-expert totals -> offsets; per-range exclusive bases
  if (tid < NX) {
    int acc = 0;
    for (int w = 0; w < RL_WAVES; ++w) {
      const int c = wcnt[w][tid];
      wcnt[w][tid] = acc;
      acc += c;
    }
    act[tid] = acc;  // total of expert tid (reused below as the active list)
  }
  __syncthreads();
  if (tid == 0) {
    int acc = 0, na = 0;
    for (int e = 0; e < NX; ++e) {
      const int c = act[e];
      off[e] = acc;
      acc += c;
      if (c > 0) act[na++] = e;  // na <= e: entries not yet read are never overwritten
    }
    off[NX] = acc;
    na_s = na;
    *mb.n_act = na;
    mb.stats[0] += na;
  }
  __syncthreads();
  const int na = na_s;
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
template <typename T>
void launch_router(hipStream_t s, const float* x, const float* gain, float eps, const T* wr, int M,
                   const MoeBufs& mb, const RouteTap& tap, const float* logit_override) {
#define OCR_RL_CASE(MRV)                                                                                   \
  hipLaunchKernelGGL((k_router_logits<T, MRV>), dim3(NE / 4, (M + MRV - 1) / MRV), dim3(256),              \
                     (size_t)MRV * D * 4, s, x, gain, eps, wr, M, mb.bnorm, mb.rlogit);
  if (M <= 1) OCR_RL_CASE(1)
  else if (M <= 2) OCR_RL_CASE(2)
  else if (M <= 4) OCR_RL_CASE(4)
  else OCR_RL_CASE(MRG)
#undef OCR_RL_CASE
  if (logit_override != nullptr) launch_copy_rows(s, logit_override, mb.rlogit, (long)M * NE);
  if (M <= MRG) {
    hipLaunchKernelGGL(k_route_small, dim3(1), dim3(256), 0, s, mb.rlogit, M, mb, tap);
  } else {
    hipLaunchKernelGGL(k_topk_rows, dim3((M + 3) / 4), dim3(256), 0, s, mb.rlogit, M, mb, tap);
    hipLaunchKernelGGL(k_sort_pairs, dim3(1), dim3(1024), 0, s, M, mb);
  }
}

// Gather the activation rows m < m_act <= MR (row_of(m) into src) into LDS;
// 256 threads, the loads of every row issued before any LDS store.
template <int K, int MR, typename SrcRow>
__device__ __forceinline__ void gather_rows(const float* __restrict__ src, SrcRow row_of, int m_act, float* xs) {
  static_assert(K % 256 == 0 || K == DI, "row length");
  constexpr int J = (K + 255) / 256;
  float v[MR][J];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    if (m < m_act) {
      const float* r = src + (long)row_of(m) * K;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int k = threadIdx.x + 256 * j;
        v[m][j] = (k < K) ? r[k] : 0.f;
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    if (m < m_act) {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int k = threadIdx.x + 256 * j;
        if (k < K) xs[m * K + k] = v[m][j];
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

// Down: block (x, slot s); wavefront w owns output rows n0 .. n0+RPW-1,
// n0 = RPW (4x + w):  y[pair][n] = W_d[n] . hx[pair].
template <typename T, int MR, int RPW>
__global__ __launch_bounds__(256) void k_expert_down(const T* __restrict__ wd, int M, MoeBufs mb) {
  extern __shared__ float xs[];
  const int4 info = expert_work(mb, blockIdx.y, M);
  const int e = info.x;
  if (e < 0) return;
  const int k0 = info.y;
  const int m_act = min(MR, info.z - k0);
  const int wave = wave_id();
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
  if (t.lead && t.m < m_act) mb.y[(long)(k0 + t.m) * D + n0 + t.r] = t.val;
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
  const dim3 grid(D / (4 * DN_RPW), expert_slot_cap(M));
#define OCR_DN_CASE(MRV) \
  hipLaunchKernelGGL((k_expert_down<T, MRV, DN_RPW>), grid, dim3(256), (size_t)MRV * DI * 4, s, wd, M, mb);
  if (M <= 1) OCR_DN_CASE(1)
  else if (M <= 2) OCR_DN_CASE(2)
  else if (M <= 4) OCR_DN_CASE(4)
  else if (M <= MRG) OCR_DN_CASE(MRG)
  else
    hipLaunchKernelGGL((k_expert_down_groups<T>), dim3(D / 16, expert_slot_cap(M)), dim3(256),
                       (size_t)MRG * DI * 4, s, wd, M, mb);
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
                                 const MoeBufs&, const RouteTap&, const float*);                         \
  template void launch_expert_gate_up<T>(hipStream_t, const T*, const T*, int, const MoeBufs&);                \
  template void launch_expert_down<T>(hipStream_t, const T*, int, const MoeBufs&);
OCR_INST_MOE(float)
OCR_INST_MOE(bf16)

}  // namespace ocr
