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

// Top-6 of the 64 logits of one row held one per lane (lane = expert id), ties
// to the lower id; writes the 8 routing slots of the row.  One wavefront.
__device__ __forceinline__ void top6_row(float v, int row, const MoeBufs& mb, int* tap, int* pe) {
  const int lane = lane_id();
  bool taken = false;
  int sel[TOPK];
  float selv[TOPK];
#pragma unroll
  for (int j = 0; j < TOPK; ++j) {
    float bv = taken ? -INFINITY : v;
    int bi = taken ? 0x7fffffff : lane;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    sel[j] = bi;
    selv[j] = bv;
    if (lane == bi) taken = true;
  }
  // softmax over all 64 routed experts; max = the top-1 logit
  const float mx = selv[0];
  const float ex = expf(v - mx);
  const float sum = wave_sum(ex);
  if (lane < NSLOT) {
    float gv = 1.0f;
    int gi = NE + (lane - TOPK);
#pragma unroll
    for (int j = 0; j < TOPK; ++j)
      if (lane == j) { gi = sel[j]; gv = expf(selv[j] - mx) / sum; }
    mb.ridx[row * NSLOT + lane] = gi;
    mb.rgate[row * NSLOT + lane] = gv;
    if (tap != nullptr) tap[row * NSLOT + lane] = gi;
    if (pe != nullptr) pe[row * NSLOT + lane] = gi;
  }
}

// Publish the sorted order: off[e], the active experts in increasing id and,
// per expert slot s < NX, slot_info[s] = (e, first pair, end pair, n_act)
// (e = -1 past n_act).  Counts the active experts into stats[0].
__device__ __forceinline__ void publish_slots(const int* off, const int* act, int na, const MoeBufs& mb, int tid,
                                              int nt) {
  for (int e = tid; e <= NX; e += nt) mb.off[e] = off[e];
  for (int sl = tid; sl < NX; sl += nt) {
    if (sl < na) {
      const int e = act[sl];
      mb.act[sl] = e;
      mb.slot_info[sl] = make_int4(e, off[e], off[e + 1], na);
    } else {
      mb.slot_info[sl] = make_int4(-1, 0, 0, na);
    }
  }
  if (tid == 0) {
    *mb.n_act = na;
    mb.stats[0] += na;
  }
}

// Stable counting sort of the P = 8M pairs (expert ids in pe[], LDS) by expert;
// all threads of the block take part.  cnt / off / act: LDS [NX + 1].
__device__ __forceinline__ void sort_pairs(const int* pe, int P, int* cnt, int* off, int* act, int* na_s,
                                           const MoeBufs& mb) {
  const int tid = threadIdx.x, nt = blockDim.x;
  for (int e = tid; e <= NX; e += nt) cnt[e] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += nt) atomicAdd(&cnt[pe[p]], 1);
  __syncthreads();
  if (tid == 0) {
    int acc = 0, na = 0;
    for (int e = 0; e < NX; ++e) {
      off[e] = acc;
      if (cnt[e] > 0) act[na++] = e;
      acc += cnt[e];
    }
    off[NX] = acc;
    *na_s = na;
  }
  __syncthreads();
  publish_slots(off, act, *na_s, mb, tid, nt);
  for (int p = tid; p < P; p += nt) {
    const int e = pe[p];
    int rank = 0;
    for (int q = 0; q < p; ++q) rank += (pe[q] == e);
    const int pos = off[e] + rank;
    mb.perm[pos] = p;
    mb.inv[p] = pos;
  }
}

// The same sort for P <= 64 pairs by one wavefront (lane = pair): ranks by
// ballots over the distinct experts present, offsets by a wavefront scan.
__device__ __forceinline__ void sort_pairs_wave(const int* pe, int P, int* cnt, int* off, int* act,
                                                const MoeBufs& mb) {
  const int lane = lane_id();
  const bool valid = lane < P;
  const int e = valid ? pe[lane] : -1;
  const uint64_t lt = (1ull << lane) - 1ull;
  for (int x = lane; x <= NX; x += 64) cnt[x] = 0;
  uint64_t todo = __ballot(valid);
  int rank = 0;
  while (todo) {
    const int leader = __builtin_ctzll(todo);
    const int el = __shfl(e, leader, 64);
    const uint64_t same = __ballot(valid && e == el);
    if (valid && e == el) rank = __popcll(same & lt);
    if (lane == 0) cnt[el] = __popcll(same);
    todo &= ~same;
  }
  // exclusive scan of the routed counts (lanes = experts 0..63), then the shared experts
  const int c = cnt[lane];
  int incl = c;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  off[lane] = incl - c;
  const int routed = __shfl(incl, 63, 64);
  const uint64_t amask = __ballot(c > 0);
  const int nr = __popcll(amask);
  if (c > 0) act[__popcll(amask & lt)] = lane;
  int na = nr;
  if (lane == 0) {
    off[NE] = routed;
    off[NE + 1] = routed + cnt[NE];
    off[NX] = routed + cnt[NE] + cnt[NE + 1];
    if (cnt[NE] > 0) act[na] = NE;
  }
  na += (cnt[NE] > 0);
  if (lane == 0 && cnt[NE + 1] > 0) act[na] = NE + 1;
  na += (cnt[NE + 1] > 0);
  if (valid) {
    const int pos = off[e] + rank;
    mb.perm[pos] = lane;
    mb.inv[lane] = pos;
  }
  publish_slots(off, act, na, mb, lane, 64);
}

// Small batches (M <= 8): one block of 16 wavefronts does everything.
// Wavefront w streams router rows 4w..4w+3 (loads issued first), RMSNorms
// rows w, w+16, ...; then top-6 per row and the sort, all in LDS.
template <typename T, int MR>
__global__ __launch_bounds__(1024) void k_router_small(const float* __restrict__ x, const float* __restrict__ gain,
                                                       float eps, const T* __restrict__ wr, int M, MoeBufs mb,
                                                       int* __restrict__ tap) {
  extern __shared__ float xs[];  // [MR][D]
  __shared__ float lg[MR][NE];
  __shared__ int pe[MR * NSLOT];
  __shared__ int cnt[NX + 1], off[NX + 1], act[NX + 1];
  const int wave = wave_id(), lane = lane_id();
  const T* rows[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) rows[r] = wr + (long)(wave * 4 + r) * D;
  WaveGemv<T, D, 4, MR> g;
  g.load(rows);
  norm_rows_wave<D>(x, D, RowIdentity{0}, M, gain, eps, xs, 16);
  __syncthreads();
  for (int k = threadIdx.x; k < M * D; k += 1024) mb.bnorm[k] = xs[k];
  float acc[4][MR];
  g.fma(xs, M, acc);
  wave_reduce_acc<4, MR>(acc, M);
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    if (m < M && lane < 4) {
      const float v = (lane == 0) ? acc[0][m] : (lane == 1) ? acc[1][m] : (lane == 2) ? acc[2][m] : acc[3][m];
      lg[m][wave * 4 + lane] = v;
    }
  }
  __syncthreads();
  for (int m = wave; m < M; m += 16) top6_row(lg[m][lane], m, mb, tap, pe);
  __syncthreads();
  if (wave == 0) sort_pairs_wave(pe, M * NSLOT, cnt, off, act, mb);
}

// Larger batches: one block per row computes its logits and top-6 ...
template <typename T>
__global__ __launch_bounds__(256) void k_router_rows(const float* __restrict__ x, const float* __restrict__ gain,
                                                     float eps, const T* __restrict__ wr, MoeBufs mb,
                                                     int* __restrict__ tap) {
  __shared__ float xs[D];
  __shared__ float lg[NE];
  const int row = blockIdx.x;
  const int wave = wave_id(), lane = lane_id();
  WaveGemv<T, D, 4, 1> g[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const T* rows[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) rows[r] = wr + (long)(wave * 16 + t * 4 + r) * D;
    g[t].load(rows);
  }
  if (wave == 0) norm_rows_wave<D>(x, D, RowIdentity{row}, 1, gain, eps, xs, 1);
  __syncthreads();
  for (int k = threadIdx.x; k < D; k += 256) mb.bnorm[(long)row * D + k] = xs[k];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    float acc[4][1];
    g[t].fma(xs, 1, acc);
    wave_reduce_acc<4, 1>(acc, 1);
    if (lane < 4)
      lg[wave * 16 + t * 4 + lane] =
          (lane == 0) ? acc[0][0] : (lane == 1) ? acc[1][0] : (lane == 2) ? acc[2][0] : acc[3][0];
  }
  __syncthreads();
  if (wave == 0) top6_row(lg[lane], row, mb, tap, nullptr);
}

// ... and one block sorts all pairs.
__global__ __launch_bounds__(1024) void k_sort_pairs(int M, MoeBufs mb) {
  extern __shared__ int pe[];
  __shared__ int cnt[NX + 1], off[NX + 1], act[NX + 1];
  __shared__ int na_s;
  const int P = M * NSLOT;
  for (int p = threadIdx.x; p < P; p += 1024) pe[p] = mb.ridx[p];
  __syncthreads();
  sort_pairs(pe, P, cnt, off, act, &na_s, mb);
}

int expert_slot_cap(int M) { return min(NE, TOPK * M) + NSH; }

template <typename T>
void launch_router(hipStream_t s, const float* x, const float* gain, float eps, const T* wr, int M,
                   const MoeBufs& mb, int* tap) {
#define OCR_ROUTER_CASE(MRV)                                                                                  \
  {                                                                                                           \
    static const bool lds_ok = (allow_lds(k_router_small<T, MRV>, (size_t)MRV * D * 4), true);                \
    (void)lds_ok;                                                                                             \
    hipLaunchKernelGGL((k_router_small<T, MRV>), dim3(1), dim3(1024), (size_t)MRV * D * 4, s, x, gain, eps, wr, \
                       M, mb, tap);                                                                           \
  }
  if (M <= 1) OCR_ROUTER_CASE(1)
  else if (M <= 2) OCR_ROUTER_CASE(2)
  else if (M <= 4) OCR_ROUTER_CASE(4)
  else if (M <= 8) OCR_ROUTER_CASE(8)
  else {
    hipLaunchKernelGGL((k_router_rows<T>), dim3(M), dim3(256), 0, s, x, gain, eps, wr, mb, tap);
    hipLaunchKernelGGL(k_sort_pairs, dim3(1), dim3(1024), (size_t)M * NSLOT * sizeof(int), s, M, mb);
  }
#undef OCR_ROUTER_CASE
}

// Gather the activation rows m < m_act (row_of(m) into src) into LDS;
// 256 threads, all loads of a row issued before its LDS stores.
template <int K, typename SrcRow>
__device__ __forceinline__ void gather_rows(const float* __restrict__ src, SrcRow row_of, int m_act, float* xs) {
  static_assert(K % 256 == 0 || K == DI, "row length");
  constexpr int J = (K + 255) / 256;
  for (int m = 0; m < m_act; ++m) {
    const float* r = src + (long)row_of(m) * K;
    float v[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int k = threadIdx.x + 256 * j;
      v[j] = (k < K) ? r[k] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int k = threadIdx.x + 256 * j;
      if (k < K) xs[m * K + k] = v[j];
    }
  }
}

// Gate/up: block (x, slot s) of expert e = slot_info[s].e; wavefront w owns
// units j0 .. j0+UPW-1, j0 = UPW (4x + w): rows gate[j] then up[j], all loads
// issued at once.  The (at most MR) pairs routed to e get
// hx[pair][j] = silu(gate . b) * (up . b).
template <typename T, int MR, int UPW>
__global__ __launch_bounds__(256) void k_expert_gate_up(const T* __restrict__ wg, const T* __restrict__ wu,
                                                        MoeBufs mb) {
  extern __shared__ float xs[];
  const int4 info = mb.slot_info[blockIdx.y];
  const int e = info.x;
  if (e < 0) return;
  const int k0 = info.y;
  const int m_act = min(MR, info.z - k0);
  const int wave = wave_id(), lane = lane_id();
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
  gather_rows<D>(mb.bnorm, [&](int m) { return mb.perm[k0 + m] / NSLOT; }, m_act, xs);
  __syncthreads();
  float acc[2 * UPW][MR];
  g.fma(xs, m_act, acc);
  wave_reduce_acc<2 * UPW, MR>(acc, m_act);
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    if (lane == m && m < m_act) {
      float* o = mb.hx + (long)(k0 + m) * DI + j0;
#pragma unroll
      for (int u = 0; u < UPW; ++u) o[u] = silu(acc[u][m]) * acc[UPW + u][m];
    }
  }
}

// Down: block (x, slot s); wavefront w owns output rows n0 .. n0+RPW-1,
// n0 = RPW (4x + w):  y[pair][n] = W_d[n] . hx[pair].
template <typename T, int MR, int RPW>
__global__ __launch_bounds__(256) void k_expert_down(const T* __restrict__ wd, MoeBufs mb) {
  extern __shared__ float xs[];
  const int4 info = mb.slot_info[blockIdx.y];
  const int e = info.x;
  if (e < 0) return;
  const int k0 = info.y;
  const int m_act = min(MR, info.z - k0);
  const int wave = wave_id(), lane = lane_id();
  const int n0 = (blockIdx.x * 4 + wave) * RPW;
  const T* base = wd + ((long)e * D + n0) * DI;
  const T* rows[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) rows[r] = base + (long)r * DI;
  WaveGemv<T, DI, RPW, MR> g;
  g.load(rows);
  gather_rows<DI>(mb.hx, [&](int m) { return k0 + m; }, m_act, xs);
  __syncthreads();
  float acc[RPW][MR];
  g.fma(xs, m_act, acc);
  wave_reduce_acc<RPW, MR>(acc, m_act);
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    if (lane == m && m < m_act) {
      float* o = mb.y + (long)(k0 + m) * D + n0;
#pragma unroll
      for (int r = 0; r < RPW; ++r) o[r] = acc[r][m];
    }
  }
}

// Batches with more than MRG rows: the same per-row arithmetic, MRG pairs at a
// time, one tile per wavefront, the tile re-read for every group of pairs.
template <typename T>
__global__ __launch_bounds__(256) void k_expert_gate_up_groups(const T* __restrict__ wg, const T* __restrict__ wu,
                                                               MoeBufs mb) {
  extern __shared__ float xs[];
  const int4 info = mb.slot_info[blockIdx.y];
  const int e = info.x;
  if (e < 0) return;
  const int wave = wave_id(), lane = lane_id();
  const int j = (blockIdx.x * 4 + wave) * 2;
  for (int kb = info.y; kb < info.z; kb += MRG) {
    const int m_act = min(MRG, info.z - kb);
    const T* gb = wg + ((long)e * DI + j) * D;
    const T* ub = wu + ((long)e * DI + j) * D;
    asm volatile("" : "+v"(gb), "+v"(ub));  // the weights are re-read per group, not hoisted
    const T* rows[4] = {gb, gb + D, ub, ub + D};
    WaveGemv<T, D, 4, MRG> g;
    g.load(rows);
    gather_rows<D>(mb.bnorm, [&](int m) { return mb.perm[kb + m] / NSLOT; }, m_act, xs);
    __syncthreads();
    float acc[4][MRG];
    g.fma(xs, m_act, acc);
    wave_reduce_acc<4, MRG>(acc, m_act);
#pragma unroll
    for (int m = 0; m < MRG; ++m) {
      if (lane == m && m < m_act) {
        float* o = mb.hx + (long)(kb + m) * DI + j;
        o[0] = silu(acc[0][m]) * acc[2][m];
        o[1] = silu(acc[1][m]) * acc[3][m];
      }
    }
    __syncthreads();
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_expert_down_groups(const T* __restrict__ wd, MoeBufs mb) {
  extern __shared__ float xs[];
  const int4 info = mb.slot_info[blockIdx.y];
  const int e = info.x;
  if (e < 0) return;
  const int wave = wave_id(), lane = lane_id();
  const int n0 = (blockIdx.x * 4 + wave) * 4;
  for (int kb = info.y; kb < info.z; kb += MRG) {
    const int m_act = min(MRG, info.z - kb);
    const T* b = wd + ((long)e * D + n0) * DI;
    asm volatile("" : "+v"(b));
    const T* rows[4] = {b, b + DI, b + 2 * DI, b + 3 * DI};
    WaveGemv<T, DI, 4, MRG> g;
    g.load(rows);
    gather_rows<DI>(mb.hx, [&](int m) { return kb + m; }, m_act, xs);
    __syncthreads();
    float acc[4][MRG];
    g.fma(xs, m_act, acc);
    wave_reduce_acc<4, MRG>(acc, m_act);
#pragma unroll
    for (int m = 0; m < MRG; ++m) {
      if (lane == m && m < m_act) {
        float* o = mb.y + (long)(kb + m) * D + n0;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = acc[r][m];
      }
    }
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
  hipLaunchKernelGGL((k_expert_gate_up<T, MRV, GU_UPW>), grid, dim3(256), (size_t)MRV * D * 4, s, wg, wu, mb);
  if (M <= 1) OCR_GU_CASE(1)
  else if (M <= 2) OCR_GU_CASE(2)
  else if (M <= 4) OCR_GU_CASE(4)
  else if (M <= MRG) OCR_GU_CASE(MRG)
  else
    hipLaunchKernelGGL((k_expert_gate_up_groups<T>), dim3(DI / 8, expert_slot_cap(M)), dim3(256),
                       (size_t)MRG * D * 4, s, wg, wu, mb);
#undef OCR_GU_CASE
}

template <typename T>
void launch_expert_down(hipStream_t s, const T* wd, int M, const MoeBufs& mb) {
  const dim3 grid(D / (4 * DN_RPW), expert_slot_cap(M));
#define OCR_DN_CASE(MRV) \
  hipLaunchKernelGGL((k_expert_down<T, MRV, DN_RPW>), grid, dim3(256), (size_t)MRV * DI * 4, s, wd, mb);
  if (M <= 1) OCR_DN_CASE(1)
  else if (M <= 2) OCR_DN_CASE(2)
  else if (M <= 4) OCR_DN_CASE(4)
  else if (M <= MRG) OCR_DN_CASE(MRG)
  else
    hipLaunchKernelGGL((k_expert_down_groups<T>), dim3(D / 16, expert_slot_cap(M)), dim3(256),
                       (size_t)MRG * DI * 4, s, wd, mb);
#undef OCR_DN_CASE
}

// x[r] += y_shared0 + y_shared1 + sum_j gate_j * y_routed_j, in this order.
__global__ __launch_bounds__(256) void k_moe_combine(float* __restrict__ x, MoeBufs mb) {
  const int r = blockIdx.x;
  const int* inv = mb.inv + r * NSLOT;
  const float* gt = mb.rgate + r * NSLOT;
  for (int n = threadIdx.x; n < D; n += 256) {
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
                                 const MoeBufs&, int*);                                                  \
  template void launch_expert_gate_up<T>(hipStream_t, const T*, const T*, int, const MoeBufs&);          \
  template void launch_expert_down<T>(hipStream_t, const T*, int, const MoeBufs&);
OCR_INST_MOE(float)
OCR_INST_MOE(bf16)

}  // namespace ocr
