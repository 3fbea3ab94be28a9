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

// Stable counting sort of the P = 8M pairs (expert ids in pe[], LDS) by expert;
// all threads of the block take part.  cnt / off: LDS [NX + 1].
__device__ __forceinline__ void sort_pairs(const int* pe, int P, int* cnt, int* off, const MoeBufs& mb) {
  const int tid = threadIdx.x, nt = blockDim.x;
  for (int e = tid; e <= NX; e += nt) cnt[e] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += nt) atomicAdd(&cnt[pe[p]], 1);
  __syncthreads();
  if (tid == 0) {
    int acc = 0, na = 0;
    for (int e = 0; e < NX; ++e) {
      off[e] = acc;
      if (cnt[e] > 0) mb.act[na++] = e;
      acc += cnt[e];
    }
    off[NX] = acc;
    *mb.n_act = na;
    mb.stats[0] += na;
  }
  __syncthreads();
  for (int e = tid; e <= NX; e += nt) mb.off[e] = off[e];
  for (int p = tid; p < P; p += nt) {
    const int e = pe[p];
    int rank = 0;
    for (int q = 0; q < p; ++q) rank += (pe[q] == e);
    const int pos = off[e] + rank;
    mb.perm[pos] = p;
    mb.inv[p] = pos;
  }
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
  __shared__ int cnt[NX + 1], off[NX + 1];
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
  sort_pairs(pe, M * NSLOT, cnt, off, mb);
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
  __shared__ int cnt[NX + 1], off[NX + 1];
  const int P = M * NSLOT;
  for (int p = threadIdx.x; p < P; p += 1024) pe[p] = mb.ridx[p];
  __syncthreads();
  sort_pairs(pe, P, cnt, off, mb);
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

// Gate/up: block (tile, expert slot); wavefront w computes units j, j+1 of the
// expert (rows gate[j], gate[j+1], up[j], up[j+1]) for every pair routed to it,
// MR pairs at a time, and stores hx[pair][j] = silu(gate . b) * (up . b).
template <typename T, int MR>
__global__ __launch_bounds__(256) void k_expert_gate_up(const T* __restrict__ wg, const T* __restrict__ wu,
                                                        MoeBufs mb) {
  extern __shared__ float xs[];
  const int s = blockIdx.y;
  if (s >= *mb.n_act) return;
  const int e = mb.act[s];
  const int k0 = mb.off[e], k1 = mb.off[e + 1];
  const int wave = wave_id(), lane = lane_id(), tid = threadIdx.x;
  const int j = blockIdx.x * 8 + wave * 2;
  const T* rows[4] = {wg + ((long)e * DI + j) * D, wg + ((long)e * DI + j + 1) * D,
                      wu + ((long)e * DI + j) * D, wu + ((long)e * DI + j + 1) * D};
  WaveGemv<T, D, 4, MR> g;
  g.load(rows);
  for (int kb = k0; kb < k1; kb += MR) {
    const int m_act = min(MR, k1 - kb);
    for (int m = 0; m < m_act; ++m) {
      const float* src = mb.bnorm + (long)(mb.perm[kb + m] / NSLOT) * D;
      for (int k = tid; k < D; k += 256) xs[m * D + k] = src[k];
    }
    __syncthreads();
    float acc[4][MR];
    g.fma(xs, m_act, acc);
    wave_reduce_acc<4, MR>(acc, m_act);
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      if (lane == m && m < m_act) {
        float* o = mb.hx + (long)(kb + m) * DI + j;
        o[0] = silu(acc[0][m]) * acc[2][m];
        o[1] = silu(acc[1][m]) * acc[3][m];
      }
    }
    __syncthreads();
  }
}

// Down: block (tile, expert slot); wavefront w computes output rows
// n = 16 tile + 4 w .. +3 of the expert for its pairs: y[pair][n] = W_d[n] . hx[pair].
template <typename T, int MR>
__global__ __launch_bounds__(256) void k_expert_down(const T* __restrict__ wd, MoeBufs mb) {
  extern __shared__ float xs[];
  const int s = blockIdx.y;
  if (s >= *mb.n_act) return;
  const int e = mb.act[s];
  const int k0 = mb.off[e], k1 = mb.off[e + 1];
  const int wave = wave_id(), lane = lane_id(), tid = threadIdx.x;
  const int n0 = blockIdx.x * 16 + wave * 4;
  const T* rows[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) rows[r] = wd + ((long)e * D + n0 + r) * DI;
  WaveGemv<T, DI, 4, MR> g;
  g.load(rows);
  for (int kb = k0; kb < k1; kb += MR) {
    const int m_act = min(MR, k1 - kb);
    for (int m = 0; m < m_act; ++m) {
      const float* src = mb.hx + (long)(kb + m) * DI;
      for (int k = tid; k < DI; k += 256) xs[m * DI + k] = src[k];
    }
    __syncthreads();
    float acc[4][MR];
    g.fma(xs, m_act, acc);
    wave_reduce_acc<4, MR>(acc, m_act);
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      if (lane == m && m < m_act) {
        float* o = mb.y + (long)(kb + m) * D + n0;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = acc[r][m];
      }
    }
    __syncthreads();
  }
}

template <typename T>
void launch_expert_gate_up(hipStream_t s, const T* wg, const T* wu, int M, const MoeBufs& mb) {
  const dim3 grid(DI / 8, expert_slot_cap(M));
  if (M <= 1) hipLaunchKernelGGL((k_expert_gate_up<T, 1>), grid, dim3(256), 1 * D * 4, s, wg, wu, mb);
  else if (M <= 2) hipLaunchKernelGGL((k_expert_gate_up<T, 2>), grid, dim3(256), 2 * D * 4, s, wg, wu, mb);
  else if (M <= 4) hipLaunchKernelGGL((k_expert_gate_up<T, 4>), grid, dim3(256), 4 * D * 4, s, wg, wu, mb);
  else hipLaunchKernelGGL((k_expert_gate_up<T, MRG>), grid, dim3(256), MRG * D * 4, s, wg, wu, mb);
}

template <typename T>
void launch_expert_down(hipStream_t s, const T* wd, int M, const MoeBufs& mb) {
  const dim3 grid(D / 16, expert_slot_cap(M));
  if (M <= 1) hipLaunchKernelGGL((k_expert_down<T, 1>), grid, dim3(256), 1 * DI * 4, s, wd, mb);
  else if (M <= 2) hipLaunchKernelGGL((k_expert_down<T, 2>), grid, dim3(256), 2 * DI * 4, s, wd, mb);
  else if (M <= 4) hipLaunchKernelGGL((k_expert_down<T, 4>), grid, dim3(256), 4 * DI * 4, s, wd, mb);
  else hipLaunchKernelGGL((k_expert_down<T, MRG>), grid, dim3(256), MRG * DI * 4, s, wd, mb);
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
