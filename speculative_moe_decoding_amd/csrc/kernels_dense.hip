// Dense decode kernels: fused RMSNorm -> QKV -> RoPE -> KV append, the generic
// wavefront GEMV (residual add / store / SwiGLU epilogues) and the LM head fused
// with a two-stage argmax.
//
// All of them stream weight rows with 16-byte coalesced loads; a wavefront owns
// R weight rows and keeps up to MRG activation rows in LDS (fp32), see
// WaveGemv.  Decode has at most a handful of activation rows, so these are
// HBM-bound GEMVs (arithmetic intensity ~ M flop per weight byte), and no MFMA
// is used.
#include "launch.h"

namespace ocr {

// RoPE table: tab[pos][i] = (cos, sin) of pos * theta^(-2i/HD) for i < HD/2,
// angle in fp64, rounded to fp32.  Built once per model handle.
__global__ void k_rope_table(int max_pos, float theta, float2* __restrict__ tab) {
  const long n = (long)max_pos * (HD / 2);
  for (long e = blockIdx.x * (long)blockDim.x + threadIdx.x; e < n; e += (long)gridDim.x * blockDim.x) {
    const int pos = (int)(e / (HD / 2)), i = (int)(e % (HD / 2));
    const double inv = pow((double)theta, -(double)(2 * i) / (double)HD);
    double sd, cd;
    sincos((double)pos * inv, &sd, &cd);
    tab[e] = make_float2((float)cd, (float)sd);
  }
}

void launch_rope_table(hipStream_t s, int max_pos, float theta, float2* tab) {
  hipLaunchKernelGGL(k_rope_table, dim3(256), dim3(256), 0, s, max_pos, theta, tab);
}

// Rotate the pair (a, b) = (x_i, x_{i+64}) by the angle with cosine c, sine s.
__device__ __forceinline__ void rot(float a, float b, float c, float s, float& o1, float& o2) {
  o1 = fmaf(a, c, -(b * s));
  o2 = fmaf(b, c, a * s);
}

// One wavefront = one pair of output rows: q / k pairs are rows {u, u+64} of
// one head (the two halves of a RoPE pair), v pairs are rows {2u, 2u+1}.  Weight
// loads are issued first; lane m fetches the cos/sin of its row's position
// while they are in flight; the RMSNorm of the activation rows overlaps them.
template <typename T, int MR>
__global__ __launch_bounds__(256) void k_qkv_rope(const float* __restrict__ x, const float* __restrict__ gain,
                                                  float eps, const T* __restrict__ wqkv, int M, RowPlan plan,
                                                  float* __restrict__ q, KvView<T> kv,
                                                  const float2* __restrict__ rope) {
  const int max_pos = kv.max_pos;
  extern __shared__ float smem[];
  float* xs = smem;
  const int wave = wave_id(), lane = lane_id();
  const int pr = blockIdx.x * 4 + wave;  // 0 .. 1919
  const int m0 = blockIdx.y * MR;
  const int m_act = min(MR, M - m0);
  const int sec = pr / 640, rem = pr % 640, h = rem / 64, u = rem % 64;
  int r0, r1;
  if (sec < 2) {
    r0 = sec * QD + h * HD + u;
    r1 = r0 + 64;
  } else {
    r0 = 2 * QD + h * HD + 2 * u;
    r1 = r0 + 1;
  }
  const T* rows[2] = {wqkv + (long)r0 * D, wqkv + (long)r1 * D};
  WaveGemv<T, D, 2, MR> g;
  g.load(rows);
  // lane m < m_act: this row's position, validity, cache page and rotation
  int pos = 0, b = 0, i = 0, slot = 0, page = 0;
  bool valid = false;
  float2 cs = make_float2(1.f, 0.f);
  if (lane < m_act) {
    const int row = m0 + lane;
    b = row / plan.Q;
    i = row - b * plan.Q;
    slot = plan.slot[b];
    pos = plan.base[b] + i;
    valid = i < plan.cnt[b] && pos >= 0 && pos < max_pos;
    if (sec < 2) cs = rope[(long)min(max(pos, 0), max_pos - 1) * (HD / 2) + u];
    if (sec > 0) {
      page = kv.raw_page(slot, pos);
      valid = valid && page >= 0;
    }
  }
  norm_rows_wave<D, MR>(x, D, RowIdentity{m0}, m_act, gain, eps, xs);
  __syncthreads();
  float acc[2][MR];
  g.fma(xs, m_act, acc);
  // lane with (r, m): row m's position data from lane m, the pair's other total
  const WaveTotals<2, MR> t(acc);
  const float other = t.partner(1);
  const int tpos = __shfl(pos, t.m, 64), tpage = __shfl(page, t.m, 64);
  const bool tvalid = __shfl((int)valid, t.m, 64) != 0;
  const float tc = __shfl(cs.x, t.m, 64), ts = __shfl(cs.y, t.m, 64);
  if (t.lead && t.m < m_act) {
    const int row = m0 + t.m;
    if (sec < 2) {
      // rows u (r = 0) and u + 64 (r = 1) of a head: each lane rotates its own
      float o;
      if (t.r == 0) o = fmaf(t.val, tc, -(other * ts));
      else o = fmaf(t.val, tc, other * ts);
      if (sec == 0) {
        q[(long)row * QD + h * HD + u + 64 * t.r] = o;
      } else if (tvalid) {
        kv.at(tpage, 0, h, tpos)[u + 64 * t.r] = WT<T>::store_cvt(o);
      }
    } else if (tvalid) {
      kv.at(tpage, 1, h, tpos)[2 * u + t.r] = WT<T>::store_cvt(t.val);
    }
  }
}

template <typename T>
void launch_qkv_rope(hipStream_t s, const float* x, const float* gain, float eps, const T* wqkv, int M,
                     RowPlan plan, float* q, KvView<T> kv, const float2* rope) {
  const dim3 blk(256);
#define OCR_QKV_CASE(MRV)                                                                                     \
  hipLaunchKernelGGL((k_qkv_rope<T, MRV>), dim3(480, (M + MRV - 1) / MRV), blk, (size_t)MRV * D * 4, s, x, gain, \
                     eps, wqkv, M, plan, q, kv, rope);
  if (M <= 1) OCR_QKV_CASE(1)
  else if (M <= 2) OCR_QKV_CASE(2)
  else if (M <= 4) OCR_QKV_CASE(4)
  else OCR_QKV_CASE(MRG)
#undef OCR_QKV_CASE
}

// Generic GEMV.  Each wavefront owns R consecutive output rows (EPI_SWIGLU: R/2
// units, rows j.. of W0 (gate) and W1 (up)).
template <typename T, int K, int R, int MR, int EPI>
__global__ __launch_bounds__(256) void k_gemv(const float* __restrict__ a, long lda, const float* __restrict__ gain,
                                              float eps, const T* __restrict__ W0, const T* __restrict__ W1, int N,
                                              int M, float* __restrict__ out, long ldo) {
  extern __shared__ float smem[];
  float* xs = smem;
  const int wave = wave_id();
  constexpr int UNITS = (EPI == EPI_SWIGLU) ? R / 2 : R;
  const int n0 = (blockIdx.x * 4 + wave) * UNITS;
  const int m0 = blockIdx.y * MR;
  const int m_act = min(MR, M - m0);
  const T* rows[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int n;
    const T* base;
    if (EPI == EPI_SWIGLU) {
      n = n0 + (r % UNITS);
      base = (r < UNITS) ? W0 : W1;
    } else {
      n = n0 + r;
      base = W0;
    }
    n = min(n, N - 1);
    rows[r] = base + (long)n * K;
  }
  WaveGemv<T, K, R, MR> g;
  g.load(rows);
  norm_rows_wave<K, MR>(a, lda, RowIdentity{m0}, m_act, gain, eps, xs);
  __syncthreads();
  float acc[R][MR];
  g.fma(xs, m_act, acc);
  const WaveTotals<R, MR> t(acc);
  float up = 0.f;
  if constexpr (EPI == EPI_SWIGLU) up = t.partner(UNITS);  // gate unit r pairs with up unit r (rows r, r + UNITS)
  const int n = n0 + t.r;
  if (t.lead && t.r < UNITS && t.m < m_act && n < N) {
    float* o = out + (long)(m0 + t.m) * ldo + n;
    if (EPI == EPI_SWIGLU) *o = silu(t.val) * up;
    else if (EPI == EPI_ADD) *o = *o + t.val;
    else *o = t.val;
  }
}

template <typename T, int K, int R, int EPI>
static void gemv_dispatch(hipStream_t s, const float* a, long lda, const float* gain, float eps, const T* W0,
                          const T* W1, int N, int M, float* out, long ldo) {
  constexpr int UNITS = (EPI == EPI_SWIGLU) ? R / 2 : R;
  const int nb = (N + 4 * UNITS - 1) / (4 * UNITS);
  const dim3 blk(256);
#define OCR_GEMV_CASE(MRV)                                                                                   \
  {                                                                                                          \
    const size_t lds = (size_t)MRV * K * 4;                                                            \
    if (lds > 65536) {                                                                                       \
      static const bool attr_set = (hipFuncSetAttribute((const void*)k_gemv<T, K, R, MRV, EPI>,              \
                                                        hipFuncAttributeMaxDynamicSharedMemorySize,          \
                                                        (int)lds) == hipSuccess);                            \
      (void)attr_set;                                                                                        \
    }                                                                                                        \
    hipLaunchKernelGGL((k_gemv<T, K, R, MRV, EPI>), dim3(nb, (M + MRV - 1) / MRV), blk, lds, s, a, lda, gain, \
                       eps, W0, W1, N, M, out, ldo);                                                         \
  }
  if (M <= 1) OCR_GEMV_CASE(1)
  else if (M <= 2) OCR_GEMV_CASE(2)
  else if (M <= 4) OCR_GEMV_CASE(4)
  else OCR_GEMV_CASE(MRG)
#undef OCR_GEMV_CASE
}

template <typename T>
void launch_gemv(hipStream_t s, int K, Epi epi, const float* a, long lda, const float* gain, float eps,
                 const T* W0, const T* W1, int N, int M, float* out, long ldo) {
  switch (K) {
    case D:
      if (epi == EPI_SWIGLU) gemv_dispatch<T, D, 4, EPI_SWIGLU>(s, a, lda, gain, eps, W0, W1, N, M, out, ldo);
      else if (epi == EPI_ADD) gemv_dispatch<T, D, 1, EPI_ADD>(s, a, lda, gain, eps, W0, W1, N, M, out, ldo);
      else gemv_dispatch<T, D, 2, EPI_STORE>(s, a, lda, gain, eps, W0, W1, N, M, out, ldo);
      break;
    case 2 * D:
      gemv_dispatch<T, 2 * D, 2, EPI_STORE>(s, a, lda, gain, eps, W0, W1, N, M, out, ldo);
      break;
    case DF:
      gemv_dispatch<T, DF, 1, EPI_ADD>(s, a, lda, gain, eps, W0, W1, N, M, out, ldo);
      break;
    default:
      break;
  }
}

// LM head + argmax, stage 1: block (x, y) scores LM_ROWS_PER_BLOCK vocab rows
// (4 wavefronts x LM_TILES tiles x 4 rows, next tile's loads in flight while the
// current one is reduced) for activation rows y*MR .. y*MR+MR-1 and writes the
// best (value, lowest id) per row to part[row][x].  Output row m reads
// activation row (last_valid ? m*Q + cnt[m] - 1 : m) and RMSNorms it.
constexpr int LM_TILES = LM_ROWS_PER_BLOCK / 16;

struct LmSrcRow {
  const int* cnt;
  int Q, last_valid, base;
  __device__ __forceinline__ int operator()(int m) const {
    const int om = base + m;
    return last_valid ? om * Q + cnt[om] - 1 : om;
  }
};

template <typename T, int MR>
__global__ __launch_bounds__(256) void k_lmhead(const float* __restrict__ x, const int* __restrict__ cnt, int Q,
                                                int last_valid, const float* __restrict__ gain, float eps,
                                                const T* __restrict__ W, int V, int M,
                                                float* __restrict__ part_val, int* __restrict__ part_idx,
                                                float* __restrict__ logits) {
  extern __shared__ float smem[];
  float* xs = smem;
  __shared__ float bv[4][MR];
  __shared__ int bi[4][MR];
  const int wave = wave_id(), lane = lane_id();
  const int nblk = gridDim.x;
  const int m0 = blockIdx.y * MR;
  const int m_act = min(MR, M - m0);
  const int vbase = blockIdx.x * LM_ROWS_PER_BLOCK + wave * 4;
  WaveGemv<T, D, 4, MR> g[2];
  {
    const T* rows[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) rows[r] = W + (long)min(vbase + r, V - 1) * D;
    g[0].load(rows);
  }
  norm_rows_wave<D, MR>(x, D, LmSrcRow{cnt, Q, last_valid, m0}, m_act, gain, eps, xs);
  __syncthreads();
  // Each lane keeps the running best of the (tile row r, activation row m)
  // whose totals it receives.
  constexpr int SH = WaveTotals<4, MR>::SH;
  float best = -INFINITY;
  int besti = 0x7fffffff;
#pragma unroll
  for (int t = 0; t < LM_TILES; ++t) {
    if (t + 1 < LM_TILES) {
      const T* rows[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) rows[r] = W + (long)min(vbase + (t + 1) * 16 + r, V - 1) * D;
      g[(t + 1) & 1].load(rows);
    }
    float acc[4][MR];
    g[t & 1].fma(xs, m_act, acc);
    const WaveTotals<4, MR> tot(acc);
    const int v = vbase + t * 16 + tot.r;
    if (tot.m < m_act && v < V) {
      if (tot.val > best) { best = tot.val; besti = v; }  // v increases with t: ties keep the lower id
      if (logits != nullptr && tot.lead) logits[(long)(m0 + tot.m) * V + v] = tot.val;
    }
  }
  // best over the four tile rows of each m: exchanges at offsets 2^SH and
  // 2^(SH+1) (a mirror partner may sit at r ^ 3 rather than r ^ 2 in the second
  // step, which is still the other pair of rows of the same m)
#pragma unroll
  for (int off = 1 << SH; off <= 2 << SH; off <<= 1) {
    const float ob = xchg(best, off);
    const int oi = xchg_i(besti, off);
    if (ob > best || (ob == best && oi < besti)) { best = ob; besti = oi; }
  }
  {
    const int i = lane >> SH;
    if ((lane & ((1 << SH) - 1)) == 0 && (i & 3) == 0) { bv[wave][i >> 2] = best; bi[wave][i >> 2] = besti; }
  }
  __syncthreads();
  if (threadIdx.x < m_act) {
    const int m = threadIdx.x;
    float v = bv[0][m];
    int id = bi[0][m];
    for (int w = 1; w < 4; ++w) {
      if (bv[w][m] > v || (bv[w][m] == v && bi[w][m] < id)) { v = bv[w][m]; id = bi[w][m]; }
    }
    part_val[(long)(m0 + m) * nblk + blockIdx.x] = v;
    part_idx[(long)(m0 + m) * nblk + blockIdx.x] = id;
  }
}

// Stage 2: one block per output row reduces the per-block bests.
__global__ __launch_bounds__(256) void k_argmax_final(const float* __restrict__ part_val,
                                                      const int* __restrict__ part_idx, int nblk,
                                                      int* __restrict__ tok, int tok_stride) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const int m = blockIdx.x;
  const int id = argmax_block(part_val + (long)m * nblk, part_idx + (long)m * nblk, nblk, sv, si);
  if (threadIdx.x == 0) tok[(long)m * tok_stride] = id;
}

int lmhead_blocks(int V) { return (V + LM_ROWS_PER_BLOCK - 1) / LM_ROWS_PER_BLOCK; }

void launch_argmax_final(hipStream_t s, const float* part_val, const int* part_idx, int nblk, int M, int* tok,
                         int tok_stride) {
  hipLaunchKernelGGL(k_argmax_final, dim3(M), dim3(256), 0, s, part_val, part_idx, nblk, tok, tok_stride);
}

template <typename T>
void launch_lmhead(hipStream_t s, const float* x, const int* cnt, int Q, bool last_valid, const float* gain,
                   float eps, const T* W, int V, int M, float* part_val, int* part_idx, float* logits, int* tok,
                   int tok_stride) {
  const int nb = lmhead_blocks(V);
  const dim3 blk(256);
#define OCR_LM_CASE(MRV)                                                                                       \
  hipLaunchKernelGGL((k_lmhead<T, MRV>), dim3(nb, (M + MRV - 1) / MRV), blk, (size_t)MRV * D * 4, s, x, cnt, Q, \
                     (int)last_valid, gain, eps, W, V, M, part_val, part_idx, logits);
  if (M <= 1) OCR_LM_CASE(1)
  else if (M <= 2) OCR_LM_CASE(2)
  else if (M <= 4) OCR_LM_CASE(4)
  else OCR_LM_CASE(MRG)
#undef OCR_LM_CASE
  if (tok != nullptr) launch_argmax_final(s, part_val, part_idx, nb, M, tok, tok_stride);
}

#define OCR_INST_DENSE(T)                                                                                       \
  template void launch_qkv_rope<T>(hipStream_t, const float*, const float*, float, const T*, int, RowPlan,     \
                                   float*, KvView<T>, const float2*);                                            \
  template void launch_gemv<T>(hipStream_t, int, Epi, const float*, long, const float*, float, const T*,       \
                               const T*, int, int, float*, long);                                              \
  template void launch_lmhead<T>(hipStream_t, const float*, const int*, int, bool, const float*, float,        \
                                 const T*, int, int, float*, int*, float*, int*, int);
OCR_INST_DENSE(float)
OCR_INST_DENSE(bf16)

}  // namespace ocr
