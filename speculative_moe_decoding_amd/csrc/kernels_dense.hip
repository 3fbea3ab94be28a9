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

// cos / sin of pos * theta^(-2i/HD): angle in fp64, rounded to fp32.
__device__ __forceinline__ void rope_cs(int pos, int i, float theta, float& c, float& s) {
  const double inv = pow((double)theta, -(double)(2 * i) / (double)HD);
  const double a = (double)pos * inv;
  double sd, cd;
  sincos(a, &sd, &cd);
  c = (float)cd;
  s = (float)sd;
}

// Rotate the pair (a, b) = (x_i, x_{i+64}) by the angle with cosine c, sine s.
__device__ __forceinline__ void rot(float a, float b, float c, float s, float& o1, float& o2) {
  o1 = fmaf(a, c, -(b * s));
  o2 = fmaf(b, c, a * s);
}

// One wavefront = one "quad" of 4 output rows.  q / k quads are rows
// {2u, 2u+1, 2u+64, 2u+65} of one head so that both halves of a RoPE pair land
// in the same wavefront; v quads are 4 consecutive rows.
template <typename T, int MR>
__global__ __launch_bounds__(256) void k_qkv_rope(const float* __restrict__ x, const float* __restrict__ gain,
                                                  float eps, const T* __restrict__ wqkv, int M, RowPlan plan,
                                                  float* __restrict__ q, T* __restrict__ kv, int max_pos,
                                                  float theta) {
  extern __shared__ float smem[];
  float* xs = smem;
  float* red = smem + MR * D;
  const int wave = wave_id(), lane = lane_id();
  const int quad = blockIdx.x * 4 + wave;  // 0 .. 959
  const int m0 = blockIdx.y * MR;
  const int m_act = min(MR, M - m0);
  const int sec = quad / 320, rem = quad % 320, h = rem / 32, u = rem % 32;
  int ri[4];
  if (sec < 2) {
    const int b0 = sec * QD + h * HD + 2 * u;
    ri[0] = b0; ri[1] = b0 + 1; ri[2] = b0 + 64; ri[3] = b0 + 65;
  } else {
    const int b0 = 2 * QD + h * HD + 4 * u;
    ri[0] = b0; ri[1] = b0 + 1; ri[2] = b0 + 2; ri[3] = b0 + 3;
  }
  const T* rows[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) rows[r] = wqkv + (long)ri[r] * D;
  WaveGemv<T, D, 4, MR> g;
  g.load(rows);
  norm_rows_to_lds<D>(x + (long)m0 * D, D, m_act, gain, eps, xs, red);
  __syncthreads();
  float acc[4][MR];
  g.fma(xs, m_act, acc);
  wave_reduce_acc<4, MR>(acc, m_act);
  const long slot_stride = 2L * NH * max_pos * HD;
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    if (lane == m && m < m_act) {
      const int row = m0 + m;
      const int b = row / plan.Q, i = row - b * plan.Q;
      const bool valid = i < plan.cnt[b];
      const int pos = plan.base[b] + i;
      const long slot = plan.slot[b];
      if (sec < 2) {
        float c0, s0, c1, s1, o[4];
        rope_cs(pos, 2 * u, theta, c0, s0);
        rope_cs(pos, 2 * u + 1, theta, c1, s1);
        rot(acc[0][m], acc[2][m], c0, s0, o[0], o[2]);
        rot(acc[1][m], acc[3][m], c1, s1, o[1], o[3]);
        const int dims[4] = {2 * u, 2 * u + 1, 2 * u + 64, 2 * u + 65};
        if (sec == 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r) q[(long)row * QD + h * HD + dims[r]] = o[r];
        } else if (valid && pos >= 0 && pos < max_pos) {
          T* kd = kv + slot * slot_stride + ((long)h * max_pos + pos) * HD;
#pragma unroll
          for (int r = 0; r < 4; ++r) kd[dims[r]] = WT<T>::store_cvt(o[r]);
        }
      } else if (valid && pos >= 0 && pos < max_pos) {
        T* vd = kv + slot * slot_stride + ((long)(NH + h) * max_pos + pos) * HD + 4 * u;
#pragma unroll
        for (int r = 0; r < 4; ++r) vd[r] = WT<T>::store_cvt(acc[r][m]);
      }
    }
  }
}

template <typename T>
void launch_qkv_rope(hipStream_t s, const float* x, const float* gain, float eps, const T* wqkv, int M,
                     RowPlan plan, float* q, T* kv, int max_pos, float theta) {
  const dim3 blk(256);
  if (M <= 1) {
    hipLaunchKernelGGL((k_qkv_rope<T, 1>), dim3(240, 1), blk, (1 * D + 4) * 4, s, x, gain, eps, wqkv, M, plan, q,
                       kv, max_pos, theta);
  } else if (M <= 2) {
    hipLaunchKernelGGL((k_qkv_rope<T, 2>), dim3(240, 1), blk, (2 * D + 4) * 4, s, x, gain, eps, wqkv, M, plan, q,
                       kv, max_pos, theta);
  } else if (M <= 4) {
    hipLaunchKernelGGL((k_qkv_rope<T, 4>), dim3(240, 1), blk, (4 * D + 4) * 4, s, x, gain, eps, wqkv, M, plan, q,
                       kv, max_pos, theta);
  } else {
    hipLaunchKernelGGL((k_qkv_rope<T, MRG>), dim3(240, (M + MRG - 1) / MRG), blk, (MRG * D + 4) * 4, s, x, gain,
                       eps, wqkv, M, plan, q, kv, max_pos, theta);
  }
}

// Generic GEMV.  Each wavefront owns R consecutive output rows (EPI_SWIGLU: R/2
// units, rows j.. of W0 (gate) and W1 (up)).
template <typename T, int K, int R, int MR, int EPI>
__global__ __launch_bounds__(256) void k_gemv(const float* __restrict__ a, long lda, const float* __restrict__ gain,
                                              float eps, const T* __restrict__ W0, const T* __restrict__ W1, int N,
                                              int M, float* __restrict__ out, long ldo) {
  extern __shared__ float smem[];
  float* xs = smem;
  float* red = smem + MR * K;
  const int wave = wave_id(), lane = lane_id();
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
  norm_rows_to_lds<K>(a + (long)m0 * lda, lda, m_act, gain, eps, xs, red);
  __syncthreads();
  float acc[R][MR];
  g.fma(xs, m_act, acc);
  wave_reduce_acc<R, MR>(acc, m_act);
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    if (lane == m && m < m_act) {
      float* o = out + (long)(m0 + m) * ldo;
#pragma unroll
      for (int r = 0; r < UNITS; ++r) {
        const int n = n0 + r;
        if (n < N) {
          if (EPI == EPI_SWIGLU) o[n] = silu(acc[r][m]) * acc[r + UNITS][m];
          else if (EPI == EPI_ADD) o[n] = o[n] + acc[r][m];
          else o[n] = acc[r][m];
        }
      }
    }
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
    const size_t lds = ((size_t)MRV * K + 4) * 4;                                                            \
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

// LM head + argmax, stage 1: each block scores LM_ROWS_PER_BLOCK vocab rows
// (4 wavefronts x 4 tiles x 4 rows) for up to MR activation rows, keeps the
// best (value, lowest id) per row; the last block to finish reduces the
// per-block bests.
template <typename T, int MR>
__global__ __launch_bounds__(256) void k_lmhead(const float* __restrict__ x, const int* __restrict__ cnt, int Q,
                                                int last_valid, const float* __restrict__ gain, float eps,
                                                const T* __restrict__ W, int V, int M,
                                                float* __restrict__ part_val, int* __restrict__ part_idx,
                                                int* __restrict__ counter, float* __restrict__ logits,
                                                int* __restrict__ tok, int tok_stride) {
  extern __shared__ float smem[];
  float* xs = smem;
  float* red = smem + MR * D;
  __shared__ float bv[4][MR];
  __shared__ int bi[4][MR];
  __shared__ int is_last;
  const int wave = wave_id(), lane = lane_id();
  const int nblk = gridDim.x;
  for (int m0 = 0; m0 < M; m0 += MR) {
    const int m_act = min(MR, M - m0);
    // gather + normalise the activation rows of this group
    for (int m = 0; m < m_act; ++m) {
      const int om = m0 + m;
      const int src = last_valid ? om * Q + cnt[om] - 1 : om;
      norm_rows_to_lds<D>(x + (long)src * D, D, 1, gain, eps, xs + m * D, red);
    }
    __syncthreads();
    float best[MR];
    int besti[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) { best[m] = -INFINITY; besti[m] = 0x7fffffff; }
#pragma unroll 1
    for (int t = 0; t < 4; ++t) {
      const int v0 = blockIdx.x * LM_ROWS_PER_BLOCK + wave * 16 + t * 4;
      const T* rows[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) rows[r] = W + (long)min(v0 + r, V - 1) * D;
      WaveGemv<T, D, 4, MR> g;
      g.load(rows);
      float acc[4][MR];
      g.fma(xs, m_act, acc);
      wave_reduce_acc<4, MR>(acc, m_act);
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        if (m < m_act) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int v = v0 + r;
            if (v < V) {
              const float val = acc[r][m];
              if (val > best[m]) { best[m] = val; besti[m] = v; }  // v increases: ties keep the lower id
              if (logits != nullptr && lane == r) logits[(long)(m0 + m) * V + v] = val;
            }
          }
        }
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int m = 0; m < MR; ++m) { bv[wave][m] = best[m]; bi[wave][m] = besti[m]; }
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
    __syncthreads();
  }
  // stage 2: the last block reduces the per-block bests
  __threadfence();
  if (threadIdx.x == 0) is_last = (atomicAdd(counter, 1) == nblk - 1);
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  for (int m = wave; m < M; m += 4) {
    float v = -INFINITY;
    int id = 0x7fffffff;
    for (int b = lane; b < nblk; b += 64) {
      const float pv = __builtin_nontemporal_load(part_val + (long)m * nblk + b);
      const int pi = __builtin_nontemporal_load(part_idx + (long)m * nblk + b);
      if (pv > v || (pv == v && pi < id)) { v = pv; id = pi; }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(v, off, 64);
      const int oi = __shfl_xor(id, off, 64);
      if (ov > v || (ov == v && oi < id)) { v = ov; id = oi; }
    }
    if (lane == 0) tok[(long)m * tok_stride] = id;
  }
  if (threadIdx.x == 0) *counter = 0;
}

int lmhead_blocks(int V) { return (V + LM_ROWS_PER_BLOCK - 1) / LM_ROWS_PER_BLOCK; }

template <typename T>
void launch_lmhead(hipStream_t s, const float* x, const int* cnt, int Q, bool last_valid, const float* gain,
                   float eps, const T* W, int V, int M, float* part_val, int* part_idx, int* counter,
                   float* logits, int* tok, int tok_stride) {
  const int nb = lmhead_blocks(V);
  const dim3 blk(256);
#define OCR_LM_CASE(MRV)                                                                                    \
  hipLaunchKernelGGL((k_lmhead<T, MRV>), dim3(nb), blk, ((size_t)MRV * D + 4) * 4, s, x, cnt, Q,             \
                     (int)last_valid, gain, eps, W, V, M, part_val, part_idx, counter, logits, tok, tok_stride);
  if (M <= 1) OCR_LM_CASE(1)
  else if (M <= 2) OCR_LM_CASE(2)
  else if (M <= 4) OCR_LM_CASE(4)
  else OCR_LM_CASE(MRG)
#undef OCR_LM_CASE
}

#define OCR_INST_DENSE(T)                                                                                       \
  template void launch_qkv_rope<T>(hipStream_t, const float*, const float*, float, const T*, int, RowPlan,     \
                                   float*, T*, int, float);                                                    \
  template void launch_gemv<T>(hipStream_t, int, Epi, const float*, long, const float*, float, const T*,       \
                               const T*, int, int, float*, long);                                              \
  template void launch_lmhead<T>(hipStream_t, const float*, const int*, int, bool, const float*, float,        \
                                 const T*, int, int, float*, int*, int*, float*, int*, int);
OCR_INST_DENSE(float)
OCR_INST_DENSE(bf16)

}  // namespace ocr
