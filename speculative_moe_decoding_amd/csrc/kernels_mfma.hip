// Matrix-core (MFMA) kernels for handles whose calls carry many rows: the
// grouped expert SwiGLU (gate/up with the SwiGLU product fused, then down) and
// the LM head with its argmax, for bf16 weights.
//
// Tile engine: a block of four wavefronts owns a strip of weight rows (16 per
// wavefront and per matrix) and streams the strip once per pass of up to 64
// activation rows.  The rows are staged in LDS in chunks of 128 k as ready MFMA
// A fragments, two chunk buffers deep; weights go straight from HBM into B
// fragments.  Expert inputs are split into two bf16 parts, hi = bf16(a) and
// lo = bf16(a - hi) (round to nearest even), and both are multiplied (about 16
// significant bits of the fp32 activation survive, so the rounding does not
// compound over the layers); the LM head takes hi alone (one rounding at the
// end of the network).  Each 16x16 output block accumulates
// v_mfma_f32_16x16x32_bf16 over k (hi then lo per k-step) in a fixed order, so
// a row's result depends only on that row and the weights: the row count of a
// call never changes it (speculative == autoregressive, bit for bit, on one
// handle).
//
// v_mfma_f32_16x16x32_bf16 operand layout (wave64): lane l supplies
// A[l % 16][8 (l / 16) .. +7] and B[8 (l / 16) .. +7][l % 16]; it receives
// D[4 (l / 16) + r][l % 16] in result register r.  With B[k][j] = W[j][k], a
// lane's B fragment is 16 contiguous bytes of weight row j.
#include "launch.h"

namespace ocr {

typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef float f32x4_v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_v mfma_bf16(const uint4& a, const uint4& b, f32x4_v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, a), __builtin_bit_cast(bf16x8_v, b),
                                                 c, 0, 0, 0);
}

typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float f32x2_v __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 (round to nearest even; gfx950 converts in hardware).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_v f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_v));
}

constexpr int MF_KC = 128;           // k per LDS chunk
constexpr int MF_SC = MF_KC / 32;    // MFMA k-steps per chunk
constexpr int MF_MT = 4;             // 16-row tiles per pass
constexpr int MF_ROWS = 16 * MF_MT;  // activation rows per pass

// One LDS chunk: f[tile][step][lane] is lane's A fragment, i.e. row
// 16 tile + lane % 16, k = 32 step + 8 (lane / 16) .. +7 of the chunk.
struct MfChunk {
  uint4 f[MF_MT][MF_SC][64];
};

// Passes use NT (1, 2 or 4) tiles, the fewest that hold their rows; rows of a
// tile past the pass's row count are zero.

template <int K, int NB, int NS>
__device__ __forceinline__ void mf_load_b(uint4 (&bq)[NB][NS][MF_SC], const bf16* const (&w)[NB], long woff, int c) {
#pragma unroll
  for (int s = 0; s < MF_SC; ++s)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int n = 0; n < NS; ++n) bq[b][n][s] = ldg16_stream(w[b] + (long)n * 16 * K + woff + c * MF_KC + 32 * s);
}

// Thread tid stages the 8-element group kg = tid % 16 of row tid / 16 + 16 i
// (tile i) of every chunk; rows past the pass read a valid row and are zeroed.
template <int NT>
__device__ __forceinline__ void mf_load_a(float4 (&ar)[NT][2], const float* const (&src)[NT], const bool (&ok)[NT],
                                          int c) {
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const float4* p = reinterpret_cast<const float4*>(src[i] + c * MF_KC);
    const float4 a = p[0], b = p[1];
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    ar[i][0] = ok[i] ? a : z;
    ar[i][1] = ok[i] ? b : z;
  }
}

// a - bf16(a) for the two halves of a packed pair (exact in fp32).
__device__ __forceinline__ float rem_lo(float a, uint32_t h) { return a - __uint_as_float(h << 16); }
__device__ __forceinline__ float rem_hi(float a, uint32_t h) { return a - __uint_as_float(h & 0xffff0000u); }

// Parts NP = 1: ch[0] = bf16(a); NP = 2: also ch[1] = bf16(a - bf16(a)).
template <int NT, int NP>
__device__ __forceinline__ void mf_store_a(MfChunk (&ch)[NP], const float4 (&ar)[NT][2], int kg, int ri) {
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    uint4 v;
    v.x = pack_bf16x2(ar[i][0].x, ar[i][0].y);
    v.y = pack_bf16x2(ar[i][0].z, ar[i][0].w);
    v.z = pack_bf16x2(ar[i][1].x, ar[i][1].y);
    v.w = pack_bf16x2(ar[i][1].z, ar[i][1].w);
    ch[0].f[i][kg >> 2][(kg & 3) * 16 + ri] = v;
    if constexpr (NP == 2) {
      uint4 u;
      u.x = pack_bf16x2(rem_lo(ar[i][0].x, v.x), rem_hi(ar[i][0].y, v.x));
      u.y = pack_bf16x2(rem_lo(ar[i][0].z, v.y), rem_hi(ar[i][0].w, v.y));
      u.z = pack_bf16x2(rem_lo(ar[i][1].x, v.z), rem_hi(ar[i][1].y, v.z));
      u.w = pack_bf16x2(rem_lo(ar[i][1].z, v.w), rem_hi(ar[i][1].w, v.w));
      ch[1].f[i][kg >> 2][(kg & 3) * 16 + ri] = u;
    }
  }
}

template <int NT, int NB, int NS, int NP>
__device__ __forceinline__ void mf_compute(const MfChunk (&ch)[NP], const uint4 (&bq)[NB][NS][MF_SC],
                                           f32x4_v (&acc)[NT][NB][NS]) {
  const int lane = lane_id();
#pragma unroll
  for (int s = 0; s < MF_SC; ++s) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const uint4 a = ch[p].f[i][s][lane];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int n = 0; n < NS; ++n) acc[i][b][n] = mfma_bf16(a, bq[b][n][s], acc[i][b][n]);
      }
    }
  }
}

// One pass: rows r < rows <= 16 NT (row r read from rowp(r), fp32, K long)
// against the wavefront's weight rows w[b] + (16 n + j) K, j < 16, of NB
// matrices: acc[i][b][n][q] = sum_k A[16 i + 4 (lane / 16) + q][k] *
// W_b[16 n + lane % 16][k], with A in NP bf16 parts.  All 256 threads must
// call it; contains barriers.
template <int K, int NT, int NB, int NS, int NP, typename RowPtr>
__device__ __forceinline__ void mfma_pass(const bf16* const (&w)[NB], RowPtr rowp, int rows, MfChunk (&buf)[2][NP],
                                          f32x4_v (&acc)[NT][NB][NS]) {
  static_assert(K % MF_KC == 0, "K must be a multiple of the chunk");
  static_assert(NT <= MF_MT, "too many tiles");
  constexpr int NC = K / MF_KC;
  const int tid = threadIdx.x, lane = tid & 63;
  const long woff = (long)(lane & 15) * K + 8 * (lane >> 4);
  const int kg = tid & 15, ri = tid >> 4;
  const float* src[NT];
  bool ok[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int r = ri + 16 * i;
    ok[i] = r < rows;
    src[i] = rowp(ok[i] ? r : 0) + 8 * kg;
  }
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int n = 0; n < NS; ++n) acc[i][b][n] = f32x4_v{0.f, 0.f, 0.f, 0.f};
  uint4 bq0[NB][NS][MF_SC], bq1[NB][NS][MF_SC];
  float4 ar[NT][2];
  mf_load_a(ar, src, ok, 0);
  mf_load_b<K, NB, NS>(bq0, w, woff, 0);
  mf_store_a(buf[0], ar, kg, ri);
  __syncthreads();
  // Chunk c computes from LDS buffer c % 2 and registers bq(c % 2) while
  // chunk c + 1 is loaded into the other pair; one barrier per chunk.
#pragma unroll 1
  for (int c = 0; c < NC; c += 2) {
    if (c + 1 < NC) {
      mf_load_a(ar, src, ok, c + 1);  // activations first: waiting for them does not wait for the weights
      mf_load_b<K, NB, NS>(bq1, w, woff, c + 1);
    }
    mf_compute<NT, NB, NS, NP>(buf[0], bq0, acc);
    if (c + 1 < NC) mf_store_a(buf[1], ar, kg, ri);
    __syncthreads();
    if (c + 1 < NC) {
      if (c + 2 < NC) {
        mf_load_a(ar, src, ok, c + 2);
        mf_load_b<K, NB, NS>(bq0, w, woff, c + 2);
      }
      mf_compute<NT, NB, NS, NP>(buf[1], bq1, acc);
      if (c + 2 < NC) mf_store_a(buf[0], ar, kg, ri);
      __syncthreads();
    }
  }
}

// Gate/up: block (x, slot s) computes units j0 .. j0+15, j0 = 64 x + 16 w, of
// active expert s for every pair routed to it:
// hx[pair][j] = silu(gate_j . b) * (up_j . b), b the pair's normalised row.
template <int NT>
__device__ __forceinline__ void gate_up_pass(const bf16* const (&w)[2], const float* __restrict__ bnorm,
                                             const int* __restrict__ perm, int kb, int rows, float* __restrict__ hx,
                                             int j0, MfChunk (&buf)[2][2]) {
  const int lane = lane_id();
  f32x4_v acc[NT][2][1];
  mfma_pass<D, NT, 2, 1, 2>(w, [=](int r) { return bnorm + (long)(perm[kb + r] / NSLOT) * D; }, rows, buf, acc);
#pragma unroll
  for (int i = 0; i < NT; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 16 * i + 4 * (lane >> 4) + q;
      if (r < rows) hx[(long)(kb + r) * DI + j0 + (lane & 15)] = silu(acc[i][0][0][q]) * acc[i][1][0][q];
    }
  }
}

__global__ __launch_bounds__(256) void k_expert_gate_up_mfma(const bf16* __restrict__ wg,
                                                             const bf16* __restrict__ wu, int M, MoeBufs mb) {
  __shared__ MfChunk buf[2][2];
  const int4 info = expert_work(mb, blockIdx.y, M);
  const int e = info.x;
  if (e < 0) return;
  const int j0 = blockIdx.x * 64 + wave_id() * 16;
  const bf16* const w[2] = {wg + ((long)e * DI + j0) * D, wu + ((long)e * DI + j0) * D};
  for (int kb = info.y; kb < info.z; kb += MF_ROWS) {
    const int rows = min(MF_ROWS, info.z - kb);
    if (rows <= 16) gate_up_pass<1>(w, mb.bnorm, mb.perm, kb, rows, mb.hx, j0, buf);
    else if (rows <= 32) gate_up_pass<2>(w, mb.bnorm, mb.perm, kb, rows, mb.hx, j0, buf);
    else gate_up_pass<4>(w, mb.bnorm, mb.perm, kb, rows, mb.hx, j0, buf);
  }
}

// Down: block (x, slot s) computes outputs n0 .. n0+31, n0 = 128 x + 32 w:
// y[pair][n] = W_d[n] . hx[pair].
template <int NT>
__device__ __forceinline__ void down_pass(const bf16* const (&w)[1], const float* __restrict__ hx, int kb, int rows,
                                          float* __restrict__ y, int n0, MfChunk (&buf)[2][2]) {
  const int lane = lane_id();
  f32x4_v acc[NT][1][2];
  mfma_pass<DI, NT, 1, 2, 2>(w, [=](int r) { return hx + (long)(kb + r) * DI; }, rows, buf, acc);
#pragma unroll
  for (int i = 0; i < NT; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 16 * i + 4 * (lane >> 4) + q;
      if (r < rows) {
        float* o = y + (long)(kb + r) * D + n0 + (lane & 15);
        o[0] = acc[i][0][0][q];
        o[16] = acc[i][0][1][q];
      }
    }
  }
}

__global__ __launch_bounds__(256) void k_expert_down_mfma(const bf16* __restrict__ wd, int M, MoeBufs mb) {
  __shared__ MfChunk buf[2][2];
  const int4 info = expert_work(mb, blockIdx.y, M);
  const int e = info.x;
  if (e < 0) return;
  const int n0 = blockIdx.x * 128 + wave_id() * 32;
  const bf16* const w[1] = {wd + ((long)e * D + n0) * DI};
  for (int kb = info.y; kb < info.z; kb += MF_ROWS) {
    const int rows = min(MF_ROWS, info.z - kb);
    if (rows <= 16) down_pass<1>(w, mb.hx, kb, rows, mb.y, n0, buf);
    else if (rows <= 32) down_pass<2>(w, mb.hx, kb, rows, mb.y, n0, buf);
    else down_pass<4>(w, mb.hx, kb, rows, mb.y, n0, buf);
  }
}

void launch_expert_gate_up_mfma(hipStream_t s, const bf16* wg, const bf16* wu, int M, const MoeBufs& mb) {
  hipLaunchKernelGGL(k_expert_gate_up_mfma, dim3(DI / 64, expert_slot_cap(M)), dim3(256), 0, s, wg, wu, M, mb);
}

void launch_expert_down_mfma(hipStream_t s, const bf16* wd, int M, const MoeBufs& mb) {
  hipLaunchKernelGGL(k_expert_down_mfma, dim3(D / 128, expert_slot_cap(M)), dim3(256), 0, s, wd, M, mb);
}

// LM head rows for the matrix cores: xn[m] = RMSNorm(x[src(m)]) * gain, one
// wavefront per row, src(m) = m * Q + cnt[m] - 1 when last_valid, else m.
// Lane l sums x[k]^2 over k = l + 64 j in order, then the xor butterfly.
__global__ __launch_bounds__(256) void k_lm_norm(const float* __restrict__ x, const int* __restrict__ cnt, int Q,
                                                 int last_valid, const float* __restrict__ gain, float eps, int M,
                                                 float* __restrict__ xn) {
  constexpr int J = D / 64;
  const int m = blockIdx.x * 4 + wave_id();
  if (m >= M) return;
  const int lane = lane_id();
  const float* xr = x + (long)(last_valid ? m * Q + cnt[m] - 1 : m) * D;
  float v[J];
#pragma unroll
  for (int j = 0; j < J; ++j) v[j] = xr[lane + 64 * j];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < J; ++j) ss = fmaf(v[j], v[j], ss);
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / (float)D + eps);
#pragma unroll
  for (int j = 0; j < J; ++j) xn[(long)m * D + lane + 64 * j] = (v[j] * r) * gain[lane + 64 * j];
}

// LM head + argmax stage 1 on the matrix cores (V >= 16): block x scores vocab
// rows 64 x .. 64 x + 63 (16 per wavefront) for all M rows, passes of 64 rows,
// and writes the best (value, lowest id) per row to part[row][x]; logits
// optionally stored to logits[row][V].
template <int NT>
__device__ __forceinline__ void lm_pass(const bf16* const (&w)[1], const float* __restrict__ xn, int p0, int rows,
                                        int vj, bool vok, int V, float* __restrict__ logits, float (&bv)[4][MF_ROWS],
                                        int (&bi)[4][MF_ROWS], MfChunk (&buf)[2][1]) {
  const int wave = wave_id(), lane = lane_id();
  f32x4_v acc[NT][1][1];
  mfma_pass<D, NT, 1, 1, 1>(w, [=](int r) { return xn + (long)(p0 + r) * D; }, rows, buf, acc);
#pragma unroll
  for (int i = 0; i < NT; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 16 * i + 4 * (lane >> 4) + q;
      const bool ok = vok && r < rows;
      const float val = acc[i][0][0][q];
      if (ok && logits != nullptr) logits[(long)(p0 + r) * V + vj] = val;
      float b = ok ? val : -INFINITY;
      int id = ok ? vj : 0x7fffffff;
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) {
        const float ob = __shfl_xor(b, off, 64);
        const int oi = __shfl_xor(id, off, 64);
        if (ob > b || (ob == b && oi < id)) { b = ob; id = oi; }
      }
      if ((lane & 15) == 0) { bv[wave][r] = b; bi[wave][r] = id; }
    }
  }
}

__global__ __launch_bounds__(256) void k_lmhead_mfma(const float* __restrict__ xn, const bf16* __restrict__ W,
                                                     int V, int M, float* __restrict__ part_val,
                                                     int* __restrict__ part_idx, float* __restrict__ logits) {
  __shared__ MfChunk buf[2][1];
  __shared__ float bv[4][MF_ROWS];
  __shared__ int bi[4][MF_ROWS];
  const int wave = wave_id(), lane = lane_id();
  const int nblk = gridDim.x;
  const int v0 = blockIdx.x * LM_ROWS_PER_BLOCK + wave * 16;
  // A strip reaching past the vocabulary is moved back to rows V-16 .. V-1;
  // its lanes then keep only the ids >= v0 (the others belong to the strip before).
  const bool shifted = v0 > V - 16;
  const bf16* const w[1] = {W + (long)(shifted ? V - 16 : v0) * D};
  const int vj = (shifted ? V - 16 : v0) + (lane & 15);
  const bool vok = vj >= v0 && vj < V;
  for (int p0 = 0; p0 < M; p0 += MF_ROWS) {
    const int rows = min(MF_ROWS, M - p0);
    if (rows <= 16) lm_pass<1>(w, xn, p0, rows, vj, vok, V, logits, bv, bi, buf);
    else if (rows <= 32) lm_pass<2>(w, xn, p0, rows, vj, vok, V, logits, bv, bi, buf);
    else lm_pass<4>(w, xn, p0, rows, vj, vok, V, logits, bv, bi, buf);
    __syncthreads();
    if ((int)threadIdx.x < rows) {
      const int r = threadIdx.x;
      float b = bv[0][r];
      int id = bi[0][r];
      for (int ww = 1; ww < 4; ++ww)
        if (bv[ww][r] > b || (bv[ww][r] == b && bi[ww][r] < id)) { b = bv[ww][r]; id = bi[ww][r]; }
      part_val[(long)(p0 + r) * nblk + blockIdx.x] = b;
      part_idx[(long)(p0 + r) * nblk + blockIdx.x] = id;
    }
    __syncthreads();
  }
}

void launch_lmhead_mfma(hipStream_t s, const float* x, const int* cnt, int Q, bool last_valid, const float* gain,
                        float eps, const bf16* W, int V, int M, float* xn, float* part_val, int* part_idx,
                        float* logits, int* tok, int tok_stride) {
  hipLaunchKernelGGL(k_lm_norm, dim3((M + 3) / 4), dim3(256), 0, s, x, cnt, Q, (int)last_valid, gain, eps, M, xn);
  const int nb = lmhead_blocks(V);
  hipLaunchKernelGGL(k_lmhead_mfma, dim3(nb), dim3(256), 0, s, xn, W, V, M, part_val, part_idx, logits);
  launch_argmax_final(s, part_val, part_idx, nb, M, tok, tok_stride);
}

}  // namespace ocr
