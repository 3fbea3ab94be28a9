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
// end of the network, made when its rows are normalised).  Each 16x16 output block accumulates
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


constexpr int MF_KC = 128;           // k per LDS chunk
constexpr int MF_SC = MF_KC / 32;    // MFMA k-steps per chunk
constexpr int MF_MT = 4;             // 16-row tiles per pass
constexpr int MF_ROWS = 16 * MF_MT;  // activation rows per pass
// Activation rows per block of the strip GEMMs: 32 for passes of up to 512
// rows (more blocks in flight: base-page prefill 2.94 against 3.05 ms), else
// MF_ROWS (Gundam page 6.55 against 6.68 ms).  Each output's sum over k is the
// same either way.
inline int dense_rows_per_block(int M) { return M <= 512 ? 32 : MF_ROWS; }
constexpr int MF_BP = 3;             // weight chunks in flight per wavefront

// One LDS chunk of CT tiles: f[tile][step][mf_slot(step, lane)] is lane's A
// fragment, i.e. row 16 tile + lane % 16, k = 32 step + 8 (lane / 16) .. +7
// of the chunk.  The slot swizzle (low four bits xor the fragment's k-group)
// spreads the staging writes of a wavefront, whose lanes stage four rows x
// sixteen k-groups, over all LDS banks; a wavefront's reads of one step still
// cover the 1 KiB row once.
__device__ __forceinline__ int mf_slot(int step, int lane) {
  return (lane & 48) | ((lane & 15) ^ ((4 * step + (lane >> 4)) & 15));
}
template <int CT>
struct MfChunkT {
  uint4 f[CT][MF_SC][64];
};
typedef MfChunkT<MF_MT> MfChunk;

// Passes use NT (1, 2 or 4) tiles, the fewest that hold their rows; rows of a
// tile past the pass's row count are zero.

// Weight fragments of chunk c: ordinary loads (CACHED), or non-temporal ones
// for a strip read once per launch where that measured faster.
template <int K, int NB, int NS, bool CACHED = false>
__device__ __forceinline__ void mf_load_b(uint4 (&bq)[NB][NS][MF_SC], const bf16* const (&w)[NB], long woff, int c) {
#pragma unroll
  for (int s = 0; s < MF_SC; ++s)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int n = 0; n < NS; ++n) {
        const bf16* p = w[b] + (long)n * 16 * K + woff + c * MF_KC + 32 * s;
        bq[b][n][s] = CACHED ? ldg16(p) : ldg16_stream(p);
      }
}

// Thread tid stages the 8-element group kg = tid % 16 of row tid / 16 + 16 i
// (tile i) of every chunk; rows past the pass read a valid row and are zeroed.
// With a gain g (RMSNorm rows) the gains of the group are loaded alongside.
template <int NT>
__device__ __forceinline__ void mf_load_a(float4 (&ar)[NT][2], float4 (&gq)[2], const float* const (&src)[NT],
                                          const bool (&ok)[NT], const float* __restrict__ g, int kg, int c) {
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const float4* p = reinterpret_cast<const float4*>(src[i] + c * MF_KC);
    const float4 a = p[0], b = p[1];
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    ar[i][0] = ok[i] ? a : z;
    ar[i][1] = ok[i] ? b : z;
  }
  if (g != nullptr) {
    const float4* gp = reinterpret_cast<const float4*>(g + c * MF_KC + 8 * kg);
    gq[0] = gp[0];
    gq[1] = gp[1];
  }
}

// RMSNorm of the staged group: (a * r) * g, r the row's scale.
__device__ __forceinline__ float4 mf_norm(const float4& a, float r, const float4& g) {
  return make_float4((a.x * r) * g.x, (a.y * r) * g.y, (a.z * r) * g.z, (a.w * r) * g.w);
}


// Parts NP = 1: ch[0] = bf16(a); NP = 2: also ch[1] = bf16(a - bf16(a)).
// NORM: a is first normalised with the thread's row scales rsv and gains gq.
template <int NT, int NP, bool NORM, int CT>
__device__ __forceinline__ void mf_store_a(MfChunkT<CT> (&ch)[NP], float4 (&ar)[NT][2], const float4 (&gq)[2],
                                           const float (&rsv)[NT], int kg, int ri) {
  static_assert(NT <= CT, "chunk too small for the pass");
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    if constexpr (NORM) {
      ar[i][0] = mf_norm(ar[i][0], rsv[i], gq[0]);
      ar[i][1] = mf_norm(ar[i][1], rsv[i], gq[1]);
    }
    uint4 v;
    v.x = pack_bf16x2(ar[i][0].x, ar[i][0].y);
    v.y = pack_bf16x2(ar[i][0].z, ar[i][0].w);
    v.z = pack_bf16x2(ar[i][1].x, ar[i][1].y);
    v.w = pack_bf16x2(ar[i][1].z, ar[i][1].w);
    const int slot = mf_slot(kg >> 2, (kg & 3) * 16 + ri);
    ch[0].f[i][kg >> 2][slot] = v;
    if constexpr (NP == 2) {
      uint4 u;
      u.x = pack_bf16x2(rem_lo(ar[i][0].x, v.x), rem_hi(ar[i][0].y, v.x));
      u.y = pack_bf16x2(rem_lo(ar[i][0].z, v.y), rem_hi(ar[i][0].w, v.y));
      u.z = pack_bf16x2(rem_lo(ar[i][1].x, v.z), rem_hi(ar[i][1].y, v.z));
      u.w = pack_bf16x2(rem_lo(ar[i][1].z, v.w), rem_hi(ar[i][1].w, v.w));
      ch[1].f[i][kg >> 2][slot] = u;
    }
  }
}

template <int NT, int NB, int NS, int NP, int CT>
__device__ __forceinline__ void mf_compute(const MfChunkT<CT> (&ch)[NP], const uint4 (&bq)[NB][NS][MF_SC],
                                           f32x4_v (&acc)[NT][NB][NS]) {
  const int lane = lane_id();
#pragma unroll
  for (int s = 0; s < MF_SC; ++s) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const uint4 a = ch[p].f[i][s][mf_slot(s, lane)];
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
// W_b[16 n + lane % 16][k], with A in NP bf16 parts.  With a gain g, row r of
// A is RMSNorm'ed first: (a * rs[r]) * g (rs in LDS, one scale per pass row).
// All 256 threads must call it; contains barriers.
template <int K, int NT, int NB, int NS, int NP, typename RowPtr, bool NORM = false, int CT = MF_MT,
          bool DEEP = false, bool CACHED = false>
__device__ __forceinline__ void mfma_pass(const bf16* const (&w)[NB], RowPtr rowp, int rows, MfChunkT<CT> (&buf)[2][NP],
                                          f32x4_v (&acc)[NT][NB][NS], const float* __restrict__ g = nullptr,
                                          const float* rs = nullptr) {
  static_assert(K % MF_KC == 0, "K must be a multiple of the chunk");
  static_assert(NT <= MF_MT, "too many tiles");
  constexpr int NC = K / MF_KC;
  const int tid = threadIdx.x, lane = tid & 63;
  const long woff = (long)(lane & 15) * K + 8 * (lane >> 4);
  const int kg = tid & 15, ri = tid >> 4;
  const float* src[NT];
  bool ok[NT];
  float rsv[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int r = ri + 16 * i;
    ok[i] = r < rows;
    src[i] = rowp(ok[i] ? r : 0) + 8 * kg;
    rsv[i] = NORM ? rs[ok[i] ? r : 0] : 1.f;
  }
  const float* gn = NORM ? g : nullptr;
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int n = 0; n < NS; ++n) acc[i][b][n] = f32x4_v{0.f, 0.f, 0.f, 0.f};
  if constexpr (DEEP) {
    // Long passes (prefill): weights in a ring of MF_BP chunks in registers,
    // activations two chunks in registers and two in LDS.  Chunk c + 2's rows
    // are loaded before chunk c's arithmetic and chunk c + MF_BP's weights
    // after it, so that waiting for chunk c + 1's rows (loads complete in
    // issue order) never waits for the weights of chunks c + 2 .. c + MF_BP.
    constexpr int BP = NC < MF_BP ? NC : MF_BP;
    uint4 bq[MF_BP][NB][NS][MF_SC];
    float4 ar[2][NT][2], gq[2][2];
    mf_load_a(ar[0], gq[0], src, ok, gn, kg, 0);
    if (NC > 1) mf_load_a(ar[1], gq[1], src, ok, gn, kg, 1);
#pragma unroll
    for (int c = 0; c < BP; ++c) mf_load_b<K, NB, NS, true>(bq[c], w, woff, c);
    mf_store_a<NT, NP, NORM, CT>(buf[0], ar[0], gq[0], rsv, kg, ri);
    __syncthreads();
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (c + 2 < NC) mf_load_a(ar[c & 1], gq[c & 1], src, ok, gn, kg, c + 2);
      mf_compute<NT, NB, NS, NP, CT>(buf[c & 1], bq[c % MF_BP], acc);
      if (c + MF_BP < NC) mf_load_b<K, NB, NS, true>(bq[c % MF_BP], w, woff, c + MF_BP);
      if (c + 1 < NC) mf_store_a<NT, NP, NORM, CT>(buf[(c + 1) & 1], ar[(c + 1) & 1], gq[(c + 1) & 1], rsv, kg, ri);
      __syncthreads();
    }
  } else {
    // Decode-sized passes: chunk c computes from LDS buffer c % 2 and
    // registers bq(c % 2) while chunk c + 1 is loaded into the other pair
    // (fewer registers: more workgroups in flight); one barrier per chunk.
    // CACHED: ordinary weight loads (see the launchers for where each kind
    // is used).
    float4 gq[2];
    uint4 bq0[NB][NS][MF_SC], bq1[NB][NS][MF_SC];
    float4 ar[NT][2];
    mf_load_a(ar, gq, src, ok, gn, kg, 0);
    mf_load_b<K, NB, NS, CACHED>(bq0, w, woff, 0);
    mf_store_a<NT, NP, NORM, CT>(buf[0], ar, gq, rsv, kg, ri);
    __syncthreads();
#pragma unroll 1
    for (int c = 0; c < NC; c += 2) {
      if (c + 1 < NC) {
        mf_load_a(ar, gq, src, ok, gn, kg, c + 1);  // activations first: waiting for them does not wait for the weights
        mf_load_b<K, NB, NS, CACHED>(bq1, w, woff, c + 1);
      }
      mf_compute<NT, NB, NS, NP, CT>(buf[0], bq0, acc);
      if (c + 1 < NC) mf_store_a<NT, NP, NORM, CT>(buf[1], ar, gq, rsv, kg, ri);
      __syncthreads();
      if (c + 1 < NC) {
        if (c + 2 < NC) {
          mf_load_a(ar, gq, src, ok, gn, kg, c + 2);
          mf_load_b<K, NB, NS, CACHED>(bq0, w, woff, c + 2);
        }
        mf_compute<NT, NB, NS, NP, CT>(buf[1], bq1, acc);
        if (c + 2 < NC) mf_store_a<NT, NP, NORM, CT>(buf[0], ar, gq, rsv, kg, ri);
        __syncthreads();
      }
    }
  }
}

// The same pass (decode-sized pipeline, one bf16 part) for activation rows
// already in bf16: the staging copies them into the A fragments as they are.
template <int NT>
__device__ __forceinline__ void mf_load_a_bf(uint4 (&ar)[NT], const bf16* const (&src)[NT], const bool (&ok)[NT],
                                             int c) {
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const uint4 v = *reinterpret_cast<const uint4*>(src[i] + c * MF_KC);
    ar[i] = ok[i] ? v : make_uint4(0, 0, 0, 0);
  }
}
template <int NT, int CT>
__device__ __forceinline__ void mf_store_a_bf(MfChunkT<CT>& ch, const uint4 (&ar)[NT], int kg, int ri) {
  static_assert(NT <= CT, "chunk too small for the pass");
#pragma unroll
  for (int i = 0; i < NT; ++i) ch.f[i][kg >> 2][mf_slot(kg >> 2, (kg & 3) * 16 + ri)] = ar[i];
}
template <int K, int NT, int NB, int CT, bool CACHED, typename RowPtr>
__device__ __forceinline__ void mfma_pass_abf(const bf16* const (&w)[NB], RowPtr rowp, int rows,
                                              MfChunkT<CT> (&buf)[2][1], f32x4_v (&acc)[NT][NB][1]) {
  static_assert(K % MF_KC == 0, "K must be a multiple of the chunk");
  constexpr int NC = K / MF_KC;
  const int tid = threadIdx.x, lane = tid & 63;
  const long woff = (long)(lane & 15) * K + 8 * (lane >> 4);
  const int kg = tid & 15, ri = tid >> 4;
  const bf16* src[NT];
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
    for (int b = 0; b < NB; ++b) acc[i][b][0] = f32x4_v{0.f, 0.f, 0.f, 0.f};
  uint4 bq0[NB][1][MF_SC], bq1[NB][1][MF_SC];
  uint4 ar[NT];
  mf_load_a_bf(ar, src, ok, 0);
  mf_load_b<K, NB, 1, CACHED>(bq0, w, woff, 0);
  mf_store_a_bf<NT, CT>(buf[0][0], ar, kg, ri);
  __syncthreads();
#pragma unroll 1
  for (int c = 0; c < NC; c += 2) {
    if (c + 1 < NC) {
      mf_load_a_bf(ar, src, ok, c + 1);
      mf_load_b<K, NB, 1, CACHED>(bq1, w, woff, c + 1);
    }
    mf_compute<NT, NB, 1, 1, CT>(buf[0], bq0, acc);
    if (c + 1 < NC) mf_store_a_bf<NT, CT>(buf[1][0], ar, kg, ri);
    __syncthreads();
    if (c + 1 < NC) {
      if (c + 2 < NC) {
        mf_load_a_bf(ar, src, ok, c + 2);
        mf_load_b<K, NB, 1, CACHED>(bq0, w, woff, c + 2);
      }
      mf_compute<NT, NB, 1, 1, CT>(buf[1], bq1, acc);
      if (c + 2 < NC) mf_store_a_bf<NT, CT>(buf[0][0], ar, kg, ri);
      __syncthreads();
    }
  }
}

// The same with the long pipeline of mfma_pass: weights MF_BP chunks ahead in
// a register ring, rows two chunks in registers and two in LDS (each
// output's sum over k in the same order: the same bits).
template <int K, int NT, int NB, int CT, bool CACHED, typename RowPtr>
__device__ __forceinline__ void mfma_pass_abf_deep(const bf16* const (&w)[NB], RowPtr rowp, int rows,
                                                   MfChunkT<CT> (&buf)[2][1], f32x4_v (&acc)[NT][NB][1]) {
  static_assert(K % MF_KC == 0, "K must be a multiple of the chunk");
  constexpr int NC = K / MF_KC;
  constexpr int BP = NC < MF_BP ? NC : MF_BP;
  const int tid = threadIdx.x, lane = tid & 63;
  const long woff = (long)(lane & 15) * K + 8 * (lane >> 4);
  const int kg = tid & 15, ri = tid >> 4;
  const bf16* src[NT];
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
    for (int b = 0; b < NB; ++b) acc[i][b][0] = f32x4_v{0.f, 0.f, 0.f, 0.f};
  uint4 bq[MF_BP][NB][1][MF_SC];
  uint4 ar[2][NT];
  mf_load_a_bf(ar[0], src, ok, 0);
  if (NC > 1) mf_load_a_bf(ar[1], src, ok, 1);
#pragma unroll
  for (int c = 0; c < BP; ++c) mf_load_b<K, NB, 1, CACHED>(bq[c], w, woff, c);
  mf_store_a_bf<NT, CT>(buf[0][0], ar[0], kg, ri);
  __syncthreads();
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (c + 2 < NC) mf_load_a_bf(ar[c & 1], src, ok, c + 2);
    mf_compute<NT, NB, 1, 1, CT>(buf[c & 1], bq[c % MF_BP], acc);
    if (c + MF_BP < NC) mf_load_b<K, NB, 1, CACHED>(bq[c % MF_BP], w, woff, c + MF_BP);
    if (c + 1 < NC) mf_store_a_bf<NT, CT>(buf[(c + 1) & 1][0], ar[(c + 1) & 1], kg, ri);
    __syncthreads();
  }
}

// Gate/up: block (x, slot s) computes units j0 .. j0+15, j0 = 64 x + 16 w, of
// active expert s for every pair routed to it:
// hx[pair][j] = silu(gate_j . b) * (up_j . b), b the pair's normalised row.
template <int NT, bool DEEP, bool CACHED, int CT>
__device__ __forceinline__ void gate_up_pass(const bf16* const (&w)[2], const float* __restrict__ bnorm,
                                             const int* __restrict__ perm, int kb, int rows, float* __restrict__ hx,
                                             int j0, MfChunkT<CT> (&buf)[2][2]) {
  const int lane = lane_id();
  f32x4_v acc[NT][2][1];
  auto rowp = [=](int r) { return bnorm + (long)(perm[kb + r] / NSLOT) * D; };
  mfma_pass<D, NT, 2, 1, 2, decltype(rowp), false, CT, DEEP, CACHED>(w, rowp, rows, buf, acc);
#pragma unroll
  for (int i = 0; i < NT; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 16 * i + 4 * (lane >> 4) + q;
      if (r < rows) hx[(long)(kb + r) * DI + j0 + (lane & 15)] = silu(acc[i][0][0][q]) * acc[i][1][0][q];
    }
  }
}

// Block (x, y).  ITEMS (prefill passes, and decode calls of more than 64
// rows): work item y, an expert and at most ITEM_PAIRS of its pairs, so that
// a shared expert's many rows spread over several blocks.  Otherwise expert
// slot y (the shared experts' blocks load their weights with no routing
// read).  Either way, passes of 64 pairs with the same arithmetic per row.
// DEEP: the deeper load pipeline (prefill passes).  CT: row tiles per pass
// (passes of 16 CT pairs; the LDS chunks are sized to them).
template <bool ITEMS, bool DEEP, bool CACHED, int CT>
__global__ __launch_bounds__(256) void k_expert_gate_up_mfma(const bf16* __restrict__ wg,
                                                             const bf16* __restrict__ wu, int M, MoeBufs mb) {
  __shared__ MfChunkT<CT> buf[2][2];
  const int4 it = ITEMS ? mb.items[blockIdx.y] : expert_work(mb, blockIdx.y, M);
  const int e = it.x;
  if (e < 0) return;
  const int j0 = blockIdx.x * 64 + wave_id() * 16;
  const bf16* const w[2] = {wg + ((long)e * DI + j0) * D, wu + ((long)e * DI + j0) * D};
  for (int kb = it.y; kb < it.z; kb += 16 * CT) {
    const int rows = min(16 * CT, it.z - kb);
    if (CT == 1 || rows <= 16) gate_up_pass<1, DEEP, CACHED, CT>(w, mb.bnorm, mb.perm, kb, rows, mb.hx, j0, buf);
    else if (CT == 2 || rows <= 32)
      gate_up_pass<(CT < 2 ? CT : 2), DEEP, CACHED, CT>(w, mb.bnorm, mb.perm, kb, rows, mb.hx, j0, buf);
    else gate_up_pass<CT, DEEP, CACHED, CT>(w, mb.bnorm, mb.perm, kb, rows, mb.hx, j0, buf);
  }
}

// Down: block (x, slot s) computes outputs n0 .. n0+31, n0 = 128 x + 32 w:
// y[pair][n] = W_d[n] . hx[pair].
template <int NT, bool DEEP, bool CACHED, int CT>
__device__ __forceinline__ void down_pass(const bf16* const (&w)[1], const float* __restrict__ hx, int kb, int rows,
                                          float* __restrict__ y, int n0, MfChunkT<CT> (&buf)[2][2]) {
  const int lane = lane_id();
  f32x4_v acc[NT][1][2];
  auto rowp = [=](int r) { return hx + (long)(kb + r) * DI; };
  mfma_pass<DI, NT, 1, 2, 2, decltype(rowp), false, CT, DEEP, CACHED>(w, rowp, rows, buf, acc);
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

template <bool ITEMS, bool DEEP, bool CACHED, int CT>
__global__ __launch_bounds__(256) void k_expert_down_mfma(const bf16* __restrict__ wd, int M, MoeBufs mb) {
  __shared__ MfChunkT<CT> buf[2][2];
  const int4 it = ITEMS ? mb.items[blockIdx.y] : expert_work(mb, blockIdx.y, M);
  const int e = it.x;
  if (e < 0) return;
  const int n0 = blockIdx.x * 128 + wave_id() * 32;
  const bf16* const w[1] = {wd + ((long)e * D + n0) * DI};
  for (int kb = it.y; kb < it.z; kb += 16 * CT) {
    const int rows = min(16 * CT, it.z - kb);
    if (CT == 1 || rows <= 16) down_pass<1, DEEP, CACHED, CT>(w, mb.hx, kb, rows, mb.y, n0, buf);
    else if (CT == 2 || rows <= 32) down_pass<(CT < 2 ? CT : 2), DEEP, CACHED, CT>(w, mb.hx, kb, rows, mb.y, n0, buf);
    else down_pass<CT, DEEP, CACHED, CT>(w, mb.hx, kb, rows, mb.y, n0, buf);
  }
}

// Decode calls of more than MF_ROWS rows take work items (the shared experts
// then spread over several blocks instead of looping in one), with ordinary
// weight loads, since a shared expert's blocks read the same strips.
// Row tiles per pass (CT), weight-load kind and pipeline depth of each use, as
// measured best.  Decode gate/up: passes of 32 pairs (half the LDS: more
// workgroups per compute unit keep more weight loads in flight), ordinary
// loads (a shared expert's 64 rows take two passes over its strips).  Decode
// down: passes of 64, ordinary loads.  Prefill passes (64-pair work
// items, ordinary loads): passes of 64 with the two-chunk pipeline (the
// deeper one costs registers, hence workgroups in flight, and measured slower
// since the work items keep every block's pass short).
constexpr int GU_DEC_CT = 2;
constexpr bool GU_DEC_CACHED = true;
constexpr int DN_DEC_CT = 4;
constexpr bool DN_DEC_CACHED = true;
constexpr int GU_ITEM_CT = 4;  // work items: decode calls of more than 64 rows
constexpr int DN_ITEM_CT = 4;
constexpr int GU_DEEP_CT = 4;  // prefill passes
constexpr int DN_DEEP_CT = 4;
constexpr bool GU_PF_DEEP = false;  // the deeper pipeline in prefill passes
constexpr bool DN_PF_DEEP = false;
void launch_expert_gate_up_mfma(hipStream_t s, const bf16* wg, const bf16* wu, int M, const MoeBufs& mb, bool deep) {
  const bool items = deep || M > MF_ROWS;
  const dim3 grid(DI / 64, items ? expert_item_cap(M) : expert_slot_cap(M));
  if (deep)
    hipLaunchKernelGGL((k_expert_gate_up_mfma<true, GU_PF_DEEP, true, GU_DEEP_CT>), grid, dim3(256), 0, s, wg, wu, M,
                       mb);
  else if (items)
    hipLaunchKernelGGL((k_expert_gate_up_mfma<true, false, true, GU_ITEM_CT>), grid, dim3(256), 0, s, wg, wu, M, mb);
  else
    hipLaunchKernelGGL((k_expert_gate_up_mfma<false, false, GU_DEC_CACHED, GU_DEC_CT>), grid, dim3(256), 0, s, wg,
                       wu, M, mb);
}

void launch_expert_down_mfma(hipStream_t s, const bf16* wd, int M, const MoeBufs& mb, bool deep) {
  const bool items = deep || M > MF_ROWS;
  const dim3 grid(D / 128, items ? expert_item_cap(M) : expert_slot_cap(M));
  if (deep)
    hipLaunchKernelGGL((k_expert_down_mfma<true, DN_PF_DEEP, true, DN_DEEP_CT>), grid, dim3(256), 0, s, wd, M, mb);
  else if (items)
    hipLaunchKernelGGL((k_expert_down_mfma<true, false, true, DN_ITEM_CT>), grid, dim3(256), 0, s, wd, M, mb);
  else
    hipLaunchKernelGGL((k_expert_down_mfma<false, false, DN_DEC_CACHED, DN_DEC_CT>), grid, dim3(256), 0, s, wd, M,
                       mb);
}

// ---- dense layers on the matrix cores -------------------------------------
// Block (strip x, row block y) multiplies activation rows 64 y .. 64 y + 63
// (RMSNorm'ed first when a gain is given: the scale of each row as in
// norm_rows_wave) with its strip of weight rows, one 16-row tile per
// wavefront and per matrix, in one mfma_pass of 1, 2 or 4 row tiles (inputs as
// bf16 hi + lo parts), so a strip is read once per 64 rows.
//   DM_STORE / DM_ADD: out[m][n] = / += W0[n] . a_m, strip = rows 64 x ..;
//   DM_SWIGLU: out[m][n] = silu(W0[n] . a_m) * (W1[n] . a_m);
//   DM_QKV (fused RoPE and cache append, as k_qkv_rope): strip x = section
//     x / 10 (q, k, v) of head x % 10; q / k wavefronts take rows u and u + 64
//     (u = 16 w + j) of the head, the two halves of a RoPE pair, v wavefronts
//     rows 32 w + j and 32 w + 16 + j.
enum DenseMode { DM_STORE = 0, DM_ADD = 1, DM_SWIGLU = 2, DM_QKV = 3 };

struct QkvOut {
  RowPlan plan;
  float* q;
  KvView<bf16> kv;
  const float2* rope;
};

constexpr bool DENSE_DEEP = true;  // the deeper pipeline in the strip GEMMs
template <int K, int MODE, int NT>
__device__ __forceinline__ void dense_mfma_rows(const float* __restrict__ a, long lda, const float* __restrict__ gain,
                                                const bf16* const (&w)[(MODE == DM_SWIGLU || MODE == DM_QKV) ? 2 : 1],
                                                int m0, int rows, float* __restrict__ out, long ldo,
                                                const QkvOut& qo, int sec, int h, int n0, MfChunk (&buf)[2][2],
                                                const float* rs) {
  constexpr int NB = (MODE == DM_SWIGLU || MODE == DM_QKV) ? 2 : 1;
  const int wave = wave_id(), lane = lane_id();
  auto rowp = [=](int r) { return a + (long)(m0 + r) * lda; };
  f32x4_v acc[NT][NB][1];
  if (gain != nullptr)
    mfma_pass<K, NT, NB, 1, 2, decltype(rowp), true, MF_MT, DENSE_DEEP, true>(w, rowp, rows, buf, acc, gain, rs);
  else
    mfma_pass<K, NT, NB, 1, 2, decltype(rowp), false, MF_MT, DENSE_DEEP, true>(w, rowp, rows, buf, acc);
  const int j = lane & 15;
#pragma unroll
  for (int i = 0; i < NT; ++i) {
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int r = 16 * i + 4 * (lane >> 4) + qq;
      if (r >= rows) continue;
      const int m = m0 + r;
      const float v0 = acc[i][0][0][qq];
      if constexpr (MODE == DM_STORE) {
        out[(long)m * ldo + n0 + j] = v0;
      } else if constexpr (MODE == DM_ADD) {
        out[(long)m * ldo + n0 + j] += v0;
      } else if constexpr (MODE == DM_SWIGLU) {
        out[(long)m * ldo + n0 + j] = silu(v0) * acc[i][NB - 1][0][qq];
      } else {
        const float v1 = acc[i][NB - 1][0][qq];
        const RowPlan& plan = qo.plan;
        const int b = m / plan.Q, ii = m - b * plan.Q;
        const int pos = plan.base[b] + ii;
        const bool valid = ii < plan.cnt[b] && pos >= 0 && pos < qo.kv.max_pos;
        if (sec < 2) {
          const int u = 16 * wave + j;
          const float2 cs = qo.rope[(long)min(max(pos, 0), qo.kv.max_pos - 1) * (HD / 2) + u];
          const float o0 = fmaf(v0, cs.x, -(v1 * cs.y));
          const float o1 = fmaf(v1, cs.x, v0 * cs.y);
          if (sec == 0) {
            qo.q[(long)m * QD + h * HD + u] = o0;
            qo.q[(long)m * QD + h * HD + u + 64] = o1;
          } else if (valid) {
            const int pg = qo.kv.raw_page(plan.slot[b], pos);
            if (pg >= 0) {
              bf16* kd = qo.kv.at(pg, 0, h, pos);
              kd[u] = f2bf(o0);
              kd[u + 64] = f2bf(o1);
            }
          }
        } else if (valid) {
          const int pg = qo.kv.raw_page(plan.slot[b], pos);
          if (pg >= 0) {
            bf16* vd = qo.kv.at(pg, 1, h, pos);
            vd[32 * wave + j] = f2bf(v0);
            vd[32 * wave + 16 + j] = f2bf(v1);
          }
        }
      }
    }
  }
}

// RMSNorm scales of M rows of K: rs[m] = 1 / sqrt(mean(x_m^2) + eps), one
// wavefront per row (lane l sums x[k]^2 over k = l + 64 j in order, then the
// xor butterfly, as norm_rows_wave does).
template <int K>
__global__ __launch_bounds__(256) void k_row_rms(const float* __restrict__ a, long lda, int M, float eps,
                                                 float* __restrict__ rs) {
  const int m = blockIdx.x * 4 + wave_id();
  if (m >= M) return;
  const int lane = lane_id();
  const float* xr = a + (long)m * lda;
  float v[K / 64];
#pragma unroll
  for (int j = 0; j < K / 64; ++j) v[j] = xr[lane + 64 * j];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < K / 64; ++j) ss = fmaf(v[j], v[j], ss);
  ss = wave_sum(ss);
  if (lane == 0) rs[m] = 1.0f / sqrtf(ss / (float)K + eps);
}

// rsc: the rows' RMSNorm scales (k_row_rms) when a gain is given.
template <int K, int MODE>
__global__ __launch_bounds__(256) void k_dense_mfma(const float* __restrict__ a, long lda,
                                                    const float* __restrict__ gain, const float* __restrict__ rsc,
                                                    const bf16* __restrict__ W0, const bf16* __restrict__ W1, int M,
                                                    float* __restrict__ out, long ldo, QkvOut qo, int rt) {
  constexpr int NB = (MODE == DM_SWIGLU || MODE == DM_QKV) ? 2 : 1;
  __shared__ MfChunk buf[2][2];
  __shared__ float rs[MF_ROWS];
  const int wave = wave_id(), lane = lane_id();
  const int m0 = blockIdx.y * rt;
  const int rows = min(rt, M - m0);
  const bf16* w[NB];
  int sec = 0, h = 0, n0 = 0;
  if constexpr (MODE == DM_QKV) {
    sec = blockIdx.x / NH;
    h = blockIdx.x % NH;
    const int r0 = sec < 2 ? sec * QD + h * HD + 16 * wave : 2 * QD + h * HD + 32 * wave;
    w[0] = W0 + (long)r0 * K;
    w[1] = W0 + (long)(r0 + (sec < 2 ? 64 : 16)) * K;
  } else {
    n0 = blockIdx.x * 64 + 16 * wave;
    w[0] = W0 + (long)n0 * K;
    if constexpr (NB == 2) w[1] = W1 + (long)n0 * K;
  }
  if (gain != nullptr) {
    if (threadIdx.x < MF_ROWS) rs[threadIdx.x] = rsc[m0 + min((int)threadIdx.x, rows - 1)];
    __syncthreads();
  }
  if (rows <= 16) dense_mfma_rows<K, MODE, 1>(a, lda, gain, w, m0, rows, out, ldo, qo, sec, h, n0, buf, rs);
  else if (rows <= 32) dense_mfma_rows<K, MODE, 2>(a, lda, gain, w, m0, rows, out, ldo, qo, sec, h, n0, buf, rs);
  else dense_mfma_rows<K, MODE, 4>(a, lda, gain, w, m0, rows, out, ldo, qo, sec, h, n0, buf, rs);
}

// Decode-sized calls: the same outputs with more, smaller blocks.  Block
// (strip x, row tile y) owns 16 weight rows per matrix; its four wavefronts
// split k into quarters and stream their A fragments (fp32 -> bf16 hi + lo,
// RMSNorm'ed when a gain is given) and B fragments straight from memory, a
// DKS_PF-step register ring deep, with no LDS staging; the four partial
// 16x16 tiles are added in LDS in wavefront order, wavefront w finishing
// output rows 4 (lane / 16) + w.  Strips: DM_QKV 120 (q / k: 16 pair rows
// u0 .. u0+15 and u0+64 .. of a head, 80 strips; v: 32 rows of a head as two
// tiles, 40 strips), else N / 16.
constexpr int DKS_PF = 4;

template <int K, int MODE>
__global__ __launch_bounds__(256) void k_dense_ks(const float* __restrict__ a, long lda,
                                                  const float* __restrict__ gain, float eps,
                                                  const bf16* __restrict__ W0, const bf16* __restrict__ W1, int M,
                                                  float* __restrict__ out, long ldo, QkvOut qo) {
  constexpr int NB = (MODE == DM_SWIGLU || MODE == DM_QKV) ? 2 : 1;
  constexpr int KQ = K / 4;
  constexpr int NSTEP = KQ / 32;
  static_assert(KQ % 32 == 0, "k quarter must be a multiple of 32");
  __shared__ float4 red[4][NB][64];
  __shared__ float rs[16];
  const int wave = wave_id(), lane = lane_id();
  const int m0 = blockIdx.y * 16;
  const int rows = min(16, M - m0);
  const int x = blockIdx.x;
  int sec = 0, h = 0, c0 = 0;  // c0: first output column (row of W) of the strip
  long r0, r1 = 0;
  if constexpr (MODE == DM_QKV) {
    if (x < 80) {
      sec = x / 40;
      h = (x % 40) / 4;
      c0 = 16 * (x % 4);
      r0 = sec * QD + h * HD + c0;
      r1 = r0 + 64;
    } else {
      sec = 2;
      h = (x - 80) / 4;
      c0 = 32 * ((x - 80) % 4);
      r0 = 2 * QD + h * HD + c0;
      r1 = r0 + 16;
    }
  } else {
    c0 = 16 * x;
    r0 = c0;
    r1 = c0;
  }
  // QKV: the plan entry, cache slot and rotation of the output row this lane
  // finishes (row 4 (lane / 16) + wave, column lane % 16), fetched before the
  // main loop so that the epilogue waits on no memory
  int e_pos = 0;
  long e_page = 0;
  bool e_valid = false;
  float2 e_cs = make_float2(1.f, 0.f);
  if constexpr (MODE == DM_QKV) {
    const int r = 4 * (lane >> 4) + wave;
    if (r < rows) {
      const RowPlan& plan = qo.plan;
      const int m = m0 + r, b = m / plan.Q, i = m - b * plan.Q;
      e_pos = plan.base[b] + i;
      e_valid = i < plan.cnt[b] && e_pos >= 0 && e_pos < qo.kv.max_pos;
      if (sec > 0) {
        e_page = qo.kv.raw_page(plan.slot[b], e_pos);
        e_valid = e_valid && e_page >= 0;
      }
      if (sec < 2) e_cs = qo.rope[(long)min(max(e_pos, 0), qo.kv.max_pos - 1) * (HD / 2) + c0 + (lane & 15)];
    }
  }
  if (gain != nullptr) {
    for (int r = wave; r < 16; r += 4) {
      float ss = 0.f;
      if (r < rows) {
        const float* xr = a + (long)(m0 + r) * lda;
#pragma unroll 4
        for (int j = 0; j < K / 64; ++j) {
          const float v = xr[lane + 64 * j];
          ss = fmaf(v, v, ss);
        }
      }
      ss = wave_sum(ss);
      if (lane == 0) rs[r] = 1.0f / sqrtf(ss / (float)K + eps);
    }
    __syncthreads();
  }
  const int ar = lane & 15;          // A row of this lane
  const bool aok = ar < rows;
  const float* arow = a + (long)(m0 + (aok ? ar : 0)) * lda;
  const float rscale = (gain != nullptr) ? rs[aok ? ar : 0] : 1.f;
  const int kl = wave * KQ + 8 * (lane >> 4);  // this lane's k offset within a step
  const bf16* wb[NB];
  wb[0] = W0 + (r0 + (lane & 15)) * K + kl;
  if constexpr (NB == 2) wb[1] = (MODE == DM_QKV ? W0 : W1) + (r1 + (lane & 15)) * K + kl;
  uint4 bq[DKS_PF][NB];
  float4 aq[DKS_PF][2], gq[DKS_PF][2];
  auto load = [&](int t, int slot) {
#pragma unroll
    for (int b = 0; b < NB; ++b) bq[slot][b] = ldg16(wb[b] + 32 * t);  // row tiles of a strip share it in L2
    const float4* ap = reinterpret_cast<const float4*>(arow + kl + 32 * t);
    aq[slot][0] = ap[0];
    aq[slot][1] = ap[1];
    if (gain != nullptr) {
      const float4* gp = reinterpret_cast<const float4*>(gain + kl + 32 * t);
      gq[slot][0] = gp[0];
      gq[slot][1] = gp[1];
    }
  };
#pragma unroll
  for (int t = 0; t < DKS_PF; ++t)
    if (t < NSTEP) load(t, t);
  f32x4_v acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = f32x4_v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < NSTEP; ++t) {
    const int slot = t % DKS_PF;
    float4 v0 = aq[slot][0], v1 = aq[slot][1];
    if (gain != nullptr) {
      v0 = mf_norm(v0, rscale, gq[slot][0]);
      v1 = mf_norm(v1, rscale, gq[slot][1]);
    }
    if (!aok) {
      v0 = make_float4(0.f, 0.f, 0.f, 0.f);
      v1 = v0;
    }
    uint4 hi, lo;
    hi.x = pack_bf16x2(v0.x, v0.y);
    hi.y = pack_bf16x2(v0.z, v0.w);
    hi.z = pack_bf16x2(v1.x, v1.y);
    hi.w = pack_bf16x2(v1.z, v1.w);
    lo.x = pack_bf16x2(rem_lo(v0.x, hi.x), rem_hi(v0.y, hi.x));
    lo.y = pack_bf16x2(rem_lo(v0.z, hi.y), rem_hi(v0.w, hi.y));
    lo.z = pack_bf16x2(rem_lo(v1.x, hi.z), rem_hi(v1.y, hi.z));
    lo.w = pack_bf16x2(rem_lo(v1.z, hi.w), rem_hi(v1.w, hi.w));
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      acc[b] = mfma_bf16(hi, bq[slot][b], acc[b]);
      acc[b] = mfma_bf16(lo, bq[slot][b], acc[b]);
    }
    if (t + DKS_PF < NSTEP) load(t + DKS_PF, slot);
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) red[wave][b][lane] = make_float4(acc[b][0], acc[b][1], acc[b][2], acc[b][3]);
  __syncthreads();
  // wavefront w finishes element q = w of every lane's four: row 4 (lane / 16) + w, column lane % 16
  const int r = 4 * (lane >> 4) + wave;
  if (r >= rows) return;
  const int m = m0 + r, j = lane & 15;
  float v[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    float t = reinterpret_cast<const float*>(&red[0][b][lane])[wave];
    t += reinterpret_cast<const float*>(&red[1][b][lane])[wave];
    t += reinterpret_cast<const float*>(&red[2][b][lane])[wave];
    t += reinterpret_cast<const float*>(&red[3][b][lane])[wave];
    v[b] = t;
  }
  if constexpr (MODE == DM_STORE) {
    out[(long)m * ldo + c0 + j] = v[0];
  } else if constexpr (MODE == DM_ADD) {
    out[(long)m * ldo + c0 + j] += v[0];
  } else if constexpr (MODE == DM_SWIGLU) {
    out[(long)m * ldo + c0 + j] = silu(v[0]) * v[NB - 1];
  } else {
    if (sec < 2) {
      const int u = c0 + j;
      const float o0 = fmaf(v[0], e_cs.x, -(v[NB - 1] * e_cs.y));
      const float o1 = fmaf(v[NB - 1], e_cs.x, v[0] * e_cs.y);
      if (sec == 0) {
        qo.q[(long)m * QD + h * HD + u] = o0;
        qo.q[(long)m * QD + h * HD + u + 64] = o1;
      } else if (e_valid) {
        bf16* kd = qo.kv.at(e_page, 0, h, e_pos);
        kd[u] = f2bf(o0);
        kd[u + 64] = f2bf(o1);
      }
    } else if (e_valid) {
      bf16* vd = qo.kv.at(e_page, 1, h, e_pos);
      vd[c0 + j] = f2bf(v[0]);
      vd[c0 + 16 + j] = f2bf(v[NB - 1]);
    }
  }
}

bool launch_gemv_ks(hipStream_t s, int K, Epi epi, const float* a, long lda, const float* gain, float eps,
                    const bf16* W0, const bf16* W1, int N, int M, float* out, long ldo) {
  const dim3 grid(N / 16, (M + 15) / 16);
  const QkvOut none{};
#define OCR_DK(KV, MODEV) \
  hipLaunchKernelGGL((k_dense_ks<KV, MODEV>), grid, dim3(256), 0, s, a, lda, gain, eps, W0, W1, M, out, ldo, none)
  if (K == D && epi == EPI_ADD) OCR_DK(D, DM_ADD);
  else if (K == D && epi == EPI_SWIGLU) OCR_DK(D, DM_SWIGLU);
  else if (K == D && epi == EPI_STORE) OCR_DK(D, DM_STORE);
  else if (K == 2 * D && epi == EPI_STORE) OCR_DK(2 * D, DM_STORE);
  else if (K == DF && epi == EPI_ADD) OCR_DK(DF, DM_ADD);
  else return false;
#undef OCR_DK
  return true;
}

void launch_qkv_rope_ks(hipStream_t s, const float* x, const float* gain, float eps, const bf16* wqkv, int M,
                        RowPlan plan, float* q, KvView<bf16> kv, const float2* rope) {
  const QkvOut qo{plan, q, kv, rope};
  hipLaunchKernelGGL((k_dense_ks<D, DM_QKV>), dim3(120, (M + 15) / 16), dim3(256), 0, s, x, (long)D, gain, eps, wqkv,
                     nullptr, M, nullptr, 0L, qo);
}

bool launch_gemv_mfma(hipStream_t s, int K, Epi epi, const float* a, long lda, const float* gain, float eps,
                      const bf16* W0, const bf16* W1, int N, int M, float* out, long ldo, float* rscale) {
  const int rt = dense_rows_per_block(M);
  const dim3 grid(N / 64, (M + rt - 1) / rt);
  const QkvOut none{};
  if (gain != nullptr) {
    if (K != D) return false;  // the normed inputs are model rows
    hipLaunchKernelGGL((k_row_rms<D>), dim3((M + 3) / 4), dim3(256), 0, s, a, lda, M, eps, rscale);
  }
#define OCR_DM(KV, MODEV) \
  hipLaunchKernelGGL((k_dense_mfma<KV, MODEV>), grid, dim3(256), 0, s, a, lda, gain, rscale, W0, W1, M, out, ldo, \
                     none, rt)
  if (K == D && epi == EPI_ADD) OCR_DM(D, DM_ADD);
  else if (K == D && epi == EPI_SWIGLU) OCR_DM(D, DM_SWIGLU);
  else if (K == D && epi == EPI_STORE) OCR_DM(D, DM_STORE);
  else if (K == 2 * D && epi == EPI_STORE) OCR_DM(2 * D, DM_STORE);
  else if (K == DF && epi == EPI_ADD) OCR_DM(DF, DM_ADD);
  else return false;
#undef OCR_DM
  return true;
}

void launch_qkv_rope_mfma(hipStream_t s, const float* x, const float* gain, float eps, const bf16* wqkv, int M,
                          RowPlan plan, float* q, KvView<bf16> kv, const float2* rope, float* rscale) {
  const QkvOut qo{plan, q, kv, rope};
  hipLaunchKernelGGL((k_row_rms<D>), dim3((M + 3) / 4), dim3(256), 0, s, x, (long)D, M, eps, rscale);
  const int rt = dense_rows_per_block(M);
  hipLaunchKernelGGL((k_dense_mfma<D, DM_QKV>), dim3(3 * NH, (M + rt - 1) / rt), dim3(256), 0, s, x, (long)D, gain,
                     rscale, wqkv, nullptr, M, nullptr, 0L, qo, rt);
}

// LM head rows for the matrix cores: xn[m] = RMSNorm(x[src(m)]) * gain, one
// wavefront per row, src(m) = m * Q + cnt[m] - 1 when last_valid, else m.
// Lane l sums x[k]^2 over k = l + 64 j in order, then the xor butterfly.
__global__ __launch_bounds__(256) void k_lm_norm(const float* __restrict__ x, const int* __restrict__ cnt, int Q,
                                                 int last_valid, const float* __restrict__ gain, float eps, int M,
                                                 bf16* __restrict__ xn) {
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
  // the normalised row rounded to bf16 (the LM head's one part), element
  // pairs (2 i, 2 i + 1) packed by the even lanes
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const float y = (v[j] * r) * gain[lane + 64 * j];
    const float yn = __shfl_down(y, 1, 64);
    if ((lane & 1) == 0)
      reinterpret_cast<uint32_t*>(xn + (long)m * D + 64 * j)[lane >> 1] = pack_bf16x2(y, yn);
  }
}

// LM head + argmax stage 1 on the matrix cores (V >= 16): block x scores vocab
// rows 64 x .. 64 x + 63 (16 per wavefront) for all M rows, passes of 64 rows,
// and writes the best (value, lowest id) per row to part[row][x]; logits
// optionally stored to logits[row][V].
// G groups of 16 vocab rows per wavefront: w[g] the group's rows, vj[g] this
// lane's id in it, vok[g] whether that id is the group's to score.
template <int NT, bool CACHED, int CT, int G, bool DEEP>
__device__ __forceinline__ void lm_pass(const bf16* const (&w)[G], const bf16* __restrict__ xn, int p0, int rows,
                                        const int (&vj)[G], const bool (&vok)[G], int V, float* __restrict__ logits,
                                        float (&bv)[4][16 * CT], int (&bi)[4][16 * CT], MfChunkT<CT> (&buf)[2][1]) {
  const int wave = wave_id(), lane = lane_id();
  f32x4_v acc[NT][G][1];
  auto rowp = [=](int r) { return xn + (long)(p0 + r) * D; };
  if constexpr (DEEP)
    mfma_pass_abf_deep<D, NT, G, CT, CACHED>(w, rowp, rows, buf, acc);
  else
    mfma_pass_abf<D, NT, G, CT, CACHED>(w, rowp, rows, buf, acc);
#pragma unroll
  for (int i = 0; i < NT; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 16 * i + 4 * (lane >> 4) + q;
      float b = -INFINITY;
      int id = 0x7fffffff;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const bool ok = vok[g] && r < rows;
        const float val = acc[i][g][0][q];
        if (ok && logits != nullptr) logits[(long)(p0 + r) * V + vj[g]] = val;
        if (ok && (val > b || (val == b && vj[g] < id))) { b = val; id = vj[g]; }
      }
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

constexpr int N_XCD = 8;  // dies of the chip, each with its own L2
constexpr int LM_G = 2;   // groups of 16 vocab rows per wavefront of the matrix-core LM head

// Block x scores vocab rows 64 G x .. 64 G x + 64 G - 1 (wavefront w: 16 G of
// them) and writes, per row, the best (value, lowest id) of each 64-row slab
// (the partials of the stage-2 argmax, slab k = rows 64 k ..).  More vocab
// rows per block share one staging of the activation rows.  CT: row tiles
// per pass.  One pass (SPLIT false, at most 16 CT rows): block x =
// blockIdx.x.  More rows (SPLIT): each pass of a strip is a block of its own,
// and the passes of strip x run as consecutive blocks of one XCD (the
// dispatcher deals blocks to the 8 XCDs in turn), so that one L2 serves the
// strip's repeated reads; the row passes then run side by side instead of
// one after another.  Ordinary weight loads either way (measured faster than
// non-temporal ones here, also for one pass).  The split passes take the long
// load pipeline (mfma_pass_abf_deep: 2.59-2.61 against 2.63 ms per 256-row
// verify call over 32,768 positions); one pass keeps the short one (the long
// one measured the same there, at half the occupancy).
template <bool SPLIT, int CT>
__global__ __launch_bounds__(256) void k_lmhead_mfma(const bf16* __restrict__ xn, const bf16* __restrict__ W,
                                                     int V, int M, int nblk, float* __restrict__ part_val,
                                                     int* __restrict__ part_idx, float* __restrict__ logits) {
  constexpr int RB = 16 * CT;
  constexpr bool CACHED = true;
  __shared__ MfChunkT<CT> buf[2][1];
  __shared__ float bv[4][RB];
  __shared__ int bi[4][RB];
  const int wave = wave_id(), lane = lane_id();
  const int nx = (nblk + LM_G - 1) / LM_G;  // blocks per pass
  int x = blockIdx.x, pass_lo = 0, pass_hi = (M + RB - 1) / RB;
  if constexpr (SPLIT) {
    const int L = blockIdx.x;
    x = L % N_XCD + N_XCD * (L / (N_XCD * pass_hi));
    pass_lo = (L / N_XCD) % pass_hi;
    pass_hi = pass_lo + 1;
    if (x >= nx) return;
  }
  // A group reaching past the vocabulary is moved back to rows V-16 .. V-1;
  // its lanes then keep only the ids >= its start (the others belong to the
  // group before, or lie past the vocabulary).
  const bf16* w[LM_G];
  int vj[LM_G];
  bool vok[LM_G];
#pragma unroll
  for (int g = 0; g < LM_G; ++g) {
    const int v0 = x * 64 * LM_G + wave * 16 * LM_G + 16 * g;
    const int vb = v0 > V - 16 ? V - 16 : v0;
    w[g] = W + (long)vb * D;
    vj[g] = vb + (lane & 15);
    vok[g] = vj[g] >= v0 && vj[g] < V;
  }
  const bf16* const (&wc)[LM_G] = w;
  for (int pi = pass_lo; pi < pass_hi; ++pi) {
    const int p0 = pi * RB;
    const int rows = min(RB, M - p0);
    if (CT == 1 || rows <= 16) {
      lm_pass<1, CACHED, CT, LM_G, SPLIT>(wc, xn, p0, rows, vj, vok, V, logits, bv, bi, buf);
    } else if (CT == 2 || rows <= 32) {
      lm_pass<(CT < 2 ? CT : 2), CACHED, CT, LM_G, SPLIT>(wc, xn, p0, rows, vj, vok, V, logits, bv, bi, buf);
    } else {
      lm_pass<CT, CACHED, CT, LM_G, SPLIT>(wc, xn, p0, rows, vj, vok, V, logits, bv, bi, buf);
    }
    __syncthreads();
    // slab h of the block: wavefronts 4 h / G .. 4 (h + 1) / G - 1
    for (int t = threadIdx.x; t < rows * LM_G; t += 256) {
      const int r = t % rows, h = t / rows;
      const int k = x * LM_G + h;
      if (k >= nblk) continue;
      constexpr int WPS = 4 / LM_G;  // wavefronts per slab
      float b = bv[h * WPS][r];
      int id = bi[h * WPS][r];
      for (int ww = h * WPS + 1; ww < (h + 1) * WPS; ++ww)
        if (bv[ww][r] > b || (bv[ww][r] == b && bi[ww][r] < id)) { b = bv[ww][r]; id = bi[ww][r]; }
      part_val[(long)(p0 + r) * nblk + k] = b;
      part_idx[(long)(p0 + r) * nblk + k] = id;
    }
    __syncthreads();
  }
}

constexpr int LM_CT = 4;  // row tiles per pass of the LM head
void launch_lmhead_mfma(hipStream_t s, const float* x, const int* cnt, int Q, bool last_valid, const float* gain,
                        float eps, const bf16* W, int V, int M, float* xn, float* part_val, int* part_idx,
                        float* logits, int* tok, int tok_stride) {
  bf16* xb = reinterpret_cast<bf16*>(xn);  // the rows in bf16, in the first half of the fp32 buffer
  hipLaunchKernelGGL(k_lm_norm, dim3((M + 3) / 4), dim3(256), 0, s, x, cnt, Q, (int)last_valid, gain, eps, M, xb);
  const int nb = lmhead_blocks(V);
  const int nx = (nb + LM_G - 1) / LM_G;
  const int passes = (M + 16 * LM_CT - 1) / (16 * LM_CT);
  if (passes > 1)
    hipLaunchKernelGGL((k_lmhead_mfma<true, LM_CT>), dim3((nx + N_XCD - 1) / N_XCD * N_XCD * passes), dim3(256), 0, s,
                       xb, W, V, M, nb, part_val, part_idx, logits);
  else
    hipLaunchKernelGGL((k_lmhead_mfma<false, LM_CT>), dim3(nx), dim3(256), 0, s, xb, W, V, M, nb, part_val, part_idx,
                       logits);
  if (tok != nullptr) launch_argmax_final(s, part_val, part_idx, nb, M, tok, tok_stride);
}

}  // namespace ocr
