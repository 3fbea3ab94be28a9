// Decode attention over the KV cache (split-KV with fixed, tile-aligned chunk
// boundaries) and its combine.
//
// Block (chunk c, head h, sequence b) stages the keys and values of
// ATT_TILE-key tiles of chunk c in LDS (keys transposed; the next tile's loads
// in flight while the current one is used) and serves every query row of
// sequence b from them (the K+1 verify rows, or a prefill chunk), so one KV
// read feeds all of the sequence's queries.  A
// query at position p sees keys 0..p.  Per query the block keeps an online
// softmax (running max m, sum l, output o) across its tiles and writes
// (o, m, l); the combine kernel merges chunks 0..p/C in order.  Because chunk
// boundaries are fixed multiples of C and masked keys contribute exact zeros,
// a query's result does not depend on which other queries share the launch.
#include "launch.h"

namespace ocr {

constexpr int QMAX_ATT = 8;  // query rows per sequence handled by one block
// Row stride of the transposed key tile: one spare element per row, so the
// staging writes of one key's dims (one row each) fall in different LDS banks.
constexpr int KQ_STRIDE = ATT_TILE + 1;

// LDS tile formats: the fp32 model stages keys / values widened to fp32; the
// bf16 model keeps them in bf16 (half the LDS, so more blocks per CU keep more
// KV reads in flight): its scores take the keys as they are (dot4), its
// values are widened as they are read.
template <typename T> struct AttTile;
template <> struct AttTile<float> {
  typedef float4 K4;   // 4 key dims
  typedef float2 V2;   // 2 value dims
  __device__ static __forceinline__ float4 stage_q(const float4& q) { return q; }
  __device__ static __forceinline__ float dot4(const float4& qv, const K4& kv4, float sc) {
    sc = fmaf(qv.x, kv4.x, sc);
    sc = fmaf(qv.y, kv4.y, sc);
    sc = fmaf(qv.z, kv4.z, sc);
    sc = fmaf(qv.w, kv4.w, sc);
    return sc;
  }
  __device__ static __forceinline__ float2 v(const V2& x) { return x; }
  __device__ static __forceinline__ void stage(const uint4& kr, const uint4& vr, int d0, int t, K4 (*Kq)[KQ_STRIDE],
                                               V2 (*Vs)[HD / 2]) {
    // a 16-byte chunk holds dims d0 .. d0+3
    Kq[d0 / 4][t] = make_float4(__uint_as_float(kr.x), __uint_as_float(kr.y), __uint_as_float(kr.z),
                                __uint_as_float(kr.w));
    Vs[t][d0 / 2] = make_float2(__uint_as_float(vr.x), __uint_as_float(vr.y));
    Vs[t][d0 / 2 + 1] = make_float2(__uint_as_float(vr.z), __uint_as_float(vr.w));
  }
};
template <> struct AttTile<bf16> {
  typedef uint2 K4;
  typedef uint32_t V2;
  // The query's 4 dims as bf16 pairs: hi = bf16(q), lo = bf16(q - hi) (q to
  // about 16 bits), laid out (hi d0 d1, hi d2 d3, lo d0 d1, lo d2 d3).
  __device__ static __forceinline__ float4 stage_q(const float4& q) {
    const uint32_t h01 = pack_bf16x2(q.x, q.y), h23 = pack_bf16x2(q.z, q.w);
    const uint32_t l01 = pack_bf16x2(rem_lo(q.x, h01), rem_hi(q.y, h01));
    const uint32_t l23 = pack_bf16x2(rem_lo(q.z, h23), rem_hi(q.w, h23));
    return make_float4(__uint_as_float(h01), __uint_as_float(h23), __uint_as_float(l01), __uint_as_float(l23));
  }
  // sc + q . k over 4 dims: the bf16 key pairs against the query's hi and lo
  // pairs by v_dot2c_f32_bf16 (products of bf16 values are exact in fp32)
  __device__ static __forceinline__ float dot4(const float4& qp, const K4& k, float sc) {
    sc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, __float_as_uint(qp.x)),
                                         __builtin_bit_cast(bf16x2_v, k.x), sc, false);
    sc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, __float_as_uint(qp.y)),
                                         __builtin_bit_cast(bf16x2_v, k.y), sc, false);
    sc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, __float_as_uint(qp.z)),
                                         __builtin_bit_cast(bf16x2_v, k.x), sc, false);
    sc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, __float_as_uint(qp.w)),
                                         __builtin_bit_cast(bf16x2_v, k.y), sc, false);
    return sc;
  }
  __device__ static __forceinline__ float2 v(const V2& x) {
    return make_float2(__uint_as_float(x << 16), __uint_as_float(x & 0xffff0000u));
  }
  __device__ static __forceinline__ void stage(const uint4& kr, const uint4& vr, int d0, int t, K4 (*Kq)[KQ_STRIDE],
                                               V2 (*Vs)[HD / 2]) {
    // a 16-byte chunk holds dims d0 .. d0+7
    Kq[d0 / 4][t] = make_uint2(kr.x, kr.y);
    Kq[d0 / 4 + 1][t] = make_uint2(kr.z, kr.w);
    *reinterpret_cast<uint4*>(&Vs[t][d0 / 2]) = vr;
  }
};

// One query row (query i of the block's sequence, visible keys 0..plim) against
// the staged tile of keys kt .. kt+63, by one wavefront: lane = key for the
// scores (q . k over 128 dims, 4 at a time, in order; bf16 caches: the query's
// hi and lo bf16 parts against the keys, AttTile::dot4), then lane = value-dim
// pair for the output; the online-softmax state (mrun, lrun, o0, o1) is the
// query's.  pw is the wavefront's 64-float LDS row for the probabilities.
template <typename T>
__device__ __forceinline__ void attn_tile_query(const float4* __restrict__ qrow,
                                                const typename AttTile<T>::K4 (*Kq)[KQ_STRIDE],
                                                const typename AttTile<T>::V2 (*Vs)[HD / 2], float4* pw, int kt,
                                                int plim, float& mrun, float& lrun, float& o0, float& o1) {
  typedef AttTile<T> AT;
  const int lane = lane_id();
  const float scale = 0.08838834764831845f;  // 1 / sqrt(128)
  float sc = 0.f;
#pragma unroll 8
  for (int d4 = 0; d4 < HD / 4; ++d4) sc = AT::dot4(qrow[d4], Kq[d4][lane], sc);
  sc = sc * scale;
  const bool vis = (kt + lane) <= plim;
  const float mt = wave_max_dpp(vis ? sc : -INFINITY);
  const float mnew = fmaxf(mrun, mt);
  const float corr = expf(mrun - mnew);
  const float p = vis ? expf(sc - mnew) : 0.f;
  lrun = lrun * corr + wave_sum_dpp(p);
  reinterpret_cast<float*>(pw)[lane] = p;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  float a0 = o0 * corr, a1 = o1 * corr;
#pragma unroll 4
  for (int t4 = 0; t4 < ATT_TILE / 4; ++t4) {
    const float4 pt = pw[t4];
    const float pv[4] = {pt.x, pt.y, pt.z, pt.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float2 v2 = AT::v(Vs[4 * t4 + u][lane]);
      a0 = fmaf(pv[u], v2.x, a0);
      a1 = fmaf(pv[u], v2.y, a1);
    }
  }
  o0 = a0;
  o1 = a1;
  mrun = mnew;
  __builtin_amdgcn_wave_barrier();
}

// Merge of the chunk partials pp[c * cstride] (o[128], m, l) of one query row
// for dims d, chunks 0..nc-1 in order: max of the m, then L and O with weights
// exp(m_c - max), result O / L.  The partials sit in L2, so the loads go out G
// chunks at a time (one round trip per group rather than per chunk), at chunk
// indices clamped to the last one in range so that they need no predicate;
// repeats of the last chunk leave the max unchanged, and the sums run over
// c < nc in order.
template <int G>
__device__ __forceinline__ void merge_load(const float* __restrict__ pp, long cstride, int c0, int nlim, int d,
                                           float (&mv)[G], float (&lv)[G], float (&ov)[G]) {
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const float* q = pp + min(c0 + j, nlim - 1) * cstride;
    mv[j] = q[HD];
    lv[j] = q[HD + 1];
    ov[j] = q[d];
  }
}
// nc <= G chunks already in registers
template <int G>
__device__ __forceinline__ float merge_regs(const float (&mv)[G], const float (&lv)[G], const float (&ov)[G],
                                            int nc) {
  float mg = -INFINITY;
#pragma unroll
  for (int j = 0; j < G; ++j) mg = fmaxf(mg, (j < nc) ? mv[j] : -INFINITY);
  float L = 0.f, O = 0.f;
#pragma unroll
  for (int j = 0; j < G; ++j) {
    if (j < nc) {
      const float w = expf(mv[j] - mg);
      L = fmaf(lv[j], w, L);
      O = fmaf(ov[j], w, O);
    }
  }
  return O / L;
}
// any nc: two passes over groups of 8
__device__ __forceinline__ float merge_loop(const float* __restrict__ pp, long cstride, int nc, int d) {
  constexpr int G = 8;
  float mg = -INFINITY;
  for (int c0 = 0; c0 < nc; c0 += G) {
    float mv[G];
#pragma unroll
    for (int j = 0; j < G; ++j) mv[j] = pp[min(c0 + j, nc - 1) * cstride + HD];
#pragma unroll
    for (int j = 0; j < G; ++j) mg = fmaxf(mg, mv[j]);
  }
  float L = 0.f, O = 0.f;
  for (int c0 = 0; c0 < nc; c0 += G) {
    float mv[G], lv[G], ov[G];
    merge_load<G>(pp, cstride, c0, nc, d, mv, lv, ov);
#pragma unroll
    for (int j = 0; j < G; ++j) {
      if (c0 + j < nc) {
        const float w = expf(mv[j] - mg);
        L = fmaf(lv[j], w, L);
        O = fmaf(ov[j], w, O);
      }
    }
  }
  return O / L;
}

constexpr int ATT_MAX_TPC = 4;  // tiles per chunk at most
template <typename T>
__global__ __launch_bounds__(256) void k_attn_partial(const float* __restrict__ q, KvView<T> kv, RowPlan plan,
                                                      int n_chunks, int tiles_per_chunk,
                                                      float* __restrict__ part) {
  typedef AttTile<T> AT;
  // keys transposed in groups of 4 dims: Kq[d/4][t] = (k_t[d..d+3]); values row-major
  __shared__ typename AT::K4 Kq[HD / 4][KQ_STRIDE];
  __shared__ __align__(16) typename AT::V2 Vs[ATT_TILE][HD / 2];
  __shared__ float4 qs[QMAX_ATT][HD / 4];
  __shared__ float4 ps[4][ATT_TILE / 4];
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int wave = wave_id(), lane = lane_id(), tid = threadIdx.x;
  const int Q = plan.Q;
  const int C = tiles_per_chunk * ATT_TILE;
  const int k0 = c * C;
  const int max_pos = kv.max_pos;
  // The tiles' addresses need only the slot and the pages of the chunk's
  // tiles (one page per tile): with identity slots the page reads go out with
  // the plan reads and this head's query rows (i < Q), then the first tile's
  // loads (rows past the last query's key are zeroed when staged).
  const long slot = plan.ident ? (long)b : (long)plan.slot[b];
  long pg[ATT_MAX_TPC];
#pragma unroll
  for (int tt = 0; tt < ATT_MAX_TPC; ++tt) pg[tt] = tt < tiles_per_chunk ? kv.page_of(slot, k0 + tt * ATT_TILE) : 0;
  constexpr int CE = WT<T>::CE;
  constexpr int CPR = HD / CE;                         // 16-byte chunks per key row
  constexpr int NLD = ATT_TILE * CPR / 256;            // chunks per thread per tile
  uint4 kr[NLD], vr[NLD];
  auto load_tile = [&](int tt) {
    const long p = tt == 0 ? pg[0] : tt == 1 ? pg[1] : tt == 2 ? pg[2] : pg[3];  // selects, no indexing
    const T* Kt = kv.rows(p, 0, h);
    const T* Vt = kv.rows(p, 1, h);
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const int e = tid + 256 * j, t = e / CPR, d0 = (e % CPR) * CE;
      kr[j] = ldg16(Kt + (long)t * HD + d0);
      vr[j] = ldg16(Vt + (long)t * HD + d0);
    }
  };
  load_tile(0);
  constexpr int NQV = QMAX_ATT * HD / 4 / 256;
  float4 qv[NQV];
#pragma unroll
  for (int j = 0; j < NQV; ++j) {
    const int e = tid + 256 * j, i = e / (HD / 4), d4 = e % (HD / 4);
    qv[j] = reinterpret_cast<const float4*>(q + (long)(b * Q + min(i, Q - 1)) * QD + h * HD)[d4];
  }
  const int base = plan.base[b], pcnt = plan.cnt[b];
  // rows past the cache (never produced by the library's own plans) are
  // skipped; no branch on base, so both reads go out together
  const int cnt = min(min(pcnt, Q), max_pos - base) & -(int)(base >= 0);
  const int p_last = base + cnt - 1;
  // LDS staging of the tile at key kt (rows past p_last as zeros)
  auto stage_tile = [&](int kt) {
    const int nk = min(ATT_TILE, p_last + 1 - kt);
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const int e = tid + 256 * j, t = e / CPR, d0 = (e % CPR) * CE;
      if (t >= nk) {
        kr[j] = make_uint4(0, 0, 0, 0);
        vr[j] = make_uint4(0, 0, 0, 0);
      }
      AT::stage(kr[j], vr[j], d0, t, Kq, Vs);
    }
  };
  // the first tile and the queries (rows past cnt as zeros) are staged before
  // the exit test, which keeps their loads ahead of it
  stage_tile(k0);
#pragma unroll
  for (int j = 0; j < NQV; ++j) {
    const int e = tid + 256 * j, i = e / (HD / 4);
    qs[i][e % (HD / 4)] = (i < cnt) ? AT::stage_q(qv[j]) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (cnt <= 0 || k0 > p_last) return;
  const int n_tiles = min(tiles_per_chunk, (p_last - k0) / ATT_TILE + 1);
  float mrun[2] = {-INFINITY, -INFINITY}, lrun[2] = {0.f, 0.f};
  float o0[2] = {0.f, 0.f}, o1[2] = {0.f, 0.f};
  for (int tt = 0; tt < n_tiles; ++tt) {
    const int kt = k0 + tt * ATT_TILE;
    if (tt > 0) {
      __syncthreads();  // the previous tile's LDS reads are done
      stage_tile(kt);
    }
    __syncthreads();
    if (tt + 1 < n_tiles) load_tile(tt + 1);  // next tile in flight during this one's arithmetic
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      const int i = wave + 4 * qq;
      if (i >= cnt) continue;
      const int plim = base + i;  // last visible key of query i
      if (kt > plim) continue;
      attn_tile_query<T>(qs[i], Kq, Vs, ps[wave], kt, plim, mrun[qq], lrun[qq], o0[qq], o1[qq]);
    }
  }
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) {
    const int i = wave + 4 * qq;
    if (i >= cnt || k0 > base + i) continue;
    float* pp = part + ((((long)b * NH + h) * n_chunks + c) * Q + i) * (HD + 2);
    reinterpret_cast<float2*>(pp)[lane] = make_float2(o0[qq], o1[qq]);
    if (lane == 0) { pp[HD] = mrun[qq]; pp[HD + 1] = lrun[qq]; }
  }
}

// Merge chunks 0..p/C of each (row, head) in order.  Block = 2 heads x 128 dims.
constexpr int MERGE_ONE = 32;  // chunk counts merged from one batch of loads
__global__ __launch_bounds__(256) void k_attn_combine(const float* __restrict__ part, RowPlan plan, int n_chunks,
                                                      int chunk_keys, int max_pos, float* __restrict__ out) {
  const int row = blockIdx.x;
  const int h = blockIdx.y * 2 + (threadIdx.x >> 7);
  const int d = threadIdx.x & 127;
  const int b = row / plan.Q, i = row - b * plan.Q;
  float* o = out + (long)row * QD + h * HD + d;
  const float* pp = part + (((long)b * NH + h) * n_chunks) * plan.Q * (HD + 2) + (long)i * (HD + 2);
  const long cstride = (long)plan.Q * (HD + 2);
  // the row's merge count from the plan (rows outside it: ok false, row zero)
  auto plan_nc = [&](bool& ok) {
    const int p = plan.base[b] + i;
    ok = i < plan.cnt[b] && p >= 0 && p < max_pos;
    return ok ? min(p / chunk_keys + 1, n_chunks) : 1;
  };
  bool ok;
  float r;
  // one batch of loads (as many as the launch's chunk count needs), issued
  // with the plan reads (their addresses do not depend on it); chunks past nc
  // unused.  Any batch size >= nc gives the same bits.
  auto merge_one = [&](auto g) {
    constexpr int G = decltype(g)::value;
    float mv[G], lv[G], ov[G];
    merge_load<G>(pp, cstride, 0, n_chunks, d, mv, lv, ov);
    return merge_regs<G>(mv, lv, ov, plan_nc(ok));
  };
  if (n_chunks <= 8) r = merge_one(std::integral_constant<int, 8>{});
  else if (n_chunks <= 16) r = merge_one(std::integral_constant<int, 16>{});
  else if (n_chunks <= MERGE_ONE) r = merge_one(std::integral_constant<int, MERGE_ONE>{});
  else r = merge_loop(pp, cstride, plan_nc(ok), d);
  *o = ok ? r : 0.f;
}

template <typename T>
void launch_attention(hipStream_t s, const float* q, KvView<T> kv, RowPlan plan, int B, int n_chunks,
                      int tiles_per_chunk, float* part, float* out) {
  hipLaunchKernelGGL((k_attn_partial<T>), dim3(n_chunks, NH, B), dim3(256), 0, s, q, kv, plan, n_chunks,
                     tiles_per_chunk, part);
  hipLaunchKernelGGL(k_attn_combine, dim3(B * plan.Q, NH / 2), dim3(256), 0, s, part, plan, n_chunks,
                     tiles_per_chunk * ATT_TILE, kv.max_pos, out);
}

// ---- prefill attention --------------------------------------------------
//
// Block (entry b, head h) serves the entry's PREFILL_CHUNK = 32 query rows,
// wavefront w rows 16 w .. 16 w + 15, over 64-key tiles 0, 64, .. up to the
// entry's last position.  Per tile and wavefront, on the matrix cores:
//   S = Q K^T / sqrt(128): four 16x16 blocks (keys 16 n .. 16 n + 15), Q in
//     bf16 hi + lo parts (the fp32 queries to about 16 bits), keys exact;
//   the online softmax per row: row max over the 64 keys (the four blocks in
//     a lane, then the 16 lanes of the row), correction exp(m_old - m_new),
//     p = exp(s - m_new) for visible keys (key <= the row's position), else 0;
//   O += P V: eight 16x16 blocks of 16 value dims, P (via LDS, in the A
//     layout) in hi + lo parts, values from an LDS copy of the tile stored
//     transposed, eight bf16 of one dim per 16 bytes; the values of keys past
//     the entry's last position (cache rows not yet written, whatever their
//     bits) are staged as zeros, so that p = 0 there adds exact zeros.
// Tiles start at multiples of 64 and a masked key adds exact zeros (in a
// fully masked tile the row's max, sum and output stay as they are), so a
// row's result does not depend on the other rows of the launch.
constexpr int PA_VT_STRIDE = ATT_TILE / 2 + 4;  // 32-bit words per transposed value row (+4: spreads banks)

__global__ __launch_bounds__(128) void k_attn_prefill_mfma(const float* __restrict__ q, KvView<bf16> kv,
                                                           RowPlan plan, float* __restrict__ part) {
  __shared__ __align__(16) uint32_t vt[HD][PA_VT_STRIDE];  // vt[d][k / 2] = (v[k][d], v[k + 1][d]) as bf16 pairs
  __shared__ __align__(16) float pl[2][16][ATT_TILE + 4];  // per wavefront: P rows
  const int b = blockIdx.x, h = blockIdx.y;
  const int wave = wave_id(), lane = lane_id(), tid = threadIdx.x;
  const int g = lane >> 4, c16 = lane & 15;
  const int Q = plan.Q;
  const int base = plan.base[b], cnt = min(plan.cnt[b], Q);
  const long slot = plan.slot[b];
  const int max_pos = kv.max_pos;
  const int p_last = min(base + cnt - 1, max_pos - 1);
  // this block's share of the entry's key tiles (split blockIdx.z)
  int t0, t1;
  if (!prefill_split(cnt > 0 && base >= 0 ? p_last / ATT_TILE + 1 : 0, blockIdx.z, t0, t1)) return;
  // A fragments of this wavefront's 16 query rows (row c16, dims 32 s + 8 g ..)
  const int qi = 16 * wave + c16;
  uint4 qh[4], ql[4];
  {
    const bool ok = qi < cnt;
    const float4* qp = reinterpret_cast<const float4*>(q + (long)(b * Q + (ok ? qi : 0)) * QD + h * HD);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      float4 a = qp[8 * st + 2 * g], c = qp[8 * st + 2 * g + 1];
      if (!ok) a = c = make_float4(0.f, 0.f, 0.f, 0.f);
      split_bf16x8(a, c, qh[st], ql[st]);
    }
  }
  // this lane's rows of the S / O blocks: i = 16 wave + 4 g + r
  int plim[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = 16 * wave + 4 * g + r;
    plim[r] = i < cnt ? base + i : -1;  // last visible key (-1: none)
  }
  float mrun[4], lrun[4];
  f32x4_v o[8];
#pragma unroll
  for (int r = 0; r < 4; ++r) { mrun[r] = -INFINITY; lrun[r] = 0.f; }
#pragma unroll
  for (int d = 0; d < 8; ++d) o[d] = f32x4_v{0.f, 0.f, 0.f, 0.f};
  // tile loads: key fragments (key kt + 16 n + c16, dims 32 s + 8 g ..) and
  // this thread's value chunks (keys 2 kp, 2 kp + 1, dims 8 dc ..), from the
  // tile's page
  uint4 kf[4][4], vc[4][2];
  auto load_tile = [&](int kt) {
    const long pgt = kv.page_of(slot, kt);
    const bf16* Kt = kv.rows(pgt, 0, h);
    const bf16* Vt = kv.rows(pgt, 1, h);
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const long k = 16 * n + c16;
#pragma unroll
      for (int st = 0; st < 4; ++st) kf[n][st] = ldg16(Kt + k * HD + 32 * st + 8 * g);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = tid + 128 * j, kp = e >> 4, dc = e & 15;  // 32 key pairs x 16 dim chunks
      vc[j][0] = ldg16(Vt + (long)(2 * kp) * HD + 8 * dc);
      vc[j][1] = ldg16(Vt + (long)(2 * kp + 1) * HD + 8 * dc);
    }
  };
  const float scale = 0.08838834764831845f;  // 1 / sqrt(128)
  load_tile(t0 * ATT_TILE);
  for (int t = t0; t < t1; ++t) {
    const int kt = t * ATT_TILE;
    // S blocks from the key fragments in registers
    f32x4_v sb[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      sb[n] = f32x4_v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        sb[n] = mfma_bf16(qh[st], kf[n][st], sb[n]);
        sb[n] = mfma_bf16(ql[st], kf[n][st], sb[n]);
      }
    }
    __syncthreads();  // the previous tile's reads of vt are done
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // transposed value staging; keys past p_last (never written) as zeros
      const int e = tid + 128 * j, kp = e >> 4, dc = e & 15;
      if (kt + 2 * kp > p_last) vc[j][0] = make_uint4(0, 0, 0, 0);
      if (kt + 2 * kp + 1 > p_last) vc[j][1] = make_uint4(0, 0, 0, 0);
      const uint32_t* a = reinterpret_cast<const uint32_t*>(&vc[j][0]);
      const uint32_t* c = reinterpret_cast<const uint32_t*>(&vc[j][1]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {  // dims 8 dc + 2 w, 8 dc + 2 w + 1
        vt[8 * dc + 2 * w][kp] = (a[w] & 0xffffu) | (c[w] << 16);
        vt[8 * dc + 2 * w + 1][kp] = (a[w] >> 16) | (c[w] & 0xffff0000u);
      }
    }
    if (t + 1 < t1) load_tile(kt + ATT_TILE);  // next tile in flight during this one's arithmetic
    // online softmax of this lane's four rows
    float corr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float s4[4];
      float mt = -INFINITY;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int key = kt + 16 * n + c16;
        s4[n] = sb[n][r] * scale;
        if (key > plim[r]) s4[n] = -INFINITY;
        mt = fmaxf(mt, s4[n]);
      }
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) mt = fmaxf(mt, xor_lane(mt, off));
      const float mnew = fmaxf(mrun[r], mt);
      corr[r] = (mnew == -INFINITY) ? 1.f : expf(mrun[r] - mnew);
      float ps = 0.f;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const float p = (s4[n] == -INFINITY) ? 0.f : expf(s4[n] - mnew);
        pl[wave][4 * g + r][16 * n + c16] = p;
        ps += p;
      }
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) ps += xor_lane(ps, off);
      lrun[r] = lrun[r] * corr[r] + ps;
      mrun[r] = mnew;
    }
#pragma unroll
    for (int d = 0; d < 8; ++d)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[d][r] *= corr[r];
    __syncthreads();  // vt staged, P written
    // O += P V over the tile's two 32-key steps
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const float* pr = &pl[wave][c16][32 * st + 8 * g];
      const float4 pa = *reinterpret_cast<const float4*>(pr), pb = *reinterpret_cast<const float4*>(pr + 4);
      uint4 ph, plo;
      split_bf16x8(pa, pb, ph, plo);
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const uint4 vb = *reinterpret_cast<const uint4*>(&vt[16 * d + c16][16 * st + 4 * g]);
        o[d] = mfma_bf16(ph, vb, o[d]);
        o[d] = mfma_bf16(plo, vb, o[d]);
      }
    }
  }
  // the split's partial of each query row: o (unnormalised), m, l (a row
  // that sees none of the split's keys: 0, -inf, 0)
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = 16 * wave + 4 * g + r;
    if (i >= cnt) continue;
    float* pp = part + ((((long)b * NH + h) * PF_SPLITS + blockIdx.z) * Q + i) * (HD + 2);
#pragma unroll
    for (int d = 0; d < 8; ++d) pp[16 * d + c16] = o[d][r];
    if (c16 == 0) {
      pp[HD] = mrun[r];
      pp[HD + 1] = lrun[r];
    }
  }
}

// Merge of the splits of each prefill row, in split order: O / L with
// weights exp(m_s - max m); rows past the entry's count are zero.  Block =
// (row, pair of heads), thread = (head, dim) as in k_attn_combine.
__global__ __launch_bounds__(256) void k_attn_prefill_merge(const float* __restrict__ part, RowPlan plan, int max_pos,
                                                            float* __restrict__ out) {
  const int row = blockIdx.x;
  const int h = blockIdx.y * 2 + (threadIdx.x >> 7);
  const int d = threadIdx.x & 127;
  const int Q = plan.Q;
  const int b = row / Q, i = row - b * Q;
  const int base = plan.base[b], cnt = min(plan.cnt[b], Q);
  const int p_last = min(base + cnt - 1, max_pos - 1);
  float* o = out + (long)row * QD + h * HD + d;
  int t0, t1, ns = 0;
  const int n_tiles = cnt > 0 && base >= 0 ? p_last / ATT_TILE + 1 : 0;
  while (ns < PF_SPLITS && prefill_split(n_tiles, ns, t0, t1)) ++ns;
  if (i >= cnt || ns == 0) {
    *o = 0.f;
    return;
  }
  const float* pp = part + (((long)b * NH + h) * PF_SPLITS * Q + i) * (HD + 2);
  const long sstride = (long)Q * (HD + 2);
  float mv[PF_SPLITS], lv[PF_SPLITS], ov[PF_SPLITS];
#pragma unroll
  for (int sp = 0; sp < PF_SPLITS; ++sp) {
    const float* q = pp + min(sp, ns - 1) * sstride;
    mv[sp] = q[HD];
    lv[sp] = q[HD + 1];
    ov[sp] = q[d];
  }
  float mg = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < PF_SPLITS; ++sp) mg = fmaxf(mg, sp < ns ? mv[sp] : -INFINITY);
  float L = 0.f, O = 0.f;
#pragma unroll
  for (int sp = 0; sp < PF_SPLITS; ++sp) {
    if (sp < ns) {
      const float w = expf(mv[sp] - mg);
      L = fmaf(lv[sp], w, L);
      O = fmaf(ov[sp], w, O);
    }
  }
  *o = O / L;
}

// The fp32 cache: block (entry b, head h), wavefront w serves rows w, w + 4,
// ..; per 64-key tile, lane = key for the scores (q . k in order over the 128
// dims), the online softmax, then lane = value-dim pair for the output.
__global__ __launch_bounds__(256) void k_attn_prefill_f32(const float* __restrict__ q, KvView<float> kv,
                                                          RowPlan plan, float* __restrict__ out) {
  __shared__ float pw[4][ATT_TILE];
  const int b = blockIdx.x, h = blockIdx.y;
  const int wave = wave_id(), lane = lane_id();
  const int Q = plan.Q;
  const int base = plan.base[b], cnt = min(plan.cnt[b], Q);
  const long slot = plan.slot[b];
  const int max_pos = kv.max_pos;
  const float scale = 0.08838834764831845f;
  for (int i = wave; i < Q; i += 4) {
    float* orow = out + (long)(b * Q + i) * QD + h * HD;
    const int plim = min(base + i, max_pos - 1);
    if (i >= cnt || base < 0) {
      orow[2 * lane] = 0.f;
      orow[2 * lane + 1] = 0.f;
      continue;
    }
    const float* qr = q + (long)(b * Q + i) * QD + h * HD;
    float mrun = -INFINITY, lrun = 0.f, o0 = 0.f, o1 = 0.f;
    for (int kt = 0; kt <= plim; kt += ATT_TILE) {
      const int key = kt + lane;
      const bool vis = key <= plim;
      const long pgt = kv.page_of(slot, kt);
      const float* kr = kv.rows(pgt, 0, h) + (long)lane * HD;
      const float* Vt = kv.rows(pgt, 1, h);
      float sc = 0.f;
      for (int d = 0; d < HD; ++d) sc = fmaf(qr[d], kr[d], sc);
      sc *= scale;
      const float mt = wave_max(vis ? sc : -INFINITY);
      const float mnew = fmaxf(mrun, mt);
      const float corr = expf(mrun - mnew);
      const float p = vis ? expf(sc - mnew) : 0.f;
      lrun = lrun * corr + wave_sum(p);
      pw[wave][lane] = p;
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      float a0 = o0 * corr, a1 = o1 * corr;
      const int nk = min(ATT_TILE, plim + 1 - kt);
      for (int t = 0; t < nk; ++t) {
        const float2 v = *reinterpret_cast<const float2*>(Vt + (long)t * HD + 2 * lane);
        a0 = fmaf(pw[wave][t], v.x, a0);
        a1 = fmaf(pw[wave][t], v.y, a1);
      }
      o0 = a0;
      o1 = a1;
      mrun = mnew;
      __builtin_amdgcn_wave_barrier();
    }
    orow[2 * lane] = o0 / lrun;
    orow[2 * lane + 1] = o1 / lrun;
  }
}

template <>
void launch_attention_prefill<bf16>(hipStream_t s, const float* q, KvView<bf16> kv, RowPlan plan, int n, float* part,
                                    float* out) {
  hipLaunchKernelGGL(k_attn_prefill_mfma, dim3(n, NH, PF_SPLITS), dim3(128), 0, s, q, kv, plan, part);
  hipLaunchKernelGGL(k_attn_prefill_merge, dim3(n * plan.Q, NH / 2), dim3(256), 0, s, part, plan, kv.max_pos, out);
}
template <>
void launch_attention_prefill<float>(hipStream_t s, const float* q, KvView<float> kv, RowPlan plan, int n,
                                     float* part, float* out) {
  (void)part;
  hipLaunchKernelGGL(k_attn_prefill_f32, dim3(n, NH), dim3(256), 0, s, q, kv, plan, out);
}

template void launch_attention<float>(hipStream_t, const float*, KvView<float>, RowPlan, int, int, int, float*,
                                      float*);
template void launch_attention<bf16>(hipStream_t, const float*, KvView<bf16>, RowPlan, int, int, int, float*,
                                     float*);

}  // namespace ocr
