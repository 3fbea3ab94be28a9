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
// KV reads in flight) and widens them as they are read.
template <typename T> struct AttTile;
template <> struct AttTile<float> {
  typedef float4 K4;   // 4 key dims
  typedef float2 V2;   // 2 value dims
  __device__ static __forceinline__ float4 k(const K4& v) { return v; }
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
  __device__ static __forceinline__ float4 k(const K4& v) {
    return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u), __uint_as_float(v.y << 16),
                       __uint_as_float(v.y & 0xffff0000u));
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
// scores (q . k over 128 dims, 4 at a time, in order), then lane = value-dim
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
  for (int d4 = 0; d4 < HD / 4; ++d4) {
    const float4 qv = qrow[d4];
    const float4 kv4 = AT::k(Kq[d4][lane]);
    sc = fmaf(qv.x, kv4.x, sc);
    sc = fmaf(qv.y, kv4.y, sc);
    sc = fmaf(qv.z, kv4.z, sc);
    sc = fmaf(qv.w, kv4.w, sc);
  }
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

template <typename T>
__global__ __launch_bounds__(256) void k_attn_partial(const float* __restrict__ q, const T* __restrict__ kv,
                                                      int max_pos, RowPlan plan, int n_chunks,
                                                      int tiles_per_chunk, float* __restrict__ part) {
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
  // The tile's addresses need only the slot: with identity slots the first
  // tile's loads go out with the plan reads and this head's query rows (i < Q)
  // (key indices clamped into the cache; rows past the last query's key are
  // zeroed when staged).
  const long slot = plan.ident ? (long)b : (long)plan.slot[b];
  const T* Kc = kv + slot * (2L * NH * max_pos * HD) + (long)h * max_pos * HD;
  const T* Vc = Kc + (long)NH * max_pos * HD;
  constexpr int CE = WT<T>::CE;
  constexpr int CPR = HD / CE;                         // 16-byte chunks per key row
  constexpr int NLD = ATT_TILE * CPR / 256;            // chunks per thread per tile
  uint4 kr[NLD], vr[NLD];
  auto load_tile = [&](int tt) {
    const int kt = k0 + tt * ATT_TILE;
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const int e = tid + 256 * j, t = e / CPR, d0 = (e % CPR) * CE;
      const long k = min(kt + t, max_pos - 1);
      kr[j] = ldg16(Kc + k * HD + d0);
      vr[j] = ldg16(Vc + k * HD + d0);
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
    qs[i][e % (HD / 4)] = (i < cnt) ? qv[j] : make_float4(0.f, 0.f, 0.f, 0.f);
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
void launch_attention(hipStream_t s, const float* q, const T* kv, int max_pos, RowPlan plan, int B, int n_chunks,
                      int tiles_per_chunk, float* part, float* out) {
  hipLaunchKernelGGL((k_attn_partial<T>), dim3(n_chunks, NH, B), dim3(256), 0, s, q, kv, max_pos, plan, n_chunks,
                     tiles_per_chunk, part);
  hipLaunchKernelGGL(k_attn_combine, dim3(B * plan.Q, NH / 2), dim3(256), 0, s, part, plan, n_chunks,
                     tiles_per_chunk * ATT_TILE, max_pos, out);
}

template void launch_attention<float>(hipStream_t, const float*, const float*, int, RowPlan, int, int, int, float*,
                                      float*);
template void launch_attention<bf16>(hipStream_t, const float*, const bf16*, int, RowPlan, int, int, int, float*,
                                     float*);

}  // namespace ocr
