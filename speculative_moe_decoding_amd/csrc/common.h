// Shared device helpers of the ocrdec kernels (gfx950, wave64).
//
// Numerics that every kernel follows, so that a row's result never depends on
// how many other rows share its launch (speculative == autoregressive, bit for
// bit):
//   * dot products: lane l of a wavefront owns the 16-byte chunks l, l+64, ...
//     of a weight row and accumulates them in order with fmaf; the 64 lane sums
//     are then added by a fixed tree (wave_reduce_t: steps at offsets 32, 16,
//     8, 4, 2, 1, exchanges in registers);
//   * row reductions of 256-thread blocks (RMSNorm): each thread sums its
//     elements k = tid + 256 j in order, then the same butterfly per wave, then
//     the four wave sums in order 0..3;
//   * no floating-point atomics anywhere.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ocr {

constexpr int D = 1280;          // d_model
constexpr int NH = 10;           // attention heads
constexpr int HD = 128;          // head dim
constexpr int QD = NH * HD;      // 1280
constexpr int NE = 64;           // routed experts
constexpr int NSH = 2;           // shared experts
constexpr int NX = NE + NSH;     // expert tensors per layer
constexpr int TOPK = 6;
constexpr int NSLOT = TOPK + NSH;  // routing slots per row: 6 routed then 2 shared
constexpr int DI = 896;          // expert width
constexpr int DF = 3584;         // draft FFN width
constexpr int MRG = 8;           // activation rows per GEMV group
constexpr int PREFILL_CHUNK = 32;  // prefix rows per prefill entry (positions 32 j .. 32 j + 31)
constexpr int ATT_TILE = 64;     // keys per LDS tile in decode attention
constexpr int LM_ROWS_PER_BLOCK = 64;

typedef uint16_t bf16;

__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename T> struct WT;
template <> struct WT<float> {
  static constexpr int CE = 4;  // elements per 16-byte chunk
  __device__ static __forceinline__ void cvt(const uint4& v, float* o) {
    o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
    o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
  }
  __device__ static __forceinline__ float load1(const float* p) { return *p; }
  __device__ static __forceinline__ float store_cvt(float v) { return v; }
};
template <> struct WT<bf16> {
  static constexpr int CE = 8;
  __device__ static __forceinline__ void cvt(const uint4& v, float* o) {
    o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xffff0000u);
    o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xffff0000u);
    o[4] = __uint_as_float(v.z << 16); o[5] = __uint_as_float(v.z & 0xffff0000u);
    o[6] = __uint_as_float(v.w << 16); o[7] = __uint_as_float(v.w & 0xffff0000u);
  }
  __device__ static __forceinline__ float load1(const bf16* p) { return __uint_as_float((uint32_t)*p << 16); }
  __device__ static __forceinline__ bf16 store_cvt(float v) { return f2bf(v); }
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// The value of lane l ^ off (off a power of two <= 32), in registers:
// permlane swaps at 32 and 16, a pair of DPP row shifts and a select at 8 and
// 4, quad permutes at 2 and 1 (lane layouts checked on the GPU).  The same
// result as __shfl_xor(v, off) without the LDS round trip; all 64 lanes must
// be active.
__device__ __forceinline__ int xor_lane_i(int v, int off) {
  switch (off) {
    case 32: {
      const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
      return (lane_id() < 32) ? p[1] : p[0];
    }
    case 16: {
      const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
      return (lane_id() & 16) ? p[0] : p[1];
    }
    case 8: {
      const int up = __builtin_amdgcn_update_dpp(0, v, 0x108, 0xF, 0xF, false);  // row_shl:8 (lane + 8)
      const int dn = __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8 (lane - 8)
      return (lane_id() & 8) ? dn : up;
    }
    case 4: {
      const int up = __builtin_amdgcn_update_dpp(0, v, 0x104, 0xF, 0xF, false);  // row_shl:4
      const int dn = __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
      return (lane_id() & 4) ? dn : up;
    }
    case 2: return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    default: return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
  }
}
__device__ __forceinline__ float xor_lane(float x, int off) {
  return __builtin_bit_cast(float, xor_lane_i(__builtin_bit_cast(int, x), off));
}

// Xor butterfly over the wavefront (offsets 32, 16, ..., 1, own + partner at
// every node): every lane gets the same bits.  All 64 lanes must be active.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += xor_lane(v, off);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, xor_lane(v, off));
  return v;
}

// Wavefront sum / max on the DPP paths, with no LDS round trip: within each
// 16-lane row, lanes exchange by quad permutes (xor 1, xor 2), then the
// half-row and row mirrors, so that every lane of a row holds the row's total
// (each step adds x + y on one lane and y + x on its partner: the same bits);
// the four row totals are then read into scalars and added in row order.
// Every lane gets the same value, whatever the call shape.
__device__ __forceinline__ float dpp_f(float v, int ctrl) {
  switch (ctrl) {  // the DPP control must be a constant
    case 0xB1: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    case 0x4E: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
    case 0x141: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
    default: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
  }
}
__device__ __forceinline__ float lane_f(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_f(v, 0xB1);   // quad_perm [1, 0, 3, 2]: lane xor 1
  v += dpp_f(v, 0x4E);   // quad_perm [2, 3, 0, 1]: lane xor 2
  v += dpp_f(v, 0x141);  // row_half_mirror: the other quad of the 8-lane half
  v += dpp_f(v, 0x140);  // row_mirror: the other half of the row
  return ((lane_f(v, 0) + lane_f(v, 16)) + lane_f(v, 32)) + lane_f(v, 48);
}
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_f(v, 0xB1));
  v = fmaxf(v, dpp_f(v, 0x4E));
  v = fmaxf(v, dpp_f(v, 0x141));
  v = fmaxf(v, dpp_f(v, 0x140));
  return fmaxf(fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), lane_f(v, 32)), lane_f(v, 48));
}

__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// v_mfma_f32_16x16x32_bf16 (wave64): lane l supplies A[l % 16][8 (l / 16) ..
// +7] and B[8 (l / 16) .. +7][l % 16] (8 bf16 in 16 bytes each) and receives
// D[4 (l / 16) + r][l % 16] in result register r.
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

// a - bf16(a) for the two halves of a packed pair (exact in fp32).
__device__ __forceinline__ float rem_lo(float a, uint32_t h) { return a - __uint_as_float(h << 16); }
__device__ __forceinline__ float rem_hi(float a, uint32_t h) { return a - __uint_as_float(h & 0xffff0000u); }

// Eight fp32 as bf16 hi = bf16(a) and lo = bf16(a - hi) fragments.
__device__ __forceinline__ void split_bf16x8(const float4& a, const float4& b, uint4& hi, uint4& lo) {
  hi.x = pack_bf16x2(a.x, a.y);
  hi.y = pack_bf16x2(a.z, a.w);
  hi.z = pack_bf16x2(b.x, b.y);
  hi.w = pack_bf16x2(b.z, b.w);
  lo.x = pack_bf16x2(rem_lo(a.x, hi.x), rem_hi(a.y, hi.x));
  lo.y = pack_bf16x2(rem_lo(a.z, hi.y), rem_hi(a.w, hi.y));
  lo.z = pack_bf16x2(rem_lo(b.x, hi.z), rem_hi(b.y, hi.z));
  lo.w = pack_bf16x2(rem_lo(b.z, hi.w), rem_hi(b.w, hi.w));
}

// Streaming (non-temporal) 16-byte load of weights that are read once per
// launch: keeps them from displacing the activations and KV tiles in the caches.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ldg16_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Sum over a 256-thread block in the fixed order described above.  `red` is
// LDS scratch of at least 4 floats; contains a barrier.
__device__ __forceinline__ float block_sum256(float v, float* red) {
  v = wave_sum(v);
  if (lane_id() == 0) red[wave_id()] = v;
  __syncthreads();
  float t = red[0];
  t += red[1];
  t += red[2];
  t += red[3];
  __syncthreads();
  return t;
}


// RMSNorm of `m_rows` (<= MR) activation rows into LDS, by the block's four
// wavefronts, one per row (rows w, w + 4, ...): lane l sums x[k]^2 over
// k = l + 64 j in order, the 64 lane sums go through the xor butterfly,
// r = 1 / sqrt(sum / K + eps), and xs[m][k] = (x[k] * r) * g[k].  g == nullptr
// copies the rows unchanged.  Row m is read from x + src_row(m) * ldx.  When
// a wavefront has two or more rows and they fit in registers, all of their
// loads go out before the first sum (row indices clamped to the last row, so
// the loads need no predicate).  No barrier inside.
template <int K, int MR, typename SrcRow>
__device__ __forceinline__ void norm_rows_wave(const float* __restrict__ x, long ldx, SrcRow src_row, int m_rows,
                                               const float* __restrict__ g, float eps, float* xs) {
  static_assert(K % 64 == 0, "row length must be a multiple of 64");
  constexpr int J = K / 64;
  constexpr int RW = (MR + 3) / 4;  // rows per wavefront
  const int lane = lane_id(), w = wave_id();
  auto finish = [&](int m, const float (&v)[J]) {
    if (g != nullptr) {
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < J; ++j) ss = fmaf(v[j], v[j], ss);
      ss = wave_sum(ss);
      const float r = 1.0f / sqrtf(ss / (float)K + eps);
#pragma unroll
      for (int j = 0; j < J; ++j) xs[m * K + lane + 64 * j] = (v[j] * r) * g[lane + 64 * j];
    } else {
#pragma unroll
      for (int j = 0; j < J; ++j) xs[m * K + lane + 64 * j] = v[j];
    }
  };
  if constexpr (RW > 1 && RW * J <= 48) {
    if (w >= m_rows) return;
    float v[RW][J];
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const float* xr = x + (long)src_row(min(w + 4 * i, m_rows - 1)) * ldx;
#pragma unroll
      for (int j = 0; j < J; ++j) v[i][j] = xr[lane + 64 * j];
    }
#pragma unroll
    for (int i = 0; i < RW; ++i)
      if (w + 4 * i < m_rows) finish(w + 4 * i, v[i]);
  } else {
    for (int m = w; m < m_rows; m += 4) {
      const float* xr = x + (long)src_row(m) * ldx;
      float v[J];
#pragma unroll
      for (int j = 0; j < J; ++j) v[j] = xr[lane + 64 * j];
      finish(m, v);
    }
  }
}

// Raise a kernel's dynamic-LDS limit once (needed above 64 KiB).
template <typename F>
inline void allow_lds(F* kernel, size_t bytes) {
  if (bytes > 65536) (void)hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

struct RowIdentity {
  int base;
  __device__ __forceinline__ int operator()(int m) const { return base + m; }
};

// Wavefront GEMV core: R weight rows (pointers rows[r], each K elements of T)
// against `m_act` (<= MR) activation rows held in LDS (xs[m][K], fp32).
// acc[r][m] holds the lane partial sums; WaveTotals adds them up.
// Loads of all R rows are issued before any arithmetic.
template <typename T, int K, int R, int MR>
struct WaveGemv {
  static constexpr int CE = WT<T>::CE;
  static constexpr int NCH = K / CE;          // 16-byte chunks per row
  static constexpr int NT = (NCH + 63) / 64;  // per-lane chunk iterations
  static_assert(K % CE == 0, "K must be a multiple of the chunk size");
  uint4 w[R][NT];

  __device__ __forceinline__ void load(const T* const* rows) {
    const int lane = lane_id();
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int c = lane + 64 * t;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (c < NCH) w[r][t] = ldg16_stream(rows[r] + (long)c * CE);
      }
    }
  }

  __device__ __forceinline__ void fma(const float* xs, int m_act, float (&acc)[R][MR]) const {
    int rows[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) rows[m] = m;
    fma_rows(xs, rows, m_act, acc);
  }

  // The same with activation row m at xs[rows[m]][.] (rows picked out of a
  // larger LDS block; the arithmetic of each row is unchanged).
  __device__ __forceinline__ void fma_rows(const float* xs, const int (&rows)[MR], int m_act,
                                           float (&acc)[R][MR]) const {
    const int lane = lane_id();
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < MR; ++m) acc[r][m] = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int c = lane + 64 * t;
      if (c < NCH) {
        float wf[R][CE];
#pragma unroll
        for (int r = 0; r < R; ++r) WT<T>::cvt(w[r][t], wf[r]);
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          if (m < m_act) {
            float xa[CE];
            const float4* xp = reinterpret_cast<const float4*>(xs + rows[m] * K + c * CE);
#pragma unroll
            for (int q = 0; q < CE / 4; ++q) {
              float4 f = xp[q];
              xa[4 * q] = f.x; xa[4 * q + 1] = f.y; xa[4 * q + 2] = f.z; xa[4 * q + 3] = f.w;
            }
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
              for (int e = 0; e < CE; ++e) acc[r][m] = fmaf(wf[r][e], xa[e], acc[r][m]);
          }
        }
      }
    }
  }
};

// Exchange with the partner lane of a reduction step at offset off, in
// registers: off = 32 and 16 by the permlane swaps (partner l ^ off), 8 and 4
// by the row and half-row mirrors (partner 15 - i / 7 - i within the 16 / 8
// lanes), 2 and 1 by quad permutes (l ^ off).  At each step of a reduction
// that goes 32, 16, 8, 4, 2, 1, the partner agrees with the lane on every bit
// already reduced and differs in bit off, which is all a reduction needs.
// All 64 lanes must be active.
__device__ __forceinline__ int xchg_i(int v, int off) {
  int r;
  switch (off) {
    case 32: {
      const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
      r = (lane_id() < 32) ? p[1] : p[0];
      break;
    }
    case 16: {
      const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
      r = (lane_id() & 16) ? p[0] : p[1];
      break;
    }
    case 8: r = __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false); break;  // row_mirror
    case 4: r = __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false); break;  // row_half_mirror
    case 2: r = __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false); break;   // quad_perm [2,3,0,1]
    default: r = __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false); break;  // quad_perm [1,0,3,2]
  }
  return r;
}
__device__ __forceinline__ float xchg(float x, int off) {
  return __builtin_bit_cast(float, xchg_i(__builtin_bit_cast(int, x), off));
}

// Sums each of N (a power of two <= 64) per-lane values over the wavefront
// with a fixed tree (steps at offsets 32, 16, ..., 1, own + partner at every
// node, partners as in xchg), transposed: at each of the first log2 N steps a
// lane keeps half of its values -- the half its own bit at that offset
// selects -- and trades the other half with its partner, so the wavefront
// spends N - 1 + 6 - log2 N exchanges instead of 6 N, all in registers.  Lane
// l returns the total of value i = l >> (6 - log2 N), and every lane holding
// value i has the same bits; v is overwritten.
template <int N>
__device__ __forceinline__ float wave_reduce_t(float (&v)[N]) {
  static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "N must be a power of two <= 64");
  constexpr int B = __builtin_ctz(N);
  const int lane = lane_id();
#pragma unroll
  for (int s = 0; s < B; ++s) {
    const int n = N >> s;
    const int off = 32 >> s;
    const bool up = (lane & off) != 0;
#pragma unroll
    for (int j = 0; j < n / 2; ++j) {
      const float lo = v[j], hi = v[j + n / 2];
      const float recv = xchg(up ? lo : hi, off);
      v[j] = (up ? hi : lo) + recv;
    }
  }
  float t = v[0];
#pragma unroll
  for (int off = 32 >> B; off >= 1; off >>= 1) t += xchg(t, off);
  return t;
}

// Argmax stage 2 of one output row over the per-block bests rv[0..nblk),
// ri[0..nblk) of the LM head (largest value, lowest id among equal ones: the
// order of the comparisons does not matter), by a 256-thread block.  Each
// thread loads AMG of them at a time, at indices clamped to the last block (a
// repeat changes nothing), so the loads need no predicate and go out together.
// `sv` / `si` are LDS scratch of 4 entries; two barriers inside; every thread
// gets the id.
constexpr int AMG = 8;
__device__ __forceinline__ int argmax_block(const float* __restrict__ rv, const int* __restrict__ ri, int nblk,
                                            float* sv, int* si) {
  const int wave = wave_id(), lane = lane_id();
  float v = -INFINITY;
  int id = 0x7fffffff;
  for (int b0 = 0; b0 < nblk; b0 += 256 * AMG) {
    float pv[AMG];
    int pi[AMG];
#pragma unroll
    for (int j = 0; j < AMG; ++j) {
      const int b = min(b0 + (int)threadIdx.x + 256 * j, nblk - 1);
      pv[j] = rv[b];
      pi[j] = ri[b];
    }
#pragma unroll
    for (int j = 0; j < AMG; ++j)
      if (pv[j] > v || (pv[j] == v && pi[j] < id)) { v = pv[j]; id = pi[j]; }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {  // any pairing gives the same result
    const float ov = xchg(v, off);
    const int oi = xchg_i(id, off);
    if (ov > v || (ov == v && oi < id)) { v = ov; id = oi; }
  }
  if (lane == 0) { sv[wave] = v; si[wave] = id; }
  __syncthreads();
  v = sv[0];
  id = si[0];
#pragma unroll
  for (int w = 1; w < 4; ++w)
    if (sv[w] > v || (sv[w] == v && si[w] < id)) { v = sv[w]; id = si[w]; }
  __syncthreads();
  return id;
}

// Totals of a WaveGemv's lane partials acc[r][m] (R a power of two): lane l
// receives the total of value i = l >> SH, i = m R + r, SH = 6 - log2(R MR),
// through the transposed reduction; `lead` marks one lane per value.  All
// lanes construct it.
template <int R, int MR>
struct WaveTotals {
  static constexpr int N = R * MR;
  static constexpr int SH = 6 - __builtin_ctz(N);
  static_assert((R & (R - 1)) == 0, "R must be a power of two");
  float val;
  int r, m;
  bool lead;
  __device__ __forceinline__ explicit WaveTotals(float (&acc)[R][MR]) {
    float v[N];
#pragma unroll
    for (int mm = 0; mm < MR; ++mm)
#pragma unroll
      for (int rr = 0; rr < R; ++rr) v[mm * R + rr] = acc[rr][mm];
    val = wave_reduce_t<N>(v);
    const int lane = lane_id();
    const int i = lane >> SH;
    r = i % R;
    m = i / R;
    lead = (lane & ((1 << SH) - 1)) == 0;
  }
  // The total of (r ^ x, m), from the lane that holds it (x << SH a power of
  // two); all lanes call it.
  __device__ __forceinline__ float partner(int x) const { return xor_lane(val, x << SH); }
};

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// Data that crosses workgroups inside one launch: loads that see the stores
// other workgroups made (agent scope: they do not stop at this XCD's L2) and
// the stores they see, agent-scope atomics for the counters, and the point
// after which this wavefront's stores are complete (s_waitcnt; the compiler
// moves no memory access across it).  No L2 write-back or invalidate is needed.
__device__ __forceinline__ float ld_agent(const float* p) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<const unsigned*>(p), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ unsigned ld_agent_u(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<unsigned*>(p), __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent_u(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned atomic_add_agent(unsigned* p, unsigned v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stores_done() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Paged KV cache of one layer (verifier or draft).  A page holds KV_PAGE
// consecutive positions (one attention tile) of one sequence, keys and
// values of every head: [K|V][head][KV_PAGE][128].  table[slot * max_blocks
// + pos / KV_PAGE] is the page of that block of positions, negative for none.
// Readers take a missing page as page 0 (they only read rows they mask: chunks
// past a sequence's end, or a slot released while the caller still decodes
// it); writers skip rows without a page.  max_pos: positions per slot.
constexpr int KV_PAGE = 64;
template <typename T>
struct KvView {
  T* base;
  const int* table;
  int max_blocks;
  int max_pos;
  __device__ __forceinline__ int raw_page(long slot, int pos) const {
    return table[slot * max_blocks + (min(max(pos, 0), max_pos - 1) / KV_PAGE)];
  }
  __device__ __forceinline__ long page_of(long slot, int pos) const {
    const int p = raw_page(slot, pos);
    return p < 0 ? 0 : p;
  }
  // the KV_PAGE rows of head h (kvsel 0: keys, 1: values) in a page
  __device__ __forceinline__ T* rows(long page, int kvsel, int h) const {
    return base + ((page * 2 + kvsel) * NH + h) * (long)(KV_PAGE * HD);
  }
  __device__ __forceinline__ T* at(long page, int kvsel, int h, int pos) const {
    return rows(page, kvsel, h) + (long)(pos % KV_PAGE) * HD;
  }
};

// Per-call row plan: sequence b of a call owns rows b*Q .. b*Q+Q-1; row i of
// it is valid when i < cnt[b] and sits at position base[b] + i.
struct RowPlan {
  const int* base;
  const int* cnt;
  const int* slot;   // state slot of sequence b
  int Q;
  int ident;         // 1: the slot of sequence b is b (slot[] holds the same)
};

}  // namespace ocr
