// gfx950 (CDNA4) kernels for R-SWA / SR-SWA single-step decode attention.
//
// Decode attention here is a memory-bound matrix-vector product (one query
// per (sequence, head)), so the kernels are built around streaming K/V rows
// from HBM with 16-byte loads per lane, not around MFMA:
//   * one head row (D = 128 bf16 = 256 B) is read by 16 lanes, a wave64 covers
//     4 rows per load instruction and keeps U such loads of K and of V in
//     flight before using any of them;
//   * the q.k dot product is reduced across the 16 lanes of a row with
//     cross-lane shuffles, the softmax is online (running max / sum in the
//     base-2 domain) per group of rows and merged across groups at the end;
//   * the waves of a workgroup take disjoint slices of a unit's keys and
//     merge their (max, sum, partial output) through LDS by log-sum-exp; the
//     dense decode can also cut a unit into several workgroups, whose partials
//     a second, small kernel merges.  No device-wide fence or atomic is used:
//     on gfx950 every agent-scope fence writes back and invalidates the L2.
//
// Method sources (web pages): R-SWA key set = permanent prefix + last n
// generated tokens ("百度Unlimited OCR" paper summary, lshu.cn, section 二);
// ring buffer overwriting the oldest slot (Unlimited-OCR-2 explainer,
// nxmr.cn, section "环形缓冲"); 32-token blocks, index-projection scores,
// 1.5-entmax top-k and log bias (same explainer, section "稀疏路由").
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "uocr_internal.h"

namespace uocr {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
// Floor of the running maximum: finite, so that exp2(m_old - m_new) never
// sees (-inf) - (-inf).  Logits (scaled, biased, base 2) are far above it.
constexpr float kFloor = -1.0e30f;
constexpr int kWaves = 4;  // waves per workgroup of the block-index kernel

// Phase stamps of the fused SR-SWA step, compiled in only with
// UOCR_PHASE_STAMPS (the library libuocr_stamps.so; libuocr.so has none of
// this code).  One thread records the device's constant-rate real-time
// counter (100 MHz) into LDS as a phase ends, and the workgroup copies its
// 64 slots to g_stamps[unit] once at the very end, so that no global store
// adds a wait to the step's barriers.  UOCR_STAMP_DONE first waits for every
// load in flight, so that a phase counts as done when its data has arrived,
// not when its last load was issued.  The slots are listed with
// uocr_phase_stamps in include/uocr_calib.h.
#ifdef UOCR_PHASE_STAMPS
constexpr int kStampSlots = 64;
__device__ unsigned long long g_stamps[kMaxStampUnits * kStampSlots];
#define UOCR_STAMP_LDS __shared__ unsigned long long s_stamp[kStampSlots]
#define UOCR_STAMP(st, cond, slot)                 \
  do {                                             \
    if (cond) (st)[slot] = wall_clock64();         \
  } while (0)
#define UOCR_STAMP_DONE(st, cond, slot)            \
  do {                                             \
    __builtin_amdgcn_s_waitcnt(0);                 \
    if (cond) (st)[slot] = wall_clock64();         \
  } while (0)
#else
#define UOCR_STAMP_LDS unsigned long long* const s_stamp = nullptr
#define UOCR_STAMP(st, cond, slot) ((void)(st))
#define UOCR_STAMP_DONE(st, cond, slot) ((void)(st))
#endif

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// element types and row geometry
// ---------------------------------------------------------------------------
// DT 0 = fp32, 1 = bf16.  A lane handles one 16-byte chunk of a row.
template <int DT, int D>
struct Geo {
  static constexpr int ES = DT == 0 ? 4 : 2;  // bytes per element
  static constexpr int E = 16 / ES;           // elements per lane chunk
  static constexpr int LPR = D * ES / 16;     // lanes per row
  static constexpr int RPL = 64 / LPR;        // rows per wave load
  static constexpr int ROWB = D * ES;         // bytes per row
  static constexpr int U = (32 / RPL) < 8 ? (32 / RPL) : 8;  // loads in flight
};

__device__ __forceinline__ uint4 ld16(const char* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Streaming 16-byte load: K/V rows and block keys are read once per step, so
// they are fetched with the nontemporal hint (measured on MI355X: ~7.0 TB/s
// for a pure read stream against ~6.2 TB/s with plain loads).
typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const char* p) {
  const v4u32 t = __builtin_nontemporal_load(reinterpret_cast<const v4u32*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ float4 ld16f_stream(const float* p) {
  typedef float v4f32 __attribute__((ext_vector_type(4)));
  const v4f32 t = __builtin_nontemporal_load(reinterpret_cast<const v4f32*>(p));
  return make_float4(t.x, t.y, t.z, t.w);
}

__device__ __forceinline__ void unpack(const uint4& v, float (&x)[4]) {
  x[0] = __uint_as_float(v.x);
  x[1] = __uint_as_float(v.y);
  x[2] = __uint_as_float(v.z);
  x[3] = __uint_as_float(v.w);
}

__device__ __forceinline__ void unpack(const uint4& v, float (&x)[8]) {
  x[0] = __uint_as_float(v.x << 16);
  x[1] = __uint_as_float(v.x & 0xffff0000u);
  x[2] = __uint_as_float(v.y << 16);
  x[3] = __uint_as_float(v.y & 0xffff0000u);
  x[4] = __uint_as_float(v.z << 16);
  x[5] = __uint_as_float(v.z & 0xffff0000u);
  x[6] = __uint_as_float(v.w << 16);
  x[7] = __uint_as_float(v.w & 0xffff0000u);
}

// fp32 -> bf16 bits, round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Cross-lane moves inside a row of 16 lanes with DPP (register to register,
// no LDS round trip).  After xor-1 and xor-2 quad permutes every lane of a
// quad holds the quad's value; the half-row mirror (lane i <- 7 - i) then
// pairs the two quads of each half row, and the row mirror (i <- 15 - i) the
// two halves, so the four steps reduce 2, 4, 8 and 16 lanes.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppMirror = 0x140;     // row_mirror

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ double dpp(double x) {
  const long long u = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(u & 0xffffffffll), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(u >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

// Value of the lane 16 (32) positions away, through the gfx950 row / half
// swaps: with both operands equal, permlane16_swap returns rows (0, 0, 2, 2)
// and (1, 1, 3, 3), permlane32_swap the halves (lo, lo) and (hi, hi).
__device__ __forceinline__ float xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]);
}
__device__ __forceinline__ float xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}
// x plus the value of the lane 16 (32) positions away.  A swap with both
// operands equal hands each lane its own and its partner's value in a fixed
// order (lower row first), so both lanes of a pair add the same two numbers
// in the same order and get bit-identical sums, with no lane select.
__device__ __forceinline__ float sum16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ double join(unsigned lo, unsigned hi) {
  return __longlong_as_double(((long long)hi << 32) | lo);
}
__device__ __forceinline__ double sum16(double x) {
  const long long u = __double_as_longlong(x);
  const unsigned lo = (unsigned)(u & 0xffffffffll), hi = (unsigned)(u >> 32);
  const auto l = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  const auto h = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  return join(l[0], h[0]) + join(l[1], h[1]);
}
__device__ __forceinline__ double sum32(double x) {
  const long long u = __double_as_longlong(x);
  const unsigned lo = (unsigned)(u & 0xffffffffll), hi = (unsigned)(u >> 32);
  const auto l = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  const auto h = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  return join(l[0], h[0]) + join(l[1], h[1]);
}

// Sum over groups of N lanes (N = 2 .. 32, aligned); every lane of a group
// gets the group's sum.
template <int N, typename T>
__device__ __forceinline__ T group_sum(T x) {
  if constexpr (N > 1) x += dpp<kDppXor1>(x);
  if constexpr (N > 2) x += dpp<kDppXor2>(x);
  if constexpr (N > 4) x += dpp<kDppHalfMirror>(x);
  if constexpr (N > 8) x += dpp<kDppMirror>(x);
  if constexpr (N > 16) x = sum16(x);
  return x;
}

template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
  return group_sum<LPR>(x);
}

// Sum of a float over the 64 lanes of a wave, returned to every lane.
__device__ __forceinline__ float wave_sum_f(float x) {
  x = group_sum<16>(x);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
}

// Sum of an int over the 64 lanes of a wave, returned to every lane.
__device__ __forceinline__ int wave_sum(int x) {
  x = group_sum<16>(x);
  return __builtin_amdgcn_readlane(x, 0) + __builtin_amdgcn_readlane(x, 16) + __builtin_amdgcn_readlane(x, 32) +
         __builtin_amdgcn_readlane(x, 48);
}

// Number of (lane, e) over the wave with v[e] < T: one compare per element
// into a lane mask and a scalar popcount, no cross-lane arithmetic.
template <int NS>
__device__ __forceinline__ int wave_count_below(const float (&v)[NS], float T) {
  int c = 0;
#pragma unroll
  for (int e = 0; e < NS; ++e) c += __popcll(__ballot(v[e] < T));
  return c;
}

__device__ __forceinline__ float readlane_f(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}
__device__ __forceinline__ double readlane_d(double x, int lane) {
  const long long u = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_readlane((int)(u & 0xffffffffll), lane);
  const int hi = __builtin_amdgcn_readlane((int)(u >> 32), lane);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

// Maximum over the 64 lanes of a wave, returned to every lane.
template <typename T>
__device__ __forceinline__ T wave_max(T x) {
  T y = dpp<kDppXor1>(x);
  x = y > x ? y : x;
  y = dpp<kDppXor2>(x);
  x = y > x ? y : x;
  y = dpp<kDppHalfMirror>(x);
  x = y > x ? y : x;
  y = dpp<kDppMirror>(x);
  x = y > x ? y : x;
  T r = x;
#pragma unroll
  for (int row = 1; row < 4; ++row) {
    T v;
    if constexpr (sizeof(T) == 4) {
      v = __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16 * row));
    }
    r = v > r ? v : r;
  }
  if constexpr (sizeof(T) == 4) r = __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, r), 0));
  return r;
}

// Online-softmax state of one lane: running max m (base-2 logits), running
// sum l and the partial output of the lane's E dimensions.
template <int E>
struct State {
  float m, l, acc[E];
  __device__ __forceinline__ void init() {
    m = kFloor;
    l = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
  }
};

// Attend over `nrows` consecutive rows starting at K / V (already offset to
// the lane's chunk).  q holds the lane's chunk of scale*log2(e)*q; bias2 is
// the additive logit bias of these rows in base 2.  Lanes of row group `grp`
// take rows grp, grp + RPL, ...
// Row `srow` (if in range) is read from sK / sV instead of K / V.  Rows in
// [nvalid, nrows) are read (they must be addressable) but carry no weight:
// this lets a caller issue loads before it knows how many rows count.  U =
// row loads of K and of V in flight per lane.  The K loads go out before the
// V loads, and every lane issues all of them (a lane past the last row
// re-reads row nrows - 1, with no weight): with no branch around a load the
// compiler waits for each load only where its value is used, so the q.k
// products start while the rest is in flight.
template <int DT, int D, int U = Geo<DT, D>::U, bool STREAM = true>
__device__ __forceinline__ void attend_range(const char* __restrict__ K, const char* __restrict__ V,
                                             int nrows, float bias2,
                                             const float (&q)[Geo<DT, D>::E],
                                             State<Geo<DT, D>::E>& st, int grp, int srow = -1,
                                             const char* sK = nullptr, const char* sV = nullptr,
                                             int nvalid = 1 << 30) {
  using G = Geo<DT, D>;
  constexpr int E = G::E;
  const int nv = min(nvalid, nrows);
  for (int r0 = 0; r0 < nrows; r0 += G::RPL * U) {
    uint4 kr[U], vr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = min(r0 + u * G::RPL + grp, nrows - 1);
      const char* kp = row == srow ? sK : K + (size_t)row * G::ROWB;
      kr[u] = STREAM ? ld16_stream(kp) : ld16(kp);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = min(r0 + u * G::RPL + grp, nrows - 1);
      const char* vp = row == srow ? sV : V + (size_t)row * G::ROWB;
      vr[u] = STREAM ? ld16_stream(vp) : ld16(vp);
    }
    float s[U];
    float mt = kFloor;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float k[E];
      unpack(kr[u], k);
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) d = fmaf(q[e], k[e], d);
      d = row_sum<G::LPR>(d);
      const bool valid = r0 + u * G::RPL + grp < nv;
      s[u] = valid ? d + bias2 : -INFINITY;
      if (!valid) vr[u] = make_uint4(0u, 0u, 0u, 0u);  // weight 0 must not meet a NaN
      mt = fmaxf(mt, s[u]);
    }
    const float mn = fmaxf(st.m, mt);
    const float alpha = fexp2(st.m - mn);
    st.l *= alpha;
#pragma unroll
    for (int e = 0; e < E; ++e) st.acc[e] *= alpha;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float p = fexp2(s[u] - mn);
      st.l += p;
      float v[E];
      unpack(vr[u], v);
#pragma unroll
      for (int e = 0; e < E; ++e) st.acc[e] = fmaf(p, v[e], st.acc[e]);
    }
    st.m = mn;
  }
}

// attend_range with no more loads in flight than the rows need (up to the
// geometry's U): a short range (a live-block chunk, a window share) issues no
// loads for rows past its end.
template <int DT, int D, bool STREAM = true>
__device__ __forceinline__ void attend_fit(const char* __restrict__ K, const char* __restrict__ V, int nrows,
                                           float bias2, const float (&q)[Geo<DT, D>::E],
                                           State<Geo<DT, D>::E>& st, int grp, int srow = -1,
                                           const char* sK = nullptr, const char* sV = nullptr,
                                           int nvalid = 1 << 30) {
  using G = Geo<DT, D>;
  const int need = (nrows + G::RPL - 1) / G::RPL;
  if (G::U > 2 && need <= 2)
    attend_range<DT, D, 2, STREAM>(K, V, nrows, bias2, q, st, grp, srow, sK, sV, nvalid);
  else if (G::U > 4 && need <= 4)
    attend_range<DT, D, 4, STREAM>(K, V, nrows, bias2, q, st, grp, srow, sK, sV, nvalid);
  else if (G::U > 6 && need <= 6)
    attend_range<DT, D, 6, STREAM>(K, V, nrows, bias2, q, st, grp, srow, sK, sV, nvalid);
  else
    attend_range<DT, D, G::U, STREAM>(K, V, nrows, bias2, q, st, grp, srow, sK, sV, nvalid);
}

// Merge the RPL row groups of a wave: afterwards every lane holds the wave's
// state for its chunk.
template <int OFF>
__device__ __forceinline__ float lane_xor(float x) {
  if constexpr (OFF == 16) return xor16(x);
  else if constexpr (OFF == 32) return xor32(x);
  else return __shfl_xor(x, OFF);
}

template <int LPR, int E, int OFF = LPR>
__device__ __forceinline__ void merge_groups(State<E>& st) {
  if constexpr (OFF < 64) {
    const float mo = lane_xor<OFF>(st.m);
    const float lo = lane_xor<OFF>(st.l);
    const float mn = fmaxf(st.m, mo);
    const float a = fexp2(st.m - mn), b = fexp2(mo - mn);
    st.l = st.l * a + lo * b;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float ao = lane_xor<OFF>(st.acc[e]);
      st.acc[e] = st.acc[e] * a + ao * b;
    }
    st.m = mn;
    merge_groups<LPR, E, OFF * 2>(st);
  }
}

template <int DT, int D>
__device__ __forceinline__ void load_q(const void* q, int unit, int c, float scale,
                                       float (&x)[Geo<DT, D>::E]) {
  using G = Geo<DT, D>;
  const uint4 v = ld16(static_cast<const char*>(q) + (size_t)unit * G::ROWB + c * 16);
  unpack(v, x);
#pragma unroll
  for (int e = 0; e < G::E; ++e) x[e] *= scale;
}

// Store E output values (already normalised) of chunk c of `unit`.
template <int DT, int D>
__device__ __forceinline__ void store_chunk(void* out, int unit, int c, const float* o) {
  using G = Geo<DT, D>;
  char* p = static_cast<char*>(out) + (size_t)unit * G::ROWB + c * 16;
  if constexpr (DT == 0) {
    *reinterpret_cast<float4*>(p) = make_float4(o[0], o[1], o[2], o[3]);
  } else {
    uint4 w;
    w.x = bf16_bits(o[0]) | (bf16_bits(o[1]) << 16);
    w.y = bf16_bits(o[2]) | (bf16_bits(o[3]) << 16);
    w.z = bf16_bits(o[4]) | (bf16_bits(o[5]) << 16);
    w.w = bf16_bits(o[6]) | (bf16_bits(o[7]) << 16);
    *reinterpret_cast<uint4*>(p) = w;
  }
}

// End of a workgroup's work: the W waves merge their states through LDS.
// With one split per unit wave 0 normalises and writes the output; otherwise
// it leaves the workgroup's (max, sum, partial output) in the workspace for
// k_split_merge, which runs after this kernel in the same stream (the kernel
// boundary makes the partials visible; no device-wide fence or atomic is
// needed).
// WC > 0 gives the number of waves at compile time, so that the reads of the
// W partial states are issued back to back instead of one LDS round trip per
// wave (about 1 us of the fused SR-SWA step with a runtime count).
constexpr int kMaxWaves = 16;

template <int DT, int D, int WC = 0>
__device__ __forceinline__ void wg_finish(State<Geo<DT, D>::E>& st, float (*lds_ml)[2], float* lds_o,
                                          const DecodeArgs& a, int unit, int split,
                                          unsigned long long* stamps = nullptr) {
  using G = Geo<DT, D>;
  constexpr int E = G::E;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, W = WC > 0 ? WC : blockDim.x >> 6;
  const int grp = lane / G::LPR, c = lane % G::LPR;
  merge_groups<G::LPR, E>(st);
  UOCR_STAMP(stamps, stamps && lane == 0, 56 + wave);
  if (grp == 0) {
    float4* dst = reinterpret_cast<float4*>(lds_o + wave * D + c * E);
#pragma unroll
    for (int e = 0; e < E; e += 4) dst[e / 4] = make_float4(st.acc[e], st.acc[e + 1], st.acc[e + 2], st.acc[e + 3]);
  }
  if (lane == 0) {
    lds_ml[wave][0] = st.m;
    lds_ml[wave][1] = st.l;
  }
  __syncthreads();
  UOCR_STAMP(stamps, stamps && threadIdx.x == 0, 7);
  // every thread takes the common maximum, then output dimensions are dealt
  // to the threads; each sums the W waves' weighted partials in wave order
  // (a wave that saw no key has l = 0 and acc = 0 and adds exactly nothing)
  float M = kFloor;
  float mw[WC > 0 ? WC : 1], fw[WC > 0 ? WC : 1];
  if constexpr (WC > 0) {
#pragma unroll
    for (int w = 0; w < WC; ++w) {
      mw[w] = lds_ml[w][0];
      M = fmaxf(M, mw[w]);
    }
#pragma unroll
    for (int w = 0; w < WC; ++w) fw[w] = fexp2(mw[w] - M);
  } else {
    for (int w = 0; w < W; ++w) M = fmaxf(M, lds_ml[w][0]);
  }
  // the stride is a constant where the wave count is, which spares a
  // scalar load of the launch's group size from the kernel arguments here
  const int nth = WC > 0 ? WC * 64 : (int)blockDim.x;
  for (int t = threadIdx.x; t < D; t += nth) {
    float L = 0.f, O = 0.f;
    if constexpr (WC > 0) {
#pragma unroll
      for (int w = 0; w < WC; ++w) {
        L = fmaf(fw[w], lds_ml[w][1], L);
        O = fmaf(fw[w], lds_o[w * D + t], O);
      }
    } else {
      for (int w = 0; w < W; ++w) {
        const float f = fexp2(lds_ml[w][0] - M);
        L = fmaf(f, lds_ml[w][1], L);
        O = fmaf(f, lds_o[w * D + t], O);
      }
    }
    if (a.splits == 1) {
      const float inv = L > 0.f ? 1.f / L : 0.f;
      char* dst = static_cast<char*>(a.out) + (size_t)unit * G::ROWB;
      if constexpr (DT == 0)
        reinterpret_cast<float*>(dst)[t] = O * inv;
      else
        reinterpret_cast<uint16_t*>(dst)[t] = (uint16_t)bf16_bits(O * inv);
    } else {
      const size_t part = (size_t)unit * a.splits + split;
      if (t == 0) *reinterpret_cast<float2*>(a.part_ml + part * 2) = make_float2(M, L);
      a.part_o[part * D + t] = O;
    }
  }
}

// The fused SR-SWA step's finish (W <= 8 waves, splits == 1): the row groups
// of every wave are not merged inside the wave first; each of the
// P = W * 64 / LPR row groups leaves its partial (max, sum, output chunk) in
// LDS, and after one barrier the whole workgroup merges them: wave w takes
// output dims [w * D / W, (w + 1) * D / W), TPD = 64 W / D lanes per dim,
// each lane merging P / TPD partials, then the TPD lanes of a dim merge by
// cross-lane swaps.  The wave that finishes last then pays for a few LDS
// stores instead of the whole in-wave merge.  part_o (P * D floats) and
// part_ml (P pairs) are the caller's LDS; every partial is read after the
// barrier only.
template <int DT, int D, int W>
struct PartGeo {
  static constexpr int GPW = 64 / Geo<DT, D>::LPR;  // row groups per wave
  static constexpr int P = W * GPW;                 // partials
  static constexpr int TPD = 64 * W / D;            // lanes per output dim
  static constexpr int DPW = D / W;                 // dims per wave
  static constexpr int PPT = P / TPD;               // partials per lane
};

template <int DT, int D, int W>
__device__ __forceinline__ void wg_finish_parts(const State<Geo<DT, D>::E>& st, float* part_o, float2* part_ml,
                                                const DecodeArgs& a, int unit,
                                                unsigned long long* stamps = nullptr) {
  using G = Geo<DT, D>;
  using PG = PartGeo<DT, D, W>;
  constexpr int E = G::E;
  static_assert(64 * W % D == 0 && PG::P % PG::TPD == 0 && PG::DPW * PG::TPD == 64, "finish geometry");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane / G::LPR, c = lane % G::LPR;
  const int p = wave * PG::GPW + grp;
  float4* dst = reinterpret_cast<float4*>(part_o + p * D + c * E);
#pragma unroll
  for (int e = 0; e < E; e += 4) dst[e / 4] = make_float4(st.acc[e], st.acc[e + 1], st.acc[e + 2], st.acc[e + 3]);
  if (c == 0) part_ml[p] = make_float2(st.m, st.l);
  UOCR_STAMP(stamps, stamps && lane == 0, 56 + wave);
  __syncthreads();
  UOCR_STAMP(stamps, stamps && threadIdx.x == 0, 7);
  // lane (qq, dl) of wave w: dim d = w * DPW + dl, partials qq, qq + TPD, ...
  const int dl = lane % PG::DPW, qq = lane / PG::DPW, d = wave * PG::DPW + dl;
  float mw[PG::PPT];
  float M = kFloor;
#pragma unroll
  for (int i = 0; i < PG::PPT; ++i) {
    mw[i] = part_ml[i * PG::TPD + qq].x;
    M = fmaxf(M, mw[i]);
  }
  float L = 0.f, O = 0.f;
#pragma unroll
  for (int i = 0; i < PG::PPT; ++i) {
    const int pi = i * PG::TPD + qq;
    const float f = fexp2(mw[i] - M);
    L = fmaf(f, part_ml[pi].y, L);
    O = fmaf(f, part_o[pi * D + d], O);
  }
#pragma unroll
  for (int off = PG::DPW; off < 64; off *= 2) {
    float mo, lo, oo;
    if (off == 16) {
      mo = xor16(M), lo = xor16(L), oo = xor16(O);
    } else if (off == 32) {
      mo = xor32(M), lo = xor32(L), oo = xor32(O);
    } else {
      mo = __shfl_xor(M, off), lo = __shfl_xor(L, off), oo = __shfl_xor(O, off);
    }
    const float mn = fmaxf(M, mo);
    const float fa = fexp2(M - mn), fb = fexp2(mo - mn);
    L = L * fa + lo * fb;
    O = O * fa + oo * fb;
    M = mn;
  }
  if (qq == 0) {
    const float inv = L > 0.f ? 1.f / L : 0.f;
    char* dst_row = static_cast<char*>(a.out) + (size_t)unit * G::ROWB;
    if constexpr (DT == 0)
      reinterpret_cast<float*>(dst_row)[d] = O * inv;
    else
      reinterpret_cast<uint16_t*>(dst_row)[d] = (uint16_t)bf16_bits(O * inv);
  }
}

// ---------------------------------------------------------------------------
// uocr_ring_append: one workgroup per sequence
// ---------------------------------------------------------------------------
template <int DT, int D>
__global__ __launch_bounds__(256) void k_ring_append(AppendArgs a) {
  using G = Geo<DT, D>;
  const int b = blockIdx.x;
  __shared__ int slot_s;
  int t = 0;
  if (threadIdx.x == 0) {
    t = max(a.t_gen[b], 0);
    slot_s = t % a.window;
  }
  __syncthreads();
  const int slot = slot_s;
  constexpr int CPR = G::ROWB / 16;  // 16-byte chunks per row
  const int per = a.heads * CPR;
  for (int i = threadIdx.x; i < 2 * per; i += blockDim.x) {
    const int which = i / per, ci = i - which * per;
    const int h = ci / CPR, off = ci - h * CPR;
    const size_t unit = (size_t)b * a.heads + h;
    const char* src = static_cast<const char*>(which ? a.v_new : a.k_new) + unit * G::ROWB + off * 16;
    char* dst = static_cast<char*>(which ? a.v_ring : a.k_ring) +
                (unit * a.window + slot) * G::ROWB + off * 16;
    *reinterpret_cast<uint4*>(dst) = ld16(src);
  }
  if (threadIdx.x == 0) a.t_gen[b] = t + 1;
}

// ---------------------------------------------------------------------------
// uocr_rswa_decode: dense prefix + window.  One workgroup per (unit, split);
// its W waves take contiguous slices of the split's keys.
// ---------------------------------------------------------------------------
template <int DT, int D>
__global__ __launch_bounds__(1024) void k_rswa_decode(DecodeArgs a) {
  using G = Geo<DT, D>;
  __shared__ float lds_ml[kMaxWaves][2];
  __shared__ __attribute__((aligned(16))) float lds_o[kMaxWaves * D];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, W = blockDim.x >> 6;
  const int unit = blockIdx.x / a.splits, split = blockIdx.x - unit * a.splits;
  const int b = unit / a.heads;
  const int m = min(max(a.prefix_len[b], 0), a.prefix_cap);
  const int w = min(max(a.t_gen[b], 0), a.window);
  // virtual key index: [0, m) prefix rows, [m, m + w) ring slots 0 .. w-1
  const int lo = split * a.chunk, hi = min(lo + a.chunk, m + w);
  const int per = hi > lo ? (hi - lo + W - 1) / W : 0;
  const int wlo = lo + wave * per, whi = min(wlo + per, hi);
  const int grp = lane / G::LPR, c = lane % G::LPR;

  float q[G::E];
  load_q<DT, D>(a.q, unit, c, a.qscale, q);
  State<G::E> st;
  st.init();
  const size_t cb = (size_t)c * 16;
  if (wlo < min(whi, m)) {
    const size_t base = ((size_t)unit * a.prefix_cap + wlo) * G::ROWB + cb;
    attend_range<DT, D>(static_cast<const char*>(a.k_prefix) + base,
                        static_cast<const char*>(a.v_prefix) + base, min(whi, m) - wlo, 0.f, q, st, grp);
  }
  const int w0 = max(wlo, m) - m, w1 = whi - m;
  if (w0 < w1) {
    const size_t base = ((size_t)unit * a.window + w0) * G::ROWB + cb;
    attend_range<DT, D>(static_cast<const char*>(a.k_ring) + base,
                        static_cast<const char*>(a.v_ring) + base, w1 - w0, 0.f, q, st, grp);
  }
  if (W == 4)
    wg_finish<DT, D, 4>(st, lds_ml, lds_o, a, unit, split);
  else
    wg_finish<DT, D>(st, lds_ml, lds_o, a, unit, split);
}

// Merge of the splits of every unit: one wave per unit.  Lane s holds the
// (max, sum) of split s, so the maximum, the weights and the total sum come
// from wave reductions; each lane then sums the partial outputs of its D/64
// dimensions, with the loads of 8 splits in flight at a time.
template <int DT, int D>
__global__ __launch_bounds__(256) void k_split_merge(DecodeArgs a) {
  using G = Geo<DT, D>;
  constexpr int DPL = D / 64;
  const int lane = threadIdx.x & 63;
  const int unit = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (unit >= a.units) return;
  const int S = a.splits;
  const float2* ml = reinterpret_cast<const float2*>(a.part_ml) + (size_t)unit * S;
  const float* po = a.part_o + (size_t)unit * S * D + lane * DPL;
  float M = kFloor;
  for (int s0 = 0; s0 < S; s0 += 64) {
    const float2 v = s0 + lane < S ? ml[s0 + lane] : make_float2(kFloor, 0.f);
    M = fmaxf(M, wave_max(v.y > 0.f ? v.x : kFloor));
  }
  float L = 0.f, O[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) O[i] = 0.f;
  for (int s0 = 0; s0 < S; s0 += 64) {
    const float2 v = s0 + lane < S ? ml[s0 + lane] : make_float2(kFloor, 0.f);
    const float wgt = v.y > 0.f ? fexp2(v.x - M) : 0.f;
    L += wave_sum_f(wgt * v.y);
    const int n = min(64, S - s0);
    for (int k0 = 0; k0 < n; k0 += 8) {
      float x[8][DPL];
#pragma unroll
      for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int i = 0; i < DPL; ++i) x[k][i] = k0 + k < n ? po[(size_t)(s0 + k0 + k) * D + i] : 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float f = readlane_f(wgt, min(k0 + k, 63));
#pragma unroll
        for (int i = 0; i < DPL; ++i) O[i] = fmaf(f, x[k][i], O[i]);
      }
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  char* dst = static_cast<char*>(a.out) + (size_t)unit * G::ROWB;
  if constexpr (DT == 0) {
    float* d = reinterpret_cast<float*>(dst) + lane * DPL;
#pragma unroll
    for (int i = 0; i < DPL; ++i) d[i] = O[i] * inv;
  } else {
    uint16_t* d = reinterpret_cast<uint16_t*>(dst) + lane * DPL;
#pragma unroll
    for (int i = 0; i < DPL; ++i) d[i] = (uint16_t)bf16_bits(O[i] * inv);
  }
}

// ---------------------------------------------------------------------------
// uocr_srswa_decode: `splits` workgroups per unit.  With one, the waves are
// shared between the window and the live selected blocks in proportion to
// their rows; with several, the window's 32-row chunks and the live blocks
// form one task list, cut finer when there are fewer tasks than waves in
// all, and task i goes to wave i mod (splits x W) of the unit; each
// workgroup leaves its partial state for k_split_merge.
// ---------------------------------------------------------------------------
template <int DT, int D>
__global__ __launch_bounds__(512, 4) void k_srswa_decode(DecodeArgs a) {
  using G = Geo<DT, D>;
  __shared__ float lds_ml[kMaxWaves][2];
  __shared__ __attribute__((aligned(16))) float lds_o[kMaxWaves * D];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, W = blockDim.x >> 6;
  const int unit = blockIdx.x / a.splits, split = blockIdx.x - unit * a.splits;
  const int b = unit / a.heads;
  const int m = min(max(a.prefix_len[b], 0), a.prefix_cap);
  const int w = min(max(a.t_gen[b], 0), a.window);
  const int nb = (m + kBlock - 1) / kBlock;

  // Selection entries of this unit, one per lane; a block is live when its
  // index is in range and its weight is non-zero (bias > -inf).
  int idx = -1;
  float bias = 0.f;
  bool live = false;
  if (lane < a.topk) {
    idx = a.sel_idx[(size_t)unit * a.topk + lane];
    bias = a.sel_bias ? a.sel_bias[(size_t)unit * a.topk + lane] : 0.f;
    live = idx >= 0 && idx < nb && bias > -INFINITY;
  }
  const uint64_t mask = __ballot(live);
  const int n_live = __popcll(mask);
  const int grp = lane / G::LPR, c = lane % G::LPR;

  float q[G::E];
  load_q<DT, D>(a.q, unit, c, a.qscale, q);
  State<G::E> st;
  st.init();
  const size_t cb = (size_t)c * 16;
  // rows [r0, r0 + nr) of live entry tk (counted among the live entries)
  auto live_rows = [&](int tk, int r0, int nr) {
    uint64_t mm = mask;
    for (int i = 0; i < tk; ++i) mm &= mm - 1;  // drop the tk lowest live entries
    const int slot = __ffsll((unsigned long long)mm) - 1;
    const int j = __shfl(idx, slot);
    const float bj = __shfl(bias, slot);
    const int row0 = j * kBlock + r0;
    const int n = min(nr, m - row0);
    if (n <= 0) return;
    const size_t base = ((size_t)unit * a.prefix_cap + row0) * G::ROWB + cb;
    attend_fit<DT, D>(static_cast<const char*>(a.k_prefix) + base, static_cast<const char*>(a.v_prefix) + base, n,
                      bj * kLog2e, q, st, grp);
  };
  auto window_rows = [&](int r0, int nr) {
    const int n = min(nr, w - r0);
    if (n <= 0) return;
    const size_t base = ((size_t)unit * a.window + r0) * G::ROWB + cb;
    attend_fit<DT, D>(static_cast<const char*>(a.k_ring) + base, static_cast<const char*>(a.v_ring) + base, n, 0.f,
                      q, st, grp);
  };
  if (a.splits == 1) {
    // The waves are shared between the window and the live blocks in
    // proportion to their rows, so that (up to 4 live blocks with 8 waves)
    // every wave has all of its rows in flight at once: one HBM round trip.
    const int R = w + kBlock * n_live;
    int ww = R > 0 ? (W * w + R - 1) / R : 0;  // waves on the window
    if (w > 0) ww = max(1, min(ww, n_live > 0 ? W - 1 : W));
    const int wl = max(W - ww, 1);             // waves on the live blocks (wave 0 too when W = 1)
    const int l0 = W - wl;                     // first of them
    if (wave < ww) {
      const int WR = (w + ww - 1) / ww;
      window_rows(wave * WR, WR);
    }
    if (wave >= l0 && n_live > 0) {
      // each live block cut into cpb chunks of 32 / cpb rows
      int cpb = 1;
      while (2 * cpb * n_live <= wl && 2 * cpb * G::RPL <= kBlock) cpb *= 2;
      const int rpc = kBlock / cpb;
      for (int task = wave - l0; task < n_live * cpb; task += wl) {
        const int tk = task / cpb, sub = task - tk * cpb;
        live_rows(tk, sub * rpc, rpc);
      }
    }
  } else {
    // one task list over the unit's workgroups: the window's 32-row chunks,
    // then the live blocks, each cut into cpt pieces of 32 / cpt rows
    const int V = a.splits * W, g = split * W + wave;
    const int wc = (w + kBlock - 1) / kBlock;
    int cpt = 1;
    while (2 * cpt * (wc + n_live) <= V && 2 * cpt * G::RPL <= kBlock) cpt *= 2;
    const int rpt = kBlock / cpt;
    for (int task = g; task < (wc + n_live) * cpt; task += V) {
      const int tk = task / cpt, sub = task - tk * cpt;
      if (tk < wc) window_rows(tk * kBlock + sub * rpt, rpt);
      else live_rows(tk - wc, sub * rpt, rpt);
    }
  }
  if (W == 8)
    wg_finish<DT, D, 8>(st, lds_ml, lds_o, a, unit, split);
  else
    wg_finish<DT, D>(st, lds_ml, lds_o, a, unit, split);
}

// ---------------------------------------------------------------------------
// Reduce-scatter over aligned groups of N lanes (N = 8, 16 or 32), each lane
// holding N/2 doubles v[0 .. N/2): afterwards v[0] of every lane is the group
// total of element rs_elem<N>(lane), and the two lanes of an even/odd pair
// hold the same element.  Each halving step pairs a lane with one whose step
// bit differs, keeps the half its bit names and adds the partner's copy of it:
// the row swap (N = 32) needs no select, the DPP mirrors and the quad xor do.
// ---------------------------------------------------------------------------
template <int N>
__device__ __forceinline__ int rs_elem(int lane) {
  int e = 0;
  if constexpr (N == 32) e = ((lane >> 4) & 1) * 8;
  if constexpr (N >= 16) e += ((lane & 15) >= 8) * 4;
  e += ((lane & 7) >= 4) * 2;
  e += (lane & 3) >= 2;
  return e;
}

template <int CTRL, int H>
__device__ __forceinline__ void rs_dpp_step(double (&v)[H * 2], bool bit) {
#pragma unroll
  for (int k = 0; k < H; ++k) {
    const double keep = bit ? v[k + H] : v[k], send = bit ? v[k] : v[k + H];
    v[k] = keep + dpp<CTRL>(send);
  }
}

template <int N>
__device__ __forceinline__ void reduce_scatter(double (&v)[N / 2], int lane) {
  constexpr int K = N / 2;
  if constexpr (N == 32) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const long long ua = __double_as_longlong(v[k]), ub = __double_as_longlong(v[k + 8]);
      const auto l = __builtin_amdgcn_permlane16_swap((unsigned)(ua & 0xffffffffll), (unsigned)(ub & 0xffffffffll),
                                                      false, false);
      const auto h = __builtin_amdgcn_permlane16_swap((unsigned)(ua >> 32), (unsigned)(ub >> 32), false, false);
      v[k] = join(l[0], h[0]) + join(l[1], h[1]);
    }
  }
  if constexpr (N >= 16) rs_dpp_step<kDppMirror, 4>(*reinterpret_cast<double(*)[8]>(&v[0]), (lane & 15) >= 8);
  rs_dpp_step<kDppHalfMirror, 2>(*reinterpret_cast<double(*)[4]>(&v[0]), (lane & 7) >= 4);
  rs_dpp_step<kDppXor2, 1>(*reinterpret_cast<double(*)[2]>(&v[0]), (lane & 3) >= 2);
  v[0] += dpp<kDppXor1>(v[0]);
  (void)K;
}

// ---------------------------------------------------------------------------
// uocr_block_index_build / _range: each wave owns a contiguous run of
// (unit, block in [first_block, first_block + n_blocks)) items and streams
// it, loading the next block's rows while it reduces the current one; fp64
// accumulation, in an order that does not depend on the range, so a rebuilt
// block is bit-identical to its full-build value.  Per block: the row sums of every lane's
// dimensions (exchanged between the row groups of the wave), then the
// projection with P held transposed in LDS (Pt[i][d], rows padded by 4 floats
// so the 16-byte reads and the transposing stores spread over the banks):
// row group g owns outputs g, g + RPL, ... and its lanes split the
// dimensions, reduced with one reduce-scatter.
// ---------------------------------------------------------------------------
template <int DT, int D>
__global__ __launch_bounds__(256) void k_block_index(IndexArgs a) {
  using G = Geo<DT, D>;
  constexpr int E = G::E;
  constexpr int PD = D + 4;                      // padded row of Pt
  constexpr int NR = kBlock / G::RPL;            // row loads per lane for a full block
  constexpr int K = kIdxDim / G::RPL;            // outputs per row group (= LPR / 2)
  static_assert(K * 2 == G::LPR, "one reduce-scatter element per lane pair");
  __shared__ __attribute__((aligned(16))) float Pt[kIdxDim * PD];
  for (int t = threadIdx.x; t < D * kIdxDim; t += blockDim.x) {  // coalesced read of P[d][i]
    const int d = t / kIdxDim, i = t - d * kIdxDim;
    Pt[i * PD + d] = a.proj[t];
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int grp = lane / G::LPR, c = lane % G::LPR;
  const long long total = (long long)a.units * a.n_blocks;  // items (unit, block in range)
  const long long nw = (long long)gridDim.x * kWaves;
  const long long per = (total + nw - 1) / nw;
  const long long beg = ((long long)blockIdx.x * kWaves + (threadIdx.x >> 6)) * per;
  const long long end = min(total, beg + per);
  if (beg >= end) return;  // no barrier follows

  auto limit = [&](int unit) { return min(max(a.prefix_len[unit / a.heads], 0), a.prefix_cap); };
  auto load = [&](uint4 (&kv)[NR], int unit, int j, int nr) {
    const char* K0 = static_cast<const char*>(a.k_prefix) +
                     ((size_t)unit * a.prefix_cap + (size_t)j * kBlock) * G::ROWB + c * 16;
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      const int r = grp + u * G::RPL;
      kv[u] = r < nr ? ld16_stream(K0 + (size_t)r * G::ROWB) : make_uint4(0u, 0u, 0u, 0u);
    }
  };

  const int jend = a.first_block + a.n_blocks;
  int unit = (int)(beg / a.n_blocks), j = a.first_block + (int)(beg - (long long)unit * a.n_blocks);
  int m = limit(unit);
  int nr = min(kBlock, m - j * kBlock);  // rows of the block inside the prefix (<= 0: none)
  uint4 kv[NR];
  load(kv, unit, j, nr);
  for (long long item = beg; item < end; ++item) {
    int nunit = unit, nj = j + 1, nm = m;
    if (nj == jend) {
      ++nunit;
      nj = a.first_block;
      nm = item + 1 < end ? limit(nunit) : 0;
    }
    const int nnr = item + 1 < end ? min(kBlock, nm - nj * kBlock) : 0;
    uint4 kn[NR];
    load(kn, nunit, nj, nnr);

    float* dst = a.kbar + ((size_t)unit * a.nb_cap + j) * kIdxDim;
    if (nr <= 0) {
      if (lane < kIdxDim) dst[lane] = 0.f;
    } else {
      double sum[E];
#pragma unroll
      for (int e = 0; e < E; ++e) sum[e] = 0.0;
#pragma unroll
      for (int u = 0; u < NR; ++u) {
        float x[E];
        unpack(kv[u], x);
#pragma unroll
        for (int e = 0; e < E; ++e) sum[e] += (double)x[e];
      }
      // totals over the row groups: every lane ends with the block sums of
      // dimensions c*E .. c*E+E-1
      const double inv = 1.0 / (double)nr;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if constexpr (G::LPR < 16) sum[e] += __shfl_xor(sum[e], 8);
        if constexpr (G::LPR < 32) sum[e] = sum16(sum[e]);
        sum[e] = sum32(sum[e]) * inv;
      }
      double acc[K];
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const float4* pr = reinterpret_cast<const float4*>(Pt + (grp + k * G::RPL) * PD + c * E);
        double t = 0.0;
#pragma unroll
        for (int e4 = 0; e4 < E / 4; ++e4) {
          const float4 p4 = pr[e4];
          t += (double)p4.x * sum[4 * e4] + (double)p4.y * sum[4 * e4 + 1] + (double)p4.z * sum[4 * e4 + 2] +
               (double)p4.w * sum[4 * e4 + 3];
        }
        acc[k] = t;
      }
      reduce_scatter<G::LPR>(acc, lane);
      if ((lane & 1) == 0) dst[grp + G::RPL * rs_elem<G::LPR>(lane)] = (float)acc[0];
    }
#pragma unroll
    for (int u = 0; u < NR; ++u) kv[u] = kn[u];
    unit = nunit;
    j = nj;
    m = nm;
    nr = nnr;
  }
}

// ---------------------------------------------------------------------------
// uocr_block_score: `parts` workgroups per unit; fp64 accumulation
// ---------------------------------------------------------------------------
template <int DT, int D>
__global__ __launch_bounds__(256) void k_block_score(ScoreArgs a) {
  using G = Geo<DT, D>;
  __shared__ double red[8][kIdxDim];
  __shared__ double qidx[kIdxDim];
  const int unit = blockIdx.x / a.parts, part = blockIdx.x - unit * a.parts;
  const int tid = threadIdx.x;
  {
    // q_idx = P^T q: thread (i = tid % 32, slice = tid / 32) sums D/8 dims
    const int i = tid % kIdxDim, sl = tid / kIdxDim;
    const char* qrow = static_cast<const char*>(a.q) + (size_t)unit * G::ROWB;
    double acc = 0.0;
    for (int d = sl * (D / 8); d < (sl + 1) * (D / 8); ++d) {
      float qd;
      if constexpr (DT == 0)
        qd = reinterpret_cast<const float*>(qrow)[d];
      else
        qd = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(qrow)[d] << 16);
      acc += (double)a.proj[d * kIdxDim + i] * (double)qd;
    }
    red[sl][i] = acc;
  }
  __syncthreads();
  if (tid < kIdxDim) {
    double s = 0.0;
#pragma unroll
    for (int k = 0; k < 8; ++k) s += red[k][tid];
    qidx[tid] = s;
  }
  __syncthreads();
  const int b = unit / a.heads;
  const int m = min(max(a.prefix_len[b], 0), a.prefix_cap);
  const int nb = (m + kBlock - 1) / kBlock;
  const int per = (a.nb_cap + a.parts - 1) / a.parts;
  const int j0 = part * per, j1 = min(j0 + per, a.nb_cap);
  // 8 lanes per block row (32 fp32 = 128 B), 32 rows per workgroup pass
  const int r = tid / 8, c = tid % 8;
  double qv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) qv[e] = qidx[c * 4 + e];
  const float* K = a.kbar + (size_t)unit * a.nb_cap * kIdxDim + c * 4;
  float* out = a.scores + (size_t)unit * a.nb_cap;
  constexpr int UNR = 4;
  for (int jb = j0; jb < j1; jb += 32 * UNR) {
    float4 kv[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int j = jb + u * 32 + r;
      kv[u] = (j < j1 && j < nb) ? ld16f_stream(K + (size_t)j * kIdxDim) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int j = jb + u * 32 + r;
      double s = qv[0] * (double)kv[u].x + qv[1] * (double)kv[u].y + qv[2] * (double)kv[u].z +
                 qv[3] * (double)kv[u].w;
      s = group_sum<8>(s);
      if (c == 0 && j < j1) out[j] = j < nb ? (float)s : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
// 1.5-entmax + top-k of one unit, computed by the NT threads of a workgroup
// ---------------------------------------------------------------------------
constexpr int kSmallCand = 256;

// Order-preserving map of a float to uint32 (larger float, larger key).
__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kPairMax = 256;  // largest candidate set ranked pairwise
constexpr int kWaveBlocks = 16; // blocks per lane on the one-wave path (nb <= 1024)

// What the one-wave routing (wave_route) uses of a PairBuf: the rank keys of
// the candidate set A (at most 64) and the entmax candidates' scores (at most
// as many).  The prefill kernel gives each wave one of these instead of a
// whole PairBuf, so that more of its workgroups fit in a CU's LDS.
struct alignas(16) WaveBuf {
  uint64_t key[64];
  int rank[64];
};

struct alignas(16) PairBuf {  // pairwise ranking (16-byte aligned rows)
  union {
    float val[kPairMax + 4];
    uint64_t key[(kPairMax + 4) / 2];  // one-wave path: rank_key of each block of A
  };
  int idx[kPairMax + 4];
  int rank[kPairMax + 4];
};

// (score descending, index ascending) as one unsigned key, larger first.
// Adding +0 turns -0 into +0, which the float order takes as equal.
__device__ __forceinline__ uint64_t rank_key(float s, int j) {
  return ((uint64_t)fkey(s + 0.f) << 32) | (uint32_t)~(uint32_t)j;
}
__device__ __forceinline__ float rank_key_score(uint64_t k) {
  const uint32_t u = (uint32_t)(k >> 32);
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

template <int NT>
struct __attribute__((aligned(16))) TopkSmem {
  uint32_t hist[256];
  int sh_i[NT / 64];
  float sh_f[NT / 64];
  double sh_d[NT / 64];
  uint32_t digit, above;
  int flag;  // selection published by the routing wave (0: not yet)
  double tau;
  union alignas(16) {
    double cand[kMaxBlocks];  // sorted path
    PairBuf a;                // pairwise paths
  };
};

// Exclusive scan of one value per thread over the workgroup; returns the
// prefix and sets `total`.
template <int NT, typename T>
__device__ __forceinline__ T block_scan_excl(T x, T& total, T* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  T inc = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const T y = __shfl_up(inc, off);
    if (lane >= off) inc += y;
  }
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  T base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const T v = sh[w];
    if (w < wave) base += v;
    tot += v;
  }
  __syncthreads();
  total = tot;
  return base + inc - x;
}

template <int NT, typename T>
__device__ __forceinline__ T block_max(T x, T* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  x = wave_max(x);
  if (lane == 0) sh[wave] = x;
  __syncthreads();
  T r = sh[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) r = sh[w] > r ? sh[w] : r;
  __syncthreads();
  return r;
}

struct NoOverlap {
  __device__ void operator()() const {}
};

// The routing wave hands its selection to the other waves of the workgroup
// through an LDS flag instead of a workgroup barrier, so that they need not
// wait for one another.  The fences order LDS only: the routing wave's LDS
// writes are complete before lane 0 stores the flag, and a reader that sees
// the flag reads the selection after it.  Global stores are not waited for.
__device__ __forceinline__ void publish_flag(int* flag, int v) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  if ((threadIdx.x & 63) == 0) __hip_atomic_store(flag, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ int wait_flag(int* flag) {
  int v;
  while ((v = __builtin_amdgcn_readfirstlane(
              __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP))) == 0)
    __builtin_amdgcn_s_sleep(1);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  return v;
}

// Sum of a double over the 64 lanes, the same value in every lane.
__device__ __forceinline__ double wave_sum_d(double x) {
  x = group_sum<16>(x);
  return readlane_d(x, 0) + readlane_d(x, 16) + readlane_d(x, 32) + readlane_d(x, 48);
}

// One-wave routing for nb <= 64 * NS blocks (see entmax_topk_block).  Returns
// false, having written nothing, when it cannot finish: more than 64 blocks
// tie around the k-th score, or (unless WIDE) the entmax candidates (d <= 2)
// alone are more than 64.
//
// WIDE: a support too large for per-candidate statistics is handled here too.
// A then only has to hold the top kk, and the threshold comes from Newton's
// method on h(tau) = || max(0, u - tau) ||_2 = 1 (a norm of convex functions
// of tau, so convex, and decreasing: from tau = u_max - 1 the iterates rise
// monotonically to the root; for equal u on a fixed support h is linear in
// tau and one step lands on the root, and near-flat supports take a few),
// followed by the closed form of the sorted algorithm on the support
// S = {u > tau} found,
// accepted only if it satisfies the optimality conditions (u > tau_S on S,
// u <= tau_S off S), which single out the exact support.
template <int NS, bool WIDE = false, typename Buf = PairBuf>
__device__ __forceinline__ bool wave_route(const float* s, int nb, int kk, int32_t* o_idx, float* o_prob,
                                           float* o_bias, int* l_idx, float* l_bias, Buf& pb,
                                           unsigned long long* stamps = nullptr) {
  const int lane = threadIdx.x & 63;
  // the routing is the critical path of the step: let this wave win the
  // issue arbitration against the waves attending over the window
  __builtin_amdgcn_s_setprio(3);
  float sv[NS];
  float lmax = -INFINITY, lmin = INFINITY;
#pragma unroll
  for (int e = 0; e < NS; ++e) {
    const int j = e * 64 + lane;
    sv[e] = j < nb ? s[j] : -INFINITY;
    lmax = fmaxf(lmax, sv[e]);
    if constexpr (WIDE) lmin = j < nb ? fminf(lmin, sv[e]) : lmin;
  }
  const float smax = wave_max(lmax);
  UOCR_STAMP(stamps, stamps && lane == 0, 9);
  // WIDE: the largest gap smax - s of a visible block (the searches below
  // start from it when the support is wide)
  const float dlast = WIDE ? smax + wave_max(-lmin) : 0.f;
  const double dmax = (double)smax;
  float dv[NS];
#pragma unroll
  for (int e = 0; e < NS; ++e) dv[e] = smax - sv[e];  // +inf past nb
  float T = 4.f;
  int nA = 0;
  for (int it = 0; it < 130; ++it) {
    nA = wave_count_below(dv, T);
    if (nA >= kk) break;
    T = T * 2.f;  // reaches +inf, where every finite d counts
  }
  // Too many blocks below T for one wave: search T in (lo, hi) for a count in
  // [kk, 64], given count(d < hi) = chi > 64 and count(d < lo) < kk (except
  // possibly at the first probe, which is lo itself).  Every other probe
  // interpolates the count linearly between the ends, aiming at the middle
  // of [kk, 64]; the others halve the interval, so the search takes at most
  // about twice the probes of a bisection.
  auto narrow = [&](float lo, float hi, int chi) -> bool {
    int clo = -1;
    for (int it = 0; it < 48; ++it) {
      float mid = it == 0 ? lo : 0.5f * (lo + hi);
      if ((it & 1) && clo >= 0) {
        const float g = lo + (hi - lo) * ((float)((kk + 64) / 2 - clo) / (float)(chi - clo));
        if (g > lo && g < hi) mid = g;
      }
      if (it > 0 && !(mid > lo && mid < hi)) return false;
      const int c = wave_count_below(dv, mid);
      if (c >= kk && c <= 64) {
        T = mid;
        nA = c;
        return true;
      }
      if (c > 64) {
        if (it == 0) return false;
        hi = mid;
        chi = c;
      } else {
        lo = mid;
        clo = c;
      }
    }
    return false;
  };
  // T never below the least float above 2 keeps every d <= 2 (every entmax
  // candidate) in A
  bool wide = false;
  if (nA > 64) {
    const float hi = T;
    if (!narrow(fmaxf(0.5f * T, __uint_as_float(0x40000001u)), hi, nA)) {
      if constexpr (WIDE) {
        // a wide support: the search starts just above the largest gap of a
        // visible block, below which all nb visible blocks count
        const float up = nextafterf(dlast, INFINITY);
        const bool tight = up < hi;
        wide = narrow(0.f, tight ? up : hi, tight ? nb : nA);
      }
    }
  }
  UOCR_STAMP(stamps, stamps && lane == 0, 10);
  if (nA <= 64) {
    // Ordered compaction of A by ballots (slot-major order is index order).
    // Two ways, with identical results (A, its rank keys and the candidate
    // list in index order):
    //  - PAIRS (prefill, and the decode step at more than 512 blocks): only
    //    (index, score bits) pairs per slot; afterwards each lane of A forms
    //    its rank key and the entmax candidates (d < 2, all in A) are
    //    compacted from the lanes, a third of the per-slot instructions;
    //  - otherwise keys and candidate scores per slot.  At up to 512 blocks
    //    the window, not the routing, is the longer branch of the step, and
    //    a routing wave that finished sooner started its live blocks while
    //    the window was still streaming: 40 pages got slower.
    constexpr bool PAIRS = WIDE || NS >= 16;
    const int nA4 = (nA + 3) & ~3;
    const bool mine = lane < nA;
    int nC, ii;
    uint64_t ki;
    float si;
    double vi;
    if constexpr (PAIRS) {
      int base = 0;
#pragma unroll
      for (int e = 0; e < NS; ++e) {
        const bool in = dv[e] < T;
        const uint64_t m = __ballot(in);
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (in) pb.key[base + below] = ((uint64_t)(uint32_t)(e * 64 + lane) << 32) | __float_as_uint(sv[e]);
        base += __popcll(m);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const uint64_t pr = mine ? pb.key[lane] : 0;
      ii = (int)(uint32_t)(pr >> 32);
      const float sraw = __uint_as_float((uint32_t)pr);
      ki = mine ? rank_key(sraw, ii) : 0;
      si = mine ? rank_key_score(ki) : -INFINITY;
      vi = ((double)si - dmax) * 0.5;
      // each lane's rank key (0 past nA: below every block's key), and the
      // candidates' scores in A's order, padded as below
      const bool cd = !wide && mine && vi > -1.0;
      const uint64_t mc = __ballot(cd);
      nC = __popcll(mc);
      const int nC4 = (nC + 3) & ~3;
      if (lane < nA4) pb.key[lane] = ki;
      if (cd)
        pb.rank[__builtin_amdgcn_mbcnt_hi((uint32_t)(mc >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mc, 0u))] =
            __float_as_int(sraw);
      if (lane >= nC && lane < nC4) pb.rank[lane] = __float_as_int(-INFINITY);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    } else {
      int base = 0, cbase = 0;
#pragma unroll
      for (int e = 0; e < NS; ++e) {
        const bool in = dv[e] < T;
        const bool cd = !wide && ((double)sv[e] - dmax) * 0.5 > -1.0;
        const uint64_t m = __ballot(in);
        const uint64_t mc = __ballot(cd);
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        const int cbelow = __builtin_amdgcn_mbcnt_hi((uint32_t)(mc >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mc, 0u));
        if (in) pb.key[base + below] = rank_key(sv[e], e * 64 + lane);
        if (cd) pb.rank[cbase + cbelow] = __float_as_int(sv[e]);  // candidate scores
        base += __popcll(m);
        cbase += __popcll(mc);
      }
      nC = cbase;
      const int nC4 = (nC + 3) & ~3;
      if (lane < nA4 - nA) pb.key[nA + lane] = 0;  // below every block's key
      if (lane < nC4 - nC) pb.rank[nC + lane] = __float_as_int(-INFINITY);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      ki = mine ? pb.key[lane] : 0;
      si = mine ? rank_key_score(ki) : -INFINITY;
      ii = (int)~(uint32_t)ki;
      vi = ((double)si - dmax) * 0.5;
    }
    const int nC4 = (nC + 3) & ~3;
    UOCR_STAMP(stamps, stamps && lane == 0, 11);
    const ulonglong2* key2 = reinterpret_cast<const ulonglong2*>(pb.key);
    int rank = 0;  // blocks of A ahead of this lane's in (score desc, index asc)
    auto rank4 = [&](int k4) {
      const ulonglong2 a0 = key2[2 * k4], a1 = key2[2 * k4 + 1];
      rank += (a0.x > ki) + (a0.y > ki) + (a1.x > ki) + (a1.y > ki);
    };
    if constexpr (WIDE) {  // throughput use (prefill): fewer registers
#pragma unroll 1
      for (int k4 = 0; k4 < nA4 / 4; ++k4) rank4(k4);
    } else {               // the decode step's latency path
#pragma unroll 2
      for (int k4 = 0; k4 < nA4 / 4; ++k4) rank4(k4);
    }
    UOCR_STAMP(stamps, stamps && lane == 0, 12);
    double tau;
    if (!wide) {
      const bool cand = mine && vi > -1.0;
      const float4* cv4 = reinterpret_cast<const float4*>(pb.rank);
      int r = 0;
      double s1 = 0.0, s2 = 0.0;
      for (int k4 = 0; k4 < nC4 / 4; ++k4) {
        const float4 c4 = cv4[k4];
        const float ck[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {  // branch-free: a zero adds nothing
          const bool ge = ck[k] >= si;
          const double vk = ge ? ((double)ck[k] - dmax) * 0.5 : 0.0;
          r += ge;
          s1 += vk;
          s2 = fma(vk, vk, s2);
        }
      }
      int rr = 0;
      double tl = 0.0;
      if (cand) {
        const double mu = s1 / r;
        const double ss = s2 - s1 * mu;
        tl = mu - sqrt(fmax(0.0, (1.0 - ss) / r));
        rr = tl <= vi ? r : 0;
      }
      const int rstar = wave_max(rr);
      const uint64_t win = __ballot(rr == rstar && rr > 0);
      tau = readlane_d(tl, __ffsll((unsigned long long)win) - 1);
    } else {
      // u' = (s - smax) / 2 in [-inf, 0]; the root lies in [-1, 0)
      // u'_e, formed where it is used (the same value every time) rather than
      // held: 2 NS registers fewer
      auto up = [&](int e) { return ((double)sv[e] - dmax) * 0.5; };
      double t = -1.0;
      for (int it = 0; it < 64; ++it) {
        double F = 0.0, G = 0.0;
#pragma unroll
        for (int e = 0; e < NS; ++e) {
          const double x = fmax(up(e) - t, 0.0);
          F = fma(x, x, F);
          G += x;
        }
        F = wave_sum_d(F);  // h = sqrt(F), -h' = G / sqrt(F)
        G = wave_sum_d(G);
        const double step = (F - sqrt(F)) / G;
        if (!(step > 0.0) || t + step == t) break;
        t += step;
      }
      int r = 0;
      double s1 = 0.0;
#pragma unroll
      for (int e = 0; e < NS; ++e)
        if (up(e) > t) {
          ++r;
          s1 += up(e);
        }
      r = wave_sum(r);
      const double mu = wave_sum_d(s1) / r;
      double ss = 0.0;
#pragma unroll
      for (int e = 0; e < NS; ++e)
        if (up(e) > t) ss += (up(e) - mu) * (up(e) - mu);
      ss = wave_sum_d(ss);
      tau = mu - sqrt(fmax(0.0, (1.0 - ss) / r));
      bool bad = false;
#pragma unroll
      for (int e = 0; e < NS; ++e) bad |= (up(e) > t) ? !(up(e) > tau) : (up(e) > tau);
      if (__ballot(bad) != 0) {
        __builtin_amdgcn_s_setprio(0);
        return false;
      }
    }
    UOCR_STAMP(stamps, stamps && lane == 0, 13);
    const bool sel = mine && rank < kk;
    const uint64_t sm_ = __ballot(sel);
    if (sel) {
      const int at = __builtin_amdgcn_mbcnt_hi((uint32_t)(sm_ >> 32),
                                               __builtin_amdgcn_mbcnt_lo((uint32_t)sm_, 0u));
      const double dd = vi - tau;
      const float p = dd > 0.0 ? (float)(dd * dd) : 0.f;
      const float bias = p > 0.f ? logf(p) : -INFINITY;
      o_idx[at] = ii;
      if (o_prob) o_prob[at] = p;
      o_bias[at] = bias;
      if (l_idx) {
        l_idx[at] = ii;
        l_bias[at] = bias;
      }
    }
  }
  __builtin_amdgcn_s_setprio(0);
  return nA <= 64;
}

// Routing of one unit from its nb scores `s` (global or LDS).  Writes topk
// entries of o_idx / o_prob (may be null) / o_bias and, when l_idx is not
// null, the same indices and biases to l_idx / l_bias.  Every thread of the
// workgroup must call it.  `others` runs exactly once on every wave but wave
// 0, while wave 0 works alone on the usual (one-wave) path: it lets a caller
// overlap independent work with the routing.
//
// Returns true when l_idx / l_bias become visible to the whole workgroup only
// after a workgroup barrier, which the caller then runs.  With EARLY, the
// one-wave path and the empty case return false instead: wave 0 publishes the
// selection through sm.flag (which the caller zeroes before a barrier that
// precedes this call), and every wave waits for that flag (wait_flag) rather
// than for the other waves.  All of l_idx / l_bias is then written by wave 0
// (topk <= 64).
template <int NT, typename F = NoOverlap, bool EARLY = false>
__device__ __forceinline__ bool entmax_topk_block(const float* s, int nb, int topk, int32_t* o_idx, float* o_prob,
                                  float* o_bias, int* l_idx, float* l_bias, TopkSmem<NT>& sm,
                                  const F& others = F(), unsigned long long* stamps = nullptr) {
  constexpr int PT = kMaxBlocks / NT;  // values per thread
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kk = min(topk, nb);
  for (int i = kk + tid; i < topk; i += NT) {
    o_idx[i] = -1;
    if (o_prob) o_prob[i] = 0.f;
    o_bias[i] = -INFINITY;
    if (l_idx) {
      l_idx[i] = -1;
      l_bias[i] = -INFINITY;
    }
  }
  if (kk == 0) {
    if (wave != 0) others();
    else if (EARLY) publish_flag(&sm.flag, 1);
    return !EARLY;
  }

  // ---- one-wave path (nb <= 1024 and a candidate set of <= 64 blocks) ----
  // Wave 0 alone: no workgroup barrier until the end.  Lane l owns blocks
  // l, l + 64, l + 128, ... (slot e holds block l + 64 e), so index order is
  // (slot, lane) order and an ordered compaction needs only ballots.  With
  // d = smax - s in fp32 (monotone in s), the set A = {d < T}, T = 4, 8, 16,
  // ... until it holds kk blocks (then bisected, never below the least float
  // above 2, while it holds more than 64), contains the top kk (ties of the
  // kk-th included) and the entmax support (exact d < 2 gives fp32 d <= 2).  A
  // is compacted in index order into LDS; each lane takes one block of A and
  // counts, over broadcast LDS reads of A, the blocks ranked before it and
  // (for an entmax candidate) the prefix statistics of the sorted order at the
  // end of its tie group.
  if (nb > 64 * kWaveBlocks && wave != 0) others();
  if (nb <= 64 * kWaveBlocks) {
    if (wave != 0) others();
    bool ok = false;
    if (wave == 0) {
      if (nb <= 64) ok = wave_route<1>(s, nb, kk, o_idx, o_prob, o_bias, l_idx, l_bias, sm.a, stamps);
      else if (nb <= 128) ok = wave_route<2>(s, nb, kk, o_idx, o_prob, o_bias, l_idx, l_bias, sm.a, stamps);
      else if (nb <= 256) ok = wave_route<4>(s, nb, kk, o_idx, o_prob, o_bias, l_idx, l_bias, sm.a, stamps);
      else if (nb <= 512) ok = wave_route<8>(s, nb, kk, o_idx, o_prob, o_bias, l_idx, l_bias, sm.a, stamps);
      else ok = wave_route<16>(s, nb, kk, o_idx, o_prob, o_bias, l_idx, l_bias, sm.a, stamps);
    }
    if constexpr (EARLY) {
      // 1: selection published; 2: the workgroup path below takes over
      if (wave == 0) publish_flag(&sm.flag, ok ? 1 : 2);
      if (wait_flag(&sm.flag) == 1) return false;
    } else {
      if (wave == 0 && lane == 0) sm.digit = ok ? 1u : 0u;
      __syncthreads();
      const bool done = sm.digit == 1u;
      __syncthreads();
      if (done) return true;
    }
  }

  // Thread t owns the contiguous blocks [t*E, t*E + E): index order equals
  // (thread, position) order, which the ordered compactions below rely on.
  const int E = (nb + NT - 1) / NT;
  const int j0 = tid * E;
  static_assert(PT <= 32, "per-thread flags are 32-bit masks");
  float v[PT];  // -inf marks a slot past nb; fkey(v) is recomputed when needed
  uint32_t valid = 0u;
  float lmax = -INFINITY;
#pragma unroll
  for (int e = 0; e < PT; ++e) {
    const int j = j0 + e;
    const bool ok = e < E && j < nb;
    v[e] = ok ? s[j] : -INFINITY;
    valid |= ok ? (1u << e) : 0u;
    lmax = fmaxf(lmax, v[e]);
  }
  const float smax = block_max<NT, float>(lmax, sm.sh_f);
  const double dmax = (double)smax;

  // ---- usual case: a small set A holding the top kk and the entmax support ----
  // Histogram of the binary exponent of d = smax - s (monotone in the
  // ranking): A = every block whose exponent is at most that of the kk-th
  // smallest d, and at least that of [2, 4), which holds every d < 2 (the
  // entmax support) even after fp32 rounding.  Ties of the kk-th score share
  // its exponent, so A holds them too.
  for (int i = tid; i < 256; i += NT) sm.hist[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < PT; ++e)
    if ((valid >> e) & 1u) atomicAdd(&sm.hist[(__float_as_uint(smax - v[e]) >> 23) & 255u], 1u);
  __syncthreads();
  if (wave == 0) {
    const uint32_t c0 = sm.hist[4 * lane], c1 = sm.hist[4 * lane + 1], c2 = sm.hist[4 * lane + 2],
                   c3 = sm.hist[4 * lane + 3];
    const uint32_t local = c0 + c1 + c2 + c3;
    uint32_t inc = local;  // inclusive count over lanes <= lane (bins 0 .. 4*lane+3)
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t y = __shfl_up(inc, off);
      if (lane >= off) inc += y;
    }
    const uint32_t before = inc - local;
    const uint32_t cnt[4] = {c0, c1, c2, c3};
    // smallest bin whose cumulative count reaches kk
    int estar = 0;
    uint32_t cum = before;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bool first = cum < (uint32_t)kk && cum + cnt[k] >= (uint32_t)kk;
      estar = first ? 4 * lane + k : estar;
      cum += cnt[k];
    }
    const uint64_t who = __ballot(before < (uint32_t)kk && inc >= (uint32_t)kk);
    estar = __shfl(estar, __ffsll((unsigned long long)who) - 1);
    const int efin = estar > 128 ? estar : 128;
    // |A| = cumulative count through bin efin
    uint32_t upto = before;
#pragma unroll
    for (int k = 0; k < 4; ++k) upto += (4 * lane + k <= efin) ? cnt[k] : 0u;
    upto = __shfl(upto, efin / 4);
    if (lane == 0) {
      sm.digit = (uint32_t)efin;
      sm.above = upto;
    }
  }
  __syncthreads();
  const uint32_t efin = sm.digit;
  const int nA = (int)sm.above;
  __syncthreads();
  if (nA <= kPairMax) {
    uint32_t inA = 0u;
#pragma unroll
    for (int e = 0; e < PT; ++e)
      inA |= (((valid >> e) & 1u) && ((__float_as_uint(smax - v[e]) >> 23) & 255u) <= efin) ? (1u << e) : 0u;
    int tot;
    int pos = block_scan_excl<NT, int>(__popc(inA), tot, sm.sh_i);
#pragma unroll
    for (int e = 0; e < PT; ++e)
      if ((inA >> e) & 1u) {
        sm.a.val[pos] = v[e];
        sm.a.idx[pos] = j0 + e;
        ++pos;
      }
    // pad to a multiple of 4 with entries that rank below every block
    const int nA4 = (nA + 3) & ~3;
    if (tid < nA4 - nA) {
      sm.a.val[nA + tid] = -INFINITY;
      sm.a.idx[nA + tid] = 0x7fffffff;
      sm.a.rank[nA + tid] = 0x7fffffff;
    }
    __syncthreads();
    const float4* val4 = reinterpret_cast<const float4*>(sm.a.val);
    const int4* idx4 = reinterpret_cast<const int4*>(sm.a.idx);
    // rank in (score desc, index asc) and, for entmax candidates, the
    // prefix statistics of the sorted order at the end of the tie group
    int rbest = 0;
    double tbest = 0.0;
    for (int i = tid; i < nA; i += NT) {
      const float si = sm.a.val[i];
      const int ii = sm.a.idx[i];
      const double vi = ((double)si - dmax) * 0.5;
      const bool cand = vi > -1.0;
      int rank = 0, r = 0;
      double s1 = 0.0, s2 = 0.0;
#pragma unroll 4
      for (int j4 = 0; j4 < nA4 / 4; ++j4) {
        const float4 sv = val4[j4];
        const int4 iv = idx4[j4];
        const float sj[4] = {sv.x, sv.y, sv.z, sv.w};
        const int ij[4] = {iv.x, iv.y, iv.z, iv.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          rank += (sj[k] > si || (sj[k] == si && ij[k] < ii)) ? 1 : 0;
          if (cand && sj[k] >= si) {
            const double vj = ((double)sj[k] - dmax) * 0.5;
            ++r;
            s1 += vj;
            s2 += vj * vj;
          }
        }
      }
      sm.a.rank[i] = rank;
      if (cand) {
        const double mu = s1 / r;
        const double ss = s2 - s1 * mu;
        const double tau = mu - sqrt(fmax(0.0, (1.0 - ss) / r));
        if (tau <= vi && r > rbest) {
          rbest = r;
          tbest = tau;
        }
      }
    }
    const int rstar = block_max<NT, int>(rbest, sm.sh_i);
    if (rbest == rstar && rbest > 0) sm.tau = tbest;
    __syncthreads();
    const double tau = sm.tau;
    for (int i = tid; i < nA; i += NT) {
      if (sm.a.rank[i] >= kk) continue;
      const int ii = sm.a.idx[i];
      int at = 0;  // output position: selected blocks with a lower index
      const int4* rank4 = reinterpret_cast<const int4*>(sm.a.rank);
#pragma unroll 4
      for (int j4 = 0; j4 < nA4 / 4; ++j4) {
        const int4 rv = rank4[j4];
        const int4 iv = idx4[j4];
        at += (rv.x < kk && iv.x < ii) + (rv.y < kk && iv.y < ii) + (rv.z < kk && iv.z < ii) +
              (rv.w < kk && iv.w < ii);
      }
      const double dd = ((double)sm.a.val[i] - dmax) * 0.5 - tau;
      const double p = dd > 0.0 ? dd * dd : 0.0;
      const float bias = p > 0.0 ? (float)log(p) : -INFINITY;
      o_idx[at] = ii;
      if (o_prob) o_prob[at] = (float)p;
      o_bias[at] = bias;
      if (l_idx) {
        l_idx[at] = ii;
        l_bias[at] = bias;
      }
    }
    return true;
  }

  // ---- general case: radix select of the kk-th key, sorted entmax ----
  uint32_t prefix = 0u, pmask = 0u;
  int rem = kk;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += NT) sm.hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < PT; ++e) {
      const uint32_t key = fkey(v[e]);
      if (((valid >> e) & 1u) && (key & pmask) == prefix) atomicAdd(&sm.hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      const uint32_t c0 = sm.hist[4 * lane], c1 = sm.hist[4 * lane + 1], c2 = sm.hist[4 * lane + 2],
                     c3 = sm.hist[4 * lane + 3];
      const uint32_t local = c0 + c1 + c2 + c3;
      uint32_t inc = local;  // sum over lanes >= lane
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_down(inc, off);
        if (lane + off < 64) inc += y;
      }
      uint32_t above = inc - local;  // counts strictly above this lane's bins
      const uint32_t cnt[4] = {c0, c1, c2, c3};
#pragma unroll
      for (int k = 3; k >= 0; --k) {
        if (above < (uint32_t)rem && (uint32_t)rem <= above + cnt[k]) {
          sm.digit = (uint32_t)(4 * lane + k);
          sm.above = above;
        }
        above += cnt[k];
      }
    }
    __syncthreads();
    prefix |= sm.digit << shift;
    pmask |= 255u << shift;
    rem -= (int)sm.above;
  }
  // prefix = key of the kk-th ranked block; take every key above it and the
  // `rem` lowest-index blocks whose key equals it.
  int ties = 0;
#pragma unroll
  for (int e = 0; e < PT; ++e) ties += (((valid >> e) & 1u) && fkey(v[e]) == prefix) ? 1 : 0;
  int tie_tot;
  int tie_before = block_scan_excl<NT, int>(ties, tie_tot, sm.sh_i);
  uint32_t sel = 0u;
#pragma unroll
  for (int e = 0; e < PT; ++e) {
    if (!((valid >> e) & 1u)) continue;
    const uint32_t key = fkey(v[e]);
    bool take = key > prefix;
    if (key == prefix) take = tie_before++ < rem;
    sel |= take ? (1u << e) : 0u;
  }
  const int nsel = __popc(sel);

  // ---- 1.5-entmax threshold, fp64 ----
  // With u = s/2 the threshold satisfies tau >= max(u) - 1, so only blocks
  // with s > max(s) - 2 can carry weight.  v = (s - smax)/2 lies in (-1, 0].
  uint32_t cmask = 0u;
#pragma unroll
  for (int e = 0; e < PT; ++e)
    cmask |= (((valid >> e) & 1u) && ((double)v[e] - dmax) * 0.5 > -1.0) ? (1u << e) : 0u;
  int C;
  int cpos = block_scan_excl<NT, int>(__popc(cmask), C, sm.sh_i);
#pragma unroll
  for (int e = 0; e < PT; ++e)
    if ((cmask >> e) & 1u) sm.cand[cpos++] = ((double)v[e] - dmax) * 0.5;
  __syncthreads();

  int rbest = 0;
  double tbest = 0.0;
  if (C <= kSmallCand) {
    // r_i = #{v_j >= v_i}: the last position of v_i's tie group in the
    // descending order; the prefix condition is checked there.
    if (tid < C) {
      const double vi = sm.cand[tid];
      int r = 0;
      double s1 = 0.0, s2 = 0.0;
      for (int j = 0; j < C; ++j) {
        const double vj = sm.cand[j];
        if (vj >= vi) {
          ++r;
          s1 += vj;
          s2 += vj * vj;
        }
      }
      const double mu = s1 / r;
      const double ss = s2 - s1 * mu;
      const double tau = mu - sqrt(fmax(0.0, (1.0 - ss) / r));
      if (tau <= vi) {
        rbest = r;
        tbest = tau;
      }
    }
  } else {
    // Many candidates: bitonic sort (descending) in LDS, then prefix sums.
    int P = 1;
    while (P < C) P <<= 1;
    for (int i = C + tid; i < P; i += NT) sm.cand[i] = -INFINITY;
    __syncthreads();
    for (int size = 2; size <= P; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = tid; i < P / 2; i += NT) {
          const int lo = 2 * stride * (i / stride) + (i % stride), hi = lo + stride;
          const bool desc = (lo & size) == 0;
          const double x = sm.cand[lo], y = sm.cand[hi];
          if ((x < y) == desc) {
            sm.cand[lo] = y;
            sm.cand[hi] = x;
          }
        }
        __syncthreads();
      }
    }
    const int per = (P + NT - 1) / NT;
    const int p0 = tid * per;
    double l1 = 0.0, l2 = 0.0;
    for (int i = 0; i < per && p0 + i < C; ++i) {
      const double x = sm.cand[p0 + i];
      l1 += x;
      l2 += x * x;
    }
    double t1, t2;
    double s1 = block_scan_excl<NT, double>(l1, t1, sm.sh_d);
    double s2 = block_scan_excl<NT, double>(l2, t2, sm.sh_d);
    for (int i = 0; i < per && p0 + i < C; ++i) {
      const double x = sm.cand[p0 + i];
      s1 += x;
      s2 += x * x;
      const int r = p0 + i + 1;
      const double mu = s1 / r;
      const double ss = s2 - s1 * mu;
      const double tau = mu - sqrt(fmax(0.0, (1.0 - ss) / r));
      if (tau <= x) {
        rbest = r;
        tbest = tau;
      }
    }
  }
  const int rstar = block_max<NT, int>(rbest, sm.sh_i);
  if (rbest == rstar && rbest > 0) sm.tau = tbest;  // equal r gives the same tau
  __syncthreads();
  const double tau = sm.tau;

  // ---- outputs in ascending index order ----
  int stot;
  int pos = block_scan_excl<NT, int>(nsel, stot, sm.sh_i);
#pragma unroll
  for (int e = 0; e < PT; ++e) {
    if (!((sel >> e) & 1u)) continue;
    const double d = ((double)v[e] - dmax) * 0.5 - tau;
    const double p = d > 0.0 ? d * d : 0.0;
    const float bias = p > 0.0 ? (float)log(p) : -INFINITY;
    o_idx[pos] = j0 + e;
    if (o_prob) o_prob[pos] = (float)p;
    o_bias[pos] = bias;
    if (l_idx) {
      l_idx[pos] = j0 + e;
      l_bias[pos] = bias;
    }
    ++pos;
  }
  return true;
}

constexpr int kTopkThreads = 256;

__global__ __launch_bounds__(kTopkThreads) void k_entmax_topk(TopkArgs a) {
  __shared__ TopkSmem<kTopkThreads> sm;
  const int unit = blockIdx.x;
  const int b = unit / a.heads;
  const int m = min(max(a.prefix_len[b], 0), a.prefix_cap);
  const int nb = min((m + kBlock - 1) / kBlock, a.nb_cap);
  const size_t o = (size_t)unit * a.topk;
  entmax_topk_block<kTopkThreads>(a.scores + (size_t)unit * a.nb_cap, nb, a.topk, a.sel_idx + o,
                                  a.sel_prob ? a.sel_prob + o : nullptr, a.sel_bias + o, nullptr, nullptr, sm);
}

// ---------------------------------------------------------------------------
// uocr_prefill_route: the routing of a prefill chunk.  A workgroup takes qt
// consecutive queries of one unit:
//   1. q_idx = P^T q of each query on the fp64 matrix cores;
//   2. the scores of every block visible to the tile's last query against the
//      tile's queries, as 16 x 16 fp64 matrix tiles (rounded once, into LDS);
//   3. wave w routes query w on the one-wave path, then claims the next
//      unrouted query of the tile.
// A query that path cannot take (more than 1024 visible blocks, more than 64
// blocks tied around the k-th score, or a wide support whose optimality check
// fails) is marked in sel_idx[0] and routed by k_prefill_fallback,
// which runs next in the same stream with the whole workgroup per query (its
// register needs would halve this kernel's occupancy).  Query i of the chunk
// sits at position q_pos[b] + i and sees the blocks all of whose prefix tokens
// come before it.
// ---------------------------------------------------------------------------
constexpr int kPrefillThreads = 512;
// Two builds of the kernel, by the most blocks a query can see (a compile-time
// bound on the routing's slots per lane, NSMAX): up to 512 blocks with 8 slots
// per lane the routing fits in 80 registers, so three workgroups (six waves
// per SIMD) share a CU, with LDS for 16 queries of 512 blocks; up to 1024
// blocks, 16 slots per lane need 112 registers and the kernel runs two
// workgroups per CU, with 12288 score slots.
constexpr int prefill_slots(int nsmax) { return nsmax >= 16 ? 12288 : 16 * 64 * nsmax; }
constexpr int prefill_nsmax(int nb_cap) { return nb_cap <= 512 ? 8 : 16; }
constexpr int kPrefillTilesInFlight = 1;  // key tiles per wave with loads in flight (2 or 4 measured slower)
constexpr int kPrefillMaxQ = 16;
constexpr int32_t kDeferred = INT32_MIN;

template <int SLOTS>
struct PrefillSmem {
  float scores[SLOTS];
  alignas(16) double qidx[kPrefillMaxQ][kIdxDim];
  WaveBuf pb[kPrefillThreads / 64];  // one per wave
  int next_q;                        // next query to route
};

// Query i of the tile starting at chunk query q0: position and visible blocks.
// Workgroups are dealt to the 8 XCDs in turn (workgroup i to XCD i mod 8),
// and each XCD has its own L2.  The workgroups of one unit all read that
// unit's block keys, so this permutation gives XCD x a contiguous range of
// the logical workgroups, i.e. of the units: each unit's keys then sit in
// one L2 instead of eight.  Any order is correct; this one only keeps reuse
// inside an L2.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_contiguous(int b, int n) {
  const int q = n / kXcds, r = n % kXcds, x = b % kXcds;
  return x * q + min(x, r) + b / kXcds;
}

struct PrefillTile {
  int unit, q0, nq, m, nb_all;
  long long pos0;
  __device__ PrefillTile(const PrefillArgs& a) {
    const int tiles = (a.tq + a.qt - 1) / a.qt;
    const int wg = xcd_contiguous((int)blockIdx.x, (int)gridDim.x);
    unit = wg / tiles;
    q0 = (wg - unit * tiles) * a.qt;
    nq = min(a.qt, a.tq - q0);
    const int b = unit / a.heads;
    m = min(max(a.prefix_len[b], 0), a.prefix_cap);
    nb_all = min((m + kBlock - 1) / kBlock, a.nb_cap);
    pos0 = (long long)a.q_pos[b] + q0;
  }
  __device__ int visible(int qi) const {  // non-decreasing in qi
    const long long t = pos0 + qi;
    return t >= m ? nb_all : (int)(max(t, 0ll) / kBlock);
  }
};

// Score of block key kv (fp64 copy) against q_idx (LDS), rounded once.
__device__ __forceinline__ float prefill_score(const double* qidx, const double (&kv)[kIdxDim]) {
  const double2* qv = reinterpret_cast<const double2*>(qidx);
  double sc = 0.0;
#pragma unroll
  for (int c = 0; c < kIdxDim / 2; ++c) {
    const double2 x = qv[c];
    sc += x.x * kv[2 * c] + x.y * kv[2 * c + 1];
  }
  return (float)sc;
}

__device__ __forceinline__ void load_key(const float* K, int j, double (&kv)[kIdxDim]) {
  const float4* kr = reinterpret_cast<const float4*>(K + (size_t)j * kIdxDim);
#pragma unroll
  for (int u = 0; u < kIdxDim / 4; ++u) {
    const float4 x = kr[u];
    kv[4 * u] = x.x;
    kv[4 * u + 1] = x.y;
    kv[4 * u + 2] = x.z;
    kv[4 * u + 3] = x.w;
  }
}

template <int DT, int D, int NSMAX>
__global__ __launch_bounds__(kPrefillThreads, NSMAX >= 16 ? 4 : 6) void k_prefill_route(PrefillArgs a) {
  constexpr int W = kPrefillThreads / 64;
  __shared__ PrefillSmem<prefill_slots(NSMAX)> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const PrefillTile t(a);
  const int nbmax = t.visible(t.nq - 1);

  typedef double v4d __attribute__((ext_vector_type(4)));
  const int lr = lane % 16, lk = lane / 16;
  const float* K = a.kbar + (size_t)t.unit * a.nb_cap * kIdxDim;
  const int ntiles = (nbmax + 15) / 16;
  // The key tiles do not depend on q_idx: this wave's first tiles are loaded
  // before it, and each tile consumed below puts the loads of the tile
  // kPrefillTilesInFlight * W later in flight.  Every lane loads (blocks past
  // the visible ones re-read the last visible one: their columns of the
  // product are never stored), with no branch around a load, so the compiler
  // waits for a tile only where it is used.
  auto load_b = [&](float4 (&bf)[2], int tile) {  // this lane's dims of one key of a tile
    const int j = min(tile * 16 + lr, max(nbmax - 1, 0));
    const float4* kr = reinterpret_cast<const float4*>(K + (size_t)j * kIdxDim) + lk;
    bf[0] = kr[0];
    bf[1] = kr[4];
  };
  float4 bq[kPrefillTilesInFlight][2];
  if (nbmax > 0) {
#pragma unroll
    for (int u = 0; u < kPrefillTilesInFlight; ++u) load_b(bq[u], wave + u * W);
  }

  // 1. q_idx on the matrix cores, fp64, with the operands read straight from
  //    global memory (P [D][32] is shared by every workgroup and stays in L2):
  //    wave w computes the 16 x 16 tile of columns 16 (w % 2) .. + 15 over the
  //    quarter w / 2 of the D terms, in the operand layout of the scores
  //    below; the four quarters are summed in a fixed order through LDS
  {
    static_assert(kPrefillThreads == 512 && kIdxDim == 32 && kPrefillMaxQ <= 16, "q_idx tiling");
    double* part = reinterpret_cast<double*>(sm.scores);  // [4][16][32], before any score is written
    const int c0 = 16 * (wave & 1), k0 = (wave >> 1) * (D / 4);
    const char* qrow = static_cast<const char*>(a.q) +
                       ((size_t)t.unit * a.tq + t.q0 + (lr < t.nq ? lr : 0)) * Geo<DT, D>::ROWB;
    float qa[D / 16], pb[D / 16];
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      const int dd = k0 + 4 * st + lk;
      if constexpr (DT == 0)
        qa[st] = reinterpret_cast<const float*>(qrow)[dd];
      else
        qa[st] = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(qrow)[dd] << 16);
      pb[st] = a.proj[dd * kIdxDim + c0 + lr];
    }
    v4d acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int st = 0; st < D / 16; ++st)
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64(lr < t.nq ? (double)qa[st] : 0.0, (double)pb[st], acc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) part[((wave >> 1) * 16 + lk + 4 * r) * kIdxDim + c0 + lr] = acc[r];
    __syncthreads();
    const int qi = tid / kIdxDim, i = tid % kIdxDim;
    if (qi < t.nq) sm.qidx[qi][i] = ((part[tid] + part[512 + tid]) + part[1024 + tid]) + part[1536 + tid];
  }
  __syncthreads();

  // 2. scores on the matrix cores, fp64: tile (16 queries) x (16 blocks),
  //    S = Qidx [16 x 32] . KBAR^T [32 x 16] in 8 steps of
  //    v_mfma_f64_16x16x4f64.  Operand layout (checked on gfx950): lane l
  //    holds A[l % 16][k] and B[k][l % 16] for the k of lane group l / 16 at
  //    each step; register r of the result holds S[l / 16 + 4 r][l % 16].
  //    Any order of the 32 index dims over (step, lane group) gives the same
  //    sum, so lane group g takes dims 4g .. 4g+3 at steps 0-3 and 16+4g ..
  //    16+4g+3 at steps 4-7: its key values are two 16-byte loads per tile.
  {
    double af[kIdxDim / 4];
#pragma unroll
    for (int st = 0; st < kIdxDim / 4; ++st)
      af[st] = lr < t.nq ? sm.qidx[lr][4 * lk + (st & 3) + 16 * (st >> 2)] : 0.0;
    int vis[4];  // blocks visible to the queries of this lane's result rows
#pragma unroll
    for (int r = 0; r < 4; ++r) vis[r] = lk + 4 * r < t.nq ? t.visible(lk + 4 * r) : 0;
    constexpr int NF = kPrefillTilesInFlight;
    for (int t0 = wave; t0 < ntiles; t0 += NF * W) {
#pragma unroll
      for (int u = 0; u < NF; ++u) {
        const int tile = t0 + u * W;
        if (tile >= ntiles) break;
        const int j = tile * 16 + lr;
        const float4 b0 = bq[u][0], b1 = bq[u][1];
        load_b(bq[u], tile + NF * W);
        const float bf[kIdxDim / 4] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
        v4d acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int st = 0; st < kIdxDim / 4; ++st)
          acc = __builtin_amdgcn_mfma_f64_16x16x4f64(af[st], (double)bf[st], acc, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (j < vis[r]) sm.scores[(lk + 4 * r) * a.nb_cap + j] = (float)acc[r];
      }
    }
  }
  if (tid == 0) sm.next_q = W;  // queries past the first W go to whichever wave is free
  __syncthreads();

  // 3. one-wave routing: wave w takes query w, then the next unclaimed one
  //    (query costs differ a lot: a wide entmax support takes several times
  //    as long as a planted one)
  for (int qi = wave; qi < t.nq;) {
    const int nbq = t.visible(qi);
    const int kk = min(a.topk, nbq);
    const size_t o = ((size_t)t.unit * a.tq + t.q0 + qi) * a.topk;
    for (int i = kk + lane; i < a.topk; i += 64) {
      a.sel_idx[o + i] = -1;
      if (a.sel_prob) a.sel_prob[o + i] = 0.f;
      a.sel_bias[o + i] = -INFINITY;
    }
    if (kk > 0) {
      const float* sq = sm.scores + qi * a.nb_cap;
      int32_t* oi = a.sel_idx + o;
      float* op = a.sel_prob ? a.sel_prob + o : nullptr;
      float* ob = a.sel_bias + o;
      bool ok = false;
      if (nbq <= 64) ok = wave_route<1, true>(sq, nbq, kk, oi, op, ob, nullptr, nullptr, sm.pb[wave]);
      else if (nbq <= 128) ok = wave_route<2, true>(sq, nbq, kk, oi, op, ob, nullptr, nullptr, sm.pb[wave]);
      else if (nbq <= 256) ok = wave_route<4, true>(sq, nbq, kk, oi, op, ob, nullptr, nullptr, sm.pb[wave]);
      else if (nbq <= 512) ok = wave_route<8, true>(sq, nbq, kk, oi, op, ob, nullptr, nullptr, sm.pb[wave]);
      else if constexpr (NSMAX >= 16)
        if (nbq <= 64 * kWaveBlocks) ok = wave_route<16, true>(sq, nbq, kk, oi, op, ob, nullptr, nullptr, sm.pb[wave]);
      if (!ok && lane == 0) oi[0] = kDeferred;
    }
    int nxt = 0;  // every path through the body claims the next query
    if (lane == 0) nxt = atomicAdd(&sm.next_q, 1);
    qi = __shfl(nxt, 0);
  }
}

// The queries k_prefill_route left marked: scores again (one query at a time)
// and the whole-workgroup routing.  The workgroups stride over the chunk's
// queries 512 at a time, reading 512 markers per pass, so a chunk with no
// marked query costs one pass of loads.
template <int DT, int D>
__global__ __launch_bounds__(kPrefillThreads) void k_prefill_fallback(PrefillArgs a) {
  __shared__ TopkSmem<kPrefillThreads> tsm;
  __shared__ float scores[kMaxBlocks];
  __shared__ alignas(16) double qidx[kIdxDim];
  __shared__ int list[kPrefillThreads];
  __shared__ int n_list;
  const int tid = threadIdx.x;
  const long long total = (long long)a.units * a.tq;
  for (long long base = (long long)blockIdx.x * kPrefillThreads; base < total;
       base += (long long)gridDim.x * kPrefillThreads) {
    if (tid == 0) n_list = 0;
    __syncthreads();
    const long long g = base + tid;
    if (g < total && a.sel_idx[g * a.topk] == kDeferred) list[atomicAdd(&n_list, 1)] = tid;
    __syncthreads();
    const int nl = n_list;
    for (int l = 0; l < nl; ++l) {
      const long long gq = base + list[l];
      const int unit = (int)(gq / a.tq), i = (int)(gq - (long long)unit * a.tq);
      const int b = unit / a.heads;
      const int m = min(max(a.prefix_len[b], 0), a.prefix_cap);
      const int nb_all = min((m + kBlock - 1) / kBlock, a.nb_cap);
      const long long t = (long long)a.q_pos[b] + i;
      const int nbq = t >= m ? nb_all : (int)(max(t, 0ll) / kBlock);
      if (tid < kIdxDim) {
        using G = Geo<DT, D>;
        const char* qrow = static_cast<const char*>(a.q) + (size_t)gq * G::ROWB;
        double acc = 0.0;
        for (int dd = 0; dd < D; ++dd) {
          float qd;
          if constexpr (DT == 0)
            qd = reinterpret_cast<const float*>(qrow)[dd];
          else
            qd = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(qrow)[dd] << 16);
          acc += (double)a.proj[dd * kIdxDim + tid] * (double)qd;
        }
        qidx[tid] = acc;
      }
      __syncthreads();
      const float* K = a.kbar + (size_t)unit * a.nb_cap * kIdxDim;
      for (int j = tid; j < nbq; j += kPrefillThreads) {
        double kv[kIdxDim];
        load_key(K, j, kv);
        scores[j] = prefill_score(qidx, kv);
      }
      __syncthreads();
      const size_t o = (size_t)gq * a.topk;
      entmax_topk_block<kPrefillThreads>(scores, nbq, a.topk, a.sel_idx + o, a.sel_prob ? a.sel_prob + o : nullptr,
                                         a.sel_bias + o, nullptr, nullptr, tsm);
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// uocr_ngram_ban: one workgroup per sequence.  The last min(window, n_gen)
// generated tokens go to LDS in position order; each thread takes start
// positions p of the n-grams lying wholly in that window and compares their
// first n-1 tokens with the last n-1 generated ones (stopping at the first
// difference); a match writes -inf over the logit of the n-gram's last token.
// The page guard, when on, first writes -inf over every logit but the page
// marker's and end-of-sequence's.  Only -inf is ever written, so concurrent
// writes of the same logit agree.
// ---------------------------------------------------------------------------
constexpr int kNgramThreads = 256;

template <int DT>
__global__ __launch_bounds__(kNgramThreads) void k_ngram_ban(NgramArgs a) {
  __shared__ int hist[kMaxNgramWindow];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int T = max(a.n_gen[b], 0);
  const int wn = min(a.window, T);
  const int32_t* tok = a.tokens + (size_t)b * a.ring_cap;
  const int s0 = (T - wn) % a.ring_cap;  // slot of the window's first token
  for (int i = tid; i < wn; i += kNgramThreads) {
    const int slot = s0 + i;
    hist[i] = tok[slot < a.ring_cap ? slot : slot - a.ring_cap];
  }
  auto kill = [&](int v) {
    if (v < 0 || v >= a.vocab) return;
    if constexpr (DT == 0)
      reinterpret_cast<float*>(a.logits)[(size_t)b * a.vocab + v] = -INFINITY;
    else
      reinterpret_cast<uint16_t*>(a.logits)[(size_t)b * a.vocab + v] = 0xFF80u;  // bf16 -inf
  };
  if (a.page_tokens && a.max_page_tokens > 0 && a.page_tokens[b] >= a.max_page_tokens)
    for (int v = tid; v < a.vocab; v += kNgramThreads)
      if (v != a.page_token && v != a.eos_token) kill(v);
  __syncthreads();
  const int n = a.ngram;
  if (wn < n) return;
  const int tail = wn - n + 1;  // first of the last n-1 tokens
  for (int p = tid; p <= wn - n; p += kNgramThreads) {
    bool match = true;
    for (int k = n - 2; k >= 0 && match; --k) match = hist[p + k] == hist[tail + k];  // nearest token first
    if (match) kill(hist[p + n - 1]);
  }
}

// ---------------------------------------------------------------------------
// page2d rotary embedding of one row, shared by uocr_rope_page2d and the
// fused steps (so that both turn a row into the same bits).  Pair j < D/2 is
// the dims (j, j + D/2); pairs j < D/4 turn by offset * theta_j, the others
// by (page mod page_mod) * theta_(j - D/4) (the page itself when page_mod is
// 0), theta_i = base^(-2 i / (D/2)); negative positions count as 0.  The
// angle is formed in fp64 and brought into [-pi, pi] by Cody-Waite reduction
// with 2 pi split in two doubles (exact to ~1e-10 rad for positions below
// 2^24); cos and sin are then taken in fp32, and the pair is turned in fp32.
// ---------------------------------------------------------------------------
constexpr double kTwoPiHi = 6.283185307179586;        // 2 pi rounded to a double
constexpr double kTwoPiLo = 2.4492935982947064e-16;   // 2 pi - kTwoPiHi
constexpr double kInvTwoPi = 0.15915494309189535;     // 1 / (2 pi) rounded

__device__ __forceinline__ double rope_theta(float base, int j, int H2) {
  const int Q4 = H2 / 2;
  return pow((double)base, -2.0 * (double)(j < Q4 ? j : j - Q4) / (double)H2);
}
__device__ __forceinline__ int rope_pos(int j, int H2, int page, int offset, int page_mod) {
  page = max(page, 0);
  offset = max(offset, 0);
  return j < H2 / 2 ? offset : (page_mod > 0 ? page % page_mod : page);
}
// (cos, sin) of pos * theta
__device__ __forceinline__ float2 rope_cs(int pos, double theta) {
  const double phi = (double)pos * theta;
  const double q = rint(phi * kInvTwoPi);
  const double r = fma(-q, kTwoPiLo, fma(-q, kTwoPiHi, phi));
  float sn, cn;
  sincosf((float)r, &sn, &cn);
  return make_float2(cn, sn);
}
// (x0, x1) turned by the angle whose (cos, sin) is w
__device__ __forceinline__ void rope_turn(float& x0, float& x1, float2 w) {
  const float s0 = x0, s1 = x1;
  x0 = fmaf(s0, w.x, -s1 * w.y);
  x1 = fmaf(s0, w.y, s1 * w.x);
}
// a value rounded to the storage type and widened again
template <int DT>
__device__ __forceinline__ float to_storage(float x) {
  if constexpr (DT == 0) return x;
  else return __uint_as_float(bf16_bits(x) << 16);
}
// element i of a row in the storage type
template <int DT>
__device__ __forceinline__ float row_elem(const void* row, int i) {
  if constexpr (DT == 0) return reinterpret_cast<const float*>(row)[i];
  else return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(row)[i] << 16);
}
template <int DT>
__device__ __forceinline__ void set_row_elem(void* row, int i, float x) {
  if constexpr (DT == 0) reinterpret_cast<float*>(row)[i] = x;
  else reinterpret_cast<uint16_t*>(row)[i] = (uint16_t)bf16_bits(x);
}
// The fused steps' rotation of one decode step (a.rope_page set): thread
// j < D/2 turns pair j of the unit's q into s_q (rounded to the storage
// type, as a separate uocr_rope_page2d call stores it) and, when kring is
// not null, pair j of k_new into the ring row kring.
template <int DT, int D>
__device__ __forceinline__ void step_rope(const StepArgs& a, int unit, int b, float* s_q, void* kring) {
  constexpr int H2 = D / 2;
  const int j = threadIdx.x;
  if (j >= H2) return;
  const float2 w = rope_cs(rope_pos(j, H2, a.rope_page[b], a.rope_offset[b], a.rope_page_mod),
                           rope_theta(a.rope_base, j, H2));
  const char* qrow = static_cast<const char*>(a.d.q) + (size_t)unit * D * (DT == 0 ? 4 : 2);
  float q0 = row_elem<DT>(qrow, j), q1 = row_elem<DT>(qrow, j + H2);
  rope_turn(q0, q1, w);
  s_q[j] = to_storage<DT>(q0);
  s_q[j + H2] = to_storage<DT>(q1);
  if (kring) {
    const char* krow = static_cast<const char*>(a.k_new) + (size_t)unit * D * (DT == 0 ? 4 : 2);
    float k0 = row_elem<DT>(krow, j), k1 = row_elem<DT>(krow, j + H2);
    rope_turn(k0, k1, w);
    set_row_elem<DT>(kring, j, k0);
    set_row_elem<DT>(kring, j + H2, k1);
  }
}

// ---------------------------------------------------------------------------
// Fused steps: append + (route +) decode in one launch
// ---------------------------------------------------------------------------
// uocr_srswa_step: one workgroup of NT threads per unit runs the whole step.
// STREAM selects nontemporal loads (better when the grid fills the chip and
// the step is bandwidth-bound) or plain loads (lower latency, better for a
// few units per CU).
//   1. issue the loads of the new token's row, P, q and the block keys;
//      q_idx = P^T q (fp64); write the new row into its ring slot;
//   2. block scores into LDS;
//   3. entmax + top-k on wave 0 while waves 1 .. W-1 attend over the window,
//      which does not depend on the routing (the new token's row is taken
//      from k_new / v_new, so no wave waits for the ring write); wave 0
//      hands the selection over through an LDS flag, not a barrier;
//   4. each wave attends over its share of the live selected blocks as soon
//      as it has the selection and its window share is done; the waves merge
//      through LDS.
template <int DT, int D, int NT, bool STREAM>
__global__ __launch_bounds__(NT, NT >= 512 ? 4 : 3) void k_srswa_step(StepArgs a) {
  using G = Geo<DT, D>;
  constexpr int W = NT / 64;
  constexpr int SL = NT / kIdxDim;  // slices of D in the q_idx product
  constexpr int KB = 4;             // block keys loaded per thread per batch
  constexpr int RPP = NT / 8;       // block keys per pass (8 lanes per key)
  __shared__ __attribute__((aligned(16))) float s_scores[kMaxBlocks];
  __shared__ double s_red[SL][kIdxDim];
  __shared__ __attribute__((aligned(16))) double s_qidx[kIdxDim];
  __shared__ TopkSmem<NT> tsm;
  __shared__ int l_idx[kMaxTopk];
  __shared__ float l_bias[kMaxTopk];
  __shared__ float lds_ml[W][2];
  __shared__ __attribute__((aligned(16))) float lds_o[W * D];
  __shared__ __attribute__((aligned(16))) float s_q[D];  // q (turned by page2d RoPE if asked)
  // the finish's partial pairs (the partial outputs reuse s_scores, which no
  // wave reads once it has the selection)
  constexpr bool kParts = W <= 8 && PartGeo<DT, D, W>::P * D <= kMaxBlocks;
  __shared__ float2 s_pml[kParts ? PartGeo<DT, D, W>::P : 1];
  UOCR_STAMP_LDS;
  const DecodeArgs& d = a.d;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int unit = blockIdx.x, b = unit / d.heads, h = unit - b * d.heads;
  const bool rope = a.rope_page != nullptr;
  const int grp = lane / G::LPR, c = lane % G::LPR;
  const size_t cb = (size_t)c * 16;
  UOCR_STAMP(s_stamp, tid == 0, 0);
#ifdef UOCR_PHASE_STAMPS
  if (tid == 0) {
    s_stamp[3] = __builtin_amdgcn_s_getreg((3 << 11) | 20);   // XCC_ID: the XCD
    s_stamp[8] = __builtin_amdgcn_s_getreg((31 << 11) | 4);   // HW_ID: CU, shader array, engine
  }
#endif

  // The loads that depend on nothing but the unit go out first, in order:
  // the new token's row (stored into its ring slot once the count is known),
  // P and q for q_idx, the block keys.  Every lane issues each of them (the
  // lanes past the new row re-read its last chunk), so that no per-lane
  // branch makes the compiler wait for a load where the paths join.
  constexpr int CPR = G::ROWB / 16;
  const int a_which = min(tid, 2 * CPR - 1) / CPR, a_off = min(tid, 2 * CPR - 1) - a_which * CPR;
  const uint4 new_chunk =
      ld16(static_cast<const char*>(a_which ? a.v_new : a.k_new) + (size_t)unit * G::ROWB + a_off * 16);

  // q_idx partial sums: the loads of P and q go out first, so that they are
  // not queued behind the block keys.  q is loaded once, one element per
  // thread of the first D, and shared through LDS (s_q) with the q_idx
  // product and the attention, instead of every thread loading its share
  // twice: fewer loads through the CU's memory pipeline in front of the keys.
  const int i_q = tid % kIdxDim, sl_q = tid / kIdxDim;
  constexpr int DPS = D / SL;
  float pv[DPS], qv_[DPS];
#pragma unroll
  for (int k = 0; k < DPS; ++k) pv[k] = a.proj[(sl_q * DPS + k) * kIdxDim + i_q];
  const float qe = tid < D ? row_elem<DT>(static_cast<const char*>(d.q) + (size_t)unit * G::ROWB, tid) : 0.f;

  // the first two batches of block keys (rows < nb_cap: no wait for
  // prefix_len), in flight while q_idx is formed.  The loads are
  // unconditional, so that the compiler keeps them all in flight and waits
  // for P and q alone before q_idx (with a branch around a load it waited
  // for the load where the paths join): rows past nb_cap read the last row
  // again, and without a prefix the first row of P stands in for the keys
  // (no score is stored for any of these).
  const int kr = tid / 8, kc = tid % 8;
  const int last_row = max(a.nb_cap - 1, 0);
  const float* K = (a.nb_cap > 0 ? a.kbar + (size_t)unit * a.nb_cap * kIdxDim : a.proj) + kc * 4;
  auto load_keys = [&](float4 (&dst)[KB], int jb) {
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const float* row = K + (size_t)min(jb + u * RPP + kr, last_row) * kIdxDim;
      dst[u] = STREAM ? ld16f_stream(row) : *reinterpret_cast<const float4*>(row);
    }
  };
  float4 kvA[KB], kvB[KB];
  load_keys(kvA, 0);
  load_keys(kvB, RPP * KB);

  const int m = min(max(d.prefix_len[b], 0), d.prefix_cap);
  const int t = max(a.t_gen_in[b], 0);
  const int n = d.window, slot = t % n, w = min(n, t + 1);
  const int nb = (m + kBlock - 1) / kBlock;

  // q into s_q; with page2d RoPE turned on the way, and the turned k_new row
  // written into its ring slot (pair-wise), before anything reads them.  The
  // block keys' loads are already in flight.
  if (rope)
    step_rope<DT, D>(a, unit, b, s_q, static_cast<char*>(a.k_ring) + ((size_t)unit * n + slot) * G::ROWB);
  else if (tid < D)
    s_q[tid] = qe;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < DPS; ++k) qv_[k] = s_q[sl_q * DPS + k];
  {
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < DPS; ++k) acc += (double)pv[k] * (double)qv_[k];
    s_red[sl_q][i_q] = acc;
  }

  // ring append of this unit's row (with RoPE the k row is already in), and
  // the new count
  if (tid < 2 * CPR && (a_which || !rope))
    *reinterpret_cast<uint4*>(static_cast<char*>(a_which ? a.v_ring : a.k_ring) +
                              ((size_t)unit * n + slot) * G::ROWB + a_off * 16) = new_chunk;
  if (h == 0 && tid == 0) a.t_gen_out[b] = t + 1;
  if (tid == 0) tsm.flag = 0;  // zeroed before the first workgroup barrier

  float q[G::E];
#pragma unroll
  for (int e = 0; e < G::E; ++e) q[e] = s_q[c * G::E + e] * d.qscale;
  State<G::E> st;
  st.init();
  __syncthreads();
  if (tid < kIdxDim) {
    double sum = 0.0;
#pragma unroll
    for (int k = 0; k < SL; ++k) sum += s_red[k][tid];
    s_qidx[tid] = sum;
  }
  __syncthreads();
  UOCR_STAMP(s_stamp, tid == 0, 5);

  // block scores (fp64 dot products, rounded once to fp32) into LDS; the
  // next batch of keys is loaded while the current one is scored
  {
    double qv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) qv[e] = s_qidx[kc * 4 + e];
    auto score = [&](const float4 (&kv)[KB], int jb) {
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const int j = jb + u * RPP + kr;
        double sc = qv[0] * (double)kv[u].x + qv[1] * (double)kv[u].y + qv[2] * (double)kv[u].z +
                    qv[3] * (double)kv[u].w;
        sc = group_sum<8>(sc);
        if (kc == 0 && j < nb) s_scores[j] = (float)sc;
      }
    };
    constexpr int BATCH = RPP * KB;
    for (int jb = 0; jb < nb; jb += 2 * BATCH) {
      score(kvA, jb);
      UOCR_STAMP(s_stamp, jb == 0 && tid == 0, 6);
      if (jb + 2 * BATCH < nb) load_keys(kvA, jb + 2 * BATCH);
      score(kvB, jb + BATCH);
      if (jb + 3 * BATCH < nb) load_keys(kvB, jb + 3 * BATCH);
    }
  }
  __syncthreads();
  UOCR_STAMP(s_stamp, tid == 0, 1);

  // Window attention on waves 1 .. W-1 while wave 0 routes: every slot of
  // the ring is addressable, so each of these waves reads its share of all n
  // slots and lets only the first w count; the new token's row is taken from
  // k_new / v_new (with RoPE, from its ring slot, written before a barrier).
  auto window = [&]() {
    const int WR = (n + W - 2) / (W - 1);
    const int r0 = (wave - 1) * WR, r1 = min(r0 + WR, n);
    if (r0 < r1) {
      const size_t base = ((size_t)unit * n + r0) * G::ROWB + cb;
      const size_t nbase = (size_t)unit * G::ROWB + cb;
      constexpr int UW = (20 + G::RPL - 1) / G::RPL < 8 ? (20 + G::RPL - 1) / G::RPL : 8;
      attend_range<DT, D, UW, STREAM>(static_cast<const char*>(d.k_ring) + base,
                                      static_cast<const char*>(d.v_ring) + base, r1 - r0, 0.f, q, st, grp,
                                      rope ? -1 : slot - r0, static_cast<const char*>(a.k_new) + nbase,
                                      static_cast<const char*>(a.v_new) + nbase, w - r0);
    }
    UOCR_STAMP_DONE(s_stamp, lane == 0, 16 + wave);
  };
  const size_t so = (size_t)unit * d.topk;
  const bool bar = entmax_topk_block<NT, decltype(window), true>(
      s_scores, nb, d.topk, a.sel_idx + so, a.sel_prob ? a.sel_prob + so : nullptr, a.sel_bias + so, l_idx,
      l_bias, tsm, window, s_stamp);
  if (bar)
    __syncthreads();
  else
    wait_flag(&tsm.flag);
  UOCR_STAMP(s_stamp, lane == 0, wave == 0 ? 2 : 32 + wave);

  // Live selected blocks, as tasks of 32 / cpb rows; task i goes to wave
  // i mod W, which starts on it as soon as it has the selection: wave 0 right
  // after routing, the others when their window share is done.  When the
  // window is the longer branch, the fewer waves a task waits for, the sooner
  // the step ends, so blocks are cut only until there are W / 4 tasks
  // (measured at 40 pages, 8 waves: 14.7 us per step against 15.6 us with a
  // barrier and W tasks).
  int idx = -1;
  float bias = 0.f;
  bool live = false;
  if (lane < d.topk) {
    idx = l_idx[lane];
    bias = l_bias[lane];
    live = idx >= 0 && idx < nb && bias > -INFINITY;
  }
  const uint64_t mask = __ballot(live);
  const int n_live = __popcll(mask);
  int cpb = 1;
  while (8 * cpb * n_live <= W && 2 * cpb * G::RPL <= kBlock) cpb *= 2;
  const int rpc = kBlock / cpb;
  for (int task = wave; task < n_live * cpb; task += W) {
    const int tk = task / cpb, sub = task - tk * cpb;
    uint64_t mm = mask;
    for (int i = 0; i < tk; ++i) mm &= mm - 1;
    const int sl = __ffsll((unsigned long long)mm) - 1;
    const int j = __shfl(idx, sl);
    const float bj = __shfl(bias, sl);
    const int r0 = j * kBlock + sub * rpc;
    const int nr = min(rpc, m - r0);
    if (nr <= 0) continue;
    const size_t base = ((size_t)unit * d.prefix_cap + r0) * G::ROWB + cb;
    attend_fit<DT, D, STREAM>(static_cast<const char*>(d.k_prefix) + base,
                              static_cast<const char*>(d.v_prefix) + base, nr, bj * kLog2e, q, st, grp);
  }
  UOCR_STAMP_DONE(s_stamp, lane == 0, 48 + wave);
  if constexpr (kParts)
    wg_finish_parts<DT, D, W>(st, s_scores, s_pml, d, unit, s_stamp);
  else
    wg_finish<DT, D, W>(st, lds_ml, lds_o, d, unit, 0, s_stamp);
#ifdef UOCR_PHASE_STAMPS
  if (tid == 0) s_stamp[4] = wall_clock64();
  __syncthreads();
  if (tid < kStampSlots && unit < kMaxStampUnits) g_stamps[(size_t)unit * kStampSlots + tid] = s_stamp[tid];
#endif
}

// uocr_rswa_step: the dense decode with the append fused in.  Every
// workgroup reads the new token's row from k_new / v_new instead of the ring
// slot it goes to; the workgroup of split 0 writes it into the ring.
// With page2d RoPE every workgroup turns q itself (into LDS), and the
// workgroup whose keys hold the new token's position writes the turned k row
// (and the v row) into the ring and reads them back from there after a
// barrier.
template <int DT, int D>
__global__ __launch_bounds__(1024) void k_rswa_step(StepArgs a) {
  using G = Geo<DT, D>;
  __shared__ float lds_ml[kMaxWaves][2];
  __shared__ __attribute__((aligned(16))) float lds_o[kMaxWaves * D];
  __shared__ __attribute__((aligned(16))) float s_q[D];
  const DecodeArgs& d = a.d;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, W = blockDim.x >> 6;
  const int unit = blockIdx.x / d.splits, split = blockIdx.x - unit * d.splits;
  const int b = unit / d.heads, h = unit - b * d.heads;
  const int m = min(max(d.prefix_len[b], 0), d.prefix_cap);
  const int t = max(a.t_gen_in[b], 0);
  const int n = d.window, slot = t % n, w = min(n, t + 1);
  const bool rope = a.rope_page != nullptr;
  const int lo = split * d.chunk, hi = min(lo + d.chunk, m + w);
  constexpr int CPR = G::ROWB / 16;
  char* const kslot = static_cast<char*>(a.k_ring) + ((size_t)unit * n + slot) * G::ROWB;
  char* const vslot = static_cast<char*>(a.v_ring) + ((size_t)unit * n + slot) * G::ROWB;
  if (rope) {
    const bool owner = m + slot >= lo && m + slot < hi;  // exactly one workgroup of the unit
    step_rope<DT, D>(a, unit, b, s_q, owner ? kslot : nullptr);
    if (owner && threadIdx.x >= D / 2 && threadIdx.x < D / 2 + CPR) {
      const int off = threadIdx.x - D / 2;
      *reinterpret_cast<uint4*>(vslot + off * 16) =
          ld16(static_cast<const char*>(a.v_new) + (size_t)unit * G::ROWB + off * 16);
    }
    __syncthreads();
  } else if (split == 0 && threadIdx.x < 2 * CPR) {
    const int which = threadIdx.x / CPR, off = threadIdx.x - which * CPR;
    const char* src = static_cast<const char*>(which ? a.v_new : a.k_new) + (size_t)unit * G::ROWB + off * 16;
    *reinterpret_cast<uint4*>((which ? vslot : kslot) + off * 16) = ld16(src);
  }
  if (split == 0 && h == 0 && threadIdx.x == 0) a.t_gen_out[b] = t + 1;

  const int per = hi > lo ? (hi - lo + W - 1) / W : 0;
  const int wlo = lo + wave * per, whi = min(wlo + per, hi);
  const int grp = lane / G::LPR, c = lane % G::LPR;
  float q[G::E];
  if (rope) {
#pragma unroll
    for (int e = 0; e < G::E; ++e) q[e] = s_q[c * G::E + e] * d.qscale;
  } else {
    load_q<DT, D>(d.q, unit, c, d.qscale, q);
  }
  State<G::E> st;
  st.init();
  const size_t cb = (size_t)c * 16;
  if (wlo < min(whi, m)) {
    const size_t base = ((size_t)unit * d.prefix_cap + wlo) * G::ROWB + cb;
    attend_range<DT, D>(static_cast<const char*>(d.k_prefix) + base,
                        static_cast<const char*>(d.v_prefix) + base, min(whi, m) - wlo, 0.f, q, st, grp);
  }
  const int w0 = max(wlo, m) - m, w1 = whi - m;
  if (w0 < w1) {
    const size_t base = ((size_t)unit * n + w0) * G::ROWB + cb;
    const size_t nb_ = (size_t)unit * G::ROWB + cb;
    attend_range<DT, D>(static_cast<const char*>(d.k_ring) + base, static_cast<const char*>(d.v_ring) + base,
                        w1 - w0, 0.f, q, st, grp, rope ? -1 : slot - w0, static_cast<const char*>(a.k_new) + nb_,
                        static_cast<const char*>(a.v_new) + nb_);
  }
  if (W == 4)
    wg_finish<DT, D, 4>(st, lds_ml, lds_o, d, unit, split);
  else
    wg_finish<DT, D>(st, lds_ml, lds_o, d, unit, split);
}

// ---------------------------------------------------------------------------
// uocr_rope_page2d: page2d two-axis rotary embedding, in place.  Pair j of a
// row is (j, j + D/2); pairs j < D/4 turn by offset * theta_j, the others by
// (page mod page_mod) * theta_(j - D/4), theta_i = base^(-2 i / (D/2)).  A
// workgroup takes up to kRopeTokens tokens of one sequence, every head, and
// both tensors when a second one (y, e.g. the keys beside the queries) is given.
// Each thread first issues the loads of its first kRopeInFlight chunk pairs
// (a 16-byte chunk of the first half of a row and the matching chunk of the
// second half), then, while they are in flight, computes the (cos, sin) of
// its (token, pair) entries into LDS; after the barrier it turns its chunks
// and stores them.  The angle is formed in fp64 and brought into [-pi, pi]
// by Cody-Waite reduction with 2 pi split in two doubles (exact to ~1e-10 rad
// for positions below 2^24); cos and sin are then taken in fp32, and the
// pairs are turned in fp32.  x is streamed with nontemporal loads and stores.
// ---------------------------------------------------------------------------
constexpr int kRopeThreads = 256;
constexpr int kRopeInFlight = 8;                       // chunk pairs per thread in flight

__device__ __forceinline__ void st16_stream(char* p, const uint4& v) {
  __builtin_nontemporal_store(v4u32{v.x, v.y, v.z, v.w}, reinterpret_cast<v4u32*>(p));
}

template <int DT, int D>
__global__ __launch_bounds__(kRopeThreads) void k_rope_page2d(RopeArgs a) {
  using G = Geo<DT, D>;
  constexpr int H2 = D / 2;
  constexpr int CPH = H2 / G::E;                        // 16-byte chunks per half row
  constexpr int AE = kRopeTokens * H2 / kRopeThreads;   // (token, pair) entries per thread
  static_assert(kRopeThreads % H2 == 0 && AE >= 1, "every entry of a thread has the same pair");
  __shared__ float2 cs[kRopeTokens][H2];
  const int tid = threadIdx.x;
  const int tiles = (a.tokens + kRopeTokens - 1) / kRopeTokens;
  const int b = blockIdx.x / tiles, t0 = (blockIdx.x - b * tiles) * kRopeTokens;
  const int nt = min(kRopeTokens, a.tokens - t0);
  const long long n1 = (long long)a.heads * nt * CPH;   // chunk pairs of one tensor
  const long long n = a.y ? 2 * n1 : n1;                 // ... of the workgroup
  const size_t base_off = ((size_t)b * a.heads * a.tokens + t0) * G::ROWB;
  char* const xb = static_cast<char*>(a.x) + base_off;
  char* const yb = a.y ? static_cast<char*>(a.y) + base_off : nullptr;
  auto chunk = [&](long long e) -> char* {              // first-half chunk of chunk pair e
    char* tb = xb;
    if (e >= n1) {
      tb = yb;
      e -= n1;
    }
    const int row = (int)(e / CPH), c = (int)(e % CPH);
    const int h = row / nt, ti = row - h * nt;
    return tb + ((size_t)h * a.tokens + ti) * G::ROWB + c * 16;
  };
  // positions of this thread's entries: token tid / H2 + k (kRopeThreads / H2), pair tid % H2
  const int j = tid % H2;
  int pos[AE];
#pragma unroll
  for (int k = 0; k < AE; ++k) {
    const int ti = tid / H2 + k * (kRopeThreads / H2);
    pos[k] = 0;
    if (ti < nt) {
      const size_t pi = (size_t)b * a.tokens + t0 + ti;
      pos[k] = rope_pos(j, H2, a.page[pi], a.offset[pi], a.page_mod);
    }
  }
  uint4 u0[kRopeInFlight], u1[kRopeInFlight];
#pragma unroll
  for (int k = 0; k < kRopeInFlight; ++k) {
    const long long e = tid + (long long)k * kRopeThreads;
    if (e < n) {
      const char* p = chunk(e);
      u0[k] = ld16_stream(p);
      u1[k] = ld16_stream(p + G::ROWB / 2);
    }
  }
  const double theta = rope_theta(a.base, j, H2);
#pragma unroll
  for (int k = 0; k < AE; ++k) {
    const int ti = tid / H2 + k * (kRopeThreads / H2);
    cs[ti][j] = rope_cs(pos[k], theta);
  }
  __syncthreads();
  auto turn = [&](const uint4& v0, const uint4& v1, long long e) {
    char* p = chunk(e);
    const long long et = e >= n1 ? e - n1 : e;
    const int row = (int)(et / CPH), c = (int)(et % CPH);
    const int ti = row % nt;
    float x0[G::E], x1[G::E];
    unpack(v0, x0);
    unpack(v1, x1);
#pragma unroll
    for (int i = 0; i < G::E; ++i) rope_turn(x0[i], x1[i], cs[ti][c * G::E + i]);
    if constexpr (DT == 0) {
      st16_stream(p, make_uint4(__float_as_uint(x0[0]), __float_as_uint(x0[1]), __float_as_uint(x0[2]),
                                __float_as_uint(x0[3])));
      st16_stream(p + G::ROWB / 2, make_uint4(__float_as_uint(x1[0]), __float_as_uint(x1[1]),
                                              __float_as_uint(x1[2]), __float_as_uint(x1[3])));
    } else {
      uint32_t w0[4], w1[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w0[i] = bf16_bits(x0[2 * i]) | (bf16_bits(x0[2 * i + 1]) << 16);
        w1[i] = bf16_bits(x1[2 * i]) | (bf16_bits(x1[2 * i + 1]) << 16);
      }
      st16_stream(p, make_uint4(w0[0], w0[1], w0[2], w0[3]));
      st16_stream(p + G::ROWB / 2, make_uint4(w1[0], w1[1], w1[2], w1[3]));
    }
  };
#pragma unroll
  for (int k = 0; k < kRopeInFlight; ++k) {
    const long long e = tid + (long long)k * kRopeThreads;
    if (e < n) turn(u0[k], u1[k], e);
  }
  // workgroups with more chunk pairs than one round (many heads, or fp32)
  for (long long e0 = (long long)kRopeInFlight * kRopeThreads; e0 < n; e0 += (long long)kRopeInFlight * kRopeThreads) {
#pragma unroll
    for (int k = 0; k < kRopeInFlight; ++k) {
      const long long e = e0 + tid + (long long)k * kRopeThreads;
      if (e < n) {
        const char* p = chunk(e);
        u0[k] = ld16_stream(p);
        u1[k] = ld16_stream(p + G::ROWB / 2);
      }
    }
#pragma unroll
    for (int k = 0; k < kRopeInFlight; ++k) {
      const long long e = e0 + tid + (long long)k * kRopeThreads;
      if (e < n) turn(u0[k], u1[k], e);
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
#define UOCR_DISPATCH(KERNEL, GRID, BLOCK, ARGS)                                   \
  do {                                                                              \
    if (dtype == 0 && head_dim == 64) KERNEL<0, 64><<<GRID, BLOCK, 0, s>>>(ARGS);   \
    else if (dtype == 0 && head_dim == 128) KERNEL<0, 128><<<GRID, BLOCK, 0, s>>>(ARGS); \
    else if (dtype == 1 && head_dim == 64) KERNEL<1, 64><<<GRID, BLOCK, 0, s>>>(ARGS);   \
    else if (dtype == 1 && head_dim == 128) KERNEL<1, 128><<<GRID, BLOCK, 0, s>>>(ARGS); \
    else return hipErrorInvalidValue;                                               \
  } while (0)

hipError_t launch_ring_append(int dtype, int head_dim, const AppendArgs& a, hipStream_t s) {
  UOCR_DISPATCH(k_ring_append, dim3(a.batch), dim3(256), a);
  return hipGetLastError();
}

hipError_t launch_rswa_decode(int dtype, int head_dim, const DecodeArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((long)a.units * a.splits));
  UOCR_DISPATCH(k_rswa_decode, grid, dim3(64 * a.waves), a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  UOCR_DISPATCH(k_split_merge, dim3((unsigned)((a.units + 3) / 4)), dim3(256), a);
  return hipGetLastError();
}

hipError_t launch_srswa_decode(int dtype, int head_dim, const DecodeArgs& a, hipStream_t s) {
  UOCR_DISPATCH(k_srswa_decode, dim3((unsigned)((long)a.units * a.splits)), dim3(64 * a.waves), a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  UOCR_DISPATCH(k_split_merge, dim3((unsigned)((a.units + 3) / 4)), dim3(256), a);
  return hipGetLastError();
}

// The index kernel streams: one resident workgroup per slot the kernel's
// register and LDS use leave on a CU, each wave walking its own run of blocks.
template <int DT, int D>
hipError_t launch_block_index_t(const IndexArgs& a, size_t items, hipStream_t s) {
  static const int cap = [] {
    int dev = 0, cus = 256, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_block_index<DT, D>, 64 * kWaves, 0) != hipSuccess ||
        per_cu <= 0)
      per_cu = 2;
    return cus * per_cu;
  }();
  size_t wgs = (items + kWaves - 1) / kWaves;
  if (wgs > (size_t)cap) wgs = (size_t)cap;
  k_block_index<DT, D><<<dim3((unsigned)wgs), dim3(64 * kWaves), 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_block_index(int dtype, int head_dim, const IndexArgs& a, hipStream_t s) {
  const size_t items = (size_t)a.units * a.n_blocks;
  if (items == 0) return hipSuccess;
  if (dtype == 0 && head_dim == 64) return launch_block_index_t<0, 64>(a, items, s);
  if (dtype == 0 && head_dim == 128) return launch_block_index_t<0, 128>(a, items, s);
  if (dtype == 1 && head_dim == 64) return launch_block_index_t<1, 64>(a, items, s);
  if (dtype == 1 && head_dim == 128) return launch_block_index_t<1, 128>(a, items, s);
  return hipErrorInvalidValue;
}

hipError_t launch_block_score(int dtype, int head_dim, const ScoreArgs& a, hipStream_t s) {
  if (a.nb_cap == 0) return hipSuccess;
  UOCR_DISPATCH(k_block_score, dim3((unsigned)(a.units * a.parts)), dim3(256), a);
  return hipGetLastError();
}

hipError_t launch_entmax_topk(const TopkArgs& a, hipStream_t s) {
  k_entmax_topk<<<dim3(a.units), dim3(kTopkThreads), 0, s>>>(a);
  return hipGetLastError();
}

int prefill_queries_per_wg(int nb_cap) {
  const int slots = prefill_nsmax(nb_cap) >= 16 ? prefill_slots(16) : prefill_slots(8);
  const int q = nb_cap > 0 ? slots / nb_cap : kPrefillMaxQ;
  return q < kPrefillMaxQ ? q : kPrefillMaxQ;
}

template <int NSMAX>
hipError_t launch_prefill_tiles(int dtype, int head_dim, const PrefillArgs& a, dim3 grid, hipStream_t s) {
  if (dtype == 0 && head_dim == 64) k_prefill_route<0, 64, NSMAX><<<grid, kPrefillThreads, 0, s>>>(a);
  else if (dtype == 0 && head_dim == 128) k_prefill_route<0, 128, NSMAX><<<grid, kPrefillThreads, 0, s>>>(a);
  else if (dtype == 1 && head_dim == 64) k_prefill_route<1, 64, NSMAX><<<grid, kPrefillThreads, 0, s>>>(a);
  else if (dtype == 1 && head_dim == 128) k_prefill_route<1, 128, NSMAX><<<grid, kPrefillThreads, 0, s>>>(a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_prefill_route(int dtype, int head_dim, const PrefillArgs& a, hipStream_t s) {
  if (a.tq == 0 || a.units == 0) return hipSuccess;
  if (a.qt != prefill_queries_per_wg(a.nb_cap)) return hipErrorInvalidValue;  // the tile must fit the LDS
  const long long tiles = (a.tq + a.qt - 1) / a.qt;
  const dim3 grid((unsigned)(a.units * tiles));
  hipError_t e = prefill_nsmax(a.nb_cap) >= 16 ? launch_prefill_tiles<16>(dtype, head_dim, a, grid, s)
                                              : launch_prefill_tiles<8>(dtype, head_dim, a, grid, s);
  if (e != hipSuccess) return e;
  long long passes = ((long long)a.units * a.tq + kPrefillThreads - 1) / kPrefillThreads;
  if (passes > 1024) passes = 1024;
  UOCR_DISPATCH(k_prefill_fallback, dim3((unsigned)passes), dim3(kPrefillThreads), a);
  return hipGetLastError();
}

hipError_t launch_ngram_ban(int dtype, const NgramArgs& a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  if (dtype == 0) k_ngram_ban<0><<<dim3(a.batch), dim3(kNgramThreads), 0, s>>>(a);
  else if (dtype == 1) k_ngram_ban<1><<<dim3(a.batch), dim3(kNgramThreads), 0, s>>>(a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_rope_page2d(int dtype, int head_dim, const RopeArgs& a, hipStream_t s) {
  if (a.batch == 0 || a.heads == 0 || a.tokens == 0) return hipSuccess;
  const dim3 grid((unsigned)(a.batch * ((a.tokens + kRopeTokens - 1) / kRopeTokens)));
  if (dtype == 0 && head_dim == 64) k_rope_page2d<0, 64><<<grid, kRopeThreads, 0, s>>>(a);
  else if (dtype == 0 && head_dim == 128) k_rope_page2d<0, 128><<<grid, kRopeThreads, 0, s>>>(a);
  else if (dtype == 1 && head_dim == 64) k_rope_page2d<1, 64><<<grid, kRopeThreads, 0, s>>>(a);
  else if (dtype == 1 && head_dim == 128) k_rope_page2d<1, 128><<<grid, kRopeThreads, 0, s>>>(a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_srswa_step(int dtype, int head_dim, const StepArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.d.units);
  // as many units as CUs or more: bandwidth-bound, stream; fewer: latency-bound
  const bool stream = a.d.units >= 256;
#define UOCR_STEP(DT_, D_, NT_)                                                        \
  do {                                                                                 \
    if (stream) k_srswa_step<DT_, D_, NT_, true><<<grid, NT_, 0, s>>>(a);             \
    else k_srswa_step<DT_, D_, NT_, false><<<grid, NT_, 0, s>>>(a);                   \
  } while (0)
  if (a.d.waves == 16) {
    if (dtype == 0 && head_dim == 64) UOCR_STEP(0, 64, 1024);
    else if (dtype == 0 && head_dim == 128) UOCR_STEP(0, 128, 1024);
    else if (dtype == 1 && head_dim == 64) UOCR_STEP(1, 64, 1024);
    else if (dtype == 1 && head_dim == 128) UOCR_STEP(1, 128, 1024);
    else return hipErrorInvalidValue;
  } else if (a.d.waves == 8) {
    if (dtype == 0 && head_dim == 64) UOCR_STEP(0, 64, 512);
    else if (dtype == 0 && head_dim == 128) UOCR_STEP(0, 128, 512);
    else if (dtype == 1 && head_dim == 64) UOCR_STEP(1, 64, 512);
    else if (dtype == 1 && head_dim == 128) UOCR_STEP(1, 128, 512);
    else return hipErrorInvalidValue;
  } else {
    if (dtype == 0 && head_dim == 64) UOCR_STEP(0, 64, 256);
    else if (dtype == 0 && head_dim == 128) UOCR_STEP(0, 128, 256);
    else if (dtype == 1 && head_dim == 64) UOCR_STEP(1, 64, 256);
    else if (dtype == 1 && head_dim == 128) UOCR_STEP(1, 128, 256);
    else return hipErrorInvalidValue;
  }
#undef UOCR_STEP
  return hipGetLastError();
}

hipError_t launch_rswa_step(int dtype, int head_dim, const StepArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((long)a.d.units * a.d.splits));
  UOCR_DISPATCH(k_rswa_step, grid, dim3(64 * a.d.waves), a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.d.splits == 1) return e;
  UOCR_DISPATCH(k_split_merge, dim3((unsigned)((a.d.units + 3) / 4)), dim3(256), a.d);
  return hipGetLastError();
}

hipError_t read_phase_stamps(void* dst, size_t bytes, hipStream_t s) {
#ifdef UOCR_PHASE_STAMPS
  if (bytes > sizeof(g_stamps)) return hipErrorInvalidValue;
  hipError_t e = hipMemcpyFromSymbolAsync(dst, HIP_SYMBOL(g_stamps), bytes, 0, hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(s);
#else
  (void)dst;
  (void)bytes;
  (void)s;
  return hipErrorNotSupported;
#endif
}

}  // namespace uocr
