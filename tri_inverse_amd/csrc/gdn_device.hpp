// gdn_device.hpp -- gfx950 (CDNA4) device helpers shared by the GDN kernels.
//
// Fragment vocabulary used by every kernel (wave64, 16x16 tiles, lane l = 16*g + c
// with g = l >> 4 in 0..3 and c = l & 15):
//
//   D-form tile (I,J) of a matrix M : lane (g,c) register r holds M[16I + 4g + r][16J + c]
//                                     (what an MFMA 16x16 accumulator holds)
//   T-form tile (I,J) of M          : lane (g,c) register r holds M[16I + c][16J + 4g + r]
//                                     (the D-form of M^T, read transposed)
//
// A 16x16x32 MFMA contracts 32 k-values; lane (g,c) supplies 8 of them for row c of
// the left operand and column c of the right operand.  We fix the slot->k map
//   slot t of lane group g  <->  k = 32p + 16*(t/4) + 4g + (t%4)        (t = 0..7)
// so that two stacked D-form tiles (2p, J), (2p+1, J) of M are, register for
// register, the right-operand fragment of M's k-pair p ("column pack", CP), and two
// side-by-side T-form tiles (I, 2p), (I, 2p+1) are the left-operand fragment of
// M's rows ("row pack", RP).  Any consistent slot->k map leaves a contraction
// unchanged, so products chain from accumulator to operand without touching LDS:
//   (X Y) in D-form  = sum_p mfma(RP(X, I, p), CP(Y, p, J))
//   (X Y) in T-form  = sum_p mfma(CP(Y, p, J), RP(X, I, p))
// The fp32 path uses 16x16x4 MFMAs with slot g of sub-step u <-> k = 16K + 4g + u,
// so register u of a D-form (T-form) tile is directly the operand of sub-step u.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;

constexpr int WAVE = 64;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---- MFMA wrappers ------------------------------------------------------------

__device__ __forceinline__ f32x4 mma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_f32(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// fp8 (OCP e4m3 on gfx950) operands: 8 codes per lane packed in a 64-bit integer
__device__ __forceinline__ f32x4 mma_fp8(long a, long b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c, 0, 0, 0);
}

// ---- packing ------------------------------------------------------------------

__device__ __forceinline__ bf16x8 pack8(const f32x4& lo, const f32x4& hi) {
  bf16x8 r;
  r[0] = (__bf16)lo[0];
  r[1] = (__bf16)lo[1];
  r[2] = (__bf16)lo[2];
  r[3] = (__bf16)lo[3];
  r[4] = (__bf16)hi[0];
  r[5] = (__bf16)hi[1];
  r[6] = (__bf16)hi[2];
  r[7] = (__bf16)hi[3];
  return r;
}

__device__ __forceinline__ bf16x4 pack4(const f32x4& v) {
  bf16x4 r;
  r[0] = (__bf16)v[0];
  r[1] = (__bf16)v[1];
  r[2] = (__bf16)v[2];
  r[3] = (__bf16)v[3];
  return r;
}

__device__ __forceinline__ bf16x8 join8(const bf16x4& lo, const bf16x4& hi) {
  bf16x8 r;
  r[0] = lo[0];
  r[1] = lo[1];
  r[2] = lo[2];
  r[3] = lo[3];
  r[4] = hi[0];
  r[5] = hi[1];
  r[6] = hi[2];
  r[7] = hi[3];
  return r;
}

__device__ __forceinline__ f32x4 unpack4(const bf16x4& v) {
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}

// ---- fp8 e4m3 (OCP) quantisation ------------------------------------------------
// Largest finite e4m3 value is 448.  Values are clamped to +-448 before the hardware
// conversion (round to nearest even), so an out-of-range input saturates instead of
// becoming NaN; the callers count how often that happens.
constexpr float FP8_MAX = 448.0f;
// A value saturates when its correctly rounded e4m3 code would lie beyond 448: the
// rounding boundary is 464, midway between 448 and the next step of that binade (480).
constexpr float FP8_SAT = 464.0f;

template <bool HI>
__device__ __forceinline__ uint32_t cvt_fp8x2(float a, float b, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

template <int BYTE>
__device__ __forceinline__ float fp8_to_f32(uint32_t word) {
  return __builtin_amdgcn_cvt_f32_fp8((int)word, BYTE);
}

// ---- LDS transpose read (gfx950 ds_read_b64_tr_b16) ------------------------------
// Within each group of 16 lanes, lane i receives element (i % 4) of the 8-byte chunk
// addressed by lane 4k + i/4 of its group, for k = 0..3.  With row-major bf16 rows
// X[r][*] in LDS, lane (g, j) addressing X[r0 + 4g + j/4][c0 + 4(j%4)] therefore
// receives X[r0 + 4g + k][c0 + j] for k = 0..3: four consecutive rows of column c0 + j.
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;

__device__ __forceinline__ bf16x4 lds_read_tr4(const __bf16* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

// ---- 16-byte bf16 stores of MFMA output tiles -------------------------------------
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Two adjacent 16-column output tiles e, e + 1 of one row tile, bf16, stored with 16
// contiguous bytes per lane.  Lane group g holds columns 4g .. 4g+3 of each tile;
// v_permlane16_swap of (tile e, tile e+1) exchanges the odd groups' tile-e values with
// the even groups' tile-(e+1) values, after which group g holds the 8 consecutive
// columns 16 (e + g % 2) + 8 (g / 2) .. +7 of the pair.
template <bool NTS = false>
__device__ __forceinline__ void store_pair_bf16(__bf16* __restrict__ row, int e, const f32x4& a0,
                                                const f32x4& a1) {
  const int g = lane_id() >> 4;
  const bf16x4 h0 = pack4(a0), h1 = pack4(a1);
  const u32x2 w0 = __builtin_bit_cast(u32x2, h0), w1 = __builtin_bit_cast(u32x2, h1);
  u32x4 out;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const unsigned x0 = w0[k], x1 = w1[k];  // vector elements to scalars before any bit cast
    const auto sw = __builtin_amdgcn_permlane16_swap(x0, x1, false, false);
    const unsigned y0 = sw[0], y1 = sw[1];
    out[k] = y0;
    out[2 + k] = y1;
  }
  u32x4* p = reinterpret_cast<u32x4*>(row + 16 * (e + (g & 1)) + 8 * (g >> 1));
  if constexpr (NTS)
    __builtin_nontemporal_store(out, p);
  else
    *p = out;
}

// ---- whole 128-byte row pieces from output tiles -----------------------------------
// An output tile in T-form gives lane (g, c) row c and columns 4g .. 4g + 3, so one store
// of a tile writes 16 rows of 64 bytes (fp32) or 32 bytes (bf16), and each 128-byte line
// reaches memory in parts.  Below, lanes c and c ^ 8 of each 16-lane row trade values
// (DPP row_ror:8) so that each store instruction covers 8 rows of 128 contiguous bytes.

// lanes c < 8 keep lo and take the partner's hi as their second value; lanes c >= 8 take
// the partner's lo as their first value and keep hi
__device__ __forceinline__ void trade8(uint32_t lo, uint32_t hi, uint32_t& v0, uint32_t& v1) {
  const bool up = (lane_id() & 15) >= 8;
  const uint32_t got = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(up ? lo : hi), 0x128, 0xf, 0xf, false);
  v0 = up ? got : lo;
  v1 = up ? hi : got;
}

template <bool NTS, class V>
__device__ __forceinline__ void store16(V* p, const V& v) {
  if constexpr (NTS)
    __builtin_nontemporal_store(v, p);
  else
    *p = v;
}

// fp32 tiles a (columns 0 .. 15) and b (16 .. 31) of a 16-row band at base (row stride
// ld elements): store k writes rows 8k + (c & 7), columns 4(g + 4(c >> 3)) .. + 3
template <bool NTS>
__device__ __forceinline__ void store_rows_f32x2(float* __restrict__ base, size_t ld, const f32x4& a,
                                                 const f32x4& b) {
  const int l = lane_id(), g = l >> 4, c = l & 15;
  f32x4 v0, v1;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float ar = a[r], br = b[r];  // vector elements to scalars before any bit cast
    uint32_t w0, w1;
    trade8(__builtin_bit_cast(uint32_t, ar), __builtin_bit_cast(uint32_t, br), w0, w1);
    v0[r] = __builtin_bit_cast(float, w0);
    v1[r] = __builtin_bit_cast(float, w1);
  }
  const size_t o = (size_t)(c & 7) * ld + 4 * (g + 4 * (c >> 3));
  store16<NTS>(reinterpret_cast<f32x4*>(base + o), v0);
  store16<NTS>(reinterpret_cast<f32x4*>(base + o + 8 * ld), v1);
}

// four bf16 tiles t[0..3] (columns 0 .. 63) of a 16-row band at base: the tile pairs
// (0, 1) and (2, 3) first become 16 contiguous bytes per lane (v_permlane16_swap: group g
// then holds columns 16(e + g % 2) + 8(g / 2) .. + 7 of pair e), then lanes c and c ^ 8
// trade, so that store k writes rows 8k + (c & 7), columns 32(c >> 3) + 16(g % 2) +
// 8(g / 2) .. + 7
template <bool NTS>
__device__ __forceinline__ void store_rows_bf16x4(__bf16* __restrict__ base, size_t ld, const f32x4 (&t)[4]) {
  const int l = lane_id(), g = l >> 4, c = l & 15;
  u32x4 pr[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const bf16x4 h0 = pack4(t[2 * e]), h1 = pack4(t[2 * e + 1]);
    const u32x2 w0 = __builtin_bit_cast(u32x2, h0), w1 = __builtin_bit_cast(u32x2, h1);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const unsigned x0 = w0[k], x1 = w1[k];
      const auto sw = __builtin_amdgcn_permlane16_swap(x0, x1, false, false);
      const unsigned y0 = sw[0], y1 = sw[1];
      pr[e][k] = y0;
      pr[e][2 + k] = y1;
    }
  }
  u32x4 v0, v1;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t lo = pr[0][k], hi = pr[1][k];
    uint32_t a0, a1;
    trade8(lo, hi, a0, a1);
    v0[k] = a0;
    v1[k] = a1;
  }
  const size_t o = (size_t)(c & 7) * ld + 32 * (c >> 3) + 16 * (g & 1) + 8 * (g >> 1);
  store16<NTS>(reinterpret_cast<u32x4*>(base + o), v0);
  store16<NTS>(reinterpret_cast<u32x4*>(base + o + 8 * ld), v1);
}

// ---- wave-wide reductions and scans (wave64) ------------------------------------
// All in the VALU (no LDS round trip): DPP within each 16-lane row, then
// v_permlane16_swap / v_permlane32_swap (or readlane) across the four rows.  Each swap
// of a value with itself returns the two rows of every row pair, so combining both
// results gives every lane the pair's value.

// DPP controls: row_shr:k = 0x110 + k, row_ror:k = 0x120 + k.  Lanes whose source lies
// outside their row read 0.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xf, 0xf, false);
}

// the two results of v_permlane16_swap (W = 16) or v_permlane32_swap (W = 32) of x
// with itself: rows (0,0,2,2) and (1,1,3,3), or rows (0,1,0,1) and (2,3,2,3)
template <int W>
__device__ __forceinline__ void self_swap(uint32_t x, uint32_t& a, uint32_t& b) {
  if constexpr (W == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    const uint32_t r0 = r[0], r1 = r[1];  // elements to scalars before use
    a = r0;
    b = r1;
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    const uint32_t r0 = r[0], r1 = r[1];
    a = r0;
    b = r1;
  }
}
template <int W>
__device__ __forceinline__ void self_swap_f(float x, float& a, float& b) {
  uint32_t ua, ub;
  self_swap<W>(__builtin_bit_cast(uint32_t, x), ua, ub);
  a = __builtin_bit_cast(float, ua);
  b = __builtin_bit_cast(float, ub);
}

// reduce over the 16 lanes of each row (rotations by 8, 4, 2, 1), then over the rows
template <typename F>
__device__ __forceinline__ float wave_reduce(float v, F op) {
  v = op(v, dpp_f<0x128>(v));
  v = op(v, dpp_f<0x124>(v));
  v = op(v, dpp_f<0x122>(v));
  v = op(v, dpp_f<0x121>(v));
  float a, b;
  self_swap_f<16>(v, a, b);
  v = op(a, b);
  self_swap_f<32>(v, a, b);
  return op(a, b);
}

__device__ __forceinline__ float wave_max(float v) {
  return wave_reduce(v, [](float x, float y) { return fmaxf(x, y); });
}

__device__ __forceinline__ float wave_min(float v) {
  return wave_reduce(v, [](float x, float y) { return fminf(x, y); });
}

__device__ __forceinline__ float wave_sum(float v) {
  return wave_reduce(v, [](float x, float y) { return x + y; });
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  v += dpp_u<0x128>(v);
  v += dpp_u<0x124>(v);
  v += dpp_u<0x122>(v);
  v += dpp_u<0x121>(v);
  uint32_t a, b;
  self_swap<16>(v, a, b);
  v = a + b;
  self_swap<32>(v, a, b);
  return a + b;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_u<0x128>(v));
  v = min(v, dpp_u<0x124>(v));
  v = min(v, dpp_u<0x122>(v));
  v = min(v, dpp_u<0x121>(v));
  uint32_t a, b;
  self_swap<16>(v, a, b);
  v = min(a, b);
  self_swap<32>(v, a, b);
  return min(a, b);
}

// true in every lane iff pred holds in every active lane
__device__ __forceinline__ bool wave_all(bool pred) { return __builtin_amdgcn_ballot_w64(!pred) == 0; }

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// inclusive prefix sum over the 64 lanes: shifts by 1, 2, 4, 8 within each row (lanes
// that would read across the row start add 0), then each row adds the totals of the
// rows before it
__device__ __forceinline__ float wave_inclusive_scan(float v) {
  v += dpp_f<0x111>(v);
  v += dpp_f<0x112>(v);
  v += dpp_f<0x114>(v);
  v += dpp_f<0x118>(v);
  const float t0 = readlane_f(v, 15), t1 = readlane_f(v, 31), t2 = readlane_f(v, 47);
  const int row = lane_id() >> 4;
  return v + ((row >= 1 ? t0 : 0.f) + (row >= 2 ? t1 : 0.f) + (row >= 3 ? t2 : 0.f));
}

// bc[X] = x of lane 16X + c, in every lane (g, c): the four row broadcasts
__device__ __forceinline__ void row_broadcasts(float x, float (&bc)[4]) {
  float a, b;
  self_swap_f<16>(x, a, b);  // rows (0,0,2,2), (1,1,3,3)
  self_swap_f<32>(a, bc[0], bc[2]);
  self_swap_f<32>(b, bc[1], bc[3]);
}

}  // namespace gdn
