// tri_block.hpp -- one wave owns one C x C block (C = 16*NT, NT = 1, 2, 4) and keeps
// every matrix of the solve in registers as 16x16 fp32 tiles (see gdn_device.hpp for
// the D-form / T-form fragment vocabulary).
//
// Steps implemented here (all per block, all in registers):
//   gates    : G = in-chunk cumsum of the per-token log-gates (wave prefix scan)
//   build_A  : A = -tril(diag(beta) (K K^T .* exp(G_i - G_j)), -1) from K row
//              fragments with MFMA (K K^T is symmetric, so the D-form tiles (J,I)
//              of K K^T are the T-form tiles (I,J) of A -- both forms come from one
//              set of MFMAs over all NT x NT tiles)
//   neumann  : T = sum_{n<=N} A^n as H <- I + A H (N-1 products), optional band mask
//              i - j <= N applied to A and to every intermediate (identical result to
//              masking the final sum, since band entries of products of lower-
//              triangular matrices only involve band entries)
//   doubling : T = prod_{q<m} (I + A^(2^q)) as P <- P + P X, X <- X X
// Pages: [GEO] "When Good Enough Is Optimal: Multiplication-Only Matrix Inversion
// Approximation for Quantized Gated DeltaNet" -- problem statement (T = (I-A)^-1,
// A strictly lower), Methodologie SS1 (truncated Neumann, Lemma 3.1), SS2 (mask).
#pragma once
#include "gdn_device.hpp"

namespace gdn {

enum : int { CMP_F32 = 0, CMP_BF16 = 1, CMP_FP8 = 2, CMP_INT8 = 3, CMP_INT16 = 4 };
enum : int { MODE_NEUMANN = 0, MODE_EXACT = 1, MODE_RESIDUAL = 2, MODE_FS = 3 };

template <int NT>
struct Mat {
  f32x4 t[NT][NT];  // only lower tiles I >= J are meaningful
};

template <int NT>
__device__ __forceinline__ f32x4 tile_or_zero(const Mat<NT>& M, int I, int J) {
  return (I < NT && J < NT && I >= J) ? M.t[I][J] : zero4();
}

// identity 16x16 tile, same in D-form and T-form: element (4g + r, c)
__device__ __forceinline__ f32x4 eye_tile() {
  const int l = lane_id(), g = l >> 4, c = l & 15;
  f32x4 e;
#pragma unroll
  for (int r = 0; r < 4; ++r) e[r] = (4 * g + r == c) ? 1.f : 0.f;
  return e;
}

// per-lane gate / beta values at the two index families a lane touches
template <int NT>
struct Gates {
  float Gl, bl;      // this lane's G and beta (lane l = chunk position l)
  bool split;        // exp(-G) finite for the whole block (min G >= -80)
  float rc[NT];      // -beta exp(G) at 16X + c      (row factor of A, T-form)
  float nc[NT];      // exp(-G) at 16X + c           (column factor of A, D-form)
  float rr[NT][4];   // -beta exp(G) at 16X + 4g + r (row factor of A, D-form)
  float nr[NT][4];   // exp(-G) at 16X + 4g + r      (column factor of A, T-form)
};

// gather G, beta and the two exponentials of G to a lane's index families
template <int NT>
__device__ __forceinline__ void gather_gates(float Gl, float bl, Gates<NT>& gt) {
  const int l = lane_id(), grp = l >> 4, c = l & 15;
  // split factors (used when exp(-G) stays finite, else the element-wise fallback
  // of gram_to_A gathers G and beta itself)
  gt.Gl = Gl;
  gt.bl = bl;
  gt.split = wave_min(Gl) >= -80.f;
  const float rl = -bl * __expf(Gl), nl = __expf(-Gl);
  float rb[4], nb[4];
  row_broadcasts(rl, rb);
  row_broadcasts(nl, nb);
#pragma unroll
  for (int X = 0; X < NT; ++X) {
    gt.rc[X] = rb[X];
    gt.nc[X] = nb[X];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ir = 16 * X + 4 * grp + r;
      gt.rr[X][r] = __shfl(rl, ir, 64);
      gt.nr[X][r] = __shfl(nl, ir, 64);
    }
  }
}

// G = inclusive in-chunk cumsum of gamma (unless already cumulative), then gathered
// to the index families.  beta, g point at this block's C values.
template <int NT>
__device__ __forceinline__ void load_gates(const float* __restrict__ beta,
                                           const float* __restrict__ g, bool g_cumulative,
                                           Gates<NT>& gt) {
  constexpr int C = 16 * NT;
  const int l = lane_id(), grp = l >> 4, c = l & 15;
  float gl = (l < C) ? g[l] : 0.f;
  float Gl = g_cumulative ? gl : wave_inclusive_scan(gl);
  float bl = (l < C) ? beta[l] : 0.f;
  gather_gates<NT>(Gl, bl, gt);
}

// S = K K^T over all NT x NT tiles in D-form (S[I][J] lane (g,c) reg r =
// (K K^T)[16I + 4g + r][16J + c]).  K points at the block's [C][dk] rows.
// bf16 K: 16x16x32 bf16 MFMA over 32-wide d slices (lane reads 16 contiguous bytes).
template <int NT, int DK>
__device__ __forceinline__ void gram_bf16(const __bf16* __restrict__ K, Mat<NT>& S) {
  constexpr int NS = DK / 32;
  const int l = lane_id(), g = l >> 4, c = l & 15;
  bf16x8 kf[NT][NS];
#pragma unroll
  for (int I = 0; I < NT; ++I)
#pragma unroll
    for (int s = 0; s < NS; ++s)
      kf[I][s] = __builtin_nontemporal_load(
          reinterpret_cast<const bf16x8*>(K + (size_t)(16 * I + c) * DK + 32 * s + 8 * g));
#pragma unroll
  for (int I = 0; I < NT; ++I)
#pragma unroll
    for (int J = 0; J < NT; ++J) {
      f32x4 acc = zero4();
#pragma unroll
      for (int s = 0; s < NS; ++s) acc = mma_bf16(kf[I][s], kf[J][s], acc);
      S.t[I][J] = acc;
    }
}

// fp32 K: 16x16x4 f32 MFMA; lane (g,c) reads K[16I + c][16s + 4g .. +3] and uses
// component u in sub-step u (slot g of sub-step u <-> d = 16s + 4g + u).
template <int NT, int DK>
__device__ __forceinline__ void gram_f32(const float* __restrict__ K, Mat<NT>& S) {
  constexpr int NS = DK / 16;
  const int l = lane_id(), g = l >> 4, c = l & 15;
#pragma unroll
  for (int I = 0; I < NT; ++I)
#pragma unroll
    for (int J = 0; J < NT; ++J) S.t[I][J] = zero4();
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    f32x4 kf[NT];
#pragma unroll
    for (int I = 0; I < NT; ++I)
      kf[I] = __builtin_nontemporal_load(
          reinterpret_cast<const f32x4*>(K + (size_t)(16 * I + c) * DK + 16 * s + 4 * g));
#pragma unroll
    for (int I = 0; I < NT; ++I)
#pragma unroll
      for (int J = 0; J < NT; ++J)
#pragma unroll
        for (int u = 0; u < 4; ++u) S.t[I][J] = mma_f32(kf[I][u], kf[J][u], S.t[I][J]);
  }
}

// ---- raw per-block inputs, loaded separately from their use so that a wave can
// prefetch the next block while it computes the current one --------------------

// K rows as 16x16x32 operand fragments (lane (g,c): K[16I + c][32s + 8g .. +7]) plus
// this lane's gate and beta (lane l holds position l of the chunk, l < C)
template <int NT, int DK>
struct KBlock {
  bf16x8 kf[NT][DK / 32];
  float gl, bl;
};

// GATES_FIRST: the gate inputs are loaded before the key rows (loads complete in order),
// so the gate factors can be formed while the keys are still arriving
// ORDERED: the loads are issued in program order (gates, then key row tile 0, 1, ...),
// for a consumer that starts on the first row tiles while the rest still arrive
template <int NT, int DK, bool NT_LOAD = false, bool GATES_FIRST = false, bool ORDERED = false>
__device__ __forceinline__ void load_kblock(const __bf16* __restrict__ K,
                                            const float* __restrict__ beta,
                                            const float* __restrict__ g, KBlock<NT, DK>& kb) {
  constexpr int C = 16 * NT;
  const int l = lane_id(), grp = l >> 4, c = l & 15;
  if constexpr (GATES_FIRST) {
    kb.gl = (l < C) ? g[l] : 0.f;
    kb.bl = (l < C) ? beta[l] : 0.f;
    if constexpr (ORDERED) __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int I = 0; I < NT; ++I) {
#pragma unroll
    for (int s = 0; s < DK / 32; ++s)
      {
        const bf16x8* src = reinterpret_cast<const bf16x8*>(K + (size_t)(16 * I + c) * DK + 32 * s + 8 * grp);
        // streaming (non-temporal) when nothing reads these rows again
        kb.kf[I][s] = NT_LOAD ? __builtin_nontemporal_load(src) : *src;
      }
    if constexpr (ORDERED) __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (!GATES_FIRST) {
    kb.gl = (l < C) ? g[l] : 0.f;
    kb.bl = (l < C) ? beta[l] : 0.f;
  }
}

// gate cumsum and gather to the two index families from the raw lane values
template <int NT>
__device__ __forceinline__ void gates_from_lanes(float gl, float bl, bool g_cumulative,
                                                 Gates<NT>& gt) {
  float Gl = g_cumulative ? gl : wave_inclusive_scan(gl);
  gather_gates<NT>(Gl, bl, gt);
}

// Gram tiles from preloaded fragments (D-form), only tiles with |I - J| <= MAXD, and of
// those only the ones A's rows ILO .. IHI are formed from
template <int NT, int DK, int MAXD = NT - 1, int ILO = 0, int IHI = NT - 1>
__device__ __forceinline__ void gram_from_frags(const KBlock<NT, DK>& kb, Mat<NT>& S) {
  constexpr bool ALL = ILO == 0 && IHI == NT - 1;
#pragma unroll
  for (int I = 0; I < NT; ++I)
#pragma unroll
    for (int J = 0; J < NT; ++J) {
      if (I - J > MAXD || J - I > MAXD) {
        if constexpr (ALL) S.t[I][J] = zero4();
        continue;
      }
      const int row = I > J ? I : J;  // tile (I, J) and its mirror serve A's row `row`
      if (row < ILO || row > IHI) continue;
      f32x4 acc = zero4();
#pragma unroll
      for (int s = 0; s < DK / 32; ++s) acc = mma_bf16(kb.kf[I][s], kb.kf[J][s], acc);
      S.t[I][J] = acc;
    }
}

// A given in memory: raw lower tiles in both forms
template <int NT>
struct ABlock {
  f32x4 t[NT][NT];  // T-form reads (row 16I + c, cols 16J + 4g .. +3)
  f32x4 d[NT][NT];  // D-form reads (rows 16I + 4g + r, col 16J + c)
};

template <int NT>
__device__ __forceinline__ void load_ablock(const float* __restrict__ A, ABlock<NT>& ab) {
  constexpr int C = 16 * NT;
  const int l = lane_id(), g = l >> 4, c = l & 15;
#pragma unroll
  for (int I = 0; I < NT; ++I)
#pragma unroll
    for (int J = 0; J <= I; ++J) {
      ab.t[I][J] = *reinterpret_cast<const f32x4*>(A + (size_t)(16 * I + c) * C + 16 * J + 4 * g);
#pragma unroll
      for (int r = 0; r < 4; ++r) ab.d[I][J][r] = A[(size_t)(16 * I + 4 * g + r) * C + 16 * J + c];
    }
}

// strict-lower and band masking of the raw A tiles
template <int NT, int MAXD, bool BANDED>
__device__ __forceinline__ void ablock_to_A(const ABlock<NT>& ab, int band, Mat<NT>& AD,
                                            Mat<NT>& AT);

// Lane-dependent part of (row - col) for an element of a 16x16 tile:
//   D-form: i - j = 16(I - J) + r + lane_off,  T-form: i - j = 16(I - J) - r - lane_off,
// with lane_off = 4g - c.  Masks compare against it instead of rebuilding indices.
__device__ __forceinline__ int lane_off() {
  const int l = lane_id();
  return 4 * (l >> 4) - (l & 15);
}

// keep element iff lo <= (i - j) <= hi; tile-level uniform checks skip whole tiles
template <int NT>
__device__ __forceinline__ f32x4 band_select_D(f32x4 v, int IJ, int lo, int hi) {
  const int lo_ = lane_off();
  f32x4 o;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    int d = 16 * IJ + r + lo_;
    o[r] = (d >= lo && d <= hi) ? v[r] : 0.f;
  }
  return o;
}
template <int NT>
__device__ __forceinline__ f32x4 band_select_T(f32x4 v, int IJ, int lo, int hi) {
  const int lo_ = lane_off();
  f32x4 o;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    int d = 16 * IJ - r - lo_;
    o[r] = (d >= lo && d <= hi) ? v[r] : 0.f;
  }
  return o;
}

template <int NT, int MAXD = NT - 1, bool BANDED = false>
__device__ __forceinline__ void ablock_to_A(const ABlock<NT>& ab, int band, Mat<NT>& AD,
                                            Mat<NT>& AT) {
  const int hi = band < 0 ? (1 << 30) : band;
#pragma unroll
  for (int I = 0; I < NT; ++I)
#pragma unroll
    for (int J = 0; J <= I; ++J) {
      if (I - J > MAXD) {
        AD.t[I][J] = zero4();
        AT.t[I][J] = zero4();
      } else if (BANDED || I == J) {
        AD.t[I][J] = band_select_D<NT>(ab.d[I][J], I - J, 1, hi);
        AT.t[I][J] = band_select_T<NT>(ab.t[I][J], I - J, 1, hi);
      } else {
        AD.t[I][J] = ab.d[I][J];
        AT.t[I][J] = ab.t[I][J];
      }
    }
}

// ---- band-masked sum with N <= 3 ([GEO] Methodologie SS2, the band mask) ---------
// Inside the band (0 < i - j <= N) every chain i > m > ... > j of the power series has
// at most i - j <= N steps, so there the masked truncated sum is the exact inverse, and
// outside it T - I is zero.  With a_d(i) = A[i][i - d] (zero where i - d < 0 or d > N)
// the band is
//   t_1(i) = a_1(i)
//   t_2(i) = a_2(i) + a_1(i) a_1(i-1)
//   t_3(i) = a_3(i) + a_1(i) a_2(i-1) + a_2(i) a_1(i-2) + a_1(i) a_1(i-1) a_1(i-2),
// formed element by element in fp32 with lane i holding row i.
constexpr int XR_LD = 20;  // LDS row of the Gram band: 4 columns left of the tile + 16

// lane i receives lane i - 1's x, lane 0 receives 0 (DPP wave_shr:1, across the rows)
__device__ __forceinline__ float lane_shr1(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x138, 0xf, 0xf, false));
}

// ad[d] = a_d(lane) for d = 1..3 -> t[d] = t_d(lane); t_d = 0 for d > N
__device__ __forceinline__ void band3_from_subdiag(const float (&ad)[4], int N, float (&t)[4]) {
  const float a1m1 = lane_shr1(ad[1]), a1m2 = lane_shr1(a1m1), a2m1 = lane_shr1(ad[2]);
  t[0] = 0.f;
  t[1] = N >= 1 ? ad[1] : 0.f;
  t[2] = N >= 2 ? ad[2] + ad[1] * a1m1 : 0.f;
  t[3] = N >= 3 ? ad[3] + ad[1] * a2m1 + ad[2] * a1m2 + ad[1] * a1m1 * a1m2 : 0.f;
}

// Gram entries S[i][i - d] (d = 1..3, rows i < 16 NT) from preloaded fragments: the
// diagonal tiles and the tile left of each in T-form (lane (g,c) reg r: row 16I + c,
// column 16J + 4g + r; the left tile's group g = 3 holds columns 16I - 4 .. 16I - 1)
// go to xr[row][4 ..] and xr[row][0 .. 3]; lane i then reads its row.  Entries with
// i - d < 0 are garbage (never written) and must be discarded by the caller.
template <int NT, int DK>
__device__ __forceinline__ void gram_band3(const bf16x8 (&kf)[NT][DK / 32], float (&xr)[64][XR_LD],
                                           float (&sv)[4]) {
  const int l = lane_id(), g = l >> 4, c = l & 15;
#pragma unroll
  for (int I = 0; I < NT; ++I) {
    f32x4 d = zero4();
#pragma unroll
    for (int p = 0; p < DK / 32; ++p) d = mma_bf16(kf[I][p], kf[I][p], d);
    *reinterpret_cast<f32x4*>(&xr[16 * I + c][4 + 4 * g]) = d;
    if (I > 0) {
      f32x4 e = zero4();
#pragma unroll
      for (int p = 0; p < DK / 32; ++p) e = mma_bf16(kf[I - 1][p], kf[I][p], e);
      if (g == 3) *reinterpret_cast<f32x4*>(&xr[16 * I + c][0]) = e;
    }
  }
  sv[0] = 0.f;
#pragma unroll
  for (int d = 1; d <= 3; ++d) sv[d] = xr[l][4 + c - d];
}

// A from the Gram tiles: AD (D-form) and AT (T-form), strictly lower.  With BANDED
// the band mask (keep i - j <= band, band < 0 = none) is applied too.  The gate factor
// is split as exp(G_i - G_j) = exp(G_i) exp(-G_j) when every exp(-G) of the block is
// finite (G >= -80); otherwise each element takes exp of the difference.
template <int NT, int MAXD = NT - 1, bool BANDED = false, int ILO = 0, int IHI = NT - 1>
__device__ __forceinline__ void gram_to_A(const Mat<NT>& S, const Gates<NT>& gt, int band,
                                          Mat<NT>& AD, Mat<NT>& AT) {
  const int hi = band < 0 ? (1 << 30) : band;
  const bool split = gt.split;
  const int lane = lane_id(), grp = lane >> 4, cl = lane & 15;
#pragma unroll
  for (int I = ILO; I <= IHI; ++I)
#pragma unroll
    for (int J = 0; J <= I; ++J) {
      if (I - J > MAXD || (BANDED && 16 * (I - J) - 15 > hi)) {  // tile outside (uniform)
        AD.t[I][J] = zero4();
        AT.t[I][J] = zero4();
        continue;
      }
      f32x4 d, t;
      if (split) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          d[r] = gt.rr[I][r] * S.t[I][J][r] * gt.nc[J];
          t[r] = gt.rc[I] * S.t[J][I][r] * gt.nr[J][r];
        }
      } else {
        const float GcI = __shfl(gt.Gl, 16 * I + cl, 64), bcI = __shfl(gt.bl, 16 * I + cl, 64);
        const float GcJ = __shfl(gt.Gl, 16 * J + cl, 64);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float GrI = __shfl(gt.Gl, 16 * I + 4 * grp + r, 64);
          const float brI = __shfl(gt.bl, 16 * I + 4 * grp + r, 64);
          const float GrJ = __shfl(gt.Gl, 16 * J + 4 * grp + r, 64);
          d[r] = -brI * __expf(GrI - GcJ) * S.t[I][J][r];
          t[r] = -bcI * __expf(GcI - GrJ) * S.t[J][I][r];
        }
      }
      if (BANDED || I == J) {
        AD.t[I][J] = band_select_D<NT>(d, I - J, 1, hi);
        AT.t[I][J] = band_select_T<NT>(t, I - J, 1, hi);
      } else {
        AD.t[I][J] = d;
        AT.t[I][J] = t;
      }
    }
}

// band mask on a D-form / T-form matrix (keep i - j <= band)
template <int NT>
__device__ __forceinline__ void mask_D(Mat<NT>& M, int band) {
#pragma unroll
  for (int I = 0; I < NT; ++I)
#pragma unroll
    for (int J = 0; J <= I; ++J) {
      if (16 * (I - J) + 15 <= band) continue;  // whole tile inside the band
      if (16 * (I - J) - 15 > band) {
        M.t[I][J] = zero4();
        continue;
      }
      M.t[I][J] = band_select_D<NT>(M.t[I][J], I - J, -(1 << 30), band);
    }
}
template <int NT, int ILO = 0, int IHI = NT - 1>
__device__ __forceinline__ void mask_T(Mat<NT>& M, int band) {
#pragma unroll
  for (int I = ILO; I <= IHI; ++I)
#pragma unroll
    for (int J = 0; J <= I; ++J) {
      if (16 * (I - J) + 15 <= band) continue;
      if (16 * (I - J) - 15 > band) {
        M.t[I][J] = zero4();
        continue;
      }
      M.t[I][J] = band_select_T<NT>(M.t[I][J], I - J, -(1 << 30), band);
    }
}

template <int NT>
__device__ __forceinline__ void add_eye(Mat<NT>& M) {
  const f32x4 e = eye_tile();
#pragma unroll
  for (int I = 0; I < NT; ++I) M.t[I][I] += e;
}

// ---- products of lower-triangular matrices -----------------------------------
// Z = X Y (+ I when EYE) for lower-triangular X (given in T-form, XT) and Y (given in
// D-form, YD).  TFORM = false: Z in D-form; TFORM = true: Z in T-form.  Only tiles
// with I - J <= MAXD are formed (the others are set to zero): with MAXD < NT - 1 the
// caller guarantees that X and Y vanish beyond that tile distance and that the
// result is band-masked afterwards, so no kept entry depends on a skipped tile.
// The tile sum runs over the k-pairs p with J/2 <= p <= I/2.

template <int NT>
__device__ __forceinline__ f32x4 tile_init(int I, int J, bool eye) {
  return (eye && I == J) ? eye_tile() : zero4();
}

template <int NT, bool TFORM, int MAXD, bool EYE, int ILO = 0, int IHI = NT - 1>
__device__ __forceinline__ void lmul_bf16(const Mat<NT>& XT, const Mat<NT>& YD, Mat<NT>& Z) {
  constexpr int NP = (NT + 1) / 2;
  bf16x8 rp[NT][NP], cp[NP][NT];
#pragma unroll
  for (int I = 0; I < NT; ++I)
#pragma unroll
    for (int p = 0; p < NP; ++p)
      if (2 * p <= I && I - (2 * p + 1) <= MAXD)
        rp[I][p] = pack8(tile_or_zero(XT, I, 2 * p), tile_or_zero(XT, I, 2 * p + 1));
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int J = 0; J < NT; ++J)
      if (J <= 2 * p + 1 && 2 * p - J <= MAXD)
        cp[p][J] = pack8(tile_or_zero(YD, 2 * p, J), tile_or_zero(YD, 2 * p + 1, J));
  // output rows ILO .. IHI only (the packs no such row reads are never formed)
#pragma unroll
  for (int I = ILO; I <= IHI; ++I)
#pragma unroll
    for (int J = 0; J <= I; ++J) {
      if (I - J > MAXD) {
        Z.t[I][J] = zero4();
        continue;
      }
      f32x4 acc = tile_init<NT>(I, J, EYE);
#pragma unroll
      for (int p = J / 2; p <= I / 2; ++p)
        acc = TFORM ? mma_bf16(cp[p][J], rp[I][p], acc) : mma_bf16(rp[I][p], cp[p][J], acc);
      Z.t[I][J] = acc;
    }
}

template <int NT, bool TFORM, int MAXD, bool EYE>
__device__ __forceinline__ void lmul_f32(const Mat<NT>& XT, const Mat<NT>& YD, Mat<NT>& Z) {
#pragma unroll
  for (int I = 0; I < NT; ++I)
#pragma unroll
    for (int J = 0; J <= I; ++J) {
      if (I - J > MAXD) {
        Z.t[I][J] = zero4();
        continue;
      }
      f32x4 acc = tile_init<NT>(I, J, EYE);
#pragma unroll
      for (int K = J; K <= I; ++K)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          acc = TFORM ? mma_f32(YD.t[K][J][u], XT.t[I][K][u], acc)
                      : mma_f32(XT.t[I][K][u], YD.t[K][J][u], acc);
      Z.t[I][J] = acc;
    }
}

template <int NT, int CMP, bool TFORM, int MAXD = NT - 1, bool EYE = false>
__device__ __forceinline__ void lmul(const Mat<NT>& XT, const Mat<NT>& YD, Mat<NT>& Z) {
  if constexpr (CMP == CMP_F32)
    lmul_f32<NT, TFORM, MAXD, EYE>(XT, YD, Z);
  else
    lmul_bf16<NT, TFORM, MAXD, EYE>(XT, YD, Z);
}

// ---- fp8 (e4m3) variant of the product, with per-block absmax scales ----------

struct Fp8Counts {
  uint32_t nonfinite, sat_dyn, sat_static, underflow;
};

// quantise 8 values (two tiles) to e4m3 codes with scale 1/inv_s applied first
__device__ __forceinline__ long quant8(const f32x4& lo, const f32x4& hi, float inv_s) {
  uint32_t w0 = cvt_fp8x2<false>(fminf(fmaxf(lo[0] * inv_s, -FP8_MAX), FP8_MAX),
                                 fminf(fmaxf(lo[1] * inv_s, -FP8_MAX), FP8_MAX), 0u);
  w0 = cvt_fp8x2<true>(fminf(fmaxf(lo[2] * inv_s, -FP8_MAX), FP8_MAX),
                       fminf(fmaxf(lo[3] * inv_s, -FP8_MAX), FP8_MAX), w0);
  uint32_t w1 = cvt_fp8x2<false>(fminf(fmaxf(hi[0] * inv_s, -FP8_MAX), FP8_MAX),
                                 fminf(fmaxf(hi[1] * inv_s, -FP8_MAX), FP8_MAX), 0u);
  w1 = cvt_fp8x2<true>(fminf(fmaxf(hi[2] * inv_s, -FP8_MAX), FP8_MAX),
                       fminf(fmaxf(hi[3] * inv_s, -FP8_MAX), FP8_MAX), w1);
  return (long)(((uint64_t)w1 << 32) | (uint64_t)w0);
}

// count diagnostics of quantising the lower tiles of M (those within MAXD tile-diagonals
// of the main one; the rest are zero and count nothing) under the reciprocal scales
// inv_s (dynamic) and inv_st (static), per lane, element by element
__device__ __forceinline__ void fp8_count1(float x, float inv_s, float inv_st, Fp8Counts& cnt) {
  constexpr float UNDER = 0.0009765625f;  // 2^-10: half the smallest e4m3 subnormal
  const float a = fabsf(x);
  const bool fin = __builtin_isfinite(x);
  cnt.nonfinite += fin ? 0u : 1u;
  cnt.sat_dyn += (fin && a * inv_s >= FP8_SAT) ? 1u : 0u;
  cnt.sat_static += (fin && a * inv_st >= FP8_SAT) ? 1u : 0u;
  cnt.underflow += (fin && x != 0.f && a * inv_s <= UNDER) ? 1u : 0u;
}

template <int NT, int MAXD>
__device__ __forceinline__ void fp8_count(const Mat<NT>& M, float inv_s, float inv_st, Fp8Counts& cnt) {
#pragma unroll
  for (int I = 0; I < NT; ++I)
#pragma unroll
    for (int J = 0; J <= I; ++J) {
      if (I - J > MAXD) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) fp8_count1(M.t[I][J][r], inv_s, inv_st, cnt);
    }
}

// the wave's counters added to stats[0..3] (one atomic per counter and wave)
__device__ __forceinline__ void flush_counts(const Fp8Counts& cnt, unsigned long long* stats) {
  const uint32_t v0 = wave_sum_u32(cnt.nonfinite), v1 = wave_sum_u32(cnt.sat_dyn);
  const uint32_t v2 = wave_sum_u32(cnt.sat_static), v3 = wave_sum_u32(cnt.underflow);
  if (lane_id() == 0) {
    if (v0) atomicAdd(stats + 0, (unsigned long long)v0);
    if (v1) atomicAdd(stats + 1, (unsigned long long)v1);
    if (v2) atomicAdd(stats + 2, (unsigned long long)v2);
    if (v3) atomicAdd(stats + 3, (unsigned long long)v3);
  }
}

// block absmax of the lower tiles within MAXD tile-diagonals (a NaN never becomes the
// maximum: fmaxf returns the other operand)
template <int NT, int MAXD = NT - 1>
__device__ __forceinline__ float absmax(const Mat<NT>& M) {
  float m = 0.f;
#pragma unroll
  for (int I = 0; I < NT; ++I)
#pragma unroll
    for (int J = 0; J <= I; ++J) {
      if (I - J > MAXD) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(M.t[I][J][r]));
    }
  return wave_max(m);
}

__device__ __forceinline__ float fp8_scale(float amax) {
  return (amax > 0.f && __builtin_isfinite(amax)) ? amax / FP8_MAX : 1.f;
}

// The scale absmax/448 of M and, when count is set, the four counters of quantising M
// under it and under the static scale s_static (s_static <= 0: M's own scale).
// Counting element by element is skipped when block-wide aggregates show that every
// counter is zero; this is exact, because a correctly rounded product a * c (c > 0) does
// not decrease as a grows:
//   - every element finite (x * 0 + acc stays 0 unless some x is infinite or NaN);
//   - absmax * inv < 464 for both scales: no finite |x| <= absmax reaches 464;
//   - the smallest non-zero |x| times inv_s exceeds 2^-10: no non-zero |x| underflows.
// The smallest non-zero magnitude comes from an unsigned minimum over
// (bits(x) << 1) - 1, which drops the sign and sends both zeros to the largest value.
template <int NT, int MAXD>
__device__ __forceinline__ float fp8_scale_count(const Mat<NT>& M, float s_static, Fp8Counts& cnt, bool count) {
  constexpr float UNDER = 0.0009765625f;
  float m = 0.f, nf = 0.f;
  uint32_t mn = 0xffffffffu;
#pragma unroll
  for (int I = 0; I < NT; ++I)
#pragma unroll
    for (int J = 0; J <= I; ++J) {
      if (I - J > MAXD) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x = M.t[I][J][r];
        m = fmaxf(m, fabsf(x));
        if (count) {
          nf = __builtin_fmaf(x, 0.f, nf);
          mn = min(mn, (__builtin_bit_cast(uint32_t, x) << 1) - 1u);
        }
      }
    }
  const float amax = wave_max(m);
  const float s = fp8_scale(amax);
  if (count) {
    const float inv_s = 1.f / s, inv_st = 1.f / (s_static > 0.f ? s_static : s);
    const uint32_t mnw = wave_min_u32(mn);
    bool quiet = wave_all(nf == 0.f) && amax * inv_s < FP8_SAT && amax * inv_st < FP8_SAT;
    if (mnw != 0xffffffffu) quiet = quiet && __builtin_bit_cast(float, (mnw + 1u) >> 1) * inv_s > UNDER;
    if (!quiet) fp8_count<NT, MAXD>(M, inv_s, inv_st, cnt);
  }
  return s;
}

// fake-quantise the lower tiles of M within MAXD tile-diagonals (x -> s * q(x / s))
template <int NT, int MAXD = NT - 1>
__device__ __forceinline__ void fp8_roundtrip(Mat<NT>& M, float s) {
  const float inv_s = 1.f / s;
#pragma unroll
  for (int I = 0; I < NT; ++I)
#pragma unroll
    for (int J = 0; J <= I; ++J) {
      if (I - J > MAXD) continue;
      long q = quant8(M.t[I][J], zero4(), inv_s);
      uint32_t w = (uint32_t)(uint64_t)q;
      M.t[I][J][0] = fp8_to_f32<0>(w) * s;
      M.t[I][J][1] = fp8_to_f32<1>(w) * s;
      M.t[I][J][2] = fp8_to_f32<2>(w) * s;
      M.t[I][J][3] = fp8_to_f32<3>(w) * s;
    }
}

// ---- the masked fp8 chain for N <= 3 in band form (lane i = row i of a 64-row block) --
// [GEO] "Adaptation a la Quantification" with the band mask of Methodologie SS2.  With the
// mask, A and every X_k live on sub-diagonals 1..N, so the chain of neumann_T_fp8 needs
// only x_d(i) = X[i][i - d], d <= 3: the same scales (absmax / 448 over the block, here a
// wave reduction), the same e4m3 codes and counters, and X_{k+1} = A' + s_A s_X (q(A) q(X_k))
// with
//   (q(A) q(X))[i][i-1] = 0,
//   (q(A) q(X))[i][i-2] = qa_1(i) qx_1(i-1),
//   (q(A) q(X))[i][i-3] = qa_1(i) qx_2(i-1) + qa_2(i) qx_1(i-2).
// A product of two e4m3 values is exact in fp32, so one fused multiply-add over the exact
// second product rounds the exact sum once: the oracle's arithmetic, bit for bit.

// e4m3 code values (as fp32 numbers, before scaling back) of x1..x3 under the reciprocal
// scale inv: clamp to +-448, then the hardware's round-to-nearest-even conversion
__device__ __forceinline__ void fp8_code3(float x1, float x2, float x3, float inv, float& q1, float& q2,
                                          float& q3) {
  const float y1 = fminf(fmaxf(x1 * inv, -FP8_MAX), FP8_MAX);
  const float y2 = fminf(fmaxf(x2 * inv, -FP8_MAX), FP8_MAX);
  const float y3 = fminf(fmaxf(x3 * inv, -FP8_MAX), FP8_MAX);
  const uint32_t w = cvt_fp8x2<true>(y3, 0.f, cvt_fp8x2<false>(y1, y2, 0u));
  q1 = fp8_to_f32<0>(w);
  q2 = fp8_to_f32<1>(w);
  q3 = fp8_to_f32<2>(w);
}

// the scale absmax / 448 of a band tensor (x1..x3 on every lane) and, when count is set,
// its four counters under that scale and under s_static (<= 0: its own)
__device__ __forceinline__ float band_scale_count(float x1, float x2, float x3, float s_static, Fp8Counts& cnt,
                                                  bool count) {
  const float s = fp8_scale(wave_max(fmaxf(fmaxf(fabsf(x1), fabsf(x2)), fabsf(x3))));
  if (count) {
    const float inv_s = 1.f / s, inv_st = 1.f / (s_static > 0.f ? s_static : s);
    fp8_count1(x1, inv_s, inv_st, cnt);
    fp8_count1(x2, inv_s, inv_st, cnt);
    fp8_count1(x3, inv_s, inv_st, cnt);
  }
  return s;
}

// ad[d] = A[i][i - d] for d = 1..3 (zero where i - d < 0 or d > N), 1 <= N <= 3 ->
// t[d] = (T - I)[i][i - d]
__device__ __forceinline__ void band3_fp8(const float (&ad)[4], int N, float (&t)[4], Fp8Counts& cnt, bool count) {
  const float sA = band_scale_count(ad[1], ad[2], ad[3], 0.f, cnt, count);
  float qa1, qa2, qa3;
  fp8_code3(ad[1], ad[2], ad[3], 1.f / sA, qa1, qa2, qa3);
  const float ap1 = qa1 * sA, ap2 = qa2 * sA, ap3 = qa3 * sA;  // A' = s_A q(A)
  float x1 = ap1, x2 = ap2, x3 = ap3;                            // X_1 = A'
  for (int k = 1; k < N; ++k) {
    const float sX = band_scale_count(x1, x2, x3, sA, cnt, count);
    const float sxy = sA * sX;
    float qx1, qx2, qx3;
    fp8_code3(x1, x2, x3, 1.f / sX, qx1, qx2, qx3);
    const float qx1m1 = lane_shr1(qx1), qx1m2 = lane_shr1(qx1m1), qx2m1 = lane_shr1(qx2);
    const float p2 = qa1 * qx1m1;
    const float p3 = __builtin_fmaf(qa2, qx1m2, qa1 * qx2m1);
    x1 = __builtin_fmaf(0.f, sxy, ap1);
    x2 = __builtin_fmaf(p2, sxy, ap2);
    x3 = N >= 3 ? __builtin_fmaf(p3, sxy, ap3) : 0.f;
  }
  // T - I = s_T q(X_N), or A' itself for N = 1
  float t1 = ap1, t2 = 0.f, t3 = 0.f;
  if (N >= 2) {
    const float sT = band_scale_count(x1, x2, x3, sA, cnt, count);
    float q1, q2, q3;
    fp8_code3(x1, x2, x3, 1.f / sT, q1, q2, q3);
    t1 = q1 * sT;
    t2 = q2 * sT;
    t3 = q3 * sT;
  }
  t[0] = 0.f;
  t[1] = t1;
  t[2] = t2;
  t[3] = t3;
}

// ---- int8 variant: per-block power-of-two scales, int32 accumulation ----------
// [GEO] "Adaptation a la Quantification" runs the power chain on INT8 operands.  Codes
// are round_half_even(x / 2^e) with one scale 2^e per block and operand, e the smallest
// integer with max|x| <= 127 2^e.  Every scaling is by a power of two and so exact;
// the products of codes are exact in int32 (|sum| <= 64 * 127^2 < 2^24).

typedef int i32x4 __attribute__((ext_vector_type(4)));

// amax = m 2^E with m in [0.5, 1): 127 2^(E-7) = (127/128) 2^E covers amax iff
// m <= 127/128, else 127 2^(E-6) does; 127 2^(E-8) < 2^(E-1) <= amax never does.
__device__ __forceinline__ int i8_exponent(float amax) {
  if (!(amax > 0.f) || !__builtin_isfinite(amax)) return 0;
  int E;
  const float m = frexpf(amax, &E);
  return (m <= 127.f / 128.f) ? E - 7 : E - 6;
}

// int8 codes of one tile's 4 registers, packed in register order (byte r = register r)
__device__ __forceinline__ int q8x4(const f32x4& v, int neg_e) {
  uint32_t w = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int q = (int)__builtin_rintf(ldexpf(v[r], neg_e));
    w |= ((uint32_t)q & 0xffu) << (8 * r);
  }
  return (int)w;
}

// x -> round(x / 2^e) 2^e on the lower tiles (the dequantised operand)
template <int NT>
__device__ __forceinline__ void i8_roundtrip(Mat<NT>& M, int e) {
#pragma unroll
  for (int I = 0; I < NT; ++I)
#pragma unroll
    for (int J = 0; J <= I; ++J)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        M.t[I][J][r] = ldexpf(__builtin_rintf(ldexpf(M.t[I][J][r], -e)), e);
}

// One 16x16x64 int8 MFMA covers the whole contraction of a 64-wide block.  Slot map:
// byte 4K + r of lane (g, c) <-> k = 16K + 4g + r, so the T-form tiles (I, 0..3) of A
// give A's left fragment for row tile I and the D-form tiles (0..3, J) of X give X's
// right fragment for column tile J (tiles beyond the block or above the diagonal are
// zero codes).
template <int NT>
__device__ __forceinline__ i32x4 i8_rowfrag(const Mat<NT>& XT, int I, int neg_e) {
  i32x4 f;
#pragma unroll
  for (int K = 0; K < 4; ++K) f[K] = q8x4(tile_or_zero(XT, I, K), neg_e);
  return f;
}
template <int NT>
__device__ __forceinline__ i32x4 i8_colfrag(const Mat<NT>& YD, int J, int neg_e) {
  i32x4 f;
#pragma unroll
  for (int K = 0; K < 4; ++K) f[K] = q8x4(tile_or_zero(YD, K, J), neg_e);
  return f;
}

__device__ __forceinline__ i32x4 mma_i8(const i32x4& a, const i32x4& b) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, i32x4{0, 0, 0, 0}, 0, 0, 0);
}

// Horner on X = H - I:  X_1 = A',  X_{k+1} = A' + A' X_k,  T = I + X_N, with A' the
// dequantised A and every X_k quantised before its product; each sum is rounded once
// to fp32.  AD, AT arrive band-masked when the mask is on (the band sets the scales),
// and each X_k is masked before it is quantised.  C <= 64.
template <int NT, int MAXD = NT - 1>
__device__ __forceinline__ void neumann_T_i8(Mat<NT>& AD, Mat<NT>& AT, int N, bool mask, Mat<NT>& TT) {
  static_assert(NT <= 4, "one 64-wide MFMA contraction per tile");
  const int band = mask ? N : (1 << 30);
  const int eA = i8_exponent(absmax(AT));
  i8_roundtrip(AD, eA);
  i8_roundtrip(AT, eA);
  if (N <= 1) {
    TT = AT;
    add_eye(TT);
    return;
  }
  i32x4 ra[NT];
#pragma unroll
  for (int I = 0; I < NT; ++I) ra[I] = i8_rowfrag(AT, I, -eA);
  Mat<NT> X = AD;
  for (int k = 1; k < N; ++k) {
    const int eX = i8_exponent(absmax(X));
    i32x4 cx[NT];
#pragma unroll
    for (int J = 0; J < NT; ++J) cx[J] = i8_colfrag(X, J, -eX);
    const int es = eA + eX;
    const bool last = (k == N - 1);
#pragma unroll
    for (int I = 0; I < NT; ++I)
#pragma unroll
      for (int J = 0; J <= I; ++J) {
        if (I - J > MAXD) {
          (last ? TT : X).t[I][J] = zero4();
          continue;
        }
        if (last) {  // T-form: operands swapped
          const i32x4 p = mma_i8(cx[J], ra[I]);
#pragma unroll
          for (int r = 0; r < 4; ++r) TT.t[I][J][r] = AT.t[I][J][r] + ldexpf((float)p[r], es);
        } else {
          const i32x4 p = mma_i8(ra[I], cx[J]);
#pragma unroll
          for (int r = 0; r < 4; ++r) X.t[I][J][r] = AD.t[I][J][r] + ldexpf((float)p[r], es);
        }
      }
    if (mask) {
      if (last)
        mask_T(TT, band);
      else
        mask_D(X, band);
    }
  }
  add_eye(TT);
}

// ---- int16 variant: 16-bit codes as two signed 8-bit digits ------------------------
// [GEO] "Adaptation a la Quantification" names INT16 beside INT8; gfx950's integer matrix
// cores multiply 8-bit operands, so a 16-bit code q is carried as its balanced base-256
// digits q = 256 hi + lo, lo in [-128, 127].  Codes are limited to |q| <= 32639 = 127 * 257
// so that hi fits int8 as well; one power-of-two scale per block and operand, as for
// int8.  A product of codes is four 16x16x64 i8 MFMAs (hi hi, hi lo, lo hi, lo lo), each
// exact in int32, recombined exactly in fp64; A' + P 2^(eA + eX) is formed in fp64 and
// rounded to fp32 (two roundings, in that order, which fixes the result).

// smallest e with amax <= 32639 2^e: amax = m 2^E, m in [0.5, 1); 32639 2^(E-15) =
// (32639 / 32768) 2^E covers amax iff m <= 32639 / 32768, else 32639 2^(E-14) does
__device__ __forceinline__ int i16_exponent(float amax) {
  if (!(amax > 0.f) || !__builtin_isfinite(amax)) return 0;
  int E;
  const float m = frexpf(amax, &E);
  return (m <= 32639.f / 32768.f) ? E - 15 : E - 14;
}

// digits of one tile's 4 registers, packed in register order (byte r = register r)
__device__ __forceinline__ void q16x4(const f32x4& v, int neg_e, int& hw, int& lw) {
  uint32_t h = 0, lo = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int q = (int)__builtin_rintf(ldexpf(v[r], neg_e));
    const int ld = ((q + 128) & 255) - 128;
    const int hd = (q - ld) >> 8;
    h |= ((uint32_t)hd & 0xffu) << (8 * r);
    lo |= ((uint32_t)ld & 0xffu) << (8 * r);
  }
  hw = (int)h;
  lw = (int)lo;
}

template <int NT>
__device__ __forceinline__ void i16_rowfrag(const Mat<NT>& XT, int I, int neg_e, i32x4& hi, i32x4& lo) {
#pragma unroll
  for (int K = 0; K < 4; ++K) {
    int h, l;
    q16x4(tile_or_zero(XT, I, K), neg_e, h, l);
    hi[K] = h;
    lo[K] = l;
  }
}
template <int NT>
__device__ __forceinline__ void i16_colfrag(const Mat<NT>& YD, int J, int neg_e, i32x4& hi, i32x4& lo) {
#pragma unroll
  for (int K = 0; K < 4; ++K) {
    int h, l;
    q16x4(tile_or_zero(YD, K, J), neg_e, h, l);
    hi[K] = h;
    lo[K] = l;
  }
}

// out = fl32(fl64(base + P 2^es)) with P the product of the two digit fragments
__device__ __forceinline__ f32x4 i16_product(const i32x4& ah, const i32x4& al, const i32x4& bh, const i32x4& bl,
                                             const f32x4& base, int es) {
  const i32x4 hh = mma_i8(ah, bh), hl = mma_i8(ah, bl), lh = mma_i8(al, bh), ll = mma_i8(al, bl);
  f32x4 out;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const double p = (double)hh[r] * 65536.0 + (double)(hl[r] + lh[r]) * 256.0 + (double)ll[r];
    out[r] = (float)((double)base[r] + ldexp(p, es));
  }
  return out;
}

// Horner on X = H - I as neumann_T_i8, with 16-bit codes.  C <= 64.
template <int NT, int MAXD = NT - 1>
__device__ __forceinline__ void neumann_T_i16(Mat<NT>& AD, Mat<NT>& AT, int N, bool mask, Mat<NT>& TT) {
  static_assert(NT <= 4, "one 64-wide MFMA contraction per tile");
  const int band = mask ? N : (1 << 30);
  const int eA = i16_exponent(absmax(AT));
  i8_roundtrip(AD, eA);  // x -> round(x / 2^e) 2^e: the dequantised operand, any code width
  i8_roundtrip(AT, eA);
  if (N <= 1) {
    TT = AT;
    add_eye(TT);
    return;
  }
  i32x4 rh[NT], rl[NT];
#pragma unroll
  for (int I = 0; I < NT; ++I) i16_rowfrag(AT, I, -eA, rh[I], rl[I]);
  Mat<NT> X = AD;
  for (int k = 1; k < N; ++k) {
    const int eX = i16_exponent(absmax(X));
    i32x4 ch[NT], cl[NT];
#pragma unroll
    for (int J = 0; J < NT; ++J) i16_colfrag(X, J, -eX, ch[J], cl[J]);
    const int es = eA + eX;
    const bool last = (k == N - 1);
#pragma unroll
    for (int I = 0; I < NT; ++I)
#pragma unroll
      for (int J = 0; J <= I; ++J) {
        if (I - J > MAXD) {
          (last ? TT : X).t[I][J] = zero4();
          continue;
        }
        if (last)  // T-form: operands swapped
          TT.t[I][J] = i16_product(ch[J], cl[J], rh[I], rl[I], AT.t[I][J], es);
        else
          X.t[I][J] = i16_product(rh[I], rl[I], ch[J], cl[J], AD.t[I][J], es);
      }
    if (mask) {
      if (last)
        mask_T(TT, band);
      else
        mask_D(X, band);
    }
  }
  add_eye(TT);
}

// ---- the two inverse variants ------------------------------------------------
// Inputs: AD, AT (A in D- and T-form; for fp8 compute already band-masked when the
// mask is on, since out-of-band magnitudes would otherwise set the scales).
// Output: TT, T in T-form (row-major friendly).
// MAXD = NT - 1 is the general case; MAXD = 1 is valid when the band mask is on with
// N <= 16 (every tile two or more tile-diagonals below the main one is then zero in
// A, in every intermediate and in T).

// fp8 chain on X = H - I ([GEO] "Adaptation a la Quantification"): the identity never
// enters a quantised tensor, so the scales follow A's powers alone.
//   A' = s_A q(A),  X_1 = A',  X_{k+1} = A' + s_A s_X (q(A) q(X_k)),  T = I + s_T q(X_N)
// (T = I + A' for N = 1).  q() are e4m3 codes under the tensor's absmax/448 scale; the
// MFMA sums the code products in fp32 and one fused multiply-add scales and adds A'.
// A's left-operand codes are formed once for all products.  AD, AT arrive band-masked
// when the mask is on, and every X_{k+1} is masked before it is quantised.  Counters:
// A under its own scale, each right operand X_1 .. X_{N-1} and X_N under theirs and
// under A's (the static scale).
template <int NT, int MAXD = NT - 1>
__device__ __forceinline__ void neumann_T_fp8(const Mat<NT>& AD, const Mat<NT>& AT, int N, bool mask,
                                              Mat<NT>& TT, Fp8Counts& cnt, bool count) {
  constexpr int NP = (NT + 1) / 2;
  const int band = mask ? N : (1 << 30);
  const float sA = fp8_scale_count<NT, MAXD>(AT, 0.f, cnt, count);
  if (N <= 1) {
    TT = AT;
    fp8_roundtrip<NT, MAXD>(TT, sA);
    add_eye(TT);
    return;
  }
  const float iA = 1.f / sA;
  long ra[NT][NP];
#pragma unroll
  for (int I = 0; I < NT; ++I)
#pragma unroll
    for (int p = 0; p < NP; ++p)
      if (2 * p <= I && I - (2 * p + 1) <= MAXD)
        ra[I][p] = quant8(tile_or_zero(AT, I, 2 * p), tile_or_zero(AT, I, 2 * p + 1), iA);
  // A' in both forms; the T-form decodes A's row codes (the same quantisation)
  Mat<NT> AqD = AD, AqT;
  fp8_roundtrip<NT, MAXD>(AqD, sA);
#pragma unroll
  for (int I = 0; I < NT; ++I)
#pragma unroll
    for (int J = 0; J <= I; ++J) {
      if (I - J > MAXD) {
        AqT.t[I][J] = zero4();
        continue;
      }
      const uint64_t q = (uint64_t)ra[I][J / 2];
      const uint32_t w = (J & 1) ? (uint32_t)(q >> 32) : (uint32_t)q;
      AqT.t[I][J][0] = fp8_to_f32<0>(w) * sA;
      AqT.t[I][J][1] = fp8_to_f32<1>(w) * sA;
      AqT.t[I][J][2] = fp8_to_f32<2>(w) * sA;
      AqT.t[I][J][3] = fp8_to_f32<3>(w) * sA;
    }
  Mat<NT> X = AqD;  // X_1 (D-form)
  for (int k = 1; k < N; ++k) {
    const float sX = fp8_scale_count<NT, MAXD>(X, sA, cnt, count);
    const float iX = 1.f / sX, sxy = sA * sX;
    long cx[NP][NT];
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int J = 0; J < NT; ++J)
        if (J <= 2 * p + 1 && 2 * p - J <= MAXD)
          cx[p][J] = quant8(tile_or_zero(X, 2 * p, J), tile_or_zero(X, 2 * p + 1, J), iX);
    const bool last = (k == N - 1);
#pragma unroll
    for (int I = 0; I < NT; ++I)
#pragma unroll
      for (int J = 0; J <= I; ++J) {
        if (I - J > MAXD) {
          (last ? TT : X).t[I][J] = zero4();
          continue;
        }
        f32x4 acc = zero4();
        if (last) {  // T-form: operands swapped
#pragma unroll
          for (int p = J / 2; p <= I / 2; ++p) acc = mma_fp8(cx[p][J], ra[I][p], acc);
#pragma unroll
          for (int r = 0; r < 4; ++r) TT.t[I][J][r] = __builtin_fmaf(acc[r], sxy, AqT.t[I][J][r]);
        } else {
#pragma unroll
          for (int p = J / 2; p <= I / 2; ++p) acc = mma_fp8(ra[I][p], cx[p][J], acc);
#pragma unroll
          for (int r = 0; r < 4; ++r) X.t[I][J][r] = __builtin_fmaf(acc[r], sxy, AqD.t[I][J][r]);
        }
      }
    if (mask) {
      if (last)
        mask_T(TT, band);
      else
        mask_D(X, band);
    }
  }
  const float sT = fp8_scale_count<NT, MAXD>(TT, sA, cnt, count);
  fp8_roundtrip<NT, MAXD>(TT, sT);
  add_eye(TT);
}

template <int NT, int CMP, int MAXD = NT - 1>
__device__ __forceinline__ void neumann_T(const Mat<NT>& AD, const Mat<NT>& AT, int N, bool mask,
                                          Mat<NT>& TT, Fp8Counts& cnt, bool count) {
  if constexpr (CMP == CMP_FP8) {
    neumann_T_fp8<NT, MAXD>(AD, AT, N, mask, TT, cnt, count);
    return;
  }
  const int band = mask ? N : (1 << 30);
  if (N <= 1) {
    TT = AT;
    if (mask) mask_T(TT, band);
    add_eye(TT);
    return;
  }
  Mat<NT> H = AD;  // H_1 = I + A (D-form)
  add_eye(H);
  // Entries inside the band of a product of lower-triangular matrices only involve
  // entries inside the band of the factors, so masking the final sum gives exactly
  // (bit for bit) what masking A and every intermediate would.
  for (int k = 2; k < N; ++k) {
    Mat<NT> Z;
    lmul<NT, CMP, false, MAXD, true>(AT, H, Z);
    H = Z;
  }
  lmul<NT, CMP, true, MAXD, true>(AT, H, TT);
  if (mask) mask_T(TT, band);
}

// ---- parallel residual correction ([GEO] Methodologie SS3) ----------------------
// T(0) = the (optionally band-masked) truncated sum, E = I - (I - A) T(0) (its residual,
// supported on subdiagonals > N when masked), and T = T(0) sum_{s<=S} E^s with the sum
// of powers in Horner form R = I + E (I + E ( ... )).  E is a small difference of O(1)
// terms, so every product here runs on the fp32 MFMA.  T(0) is formed in both tile
// forms (right operand of A T(0), left operand of T(0) R).
template <int NT>
__device__ __forceinline__ void residual_T(const Mat<NT>& AD, const Mat<NT>& AT, int N, bool mask, int S,
                                           Mat<NT>& TT) {
  Mat<NT> HD = AD, HT = AT;  // H_1 = I + A
  add_eye(HD);
  add_eye(HT);
  for (int k = 2; k <= N; ++k) {
    Mat<NT> ZD, ZT;
    lmul<NT, CMP_F32, false, NT - 1, true>(AT, HD, ZD);
    lmul<NT, CMP_F32, true, NT - 1, true>(AT, HD, ZT);
    HD = ZD;
    HT = ZT;
  }
  if (mask) {
    mask_D(HD, N);
    mask_T(HT, N);
  }
  // E = A T(0) - (T(0) - I), T-form
  Mat<NT> E;
  lmul<NT, CMP_F32, true, NT - 1, false>(AT, HD, E);
#pragma unroll
  for (int I = 0; I < NT; ++I)
#pragma unroll
    for (int J = 0; J <= I; ++J) E.t[I][J] -= HT.t[I][J];
  add_eye(E);
  // R = I + E R, S times, D-form
  Mat<NT> R;
#pragma unroll
  for (int I = 0; I < NT; ++I)
#pragma unroll
    for (int J = 0; J < NT; ++J) R.t[I][J] = zero4();
  add_eye(R);
  for (int s = 0; s < S; ++s) {
    Mat<NT> Z;
    lmul<NT, CMP_F32, false, NT - 1, true>(E, R, Z);
    R = Z;
  }
  lmul<NT, CMP_F32, true, NT - 1, false>(HT, R, TT);
}

// exact doubling: P = I + A; X = A; for q = 1..m-1: X <- X X; P <- P + P X
template <int NT, int CMP>
__device__ __forceinline__ void doubling_T(const Mat<NT>& AD, const Mat<NT>& AT, Mat<NT>& PT) {
  constexpr int C = 16 * NT;
  constexpr int M = (C <= 16) ? 4 : (C <= 32) ? 5 : 6;  // ceil(log2 C)
  PT = AT;
  add_eye(PT);
  Mat<NT> XD = AD, XT = AT;
#pragma unroll
  for (int q = 1; q < M; ++q) {
    Mat<NT> ND, NTm;
    lmul<NT, CMP, false>(XT, XD, ND);  // X^2, D-form
    if (q + 1 < M) lmul<NT, CMP, true>(XT, XD, NTm);  // X^2, T-form (not needed last)
    XD = ND;
    XT = NTm;
    // P <- P + P X  (P X = X P: every factor is a polynomial in A)
    Mat<NT> PX;
    lmul<NT, CMP, true>(PT, XD, PX);
#pragma unroll
    for (int I = 0; I < NT; ++I)
#pragma unroll
      for (int J = 0; J <= I; ++J) PT.t[I][J] += PX.t[I][J];
  }
}

// Exact doubling at C = 64 on bf16 products, the method's m - 1 squarings and m - 1
// products and no more: P = I + A; for q = 1..m-1: X <- X X (D-form); P <- P + P X.
// A product needs its left factor in T-form and its right factor in D-form, so the
// square is formed once (D-form) and its T-form row packs are read back from a bf16 copy
// of X^T in LDS (xt: this wave's 64 x XT_LD scratch) with the transpose read.  Tiles
// that Lemma 3.1 makes zero are skipped: X = A^d vanishes below sub-diagonal d, so
// tile (I, J) of X is zero when 16 (I - J) + 15 < d, and a product's tile (I, J) only
// sums over the tiles K where both factors can be non-zero.  P + P X accumulates onto
// P's own tile inside the MFMA.
constexpr int XT_LD = 72;  // bf16 row stride of the X^T scratch (64 + 8: bank spread)

// first and last tile index K of a product's tile (I, J) given the smallest non-zero tile
// distance of the left (kl) and right (kr) factor
__device__ __forceinline__ constexpr int tile_kmin(int J, int kr) { return J + kr; }
__device__ __forceinline__ constexpr int tile_kmax(int I, int kl) { return I - kl; }
// smallest tile distance I - J at which A^d can be non-zero (entries only at i - j >= d)
__device__ __forceinline__ constexpr int tile_dist(int d) { return d <= 15 ? 0 : (d - 15 + 15) / 16; }

// AD_FROM_AT: A's column packs are not formed from AD (which the caller then need not
// build, nor the Gram tiles below the diagonal that only AD reads) but read back from a
// bf16 copy of A's rows through the same transpose read, as the squares' row packs are:
// the column packs of A are the row packs of A^T.
template <bool AD_FROM_AT = false>
__device__ __forceinline__ void doubling_T_lds(const Mat<4>& AD, const Mat<4>& AT, Mat<4>& PT,
                                               __bf16 (*xt)[XT_LD]) {
  constexpr int NT = 4, NP = 2;
  const int l = lane_id(), g = l >> 4, c = l & 15;
  bf16x8 xr[NT][NP], xc[NP][NT];  // row packs (T-form) and column packs (D-form) of X
#pragma unroll
  for (int I = 0; I < NT; ++I)
#pragma unroll
    for (int p = 0; p < NP; ++p) xr[I][p] = pack8(tile_or_zero(AT, I, 2 * p), tile_or_zero(AT, I, 2 * p + 1));
  if constexpr (AD_FROM_AT) {
    // A's rows 16I + c, columns 32p + 16h + 4g .. +3 into the scratch (every pack, the
    // zero ones above the diagonal included), then A^T's row packs back transposed
#pragma unroll
    for (int I = 0; I < NT; ++I)
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const u32x4 w = __builtin_bit_cast(u32x4, xr[I][p]);
        *reinterpret_cast<u32x2*>(&xt[16 * I + c][32 * p + 4 * g]) = u32x2{w[0], w[1]};
        *reinterpret_cast<u32x2*>(&xt[16 * I + c][32 * p + 16 + 4 * g]) = u32x2{w[2], w[3]};
      }
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int J = 0; J < NT; ++J) {
        const __bf16* b0 = &xt[32 * p + 4 * g + (c >> 2)][16 * J + 4 * (c & 3)];
        xc[p][J] = join8(lds_read_tr4(b0), lds_read_tr4(b0 + 16 * XT_LD));
      }
  } else {
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int J = 0; J < NT; ++J) xc[p][J] = pack8(tile_or_zero(AD, 2 * p, J), tile_or_zero(AD, 2 * p + 1, J));
  }
  PT = AT;
  add_eye(PT);
#pragma unroll
  for (int q = 1; q < 6; ++q) {
    const int d = 1 << (q - 1);  // X = A^d
    const int kx = tile_dist(d), kx2 = tile_dist(2 * d);
    // X <- X X (D-form)
    Mat<NT> XD;
#pragma unroll
    for (int I = 0; I < NT; ++I)
#pragma unroll
      for (int J = 0; J <= I; ++J) {
        f32x4 acc = zero4();
        if (I - J >= kx2) {
          const int k0 = tile_kmin(J, kx), k1 = tile_kmax(I, kx);
#pragma unroll
          for (int p = 0; p < NP; ++p)
            if (2 * p + 1 >= k0 && 2 * p <= k1) acc = mma_bf16(xr[I][p], xc[p][J], acc);
        }
        XD.t[I][J] = acc;
      }
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int J = 0; J < NT; ++J) xc[p][J] = pack8(tile_or_zero(XD, 2 * p, J), tile_or_zero(XD, 2 * p + 1, J));
    // P <- P + P X (T-form: operands swapped), accumulated onto P's tile
    bf16x8 pr[NT][NP];
#pragma unroll
    for (int I = 0; I < NT; ++I)
#pragma unroll
      for (int p = 0; p < NP; ++p)
        if (2 * p <= I) pr[I][p] = pack8(tile_or_zero(PT, I, 2 * p), tile_or_zero(PT, I, 2 * p + 1));
#pragma unroll
    for (int I = 0; I < NT; ++I)
#pragma unroll
      for (int J = 0; J <= I; ++J) {
        if (I - J < kx2) continue;  // (P X)(I, J) needs K - J >= kx2 with K <= I
        const int k0 = tile_kmin(J, kx2), k1 = I;
        f32x4 acc = PT.t[I][J];
#pragma unroll
        for (int p = 0; p < NP; ++p)
          if (2 * p + 1 >= k0 && 2 * p <= k1) acc = mma_bf16(xc[p][J], pr[I][p], acc);
        PT.t[I][J] = acc;
      }
    if (q < 5) {
      // the new X's row packs: its column packs hold X^T's rows 16J + c, columns
      // 32p + 16h + 4g .. +3; write them and read the T-form back transposed
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int J = 0; J < NT; ++J) {
          const u32x4 w = __builtin_bit_cast(u32x4, xc[p][J]);
          *reinterpret_cast<u32x2*>(&xt[16 * J + c][32 * p + 4 * g]) = u32x2{w[0], w[1]};
          *reinterpret_cast<u32x2*>(&xt[16 * J + c][32 * p + 16 + 4 * g]) = u32x2{w[2], w[3]};
        }
#pragma unroll
      for (int I = 0; I < NT; ++I)
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const __bf16* b0 = &xt[32 * p + 4 * g + (c >> 2)][16 * I + 4 * (c & 3)];
          xr[I][p] = join8(lds_read_tr4(b0), lds_read_tr4(b0 + 16 * XT_LD));
        }
    }
  }
}

// ---- stores ------------------------------------------------------------------
// T-form tile (I,J): lane (g,c) holds row 16I + c, columns 16J + 4g .. +3.

// T is written once per launch (and K read once): both use non-temporal accesses, the
// streaming cache policy, so they do not displace other lines on their way to HBM.
template <int NT, int MAXD = NT - 1>
__device__ __forceinline__ void store_T_f32(float* __restrict__ out, const Mat<NT>& M) {
  constexpr int C = 16 * NT;
  const int l = lane_id(), g = l >> 4, c = l & 15;
#pragma unroll
  for (int I = 0; I < NT; ++I)
#pragma unroll
    for (int J = 0; J < NT; ++J) {
      f32x4 v = (J <= I && I - J <= MAXD) ? M.t[I][J] : zero4();
      __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(out + (size_t)(16 * I + c) * C + 16 * J + 4 * g));
    }
}

template <int NT, int MAXD = NT - 1>
__device__ __forceinline__ void store_T_bf16(__bf16* __restrict__ out, const Mat<NT>& M) {
  constexpr int C = 16 * NT;
  const int l = lane_id(), g = l >> 4, c = l & 15;
#pragma unroll
  for (int I = 0; I < NT; ++I)
#pragma unroll
    for (int J = 0; J < NT; ++J) {
      f32x4 v = (J <= I && I - J <= MAXD) ? M.t[I][J] : zero4();
      __builtin_nontemporal_store(pack4(v), reinterpret_cast<bf16x4*>(out + (size_t)(16 * I + c) * C + 16 * J + 4 * g));
    }
}

// ---- T of a 32 x 32 or 64 x 64 block as whole 128-byte row pieces ------------------
// Tiles beyond MAXD tile-diagonals and above the diagonal are zero.
template <int NT, int MAXD>
__device__ __forceinline__ f32x4 tile_kept(const Mat<NT>& M, int I, int J) {
  return (J <= I && I - J <= MAXD) ? M.t[I][J] : zero4();
}

// fp32: tile pairs through store_rows_f32x2 (a pair is 128 bytes of a row)
template <int NT, int MAXD, int ILO = 0, int IHI = NT - 1>
__device__ __forceinline__ void store_T_rows_f32(float* __restrict__ out, const Mat<NT>& M) {
  static_assert(NT == 2 || NT == 4, "32 x 32 or 64 x 64 blocks");
  constexpr int C = 16 * NT;
#pragma unroll
  for (int I = ILO; I <= IHI; ++I)
#pragma unroll
    for (int J = 0; J < NT; J += 2)
      store_rows_f32x2<true>(out + (size_t)16 * I * C + 16 * J, C, tile_kept<NT, MAXD>(M, I, J),
                             tile_kept<NT, MAXD>(M, I, J + 1));
}

// bf16: at C = 64 four tiles through store_rows_bf16x4; at C = 32 a row is 64 bytes and
// one tile pair through store_pair_bf16 writes 16 contiguous rows
template <int NT, int MAXD, int ILO = 0, int IHI = NT - 1>
__device__ __forceinline__ void store_T_rows_bf16(__bf16* __restrict__ out, const Mat<NT>& M) {
  static_assert(NT == 2 || NT == 4, "32 x 32 or 64 x 64 blocks");
  constexpr int C = 16 * NT;
  const int c = lane_id() & 15;
#pragma unroll
  for (int I = ILO; I <= IHI; ++I) {
    if constexpr (NT == 4) {
      const f32x4 t[4] = {tile_kept<NT, MAXD>(M, I, 0), tile_kept<NT, MAXD>(M, I, 1),
                          tile_kept<NT, MAXD>(M, I, 2), tile_kept<NT, MAXD>(M, I, 3)};
      store_rows_bf16x4<true>(out + (size_t)16 * I * C, C, t);
    } else {
      store_pair_bf16<true>(out + (size_t)(16 * I + c) * C, 0, tile_kept<NT, MAXD>(M, I, 0),
                            tile_kept<NT, MAXD>(M, I, 1));
    }
  }
}

// T - I of a 64 x 64 block as the six left-operand row packs of the chunk forward's
// product (T - I) Y: pack k <-> (I, p) in the order (0,0) (1,0) (2,0) (2,1) (3,0) (3,1),
// tiles (I, 2p) and (I, 2p + 1) in T-form, 16 bytes per lane at out[64 k + lane].  The
// packs with 2p > I lie above the diagonal and are not stored.
constexpr int T_PACKS = 6;

__device__ __forceinline__ int t_pack_index(int I, int p) { return I <= 1 ? I : 2 * I - 2 + p; }

__device__ __forceinline__ void store_T_packs(bf16x8* __restrict__ out, const Mat<4>& TT) {
  const int l = lane_id();
  const f32x4 e = eye_tile();
#pragma unroll
  for (int I = 0; I < 4; ++I)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      if (2 * p > I) continue;
      const f32x4 t0 = (2 * p == I) ? TT.t[I][2 * p] - e : TT.t[I][2 * p];
      const f32x4 t1 = (2 * p + 1 == I) ? TT.t[I][2 * p + 1] - e : tile_or_zero(TT, I, 2 * p + 1);
      out[WAVE * t_pack_index(I, p) + l] = pack8(t0, t1);
    }
}

}  // namespace gdn
