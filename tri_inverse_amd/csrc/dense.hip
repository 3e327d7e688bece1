// dense.hip -- T = (I - A)^-1 for C = 128 and 256 over the full lower triangle: the
// truncated Neumann sum (any N, masked or not) and the exact doubling product, as T
// itself or as the WY products; also the WY products of a given T.
//
// [GEO] "When Good Enough Is Optimal: Multiplication-Only Matrix Inversion
// Approximation for Quantized Gated DeltaNet", problem statement and Methodologie
// SS1-2: T approximated by the Horner form of sum_{n<=N} A^n, optionally band-masked.
// The exact variant multiplies (I + A^(2^i)) for i < ceil(log2 C), exact because A is
// strictly lower-triangular, hence nilpotent (A^C = 0).
//
// One workgroup of NT/2 waves per block (NT = C/16 tile rows).  Wave w owns tile rows
// w and NT-1-w (equal tile counts), holding their 16x16 tiles in registers in T-form
// (lane (g,c) reg r = M[16I + c][16J + 4g + r]), fp32.  A product Z = X Y of
// lower-triangular tile matrices is formed row by row by the owners of Z's rows with
// the 16x16x16 bf16 MFMA: D-form of (X Y)^T = Y^T X^T, i.e. operand a = Y tile read
// column-wise (LDS transpose read) and operand b = X tile read row-wise, which gives Z
// in T-form directly.  Both operands come from bf16 copies of the tile matrices in LDS
// (16x16 tiles, rows XOR-swizzled in 8-byte chunks); a matrix changes only between
// barriers.  In the doubling
// product A^(2^q) vanishes on subdiagonals below 2^q, and the tiles that lie entirely
// there are skipped.
#include "gdn_kernels.hpp"
#include "tri_block.hpp"

#include <utility>

namespace gdn {

template <class F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// 16x16x16 bf16 MFMA: lane (g,c) holds a = A[c][4g..4g+3] and b = B[4g..4g+3][c];
// the result is D-form (lane (g,c) reg r = D[4g + r][c])
__device__ __forceinline__ f32x4 mma16(const bf16x4& a, const bf16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a), __builtin_bit_cast(i16x4, b),
                                                   c, 0, 0, 0);
}

__device__ __forceinline__ int tri_idx(int I, int J) { return I * (I + 1) / 2 + J; }

// lower-triangular tile matrix in LDS, bf16, row-major 16x16 tiles
template <int NT>
struct alignas(16) LTiles {
  __bf16 t[NT * (NT + 1) / 2][16][16];
};

// Each tile row holds four 8-byte chunks; chunk q of row r sits at chunk position
// q ^ (r / 4) (rows r and r + 4 would otherwise start on the same banks).
// lane (g,c): M(I,J)[c][4g .. 4g+3]
template <int NT>
__device__ __forceinline__ bf16x4 rowfrag(const LTiles<NT>& M, int I, int J) {
  const int l = lane_id(), g = l >> 4, c = l & 15;
  return *reinterpret_cast<const bf16x4*>(&M.t[tri_idx(I, J)][c][4 * (g ^ (c >> 2))]);
}
// lane (g,c): M(I,J)[4g .. 4g+3][c] (transpose read; lane (g, j) addresses row
// 4g + j / 4, chunk j % 4)
template <int NT>
__device__ __forceinline__ bf16x4 colfrag(const LTiles<NT>& M, int I, int J) {
  const int l = lane_id(), g = l >> 4, j = l & 15;
  return lds_read_tr4(&M.t[tri_idx(I, J)][4 * g + (j >> 2)][4 * ((j & 3) ^ g)]);
}
// store a T-form tile
template <int NT>
__device__ __forceinline__ void put_tile(LTiles<NT>& M, int I, int J, const f32x4& v) {
  const int l = lane_id(), g = l >> 4, c = l & 15;
  *reinterpret_cast<bf16x4*>(&M.t[tri_idx(I, J)][c][4 * (g ^ (c >> 2))]) = pack4(v);
}

// the two tile rows a wave owns: row I0 = w (at most NT/2 tiles), row I1 = NT-1-w
template <int NT>
struct OwnRows {
  f32x4 a[NT / 2];
  f32x4 b[NT];
};

// f(row, J, tile) for every owned tile, J compile-time
template <int NT, class F>
__device__ __forceinline__ void for_owned(OwnRows<NT>& R, int I0, int I1, F&& f) {
  static_for<NT / 2>([&](auto Jc) {
    constexpr int J = decltype(Jc)::value;
    if (J <= I0) f(I0, J, R.a[J]);
  });
  static_for<NT>([&](auto Jc) {
    constexpr int J = decltype(Jc)::value;
    if (J <= I1) f(I1, J, R.b[J]);
  });
}

// Z(I, J0 + j) (+)= sum_K X(I,K) Y(K, J0 + j), j < NJ, over one owned row: K runs over
// the contraction (runtime), the output tile is compile-time; only pairs with K - J >= dy
// (Y's vanishing tile-subdiagonals) and I - K >= dx (X's) are formed
template <int NT, int NJ, int J0 = 0>
__device__ __forceinline__ void row_product(const LTiles<NT>& X, const LTiles<NT>& Y, int I, int dx, int dy,
                                            f32x4 (&z)[NJ]) {
  for (int K = J0; K + dx <= I; ++K) {
    const bf16x4 xb = rowfrag<NT>(X, I, K);
    static_for<NJ>([&](auto jc) {
      constexpr int J = J0 + decltype(jc)::value;
      if (J + dy <= K) z[J - J0] = mma16(colfrag<NT>(Y, K, J), xb, z[J - J0]);
    });
  }
}

// The squarings X <- X X of the doubling product feed only the bf16 copy in LDS, so their
// output tiles need not follow row ownership.  A tile (I, J) of a product of lower-
// triangular tile matrices sums I - J + 1 tile products, so the owner pairs (w, NT-1-w)
// carry from (NT/2)(NT/2 + 1) to NT/2 + NT(NT + 1)/2 of them: 81 to 137 at NT = 16, with
// every barrier waiting for the heaviest.  The squarings are dealt out instead as row
// halves (column tiles 0 .. NT/2-1, "left", and NT/2 .. NT-1, "right"), assigned by
// longest-first greedy packing: at most 103 (NT = 16) and 31 (NT = 8) tile products per
// wave for the unskipped squarings, against a mean of 102 and 30.
template <int NT>
__device__ __forceinline__ int sq_left_row(int w, int s) {  // -1: none
  static constexpr int L8[4][3] = {{7, 1, -1}, {6, 2, -1}, {5, 0, -1}, {4, 3, -1}};
  static constexpr int L16[8][3] = {{15, 0, -1}, {14, -1, -1}, {13, 4, -1}, {12, 5, -1},
                                    {11, 2, -1}, {10, 6, -1}, {9, 3, 1},   {8, 7, -1}};
  if constexpr (NT == 8) return L8[w][s];
  else return L16[w][s];
}
template <int NT>
__device__ __forceinline__ int sq_right_row(int w) {
  static constexpr int R8[4] = {4, 5, 7, 6};
  static constexpr int R16[8] = {8, 11, 9, 10, 14, 12, 15, 13};
  if constexpr (NT == 8) return R8[w];
  else return R16[w];
}

// wave w's share of X^2 (the tiles of A^(2n) that vanish skipped through d) into out
template <int NT>
__device__ __forceinline__ void square_share(const LTiles<NT>& X, LTiles<NT>& out, int w, int d) {
  static_assert(NT == 8 || NT == 16, "C = 128 or 256");
  auto half = [&](int I, auto j0) {
    constexpr int J0 = decltype(j0)::value;
    f32x4 z[NT / 2];
    static_for<NT / 2>([&](auto jc) { z[decltype(jc)::value] = zero4(); });
    row_product<NT, NT / 2, J0>(X, X, I, d, d, z);
    static_for<NT / 2>([&](auto jc) {
      constexpr int J = J0 + decltype(jc)::value;
      if (J <= I) put_tile<NT>(out, I, J, z[J - J0]);
    });
  };
  for (int s = 0; s < 3; ++s) {
    const int I = sq_left_row<NT>(w, s);
    if (I < 0) break;
    half(I, std::integral_constant<int, 0>{});
  }
  half(sq_right_row<NT>(w), std::integral_constant<int, NT / 2>{});
}

// T = I + A on the owned rows
template <int NT>
__device__ __forceinline__ void init_eye_plus(const OwnRows<NT>& A, OwnRows<NT>& T, int I0, int I1,
                                              const f32x4& eye) {
  static_for<NT / 2>([&](auto Jc) {
    constexpr int J = decltype(Jc)::value;
    if (J <= I0) T.a[J] = (J == I0) ? A.a[J] + eye : A.a[J];
  });
  static_for<NT>([&](auto Jc) {
    constexpr int J = decltype(Jc)::value;
    if (J <= I1) T.b[J] = (J == I1) ? A.b[J] + eye : A.b[J];
  });
}

struct DenseArgs {
  BlocksArgs a;
  const void* T_in;   // given T (WY only), or NULL
  int t_in_bf16;
  const __bf16* V;
  int N, mask, gate_k;
  void* T_out;
  int t_bf16;
  void* W_out;
  void* U_out;
  int out_bf16;
};

template <int C>
struct alignas(16) DenseGates {
  float beta[C];
  float G[C];
  float rowf[C];  // -beta exp(G)
  float colf[C];  // exp(-G)
  int split;      // exp(-G) finite over the block
};

// MODE: MODE_NEUMANN / MODE_EXACT; TSRC: 0 formed here, 1 given fp32, 2 given bf16;
// DV = 0: T out, else W, U out
template <int NT, int DK, int DV, int MODE, int TSRC>
__global__ __launch_bounds__(NT * WAVE / 2, 1) void dense_kernel(DenseArgs p) {
  constexpr int C = 16 * NT;
  constexpr int KP = DK + 8, VP = (DV ? DV : 8) + 8;
  constexpr int MAT_BYTES = 2 * (int)sizeof(LTiles<NT>);
  constexpr int KV_BYTES = C * KP * 2 + (DV ? C * VP * 2 : 0);
  constexpr int SMEM = MAT_BYTES > KV_BYTES ? MAT_BYTES : KV_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  __shared__ DenseGates<C> gs;
  LTiles<NT>& MX = *reinterpret_cast<LTiles<NT>*>(smem);
  LTiles<NT>& MP = *reinterpret_cast<LTiles<NT>*>(smem + sizeof(LTiles<NT>));
  __bf16(&Ks)[C][KP] = *reinterpret_cast<__bf16(*)[C][KP]>(smem);
  __bf16(&Vs)[C][VP] = *reinterpret_cast<__bf16(*)[C][VP]>(smem + C * KP * 2);

  const BlocksArgs& a = p.a;
  const int64_t b = blockIdx.x;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const int l = lane_id(), g = l >> 4, c = l & 15;
  const int I0 = w, I1 = NT - 1 - w;
  const __bf16* Kb = reinterpret_cast<const __bf16*>(a.K) + b * C * DK;
  constexpr int NTHR = NT * WAVE / 2;

  // ---- gates: G = in-block cumsum of the log-gates (or given cumulative) ------------
  if (w == 0) {
    float carry = 0.f, gmin = 0.f;
    for (int s = 0; s < C; s += WAVE) {
      const float gv = a.g[b * C + s + l], bv = a.beta[b * C + s + l];
      const float Gv = a.g_cumulative ? gv : carry + wave_inclusive_scan(gv);
      carry = readlane_f(Gv, WAVE - 1);
      gs.beta[s + l] = bv;
      gs.G[s + l] = Gv;
      gs.rowf[s + l] = -bv * __expf(Gv);
      gs.colf[s + l] = __expf(-Gv);
      gmin = fminf(gmin, Gv);
    }
    gmin = wave_min(gmin);
    if (l == 0) gs.split = gmin >= -80.f ? 1 : 0;
  }

  OwnRows<NT> T;  // the result, T-form fp32
  if constexpr (TSRC == 0) {
    // ---- stage K, gram tiles of the owned rows, A ----------------------------------
    {
      constexpr int SEG = DK / 8, NSEG = C * SEG;
      for (int e = tid; e < NSEG; e += NTHR)
        *reinterpret_cast<bf16x8*>(&Ks[e / SEG][8 * (e % SEG)]) = *reinterpret_cast<const bf16x8*>(Kb + 8 * e);
    }
    __syncthreads();
    const bool split = gs.split != 0;
    OwnRows<NT> Am;  // A, T-form fp32
    auto gram_row = [&](int I, auto& row, auto nj) {
      constexpr int NJ = decltype(nj)::value;
      bf16x8 ki[DK / 32];
#pragma unroll
      for (int s = 0; s < DK / 32; ++s) ki[s] = *reinterpret_cast<const bf16x8*>(&Ks[16 * I + c][32 * s + 8 * g]);
      const int i = 16 * I + c;
      const float rf = gs.rowf[i], Gi = gs.G[i], bi = gs.beta[i];
      static_for<NJ>([&](auto Jc) {
        constexpr int J = decltype(Jc)::value;
        if (J <= I) {
          f32x4 s4 = zero4();
#pragma unroll
          for (int s = 0; s < DK / 32; ++s)
            s4 = mma_bf16(*reinterpret_cast<const bf16x8*>(&Ks[16 * J + c][32 * s + 8 * g]), ki[s], s4);
          // T-form: reg r <-> (i, j) = (16I + c, 16J + 4g + r); strictly lower only
          const f32x4 cf = *reinterpret_cast<const f32x4*>(&gs.colf[16 * J + 4 * g]);
          const f32x4 Gj = *reinterpret_cast<const f32x4*>(&gs.G[16 * J + 4 * g]);
          f32x4 v;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = 16 * J + 4 * g + r;
            const float f = split ? rf * cf[r] : -bi * __expf(Gi - Gj[r]);
            v[r] = (i > j) ? f * s4[r] : 0.f;
          }
          row[J] = v;
        }
      });
    };
    gram_row(I0, Am.a, std::integral_constant<int, NT / 2>{});
    gram_row(I1, Am.b, std::integral_constant<int, NT>{});
    __syncthreads();  // K no longer needed: the LDS turns into tile matrices

    const f32x4 eye = eye_tile();
    if constexpr (MODE == MODE_NEUMANN) {
      // H_1 = I + A; H_{k+1} = I + A H_k; T = H_N, masked to the band when asked
      for_owned<NT>(Am, I0, I1, [&](int I, int J, f32x4& t) { put_tile<NT>(MP, I, J, t); });  // A in MP
      init_eye_plus(Am, T, I0, I1, eye);                                                       // H_1

      for (int k = 2; k <= p.N; ++k) {
        for_owned<NT>(T, I0, I1, [&](int I, int J, f32x4& t) { put_tile<NT>(MX, I, J, t); });  // H_{k-1}
        __syncthreads();
        OwnRows<NT> Z;
        for_owned<NT>(Z, I0, I1, [&](int I, int J, f32x4& z) { z = (I == J) ? eye : zero4(); });
        row_product<NT, NT / 2>(MP, MX, I0, 0, 0, Z.a);
        row_product<NT, NT>(MP, MX, I1, 0, 0, Z.b);
        T = Z;
        __syncthreads();  // everyone done reading H_{k-1}
      }
      if (p.mask) {
        for_owned<NT>(T, I0, I1, [&](int I, int J, f32x4& t) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if ((16 * I + c) - (16 * J + 4 * g + r) > p.N) t[r] = 0.f;
        });
      }
    } else {
      // P = I + A, X = A; for q = 1 .. m-1: X <- X X; P <- P + P X.  The two LDS
      // buffers swap roles every step: X^2 goes straight into the buffer not holding X,
      // then P's bf16 copy overwrites the old X.
      constexpr int M = (C <= 128) ? 7 : 8;  // ceil(log2 C)
      for_owned<NT>(Am, I0, I1, [&](int I, int J, f32x4& t) { put_tile<NT>(MX, I, J, t); });  // X = A
      init_eye_plus(Am, T, I0, I1, eye);                                                       // P = I + A
      LTiles<NT>* xb = &MX;
      LTiles<NT>* ob = &MP;
      for (int q = 1; q < M; ++q) {
        // (A^n)_ij = 0 for i - j < n, so tile (I,J) of A^n is zero when 16(I - J) + 15 < n,
        // i.e. below tile-subdiagonal n / 16 (n a power of two)
        const int dprev = (1 << (q - 1)) / 16, dq = (1 << q) / 16;
        __syncthreads();  // X = A^(2^(q-1)) complete in *xb; *ob no longer read
        square_share<NT>(*xb, *ob, w, dprev);
        __syncthreads();  // X^2 complete in *ob; the old X is dead
        for_owned<NT>(T, I0, I1, [&](int I, int J, f32x4& t) { put_tile<NT>(*xb, I, J, t); });  // P (old)
        __syncthreads();
        row_product<NT, NT / 2>(*xb, *ob, I0, 0, dq, T.a);
        row_product<NT, NT>(*xb, *ob, I1, 0, dq, T.b);
        LTiles<NT>* t = xb;
        xb = ob;
        ob = t;
      }
    }
    __syncthreads();  // tile matrices consumed
  } else {
    // ---- given T: the owned rows, read in T-form ------------------------------------
    for_owned<NT>(T, I0, I1, [&](int I, int J, f32x4& t) {
      const int64_t o = b * C * C + (int64_t)(16 * I + c) * C + 16 * J + 4 * g;
      if constexpr (TSRC == 1)
        t = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(p.T_in) + o);
      else
        t = unpack4(*reinterpret_cast<const bf16x4*>(reinterpret_cast<const __bf16*>(p.T_in) + o));
    });
    __syncthreads();  // gates ready
  }

  if constexpr (DV == 0) {
    // ---- T out: the owned rows, zero above the diagonal, as whole 128-byte row pieces
    auto store_row = [&](int I, auto& row, auto nj) {
      constexpr int NJ = decltype(nj)::value;
      auto tile = [&](auto Jc) -> f32x4 {
        constexpr int J = decltype(Jc)::value;
        f32x4 t = zero4();
        if constexpr (J < NJ) {
          if (J <= I) t = row[J];
        }
        return t;
      };
      const int64_t rowbase = b * C * C + (int64_t)(16 * I) * C;
      if (p.t_bf16) {
        static_for<NT / 4>([&](auto qc) {
          constexpr int J = 4 * decltype(qc)::value;
          const f32x4 t[4] = {tile(std::integral_constant<int, J>{}), tile(std::integral_constant<int, J + 1>{}),
                              tile(std::integral_constant<int, J + 2>{}), tile(std::integral_constant<int, J + 3>{})};
          store_rows_bf16x4<true>(reinterpret_cast<__bf16*>(p.T_out) + rowbase + 16 * J, C, t);
        });
      } else {
        static_for<NT / 2>([&](auto pc) {
          constexpr int J = 2 * decltype(pc)::value;
          store_rows_f32x2<true>(reinterpret_cast<float*>(p.T_out) + rowbase + 16 * J, C,
                                 tile(std::integral_constant<int, J>{}), tile(std::integral_constant<int, J + 1>{}));
        });
      }
    };
    store_row(I0, T.a, std::integral_constant<int, NT / 2>{});
    store_row(I1, T.b, std::integral_constant<int, NT>{});
  } else {
    // ---- WY: stage K and V, then W = (T diag(s)) K, U = (T diag(beta)) V -----------
    {
      constexpr int SEG = DK / 8, NSEG = C * SEG;
      for (int e = tid; e < NSEG; e += NTHR)
        *reinterpret_cast<bf16x8*>(&Ks[e / SEG][8 * (e % SEG)]) = *reinterpret_cast<const bf16x8*>(Kb + 8 * e);
      constexpr int SV = DV / 8, NSV = C * SV;
      const __bf16* Vb = p.V + b * C * DV;
      for (int e = tid; e < NSV; e += NTHR)
        *reinterpret_cast<bf16x8*>(&Vs[e / SV][8 * (e % SV)]) = *reinterpret_cast<const bf16x8*>(Vb + 8 * e);
    }
    __syncthreads();
    // operand a: X tile (K, e) read column-wise (rows 16K + 4g .., column 16e + c);
    // operand b: the owned T-form tile (I, K) times the column factors, as a hi/lo pair
    auto apply_row = [&](int I, auto& row, auto nj, auto& Xs, auto dcols, bool keyside, void* out) {
      constexpr int NJ = decltype(nj)::value;
      constexpr int D = decltype(dcols)::value;
      f32x4 acc[D / 16];
#pragma unroll
      for (int e = 0; e < D / 16; ++e) acc[e] = zero4();
      static_for<NJ>([&](auto Kc) {
        constexpr int K = decltype(Kc)::value;
        if (K <= I) {
          const f32x4 bt = *reinterpret_cast<const f32x4*>(&gs.beta[16 * K + 4 * g]);
          f32x4 f = bt;
          if (keyside && p.gate_k) {
            const f32x4 Gk = *reinterpret_cast<const f32x4*>(&gs.G[16 * K + 4 * g]);
#pragma unroll
            for (int r = 0; r < 4; ++r) f[r] = bt[r] * __expf(Gk[r]);
          }
          const f32x4 x = row[K] * f;
          const bf16x4 hi = pack4(x), lo = pack4(x - unpack4(hi));
#pragma unroll
          for (int e = 0; e < D / 16; ++e) {
            const bf16x4 xa = lds_read_tr4(&Xs[16 * K + 4 * g + (c >> 2)][16 * e + 4 * (c & 3)]);
            acc[e] = mma16(xa, hi, acc[e]);
            acc[e] = mma16(xa, lo, acc[e]);
          }
        }
      });
      // bf16: two column tiles at a time, 16 contiguous bytes per lane (store_pair_bf16)
      const int64_t ro = (b * C + 16 * I + c) * D;
      if (p.out_bf16) {
#pragma unroll
        for (int e2 = 0; e2 < D / 32; ++e2)
          store_pair_bf16(reinterpret_cast<__bf16*>(out) + ro, 2 * e2, acc[2 * e2], acc[2 * e2 + 1]);
      } else {
#pragma unroll
        for (int e = 0; e < D / 16; ++e)
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + ro + 16 * e + 4 * g) = acc[e];
      }
    };
    using NJa = std::integral_constant<int, NT / 2>;
    using NJb = std::integral_constant<int, NT>;
    using Dk = std::integral_constant<int, DK>;
    using Dv = std::integral_constant<int, DV>;
    apply_row(I0, T.a, NJa{}, Ks, Dk{}, true, p.W_out);
    apply_row(I1, T.b, NJb{}, Ks, Dk{}, true, p.W_out);
    apply_row(I0, T.a, NJa{}, Vs, Dv{}, false, p.U_out);
    apply_row(I1, T.b, NJb{}, Vs, Dv{}, false, p.U_out);
  }
}

int launch_dense(const BlocksArgs& a, const void* T_in, int t_in_bf16, int mode, int N, int mask,
                 const void* V, int d_v, int gate_k, void* T_out, int t_bf16, void* W_out, void* U_out,
                 int out_bf16, hipStream_t s) {
  DenseArgs p;
  p.a = a;
  p.T_in = T_in;
  p.t_in_bf16 = t_in_bf16;
  p.V = reinterpret_cast<const __bf16*>(V);
  p.N = N;
  p.mask = mask;
  p.gate_k = gate_k;
  p.T_out = T_out;
  p.t_bf16 = t_bf16;
  p.W_out = W_out;
  p.U_out = U_out;
  p.out_bf16 = out_bf16;
  const dim3 grid((unsigned)a.n_blocks);
  auto go = [&](auto nt, auto dk, auto dv, auto md, auto ts) {
    constexpr int NT = decltype(nt)::value;
    hipLaunchKernelGGL((dense_kernel<NT, dk.value, dv.value, md.value, ts.value>), grid,
                       dim3(NT * WAVE / 2), 0, s, p);
    return 0;
  };
  using MN = std::integral_constant<int, MODE_NEUMANN>;
  using ME = std::integral_constant<int, MODE_EXACT>;
  using S0 = std::integral_constant<int, 0>;
  auto with_dv = [&](auto nt, auto dk) -> int {
    if (!W_out) return mode == MODE_EXACT ? go(nt, dk, S0{}, ME{}, S0{}) : go(nt, dk, S0{}, MN{}, S0{});
    auto with_src = [&](auto dv) -> int {
      if (T_in)
        return t_in_bf16 ? go(nt, dk, dv, MN{}, std::integral_constant<int, 2>{})
                         : go(nt, dk, dv, MN{}, std::integral_constant<int, 1>{});
      return mode == MODE_EXACT ? go(nt, dk, dv, ME{}, S0{}) : go(nt, dk, dv, MN{}, S0{});
    };
    switch (d_v) {
      case 64: return with_src(std::integral_constant<int, 64>{});
      case 128: return with_src(std::integral_constant<int, 128>{});
      default: return -1;
    }
  };
  auto with_dk = [&](auto nt) -> int {
    switch (a.d_k) {
      case 64: return with_dv(nt, std::integral_constant<int, 64>{});
      case 128: return with_dv(nt, std::integral_constant<int, 128>{});
      default: return -1;
    }
  };
  switch (a.C) {
    case 128: return with_dk(std::integral_constant<int, 8>{});
    case 256: return with_dk(std::integral_constant<int, 16>{});
    default: return -1;
  }
}

}  // namespace gdn
