// wy.hip -- WY products per block: W = T diag(s) K and U = T diag(beta) V.
//
// [GEO] "When Good Enough Is Optimal: Multiplication-Only Matrix Inversion
// Approximation for Quantized Gated DeltaNet", problem statement: the chunk update
// consumes T = (I - A)^-1; here T is applied to the key and value rows of the chunk.
// s = beta (gate_k = 0) or s = beta .* exp(G) (gate_k = 1, the key-side gate the
// chunk recurrence needs when A carries the gate).
//
// One wave per block (C <= 64).  T is either read (T-form tiles) or formed in
// registers exactly as in the inverse kernels.  The diagonal is folded into T's
// columns in fp32, and T diag(s) enters the MFMAs as a bf16 hi/lo pair, so the
// products (T diag(s)) K carry about 16 bits and the bf16 rounding of the outputs
// dominates their error.  The contraction runs over the chunk's tokens, so each wave
// copies K (then V) row-major into its own LDS slice with 16-byte stores and reads the
// column fragments back with the gfx950 transpose read.
#include "gdn_kernels.hpp"
#include "tri_block.hpp"

namespace gdn {

constexpr int WY_WAVES = 4;
constexpr int XR_PAD = 8;

template <int NT, int D>
struct alignas(16) WyLds {
  __bf16 xr[16 * NT][D + XR_PAD];  // the block's [C][D] rows X, row-major (padded rows)
};

// stage rows X[C][D] (bf16, global) into LDS row-major: consecutive lanes take
// consecutive 16-byte pieces, so every load instruction covers whole rows
template <int NT, int D>
__device__ __forceinline__ void stage_rows(const __bf16* __restrict__ X, WyLds<NT, D>& L) {
  constexpr int SEG = D / 8, N = 16 * NT * SEG / WAVE;
  const int l = lane_id();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int e = i * WAVE + l;
    *reinterpret_cast<bf16x8*>(&L.xr[e / SEG][8 * (e % SEG)]) =
        *reinterpret_cast<const bf16x8*>(X + (size_t)8 * e);
  }
}

// Z = Tc X in T-form tiles, Tc given as row packs, X's column packs read from the
// row-major LDS copy with the transpose read: lane (g, j) addressing
// xr[r0 + 4g + j/4][c0 + 4(j%4)] receives xr[r0 + 4g + k][c0 + j], k = 0..3, which is
// the token pair p column fragment (slot t <-> token 32p + 16(t/4) + 4g + t%4) of
// column c0 + j.  Four column tiles at a time, stored row-major [C][D] as whole 128-byte
// row pieces (store_rows_bf16x4, store_rows_f32x2), so that no line is written in parts
// at different times.
template <int NT, int D>
__device__ __forceinline__ void apply_rows(const bf16x8 (&rp)[NT][(NT + 1) / 2],
                                           const bf16x8 (&rl)[NT][(NT + 1) / 2],
                                           const WyLds<NT, D>& L, void* __restrict__ out,
                                           bool out_bf16) {
  constexpr int C = 16 * NT, NP = (NT + 1) / 2;
  static_assert(D % 64 == 0, "column tiles are stored four at a time");
  const int l = lane_id(), g = l >> 4, c = l & 15;
#pragma unroll
  for (int e4 = 0; e4 < D / 64; ++e4) {
    bf16x8 cp[4][NP];
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int e = 4 * e4 + h;
        const bf16x4 lo = lds_read_tr4(&L.xr[32 * p + 4 * g + (c >> 2)][16 * e + 4 * (c & 3)]);
        bf16x4 hi = bf16x4{};
        if (32 * p + 16 < C) hi = lds_read_tr4(&L.xr[32 * p + 16 + 4 * g + (c >> 2)][16 * e + 4 * (c & 3)]);
        cp[h][p] = join8(lo, hi);
      }
#pragma unroll
    for (int I = 0; I < NT; ++I) {
      f32x4 acc[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        acc[h] = zero4();
#pragma unroll
        for (int p = 0; p <= I / 2; ++p) {
          acc[h] = mma_bf16(cp[h][p], rp[I][p], acc[h]);
          acc[h] = mma_bf16(cp[h][p], rl[I][p], acc[h]);
        }
      }
      const size_t o = (size_t)16 * I * D + 64 * e4;
      if (out_bf16) {
        store_rows_bf16x4<false>(reinterpret_cast<__bf16*>(out) + o, D, acc);
      } else {
        store_rows_f32x2<false>(reinterpret_cast<float*>(out) + o, D, acc[0], acc[1]);
        store_rows_f32x2<false>(reinterpret_cast<float*>(out) + o + 32, D, acc[2], acc[3]);
      }
    }
  }
}

// T-form tiles of T scaled column-wise by f[m] (m = 16J + 4g + r), as row packs; the
// scaled values are split into a bf16 hi/lo pair so the products keep ~16 bits
template <int NT>
__device__ __forceinline__ void scaled_row_packs(const Mat<NT>& TT, const float (&f)[NT][4],
                                                 bf16x8 (&rp)[NT][(NT + 1) / 2],
                                                 bf16x8 (&rl)[NT][(NT + 1) / 2]) {
  constexpr int NP = (NT + 1) / 2;
#pragma unroll
  for (int I = 0; I < NT; ++I)
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      f32x4 a = zero4(), b = zero4();
      if (2 * p <= I) {
#pragma unroll
        for (int r = 0; r < 4; ++r) a[r] = TT.t[I][2 * p][r] * f[2 * p][r];
      }
      if (2 * p + 1 <= I && 2 * p + 1 < NT) {
#pragma unroll
        for (int r = 0; r < 4; ++r) b[r] = TT.t[I][2 * p + 1][r] * f[2 * p + 1][r];
      }
      rp[I][p] = pack8(a, b);
      rl[I][p] = pack8(a - f32x4{(float)rp[I][p][0], (float)rp[I][p][1], (float)rp[I][p][2],
                                 (float)rp[I][p][3]},
                       b - f32x4{(float)rp[I][p][4], (float)rp[I][p][5], (float)rp[I][p][6],
                                 (float)rp[I][p][7]});
    }
}

template <int NT, int DK, int DV, int TSRC, int MODE, int MAXD>
__global__ __launch_bounds__(256) void wy_kernel(BlocksArgs a, const void* __restrict__ T_in,
                                                 int N, int mask, int gate_k,
                                                 const __bf16* __restrict__ V, void* W_out,
                                                 void* U_out, int out_bf16) {
  constexpr int C = 16 * NT;
  constexpr int DMAX = DK > DV ? DK : DV;
  __shared__ WyLds<NT, DMAX> lds[WY_WAVES];
  const int wave = threadIdx.x / WAVE;
  const int l = lane_id(), g = l >> 4, c = l & 15;
  const int64_t blk = (int64_t)blockIdx.x * WY_WAVES + wave;
  const bool live = blk < a.n_blocks;  // every wave reaches every barrier
  const int64_t b = live ? blk : 0;
  WyLds<NT, DK>& LK = *reinterpret_cast<WyLds<NT, DK>*>(&lds[wave]);
  WyLds<NT, DV>& LV = *reinterpret_cast<WyLds<NT, DV>*>(&lds[wave]);

  // gates of this block
  Gates<NT> gt;
  load_gates<NT>(a.beta + (size_t)b * C, a.g + (size_t)b * C, a.g_cumulative != 0, gt);
  // T in T-form
  Mat<NT> TT;
  if constexpr (TSRC == 0 || TSRC == 1) {  // given: fp32 (0) or bf16 (1) [C][C]
#pragma unroll
    for (int I = 0; I < NT; ++I)
#pragma unroll
      for (int J = 0; J <= I; ++J) {
        const size_t o = (size_t)b * C * C + (size_t)(16 * I + c) * C + 16 * J + 4 * g;
        if constexpr (TSRC == 0)
          TT.t[I][J] = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(T_in) + o);
        else
          TT.t[I][J] = unpack4(*reinterpret_cast<const bf16x4*>(reinterpret_cast<const __bf16*>(T_in) + o));
      }
  } else {  // formed here from K, beta, g
    KBlock<NT, DK> kb;
    if constexpr (MODE == MODE_NEUMANN) {
      // K is read from HBM once, into LDS; the Gram fragments and the W product both
      // take it from there (measured faster for the truncated sums, slower for the
      // doubling product, whose longer register lifetime then costs occupancy)
      stage_rows<NT, DK>(reinterpret_cast<const __bf16*>(a.K) + (size_t)b * C * DK, LK);
#pragma unroll
      for (int I = 0; I < NT; ++I)
#pragma unroll
        for (int s = 0; s < DK / 32; ++s)
          kb.kf[I][s] = *reinterpret_cast<const bf16x8*>(&LK.xr[16 * I + c][32 * s + 8 * g]);
    } else {
      load_kblock<NT, DK>(reinterpret_cast<const __bf16*>(a.K) + (size_t)b * C * DK, a.beta + (size_t)b * C,
                          a.g + (size_t)b * C, kb);
    }
    // A from the Gram tiles and the gate factors formed at the top (gt)
    Mat<NT> S, AD, AT;
    gram_from_frags<NT, DK, MAXD>(kb, S);
    gram_to_A<NT, MAXD, false>(S, gt, -1, AD, AT);
    if constexpr (MODE == MODE_EXACT) {
      doubling_T<NT, CMP_BF16>(AD, AT, TT);
    } else {
      Fp8Counts cnt{0, 0, 0, 0};
      neumann_T<NT, CMP_BF16, MAXD>(AD, AT, N, mask != 0, TT, cnt, false);
    }
  }
  // row packs of T diag(s) and T diag(beta); s and beta at column m = 16J + 4g + r
  float fs[NT][4], fb[NT][4];
  {
    const float sl = gt.bl * (gate_k ? __expf(gt.Gl) : 1.f);
#pragma unroll
    for (int J = 0; J < NT; ++J)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        fs[J][r] = __shfl(sl, 16 * J + 4 * g + r, 64);
        fb[J][r] = __shfl(gt.bl, 16 * J + 4 * g + r, 64);
      }
  }
  bf16x8 rpw[NT][(NT + 1) / 2], rlw[NT][(NT + 1) / 2], rpu[NT][(NT + 1) / 2],
      rlu[NT][(NT + 1) / 2];
  scaled_row_packs<NT>(TT, fs, rpw, rlw);
  scaled_row_packs<NT>(TT, fb, rpu, rlu);

  // W = (T diag(s)) K
  if constexpr (TSRC != 2 || MODE != MODE_NEUMANN)  // (else K is in LDS already)
    stage_rows<NT, DK>(reinterpret_cast<const __bf16*>(a.K) + (size_t)b * C * DK, LK);
  __syncthreads();
  if (live) {
    void* wo = out_bf16 ? (void*)(reinterpret_cast<__bf16*>(W_out) + (size_t)b * C * DK)
                        : (void*)(reinterpret_cast<float*>(W_out) + (size_t)b * C * DK);
    apply_rows<NT, DK>(rpw, rlw, LK, wo, out_bf16 != 0);
  }
  __syncthreads();
  // U = (T diag(beta)) V
  stage_rows<NT, DV>(V + (size_t)b * C * DV, LV);
  __syncthreads();
  if (live) {
    void* uo = out_bf16 ? (void*)(reinterpret_cast<__bf16*>(U_out) + (size_t)b * C * DV)
                        : (void*)(reinterpret_cast<float*>(U_out) + (size_t)b * C * DV);
    apply_rows<NT, DV>(rpu, rlu, LV, uo, out_bf16 != 0);
  }
}

int launch_wy(const BlocksArgs& a, const void* T, int t_bf16, int mode, int N, int mask,
              const void* V, int d_v, int gate_k, void* W_out, void* U_out, int out_bf16,
              hipStream_t s) {
  const dim3 grid((unsigned)((a.n_blocks + WY_WAVES - 1) / WY_WAVES));
  const dim3 block(WY_WAVES * WAVE);
  const int tsrc = T ? (t_bf16 ? 1 : 0) : 2;
  const bool narrow = (mode == MODE_NEUMANN) && mask && N <= 16;
  auto go = [&](auto nt, auto dk, auto dv, auto ts, auto md, auto mx) -> int {
    hipLaunchKernelGGL((wy_kernel<nt.value, dk.value, dv.value, ts.value, md.value, mx.value>), grid,
                       block, 0, s, a, T, N, mask, gate_k, reinterpret_cast<const __bf16*>(V), W_out,
                       U_out, out_bf16);
    return 0;
  };
  auto with_t = [&](auto nt, auto dk, auto dv) -> int {
    constexpr int NTv = decltype(nt)::value;
    using Full = std::integral_constant<int, NTv - 1>;
    using Nar = std::integral_constant<int, (NTv > 2 ? 1 : NTv - 1)>;
    using M0 = std::integral_constant<int, MODE_NEUMANN>;
    using M1 = std::integral_constant<int, MODE_EXACT>;
    if (tsrc == 0) return go(nt, dk, dv, std::integral_constant<int, 0>{}, M0{}, Full{});
    if (tsrc == 1) return go(nt, dk, dv, std::integral_constant<int, 1>{}, M0{}, Full{});
    using T2 = std::integral_constant<int, 2>;
    if (mode == MODE_EXACT) return go(nt, dk, dv, T2{}, M1{}, Full{});
    return narrow ? go(nt, dk, dv, T2{}, M0{}, Nar{}) : go(nt, dk, dv, T2{}, M0{}, Full{});
  };
  auto with_dv = [&](auto nt, auto dk) -> int {
    switch (d_v) {
      case 64: return with_t(nt, dk, std::integral_constant<int, 64>{});
      case 128: return with_t(nt, dk, std::integral_constant<int, 128>{});
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
    case 32: return with_dk(std::integral_constant<int, 2>{});
    case 64: return with_dk(std::integral_constant<int, 4>{});
    default: return -1;
  }
}

}  // namespace gdn
