// band.hip -- masked truncated Neumann (band N <= 16) for any chunk size, as T or as
// the WY products, one 16-row tile of the block per wave.
//
// [GEO] "When Good Enough Is Optimal: Multiplication-Only Matrix Inversion
// Approximation for Quantized Gated DeltaNet", Methodologie SS1-2: the masked
// truncated sum keeps subdiagonals 0..N of the Neumann sum of A.  Entry (i, j) of
// any power of a strictly lower-triangular A only involves A restricted to rows and
// columns j..i, so the masked result on rows 16I..16I+15 depends on A only inside the
// 32-row window of tiles I-1 and I when N <= 16.  Each wave therefore solves its own
// 32 x 32 window (the last tile row of that window is the output), which makes the
// work linear in the chunk size and independent across tiles.
//
// A workgroup of eight waves covers 128 rows of one block; it stages those rows plus the
// 16 rows above them (K, log-gates, beta; later the V columns into the same buffer) in
// LDS with coalesced 16-byte loads (eight waves rather than four: an eighth of the rows
// staged twice instead of a quarter, 13-14 % faster at C = 128 and 256; one buffer for
// K and then V: half the LDS, 5-8 % faster again), then each wave builds its window's A (gate differences need only the
// window's own log-gates), forms the masked sum with the 2 x 2 tile products, and
// writes its tile row of T, or of W = T diag(s) K and U = T diag(beta) V.  The key
// gate s = beta exp(G) needs G itself, the block prefix sum, which the workgroup
// adds from the rows above its window.
#include "gdn_kernels.hpp"
#include "tri_block.hpp"

namespace gdn {

constexpr int BAND_WAVES = 8;        // row tiles per workgroup
constexpr int BAND_ROWS = 16 * (BAND_WAVES + 1);
constexpr int BAND_PAD = 8;

// one row buffer: the staged K rows, then (after the W product) the V rows
template <int DK, int DV>
struct alignas(16) BandLds {
  static constexpr int LD = (DK > DV ? DK : DV) + BAND_PAD;
  __bf16 x[BAND_ROWS][LD];
  float gam[BAND_ROWS];
  float bet[BAND_ROWS];
  float gpre;  // sum of the log-gates of the block's rows above the staged ones
};

struct BandArgs {
  BlocksArgs a;
  const __bf16* V;
  int d_v;
  int N;
  int gate_k;
  void* T_out;
  int t_bf16;
  void* W_out;
  void* U_out;
  int out_bf16;
};

// K^T (or V^T) operand fragment over the 32 window rows starting at local row r0,
// columns 16e .. 16e + 15: lane (g, c) slot t <-> X[r0 + 16(t/4) + 4g + t%4][16e + c]
template <int LD>
__device__ __forceinline__ bf16x8 window_colpack(const __bf16* X, int r0, int e) {
  const int l = lane_id(), g = l >> 4, j = l & 15;
  const __bf16* p0 = X + (r0 + 4 * g + (j >> 2)) * LD + 16 * e + 4 * (j & 3);
  const __bf16* p1 = X + (r0 + 16 + 4 * g + (j >> 2)) * LD + 16 * e + 4 * (j & 3);
  return join8(lds_read_tr4(p0), lds_read_tr4(p1));
}

// Z (T-form row tile) = R X over the window, R as a hi/lo pair of row packs; stored
// row-major at row `row` of out: fp32 as columns 16e + 4g .. +3, bf16 two column tiles
// at a time with 16 contiguous bytes per lane (store_pair_bf16)
template <int D, int LD>
__device__ __forceinline__ void window_apply(const bf16x8& rh, const bf16x8& rl,
                                             const __bf16* X, int r0,
                                             void* __restrict__ out, int64_t row, bool obf16) {
  static_assert(D % 32 == 0, "column tiles are stored in pairs");
  const int g = lane_id() >> 4;
#pragma unroll
  for (int e2 = 0; e2 < D / 32; ++e2) {
    f32x4 acc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bf16x8 cp = window_colpack<LD>(X, r0, 2 * e2 + h);
      acc[h] = mma_bf16(cp, rh, zero4());
      acc[h] = mma_bf16(cp, rl, acc[h]);
    }
    if (obf16) {
      store_pair_bf16(reinterpret_cast<__bf16*>(out) + row * D, 2 * e2, acc[0], acc[1]);
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + row * D + 16 * (2 * e2 + h) + 4 * g) = acc[h];
    }
  }
}

template <int DK, int DV, bool TOUT>
__global__ __launch_bounds__(BAND_WAVES * WAVE) void band_kernel(BandArgs p) {
  __shared__ BandLds<DK, DV> L;
  const BlocksArgs& a = p.a;
  const int C = a.C;
  const int parts = C / (16 * BAND_WAVES);
  const int64_t total = a.n_blocks * parts;
  // workgroup -> (block, part): the parts of one block are consecutive indices inside
  // one XCD (workgroups are dealt round-robin over the 8 XCDs), so the halo rows a part
  // shares with its neighbour come from that XCD's L2
  const int64_t wg = blockIdx.x;
  const int64_t idx = (total % 8 == 0) ? (wg % 8) * (total / 8) + wg / 8 : wg;
  const int64_t b = idx / parts;
  const int I0 = (int)(idx % parts) * BAND_WAVES;  // first row tile of this workgroup
  const int row0 = 16 * (I0 - 1);                  // block row of local row 0 (may be < 0)
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const int l = lane_id(), g = l >> 4, c = l & 15;
  const __bf16* Kb = reinterpret_cast<const __bf16*>(a.K) + b * C * DK;

  // ---- stage rows row0 .. row0 + BAND_ROWS - 1 (rows above the block are zero) ------
  {
    constexpr int SEG = DK / 8;
    constexpr int NSEG = BAND_ROWS * SEG;
    constexpr int NK = (NSEG + BAND_WAVES * WAVE - 1) / (BAND_WAVES * WAVE);
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int e = i * BAND_WAVES * WAVE + tid, r = e / SEG, s = e % SEG;
      const int gr = row0 + r;
      if (e < NSEG) {
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(Kb + (int64_t)(gr < 0 ? 0 : gr) * DK + 8 * s);
        *reinterpret_cast<bf16x8*>(&L.x[r][8 * s]) = gr < 0 ? bf16x8{} : v;
      }
    }
    if (tid < BAND_ROWS) {
      const int gr = row0 + tid;
      const float gv = a.g[b * C + (gr < 0 ? 0 : gr)], bv = a.beta[b * C + (gr < 0 ? 0 : gr)];
      L.gam[tid] = gr < 0 ? 0.f : gv;
      L.bet[tid] = gr < 0 ? 0.f : bv;
    }
    if (wave == 0) {
      // block prefix of the log-gates above the staged rows (absolute G for the key
      // gate); with cumulative gates the staged values are absolute already
      float s = 0.f;
      if (!a.g_cumulative)
        for (int r = l; r < row0; r += WAVE) s += a.g[b * C + r];
      s = wave_sum(s);
      if (l == 0) L.gpre = s;
    }
  }
  __syncthreads();

  // ---- this wave's window: local rows 16w .. 16w + 31, output row tile I0 + w -------
  const int I = I0 + wave;
  const int r0 = 16 * wave;
  const float gl = l < 32 ? L.gam[r0 + l] : 0.f;
  const float bl = l < 32 ? L.bet[r0 + l] : 0.f;
  KBlock<2, DK> kb;
#pragma unroll
  for (int J = 0; J < 2; ++J)
#pragma unroll
    for (int s = 0; s < DK / 32; ++s) kb.kf[J][s] = *reinterpret_cast<const bf16x8*>(&L.x[r0 + 16 * J + c][32 * s + 8 * g]);
  kb.gl = gl;
  kb.bl = bl;
  Gates<2> gt;
  gates_from_lanes<2>(gl, bl, a.g_cumulative != 0, gt);
  Mat<2> S, AD, AT, TT;
  gram_from_frags<2, DK, 1>(kb, S);
  gram_to_A<2, 1, false>(S, gt, -1, AD, AT);
  Fp8Counts cnt{0, 0, 0, 0};
  neumann_T<2, CMP_BF16, 1>(AD, AT, p.N, true, TT, cnt, false);

  if constexpr (TOUT) {
    // row tile I of T: tiles (I, I-1) and (I, I) from the window, zero elsewhere, as
    // whole 128-byte row pieces (store_rows_*)
    const int NTB = C / 16;
    auto tile = [&](int J) -> f32x4 { return (J == I) ? TT.t[1][1] : (J == I - 1) ? TT.t[1][0] : zero4(); };
    const int64_t rowbase = b * C * C + (int64_t)(16 * I) * C;
    if (p.t_bf16) {
      for (int J = 0; J < NTB; J += 4) {
        const f32x4 t[4] = {tile(J), tile(J + 1), tile(J + 2), tile(J + 3)};
        store_rows_bf16x4<true>(reinterpret_cast<__bf16*>(p.T_out) + rowbase + 16 * J, C, t);
      }
    } else {
      for (int J = 0; J < NTB; J += 2)
        store_rows_f32x2<true>(reinterpret_cast<float*>(p.T_out) + rowbase + 16 * J, C, tile(J), tile(J + 1));
    }
  }
  if constexpr (DV > 0) {
    // column factors at window column m = 16J + 4g + r: s_m (key side) and beta_m
    float Gabs = gt.Gl;
    if (!a.g_cumulative) {
      float pre = 0.f;  // log-gates of the staged rows above the window
      for (int r = l; r < r0; r += WAVE) pre += L.gam[r];
      Gabs += L.gpre + wave_sum(pre);
    }
    const float sl = bl * (p.gate_k ? __expf(Gabs) : 1.f);
    f32x4 tw[2], tu[2];
#pragma unroll
    for (int J = 0; J < 2; ++J)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 16 * J + 4 * g + r;
        tw[J][r] = TT.t[1][J][r] * __shfl(sl, m, 64);
        tu[J][r] = TT.t[1][J][r] * __shfl(bl, m, 64);
      }
    // T diag(s) and T diag(beta) as bf16 hi/lo pairs (x = xh + xl), so the products
    // keep about 16 bits and the rounding of the outputs dominates their error
    auto hilo = [](const f32x4& x0, const f32x4& x1, bf16x8& h, bf16x8& lo) {
      h = pack8(x0, x1);
      const f32x4 h0{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
      const f32x4 h1{(float)h[4], (float)h[5], (float)h[6], (float)h[7]};
      lo = pack8(x0 - h0, x1 - h1);
    };
    bf16x8 wh, wl, uh, ul;
    hilo(tw[0], tw[1], wh, wl);
    hilo(tu[0], tu[1], uh, ul);
    // the V rows go into registers now, so that their loads overlap the W product, and
    // into the row buffer once every wave is done with K
    constexpr int SV = DV / 8;
    constexpr int NSV = BAND_ROWS * SV;
    constexpr int NV = (NSV + BAND_WAVES * WAVE - 1) / (BAND_WAVES * WAVE);
    const __bf16* Vb = p.V + b * C * DV;
    bf16x8 vr[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = i * BAND_WAVES * WAVE + tid, r = e / SV, s = e % SV;
      const int gr = row0 + r;
      vr[i] = bf16x8{};
      if (e < NSV && gr >= 0) vr[i] = *reinterpret_cast<const bf16x8*>(Vb + (int64_t)gr * DV + 8 * s);
    }
    const int64_t row = b * C + 16 * I + c;
    constexpr int LD = BandLds<DK, DV>::LD;
    window_apply<DK, LD>(wh, wl, &L.x[0][0], r0, p.W_out, row, p.out_bf16 != 0);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = i * BAND_WAVES * WAVE + tid, r = e / SV, s = e % SV;
      if (e < NSV) *reinterpret_cast<bf16x8*>(&L.x[r][8 * s]) = vr[i];
    }
    __syncthreads();
    window_apply<DV, LD>(uh, ul, &L.x[0][0], r0, p.U_out, row, p.out_bf16 != 0);
  }
}

int launch_band(const BlocksArgs& a, const void* V, int d_v, int N, int gate_k, void* T_out, int t_bf16,
                void* W_out, void* U_out, int out_bf16, hipStream_t s) {
  if (a.C < 16 * BAND_WAVES || a.C % (16 * BAND_WAVES) != 0 || N > 16) return -1;
  BandArgs p;
  p.a = a;
  p.V = reinterpret_cast<const __bf16*>(V);
  p.d_v = d_v;
  p.N = N;
  p.gate_k = gate_k;
  p.T_out = T_out;
  p.t_bf16 = t_bf16;
  p.W_out = W_out;
  p.U_out = U_out;
  p.out_bf16 = out_bf16;
  const dim3 grid((unsigned)(a.n_blocks * (a.C / (16 * BAND_WAVES))));
  const dim3 block(BAND_WAVES * WAVE);
  auto go = [&](auto dk, auto dv, auto tout) {
    hipLaunchKernelGGL((band_kernel<dk.value, dv.value, tout.value>), grid, block, 0, s, p);
    return 0;
  };
  auto with_dk = [&](auto dk) -> int {
    if (T_out) return go(dk, std::integral_constant<int, 0>{}, std::true_type{});
    switch (d_v) {
      case 64: return go(dk, std::integral_constant<int, 64>{}, std::false_type{});
      case 128: return go(dk, std::integral_constant<int, 128>{}, std::false_type{});
      default: return -1;
    }
  };
  switch (a.d_k) {
    case 64: return with_dk(std::integral_constant<int, 64>{});
    case 128: return with_dk(std::integral_constant<int, 128>{});
    default: return -1;
  }
}

}  // namespace gdn
