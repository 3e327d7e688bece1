// chunk.hip -- chunk-wise gated delta rule forward (prefill) for C = 64.
//
// [GEO] "When Good Enough Is Optimal: Multiplication-Only Matrix Inversion
// Approximation for Quantized Gated DeltaNet", problem statement: the chunk-wise form
// needs T = (I - A)^-1 per chunk and carries a fixed-size recurrent state across
// chunks; Methodologie SS1-2 give the truncated / masked inverse used here.
// [PSDA] "A Persistent-State Dataflow Accelerator for Memory-Bound Linear Attention
// Decode on FPGA", section 2.A: keep the recurrent state on chip and stream only the
// per-token inputs.  Here the state slice lives in a wave's registers for the whole
// sequence.
//
// Per chunk (rows r = 0..63, G = in-chunk cumsum of the log-gates):
//   T   = inverse of I - A (truncated Neumann or exact doubling)
//   P   = Q K^T .* exp(G_i - G_j) .* [i >= j]
//   Y   = diag(beta) (V - diag(exp(G)) K S)
//   U'  = T Y                                (= U - W S with W = T diag(beta e^G) K)
//   O   = scale (diag(exp(G)) Q S + P U')
//   S  <- exp(G_C) S + K^T diag(exp(G_C - G)) U'
//
// Work split: one workgroup per (batch, head, 32 columns of d_v), four waves:
//   wave 0, 1  consumers: each owns 16 state columns S[:, 16v..16v+15] (fp32, in
//              registers) and runs the sequential scan;
//   wave 2     producer: gates, A and T (bf16 row-pack fragments) of the next chunk;
//   wave 3     producer: P (hi/lo bf16) of the current chunk; K and Q fragments and
//              K^T of the next chunk.
// Producers fill one half of a double-buffered LDS area while the consumers read
// the other; one barrier per chunk hands over, and every global load is issued at
// least one iteration before its data is used (see the schedule above the kernel).  Y, U' and P enter the MFMAs as hi/lo
// bf16 pairs (x = xh + xl, both bf16; products take xh yh + xl yh + xh yl), which
// brings the error of O and S to about 1e-4 relative (rounding each of them to a
// single bf16 would cost 1e-3 or more each), leaving the bf16 rounding of O itself
// as the dominant error.
#include "gdn_kernels.hpp"
#include "tri_block.hpp"

namespace gdn {

constexpr int CH = 64;           // chunk size (tokens)
constexpr int CNT = 4;           // 16-row tiles per chunk
constexpr int DVS = 32;          // d_v columns per workgroup
constexpr int KT_PAD = 8;        // padding of the K^T rows in LDS (bank spread)

struct ChunkArgs {
  const __bf16* Q;
  const __bf16* K;
  const __bf16* V;
  const float* beta;
  const float* g;
  const float* S0;
  void* O;
  float* S_out;
  unsigned long long* stats;
  int64_t T;
  int BH;
  int dv;
  int o_bf16;
  int N;
  int mask;
  float scale;
};

template <int DK>
struct ChunkLds {
  bf16x8 krp[CNT][DK / 32][WAVE];  // K rows as left-operand fragments (permuted k order)
  bf16x8 qrp[CNT][DK / 32][WAVE];  // Q rows, same
  bf16x8 trp[CNT][2][WAVE];        // T rows (T-form row packs)
  bf16x8 prh[CNT][2][WAVE];        // P rows, high part
  bf16x8 prl[CNT][2][WAVE];        // P rows, low part
  __bf16 kt[DK][CH + KT_PAD];      // K^T: kt[d][token]
  float beta[CH];
  float eg[CH];                    // exp(G_i)
  float eng[CH];                   // exp(-G_i)
  float egcg[CH];                  // exp(G_C - G_i)
  float G[CH];                     // G_i
  float egc;                       // exp(G_C)
  int split;                       // exp(-G) finite over the chunk
};

// 8 consecutive-in-slot bf16 of row `row` for k-pair p in the permuted order
// (k = 32p + 4g .. +3 and 32p + 16 + 4g .. +3)
template <int DK>
__device__ __forceinline__ bf16x8 load_rowpack(const __bf16* __restrict__ base, int row, int p) {
  const int g = lane_id() >> 4;
  const __bf16* src = base + (size_t)row * DK + 32 * p + 4 * g;
  bf16x4 lo = *reinterpret_cast<const bf16x4*>(src);
  bf16x4 hi = *reinterpret_cast<const bf16x4*>(src + 16);
  return join8(lo, hi);
}

__device__ __forceinline__ f32x4 unpack_lo(const bf16x8& v) {
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ f32x4 unpack_hi(const bf16x8& v) {
  return f32x4{(float)v[4], (float)v[5], (float)v[6], (float)v[7]};
}

// hi/lo bf16 split of two tiles packed as one operand fragment
__device__ __forceinline__ void pack8_hilo(const f32x4& a, const f32x4& b, bf16x8& hi, bf16x8& lo) {
  hi = pack8(a, b);
  lo = pack8(a - unpack_lo(hi), b - unpack_hi(hi));
}

// raw inputs of one chunk for the A/T producer (held in registers one chunk ahead)
template <int DK>
struct KChunk {
  KBlock<CNT, DK> kb;
  __device__ __forceinline__ void load(const ChunkArgs& a, int64_t row0) {
    const int l = lane_id(), c = l & 15;
#pragma unroll
    for (int I = 0; I < CNT; ++I)
#pragma unroll
      for (int p = 0; p < DK / 32; ++p) kb.kf[I][p] = load_rowpack<DK>(a.K + row0 * DK, 16 * I + c, p);
    kb.gl = a.g[row0 + l];
    kb.bl = a.beta[row0 + l];
  }
};

// ---- producer wave 2: gates, A, T, and the K layouts the other waves read ----------
template <int DK, int MODE, int CMP, int MAXD>
__device__ __forceinline__ void produce_T(const ChunkArgs& a, const KChunk<DK>& in, ChunkLds<DK>& L,
                                          Fp8Counts& cnt, bool count) {
  const int l = lane_id(), g = l >> 4, c = l & 15;
  const KBlock<CNT, DK>& kb = in.kb;
  Gates<CNT> gt;
  gates_from_lanes<CNT>(kb.gl, kb.bl, false, gt);
  Mat<CNT> S, AD, AT, TT;
  constexpr bool BANDED = (MODE == MODE_NEUMANN && CMP == CMP_FP8);
  gram_from_frags<CNT, DK, MAXD>(kb, S);
  const int band = a.mask ? a.N : -1;
  gram_to_A<CNT, MAXD, BANDED>(S, gt, BANDED ? band : -1, AD, AT);
  if constexpr (MODE == MODE_EXACT)
    doubling_T<CNT, CMP_BF16>(AD, AT, TT);
  else
    neumann_T<CNT, CMP, MAXD>(AD, AT, a.N, a.mask != 0, TT, cnt, count);
#pragma unroll
  for (int I = 0; I < CNT; ++I)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      if (2 * p <= I && I - (2 * p + 1) <= MAXD)
        L.trp[I][p][l] = pack8(tile_or_zero(TT, I, 2 * p), tile_or_zero(TT, I, 2 * p + 1));
    }
  // gate factors
  const float GC = __shfl(gt.Gl, CH - 1, 64);
  L.beta[l] = kb.bl;
  L.eg[l] = __expf(gt.Gl);
  L.eng[l] = __expf(-gt.Gl);
  L.egcg[l] = __expf(GC - gt.Gl);
  L.G[l] = gt.Gl;
  if (l == 0) {
    L.egc = __expf(GC);
    L.split = gt.split ? 1 : 0;
  }
}

// ---- producer wave 3: P = Q K^T .* exp(G_i - G_j) .* [i >= j] (hi/lo) -------------
// Reads K and Q fragments and the gates of the same chunk from LDS.
template <int DK>
__device__ __forceinline__ void produce_P(const ChunkLds<DK>& Lin, ChunkLds<DK>& Lout) {
  const int l = lane_id(), g = l >> 4, c = l & 15;
  const bool split = Lin.split != 0;
  const int lo_ = 4 * g - c;
#pragma unroll
  for (int I = 0; I < CNT; ++I) {
    const float rowf = Lin.eg[16 * I + c];  // exp(G_i), i = 16I + c
    const float Gi = Lin.G[16 * I + c];
    bf16x8 qf[DK / 32];
#pragma unroll
    for (int p = 0; p < DK / 32; ++p) qf[p] = Lin.qrp[I][p][l];
    f32x4 pt[CNT];
#pragma unroll
    for (int J = 0; J < CNT; ++J) {
      if (J > I) {
        pt[J] = zero4();
        continue;
      }
      // T-form tile (I,J): lane (g,c) reg r = q_{16I+c} . k_{16J+4g+r}
      f32x4 acc = zero4();
#pragma unroll
      for (int p = 0; p < DK / 32; ++p) acc = mma_bf16(Lin.krp[J][p][l], qf[p], acc);
      const f32x4 ncol = *reinterpret_cast<const f32x4*>(&Lin.eng[16 * J + 4 * g]);
      const f32x4 Gcol = *reinterpret_cast<const f32x4*>(&Lin.G[16 * J + 4 * g]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float f = split ? rowf * ncol[r] : __expf(Gi - Gcol[r]);
        const int d = 16 * (I - J) - r - lo_;       // i - j
        acc[r] = (d >= 0) ? acc[r] * f : 0.f;
      }
      pt[J] = acc;
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      if (2 * p <= I) {
        bf16x8 h, lw;
        pack8_hilo(pt[2 * p], (2 * p + 1 < CNT) ? pt[2 * p + 1] : zero4(), h, lw);
        Lout.prh[I][p][l] = h;
        Lout.prl[I][p][l] = lw;
      }
    }
  }
}

// ---- consumer waves: the state scan ----------------------------------------------
// Each phase first gathers the LDS fragments it needs into registers, then issues
// its MFMAs with independent accumulators adjacent, so LDS latency and MFMA latency
// overlap instead of serialising.
template <int DK, int MAXD, bool OBF16>
struct Consumer {
  static constexpr int NP = DK / 32;
  f32x4 S[DK / 16];  // D-form tiles: lane (g,c) reg r = S[16a + 4g + r][col0 + c]
  f32x4 qsg[CNT];    // previous chunk: e^{G_i} (Q S)_i in T-form (row 16I + c)
  bf16x8 cuh[2], cul[2];  // previous chunk: U' column packs, hi / lo

  __device__ __forceinline__ void load_v(const ChunkArgs& a, int64_t row0, int col0, f32x4 (&v)[CNT]) {
    const int l = lane_id(), g = l >> 4, c = l & 15;
    const __bf16* base = a.V + (row0 + 4 * g) * a.dv + col0 + c;
#pragma unroll
    for (int I = 0; I < CNT; ++I)
#pragma unroll
      for (int r = 0; r < 4; ++r) v[I][r] = (float)base[(16 * I + r) * a.dv];
  }

  // O of the previous chunk: scale (e^G Q S + P U'), T-form rows 16I + c
  __device__ __forceinline__ void emit_O(const ChunkArgs& a, int64_t row0, int col0,
                                         const ChunkLds<DK>& L) {
    const int l = lane_id(), g = l >> 4, c = l & 15;
    bf16x8 ph[CNT][2], pl[CNT][2];
#pragma unroll
    for (int I = 0; I < CNT; ++I)
#pragma unroll
      for (int p = 0; p < 2; ++p)
        if (2 * p <= I) {
          ph[I][p] = L.prh[I][p][l];
          pl[I][p] = L.prl[I][p][l];
        }
    f32x4 acc[CNT];
#pragma unroll
    for (int I = 0; I < CNT; ++I) acc[I] = qsg[I];
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int k = 0; k < 3; ++k)
#pragma unroll
        for (int I = 0; I < CNT; ++I)
          if (2 * p <= I) {
            const bf16x8& uu = (k == 1) ? cul[p] : cuh[p];
            const bf16x8& pp = (k == 2) ? pl[I][p] : ph[I][p];
            acc[I] = mma_bf16(uu, pp, acc[I]);
          }
#pragma unroll
    for (int I = 0; I < CNT; ++I) {
      const f32x4 o = acc[I] * a.scale;
      const int64_t off = (row0 + 16 * I + c) * a.dv + col0 + 4 * g;
      if constexpr (OBF16)
        *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(a.O) + off) = pack4(o);
      else
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.O) + off) = o;
    }
  }

  // state part of one chunk: K S, Q S, Y, U' = T Y, state update; keeps e^G Q S and U'
  __device__ __forceinline__ void step(const ChunkLds<DK>& L, const f32x4 (&vd)[CNT]) {
    const int l = lane_id(), g = l >> 4, c = l & 15;
    bf16x8 cps[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) cps[p] = pack8(S[2 * p], S[2 * p + 1]);
    // K S (D-form) and Q S (T-form), contraction over d_k; two row tiles at a time
    f32x4 ks[CNT];
#pragma unroll
    for (int I0 = 0; I0 < CNT; I0 += 2) {
      bf16x8 kf[2][NP], qf[2][NP];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          kf[i][p] = L.krp[I0 + i][p][l];
          qf[i][p] = L.qrp[I0 + i][p][l];
        }
      f32x4 ak[2] = {zero4(), zero4()}, aq[2] = {zero4(), zero4()};
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          ak[i] = mma_bf16(kf[i][p], cps[p], ak[i]);
          aq[i] = mma_bf16(cps[p], qf[i][p], aq[i]);
        }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        ks[I0 + i] = ak[i];
        qsg[I0 + i] = aq[i] * L.eg[16 * (I0 + i) + c];
      }
    }
    // Y = diag(beta) (V - diag(e^G) K S), D-form rows 16I + 4g + r
    f32x4 y[CNT];
#pragma unroll
    for (int I = 0; I < CNT; ++I) {
      const f32x4 b4 = *reinterpret_cast<const f32x4*>(&L.beta[16 * I + 4 * g]);
      const f32x4 e4 = *reinterpret_cast<const f32x4*>(&L.eg[16 * I + 4 * g]);
      y[I] = b4 * (vd[I] - e4 * ks[I]);
    }
    bf16x8 cyh[2], cyl[2];
    pack8_hilo(y[0], y[1], cyh[0], cyl[0]);
    pack8_hilo(y[2], y[3], cyh[1], cyl[1]);
    // U' = T Y (D-form), Y as a hi/lo pair
    bf16x8 tf[CNT][2];
#pragma unroll
    for (int I = 0; I < CNT; ++I)
#pragma unroll
      for (int p = 0; p < 2; ++p)
        if (2 * p <= I && I - (2 * p + 1) <= MAXD) tf[I][p] = L.trp[I][p][l];
    f32x4 u[CNT];
#pragma unroll
    for (int I = 0; I < CNT; ++I) u[I] = zero4();
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int I = 0; I < CNT; ++I)
          if (2 * p <= I && I - (2 * p + 1) <= MAXD) u[I] = mma_bf16(tf[I][p], k ? cyl[p] : cyh[p], u[I]);
    pack8_hilo(u[0], u[1], cuh[0], cul[0]);
    pack8_hilo(u[2], u[3], cuh[1], cul[1]);
    // S <- e^{G_C} S + K^T diag(e^{G_C - G}) U'
    f32x4 ut[CNT];
#pragma unroll
    for (int I = 0; I < CNT; ++I) ut[I] = u[I] * *reinterpret_cast<const f32x4*>(&L.egcg[16 * I + 4 * g]);
    bf16x8 cth[2], ctl[2];
    pack8_hilo(ut[0], ut[1], cth[0], ctl[0]);
    pack8_hilo(ut[2], ut[3], cth[1], ctl[1]);
    const float egc = L.egc;
#pragma unroll
    for (int A0 = 0; A0 < DK / 16; A0 += 4) {
      bf16x8 kt[4][2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const __bf16* kr = &L.kt[16 * (A0 + i) + c][32 * p + 4 * g];
          kt[i][p] = join8(*reinterpret_cast<const bf16x4*>(kr), *reinterpret_cast<const bf16x4*>(kr + 16));
        }
      f32x4 acc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = S[A0 + i] * egc;
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] = mma_bf16(kt[i][p], k ? ctl[p] : cth[p], acc[i]);
#pragma unroll
      for (int i = 0; i < 4; ++i) S[A0 + i] = acc[i];
    }
  }
};

// Schedule (iteration c = 0 .. nchunks, one barrier each, buffers by chunk parity):
//   wave 2: T and gates of chunk c+1 (its K rows were loaded one iteration earlier;
//           chunk c+2's rows are loaded now)
//   wave 3: P of chunk c from chunk c's K/Q fragments in LDS; K and Q rows of chunk
//           c+1 loaded now and staged (fragments, K^T) at the end of the iteration
//   waves 0, 1: state part of chunk c, and O of chunk c-1 (needs P of chunk c-1)
template <int DK, int MODE, int CMP, int MAXD, bool OBF16>
__global__ __launch_bounds__(256, 1) void chunk_fwd_kernel(ChunkArgs a) {
  __shared__ ChunkLds<DK> lds[2];
  const int wave = threadIdx.x / WAVE;
  const int l = lane_id(), g = l >> 4, c = l & 15;
  // workgroup -> (head, slice): the slices of one head are consecutive workgroup
  // indices inside one XCD (workgroups are dealt round-robin over the 8 XCDs), so
  // they share that XCD's L2 for the Q/K/V rows they all read
  const int n_slices = a.dv / DVS;
  const int total = a.BH * n_slices;
  const int wg = blockIdx.x;
  const int idx = (total % 8 == 0) ? (wg % 8) * (total / 8) + wg / 8 : wg;
  const int bh = idx / n_slices, slice = idx % n_slices;
  const int64_t nchunks = a.T / CH;
  const int64_t head_row0 = (int64_t)bh * a.T;
  const bool count = (CMP == CMP_FP8) && a.stats != nullptr;

  if (wave == 2) {
    Fp8Counts cnt{0, 0, 0, 0};
    // ping-pong register buffers: a buffer's rows are consumed one full iteration
    // (one barrier) after their loads are issued
    KChunk<DK> b0, b1;
    b0.load(a, head_row0);
    produce_T<DK, MODE, CMP, MAXD>(a, b0, lds[0], cnt, count);
    if (nchunks > 1) b0.load(a, head_row0 + CH);
    __syncthreads();
    for (int64_t ci = 0; ci <= nchunks; ci += 2) {
      // iteration ci: T of chunk ci+1 from b0, rows of chunk ci+2 into b1
      if (ci + 2 < nchunks) b1.load(a, head_row0 + (ci + 2) * CH);
      if (ci + 1 < nchunks) produce_T<DK, MODE, CMP, MAXD>(a, b0, lds[(ci + 1) & 1], cnt, count);
      __syncthreads();
      if (ci + 1 > nchunks) break;
      // iteration ci+1: T of chunk ci+2 from b1, rows of chunk ci+3 into b0
      if (ci + 3 < nchunks) b0.load(a, head_row0 + (ci + 3) * CH);
      if (ci + 2 < nchunks) produce_T<DK, MODE, CMP, MAXD>(a, b1, lds[(ci + 2) & 1], cnt, count);
      __syncthreads();
    }
    if constexpr (CMP == CMP_FP8) {
      if (count) {
        uint32_t v0 = wave_sum_u32(cnt.nonfinite), v1 = wave_sum_u32(cnt.sat_dyn);
        uint32_t v2 = wave_sum_u32(cnt.sat_static), v3 = wave_sum_u32(cnt.underflow);
        if (l == 0) {
          if (v0) atomicAdd(a.stats + 0, (unsigned long long)v0);
          if (v1) atomicAdd(a.stats + 1, (unsigned long long)v1);
          if (v2) atomicAdd(a.stats + 2, (unsigned long long)v2);
          if (v3) atomicAdd(a.stats + 3, (unsigned long long)v3);
        }
      }
    }
    return;
  }
  if (wave == 3) {
    // stages chunk c+1's K fragments, K^T and Q fragments at the end of iteration c;
    // their rows are loaded at the start of the iteration, so the P computation of
    // chunk c hides the load latency
    auto stage = [&](int64_t row0, ChunkLds<DK>& L, const bf16x8 (&kq)[CNT][DK / 32],
                     const bf16x8 (&qq)[CNT][DK / 32]) {
#pragma unroll
      for (int I = 0; I < CNT; ++I)
#pragma unroll
        for (int p = 0; p < DK / 32; ++p) {
          L.krp[I][p][l] = kq[I][p];
          L.qrp[I][p][l] = qq[I][p];
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const int d = 32 * p + 16 * (t >> 2) + 4 * g + (t & 3);
            L.kt[d][16 * I + c] = kq[I][p][t];
          }
        }
    };
    bf16x8 kq[CNT][DK / 32], qq[CNT][DK / 32];
    auto load = [&](int64_t row0) {
#pragma unroll
      for (int I = 0; I < CNT; ++I)
#pragma unroll
        for (int p = 0; p < DK / 32; ++p) {
          kq[I][p] = load_rowpack<DK>(a.K + row0 * DK, 16 * I + c, p);
          qq[I][p] = load_rowpack<DK>(a.Q + row0 * DK, 16 * I + c, p);
        }
    };
    load(head_row0);
    stage(head_row0, lds[0], kq, qq);
    __syncthreads();
    for (int64_t ci = 0; ci <= nchunks; ++ci) {
      const bool more = ci + 1 < nchunks;
      if (more) load(head_row0 + (ci + 1) * CH);
      if (ci < nchunks) produce_P<DK>(lds[ci & 1], lds[ci & 1]);
      if (more) stage(head_row0 + (ci + 1) * CH, lds[(ci + 1) & 1], kq, qq);
      __syncthreads();
    }
    return;
  }

  // consumers
  const int col0 = slice * DVS + 16 * wave;
  Consumer<DK, MAXD, OBF16> cs;
#pragma unroll
  for (int A = 0; A < DK / 16; ++A)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      cs.S[A][r] = a.S0 ? a.S0[((size_t)bh * DK + 16 * A + 4 * g + r) * a.dv + col0 + c] : 0.f;
  // V rows: ping-pong registers, loaded one iteration before use
  f32x4 v0[CNT], v1[CNT];
  cs.load_v(a, head_row0, col0, v0);
  __syncthreads();  // chunk 0's T, K and Q are in LDS
  for (int64_t ci = 0; ci <= nchunks; ci += 2) {
    if (ci + 1 < nchunks) cs.load_v(a, head_row0 + (ci + 1) * CH, col0, v1);
    if (ci >= 1) cs.emit_O(a, head_row0 + (ci - 1) * CH, col0, lds[(ci - 1) & 1]);
    if (ci < nchunks) cs.step(lds[ci & 1], v0);
    __syncthreads();
    if (ci + 1 > nchunks) break;
    if (ci + 2 < nchunks) cs.load_v(a, head_row0 + (ci + 2) * CH, col0, v0);
    cs.emit_O(a, head_row0 + ci * CH, col0, lds[ci & 1]);
    if (ci + 1 < nchunks) cs.step(lds[(ci + 1) & 1], v1);
    __syncthreads();
  }
#pragma unroll
  for (int A = 0; A < DK / 16; ++A)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      a.S_out[((size_t)bh * DK + 16 * A + 4 * g + r) * a.dv + col0 + c] = cs.S[A][r];
}

int launch_chunk_fwd(const ChunkLaunch& p, hipStream_t s) {
  ChunkArgs a;
  a.Q = reinterpret_cast<const __bf16*>(p.Q);
  a.K = reinterpret_cast<const __bf16*>(p.K);
  a.V = reinterpret_cast<const __bf16*>(p.V);
  a.beta = p.beta;
  a.g = p.g;
  a.S0 = p.S0;
  a.O = p.O;
  a.S_out = p.S_out;
  a.stats = p.stats;
  a.T = p.T;
  a.BH = p.B * p.H;
  a.dv = p.d_v;
  a.o_bf16 = p.o_bf16;
  a.N = p.N;
  a.mask = p.mask;
  a.scale = p.scale;
  const dim3 grid((unsigned)(a.BH * (p.d_v / DVS)));
  const dim3 block(4 * WAVE);
  const bool narrow = p.mode == 0 && p.mask && p.N <= 16;
  auto go = [&](auto dk, auto mode, auto cmp, auto maxd) {
    if (a.o_bf16)
      hipLaunchKernelGGL((chunk_fwd_kernel<dk.value, mode.value, cmp.value, maxd.value, true>), grid,
                         block, 0, s, a);
    else
      hipLaunchKernelGGL((chunk_fwd_kernel<dk.value, mode.value, cmp.value, maxd.value, false>), grid,
                         block, 0, s, a);
    return 0;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  auto with_dk = [&](auto dk) -> int {
    if (p.mode == 1) return go(dk, std::integral_constant<int, MODE_EXACT>{}, I1{}, I3{});
    if (p.cmp == CMP_FP8)
      return narrow ? go(dk, I0{}, I2{}, I1{}) : go(dk, I0{}, I2{}, I3{});
    if (p.cmp == CMP_BF16)
      return narrow ? go(dk, I0{}, I1{}, I1{}) : go(dk, I0{}, I1{}, I3{});
    return -1;
  };
  switch (p.d_k) {
    case 64: return with_dk(std::integral_constant<int, 64>{});
    case 128: return with_dk(std::integral_constant<int, 128>{});
    default: return -1;
  }
}

}  // namespace gdn
