// chunk.hip -- chunk-wise gated delta rule forward (prefill) for C = 64.
//
// [GEO] "When Good Enough Is Optimal: Multiplication-Only Matrix Inversion
// Approximation for Quantized Gated DeltaNet", problem statement: the chunk-wise form
// needs T = (I - A)^-1 per chunk and carries a fixed-size recurrent state across
// chunks; Methodologie SS1-2 give the truncated / masked inverse used here.
// [PSDA] "A Persistent-State Dataflow Accelerator for Memory-Bound Linear Attention
// Decode on FPGA", section 2.A: keep the recurrent state on chip and stream only the
// per-token inputs.  Here each state slice lives in one wave's registers for the
// whole sequence.
//
// Per chunk (rows r = 0..63, G = in-chunk cumsum of the log-gates):
//   T   = inverse of I - A (truncated Neumann or exact doubling)
//   P   = Q K^T .* exp(G_i - G_j) .* [i >= j]
//   Y   = diag(beta) (V - diag(exp(G)) K S)
//   U'  = T Y                                (= U - W S with W = T diag(beta e^G) K)
//   O   = scale (diag(exp(G)) Q S + P U')
//   S  <- exp(G_C) S + K^T diag(exp(G_C - G)) U'
//
// One workgroup per (batch, head, 32 columns of d_v) with eight waves; waves w and
// w + 4 share a SIMD, so every SIMD interleaves two waves:
//   waves 0, 1  state waves: each owns 16 columns of S (fp32, in registers) and runs
//               the sequential part of a chunk: K S, Y, U' = T Y and the state update.
//               They hand S^T (bf16) and U' (hi/lo) to the output waves.
//   waves 2, 3, 6, 7  output waves for row tiles 0, 1, 2, 3, one chunk behind: P and
//               O = scale (e^G Q S + P U') for their 16 rows, all 32 columns.  Tiles 0
//               and 2 share one SIMD, tiles 1 and 3 another (measured as fast as the
//               pairing 0 and 3, 1 and 2, which evens the two SIMDs' MFMA counts).
//   wave 5      T - I of the next chunk (beside state wave 1): formed here on the band
//               path (N <= 3 with the mask, bf16); for the masked fp8 chain with N <= 3
//               put together from the band rows of the fp8 band pre-pass; else streamed
//               from the row packs a batched pre-pass wrote (every other variant).
//   wave 4      copies K rows, V columns, log-gates and beta of the chunk after next
//               into a 4-deep LDS ring and forms that chunk's gate factors (beside
//               state wave 0).
// The state waves, heavy on MFMA and on the sequential chain, share their SIMDs only
// with the two light roles.
// One barrier per chunk hands every buffer over (schedule above the kernel).  The K
// rows sit in LDS row-major; the K^T operand of the state update comes from the same
// rows through the LDS transpose read.  Q is read once per workgroup, each lane taking
// 16 contiguous bytes (8 consecutive d), so the contractions over d that involve Q use
// that natural order of d in both operands.  U' = T Y is formed as Y + (T - I) Y: the
// identity part stays exact in fp32 and only the strictly lower part of T meets the
// bf16-rounded Y.  U' (in O) and e^{G_C - G} U' (in the state update) and P enter the
// MFMAs as hi/lo bf16 pairs (x = xh + xl; products take xh yh + xl yh + xh yl).  This
// keeps the error of S near 1e-4 relative and that of O at the level of its own bf16
// rounding.
#include "gdn_kernels.hpp"
#include "tri_block.hpp"

namespace gdn {

constexpr int CH = 64;     // chunk size (tokens)
constexpr int CNT = 4;     // 16-row tiles per chunk
constexpr int DVS = 32;    // d_v columns per workgroup
constexpr int KPAD = 16;   // bf16 padding of the LDS K rows (bank spread; measured best of 8, 16, 24)
constexpr int VPAD = 0;    // bf16 padding of the LDS V rows (measured: 0 and 16 beat 8)
constexpr int NWAVES = 8;

struct ChunkArgs {
  const __bf16* Q;
  const __bf16* K;
  const __bf16* V;
  const float* beta;
  const float* g;
  const float* S0;
  void* O;
  float* S_out;
  const bf16x8* packs;  // T - I row packs of every chunk (pre-pass), MODE_LOAD only
  const bf16x4* band;   // band rows of T - I of every chunk (fp8 band pre-pass), MODE_LOADBAND only
  int64_t T;
  int BH;
  int dv;
  int N;
  int mask;
  float scale;
};

// raw inputs of one chunk staged in LDS: K rows (row-major), this workgroup's V
// columns (row-major), log-gates and beta
template <int DK>
struct alignas(16) ChunkIn {
  __bf16 k[CH][DK + KPAD];
  __bf16 v[CH][DVS + VPAD];
  float g[CH];
  float beta[CH];
};

// gate factors of one chunk
struct alignas(16) ChunkGates {
  float beta[CH];
  float eg[CH];    // exp(G_i)
  float eng[CH];   // exp(-G_i)
  float egcg[CH];  // exp(G_C - G_i)
  float G[CH];
  float egc;       // exp(G_C)
  int split;       // exp(-G) finite over the chunk
};

// products of one chunk handed from their producers to their readers
template <int DK>
struct alignas(16) ChunkBuf {
  bf16x8 trp[CNT][2][WAVE];         // rows of T - I (row packs)
  __bf16 st[2][16][DK + KPAD];      // per state wave: S^T before the chunk, st[col][d]
  bf16x8 uh[2][2][WAVE];            // per state wave: U' column packs, high
  bf16x8 ul[2][2][WAVE];            // per state wave: U' column packs, low
};

// The state's d order.  Row 4g + r of the state's D-form tile a holds
//   d = sdim(a, g, r) = 32 (a / 2) + 8 g + 4 (a % 2) + r,
// so the two tiles 2p, 2p + 1 of one lane are, slot for slot, the natural-order
// operand fragment (slot t <-> d = 32p + 8g + t) of the k-pair p: K S then reads K rows
// with one 16-byte load per fragment, and S^T goes out with one 16-byte store.
__device__ __forceinline__ int sdim(int a, int g, int r) { return 32 * (a >> 1) + 8 * g + 4 * (a & 1) + r; }

// K^T operand fragment of state tile a (row c <-> d = sdim(a, c / 4, c % 4)), token
// pair p: lane (g, c) slot t <-> K[32p + 16(t/4) + 4g + t%4][sdim(a, c/4, c%4)].  The
// transpose read hands lane i element i % 4 of the 8-byte pieces addressed by lanes
// 4k + i / 4 (k = 0..3); lane j addresses four consecutive d starting at
// sdim(a, j % 4, 0), so lane i receives column sdim(a, i / 4, i % 4) of four
// consecutive rows.
template <int DK>
__device__ __forceinline__ bf16x8 ktpack_lds(const ChunkIn<DK>& R, int a, int p) {
  const int l = lane_id(), g = l >> 4, j = l & 15;
  const int d0 = sdim(a, j & 3, 0);
  const __bf16* p0 = &R.k[32 * p + 4 * g + (j >> 2)][d0];
  const __bf16* p1 = &R.k[32 * p + 16 + 4 * g + (j >> 2)][d0];
  return join8(lds_read_tr4(p0), lds_read_tr4(p1));
}

// natural d order (slot t <-> d = 32p + 8g + t): K row `row` from LDS, and the Q rows
// of row tiles I0, I1 of a chunk from global memory (16 contiguous bytes per lane)
template <int DK>
__device__ __forceinline__ bf16x8 rowfrag_nat(const ChunkIn<DK>& R, int row, int p) {
  const int g = lane_id() >> 4;
  return *reinterpret_cast<const bf16x8*>(&R.k[row][32 * p + 8 * g]);
}

template <int DK, int NI, int I0, int I1>
__device__ __forceinline__ void load_q_nat(const ChunkArgs& a, int64_t row0, bf16x8 (&q)[NI][DK / 32]) {
  const int l = lane_id(), g = l >> 4, c = l & 15;
  const __bf16* base = a.Q + (row0 + c) * DK + 8 * g;
#pragma unroll
  for (int p = 0; p < DK / 32; ++p) {
    q[0][p] = *reinterpret_cast<const bf16x8*>(base + (16 * I0) * DK + 32 * p);
    if constexpr (NI > 1) q[NI - 1][p] = *reinterpret_cast<const bf16x8*>(base + (16 * I1) * DK + 32 * p);
  }
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

// Gate factors of one chunk from its raw log-gates and beta (lane l = position l),
// formed by the stager as it stages the chunk: G = in-chunk cumsum by the wave scan.
__device__ __forceinline__ void write_gates(float gl, float bl, ChunkGates& GT) {
  const int l = lane_id();
  const float Gl = wave_inclusive_scan(gl);
  const bool split = wave_min(Gl) >= -80.f;
  GT.beta[l] = bl;
  GT.eg[l] = __expf(Gl);
  GT.eng[l] = __expf(-Gl);
  GT.G[l] = Gl;
  const float GC = readlane_f(Gl, CH - 1);
  GT.egcg[l] = __expf(GC - Gl);
  if (l == 0) {
    GT.egc = __expf(GC);
    GT.split = split ? 1 : 0;
  }
}

// ---- T wave -----------------------------------------------------------------------------
// Band-masked sum with N <= 3: the band of T - I by band3_from_subdiag (lane i = row i).
// The Gram entries come from the MFMA diagonal tiles and the last four columns of the
// tile left of each (T-form, through LDS to the row lanes).  Only the band slots of the
// row packs are written: the rest of both pack buffers is cleared once before the scan
// and stays zero.
constexpr int MODE_BAND = 16;  // chunk-only codes next to the MODE_* values
// Every other variant (the truncated sum on bf16 or fp8 operands, masked or not, and the
// exact product) has its T - I formed by the batched pre-pass as the row packs the
// state step reads; the T wave only streams them into LDS.
constexpr int MODE_LOAD = 17;
// The masked fp8 chain with N <= 3: the band pre-pass (band_fp8_kernel) wrote the band of
// T - I per row; the T wave puts it into the band slots of the row packs.
constexpr int MODE_LOADBAND = 18;

// row-pack slot (bf16 index into trp) of T - I at row i, column j
__device__ __forceinline__ int trp_slot(int i, int j) {
  const int I = i >> 4, c = i & 15, p = j >> 5, h = (j >> 4) & 1, gg = (j >> 2) & 3;
  return ((I * 2 + p) * WAVE + 16 * gg + c) * 8 + (j & 3) + 4 * h;
}

// a_d(l) = A[l][l - d] for d = 1..3 from the Gram band sv[d] = k_l . k_{l-d} and this
// lane's beta, G, exp(G), exp(-G): (-beta_l exp(G_l)) S exp(-G_{l-d}) when every exp(-G)
// of the chunk is finite, else -beta_l exp(G_l - G_{l-d}) S (gram_to_A's two forms, in its
// operation order); zero outside the chunk (l < d) or the band (d > N)
// (split: wave-uniform, so only one form is evaluated)
__device__ __forceinline__ void band_A(const float (&sv)[4], float bl, float Gl, float eg, float eng, bool split,
                                       int N, float (&ad)[4]) {
  const int l = lane_id();
  ad[0] = 0.f;
  if (split) {
    const float rl = -bl * eg;
    float nm = eng;
#pragma unroll
    for (int d = 1; d <= 3; ++d) {
      nm = lane_shr1(nm);
      ad[d] = (l >= d && d <= N) ? rl * sv[d] * nm : 0.f;
    }
  } else {
    float Gm = Gl;
#pragma unroll
    for (int d = 1; d <= 3; ++d) {
      Gm = lane_shr1(Gm);
      ad[d] = (l >= d && d <= N) ? -bl * __expf(Gl - Gm) * sv[d] : 0.f;
    }
  }
}

// band values t[1..3] of row l into their row-pack slots
__device__ __forceinline__ void scatter_band(const float (&t)[4], bf16x8 (&trp)[CNT][2][WAVE]) {
  const int l = lane_id();
  __bf16* tb = reinterpret_cast<__bf16*>(&trp[0][0][0]);
#pragma unroll
  for (int d = 1; d <= 3; ++d)
    if (l - d >= 0) tb[trp_slot(l, l - d)] = (__bf16)t[d];
}

template <int DK>
__device__ __forceinline__ void produce_T_band(const ChunkArgs& a, const ChunkIn<DK>& R,
                                               bf16x8 (&trp)[CNT][2][WAVE], const ChunkGates& GT,
                                               float (&xr)[CH][XR_LD]) {
  const int l = lane_id(), c = l & 15;
  bf16x8 kf[CNT][DK / 32];
#pragma unroll
  for (int I = 0; I < CNT; ++I)
#pragma unroll
    for (int p = 0; p < DK / 32; ++p) kf[I][p] = rowfrag_nat<DK>(R, 16 * I + c, p);
  const float bl = R.beta[l];
  const float Gl = GT.G[l];  // the gates were formed by the stager
  float sv[4];
  gram_band3<CNT, DK>(kf, xr, sv);
  // a_d(l) = -beta_l (k_l . k_{l-d}) exp(G_l - G_{l-d}), zero outside the chunk or band
  // (the exponential of the difference: three exponentials per row measured faster here
  // than band_A's split form, which reads two more gate rows)
  float ad[4];
  ad[0] = 0.f;
  float Gm = Gl;
#pragma unroll
  for (int d = 1; d <= 3; ++d) {
    Gm = lane_shr1(Gm);
    ad[d] = (l >= d && d <= a.N) ? -bl * __expf(Gl - Gm) * sv[d] : 0.f;
  }
  float tv[4];
  band3_from_subdiag(ad, a.N, tv);
  scatter_band(tv, trp);
}

// ---- the masked fp8 chain (N <= 3) of every chunk, ahead of the scan ------------------
// [GEO] "Adaptation a la Quantification" with the mask: band3_fp8 on A's band, formed by
// band_A in gram_to_A's gate form and order (so bit for bit the A of gdn_build_A).  One
// wave per chunk writes (T - I)[i][i - d] of row i as bf16 in slots d = 1..3 of 8 bytes
// (slot 0 zero), 512 bytes per chunk; the scan's T wave puts them into its row packs.
// The chain's serial scale reductions and divisions would otherwise sit in the scan's T
// wave, which then sets the scan's pace.
template <int DK>
__global__ __launch_bounds__(256) void band_fp8_kernel(const __bf16* __restrict__ K, const float* __restrict__ beta,
                                                       const float* __restrict__ g, int64_t n_chunks, int N,
                                                       bf16x4* __restrict__ out, unsigned long long* stats) {
  __shared__ float xr[4][CH][XR_LD];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  const int64_t ch = (int64_t)blockIdx.x * 4 + wave;
  if (ch >= n_chunks) return;
  const int l = lane_id(), gq = l >> 4, c = l & 15;
  const float gl = g[ch * CH + l], bl = beta[ch * CH + l];
  const __bf16* kb = K + ch * CH * DK;
  // plain loads: each instruction covers half of 16 rows' 128-byte lines and the next one
  // the other half; with streaming (non-temporal) loads the lines were fetched twice
  // (1.37x the key bytes, 131 against 112 us)
  bf16x8 kf[CNT][DK / 32];
#pragma unroll
  for (int I = 0; I < CNT; ++I)
#pragma unroll
    for (int p = 0; p < DK / 32; ++p)
      kf[I][p] = *reinterpret_cast<const bf16x8*>(kb + (size_t)(16 * I + c) * DK + 32 * p + 8 * gq);
  // the gate factors as the stager (and gdn_build_A) forms them
  const float Gl = wave_inclusive_scan(gl);
  const bool split = __builtin_amdgcn_readfirstlane(wave_min(Gl) >= -80.f ? 1 : 0) != 0;
  const float eg = __expf(Gl), eng = __expf(-Gl);
  float sv[4], ad[4], tv[4];
  gram_band3<CNT, DK>(kf, xr[wave], sv);
  band_A(sv, bl, Gl, eg, eng, split, N, ad);
  Fp8Counts cnt{0, 0, 0, 0};
  const bool count = stats != nullptr;
  band3_fp8(ad, N, tv, cnt, count);
  bf16x4 o;
  o[0] = (__bf16)0.f;
  o[1] = (__bf16)tv[1];
  o[2] = (__bf16)tv[2];
  o[3] = (__bf16)tv[3];
  out[ch * CH + l] = o;
  if (count) flush_counts(cnt, stats);
}

int launch_band_fp8(const BlocksArgs& a, int N, void* out, unsigned long long* stats, hipStream_t s) {
  if (a.C != CH || a.g_cumulative) return -1;
  const dim3 grid((unsigned)((a.n_blocks + 3) / 4)), block(4 * WAVE);
  auto go = [&](auto dk) {
    hipLaunchKernelGGL((band_fp8_kernel<dk.value>), grid, block, 0, s, reinterpret_cast<const __bf16*>(a.K),
                       a.beta, a.g, a.n_blocks, N, reinterpret_cast<bf16x4*>(out), stats);
    return 0;
  };
  switch (a.d_k) {
    case 64: return go(std::integral_constant<int, 64>{});
    case 128: return go(std::integral_constant<int, 128>{});
    default: return -1;
  }
}

// ---- waves 0, 1: the state scan -------------------------------------------------------
template <int DK, int MAXD>
struct StateWave {
  static constexpr int NP = DK / 32;
  static constexpr int NA = DK / 16;
  f32x4 S[NA];  // D-form tiles: lane (g,c) reg r = S[sdim(a, g, r)][col0 + c]
  // this chunk's K rows, V tiles, beta and half of the K^T fragments, read at the end
  // of the previous step
  bf16x8 kfn[CNT][NP];
  bf16x4 vtn[CNT];
  f32x4 b4n[CNT];
  // K^T fragments of state tiles 0..KTP-1 read ahead as well (all eight measured no
  // faster and leave no register headroom)
  static constexpr int KTP = 4;
  bf16x8 ktn[KTP][2];

  // a chunk's raw inputs as the step uses them: K rows as the K S operand (natural d
  // order, the state's d order), V in D-form (rows 16I + 4g + r, column 16v + c) by the
  // transpose read, beta at rows 16I + 4g + r
  __device__ __forceinline__ void read_inputs(const ChunkIn<DK>& R, int v) {
    const int l = lane_id(), g = l >> 4, c = l & 15;
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int I = 0; I < CNT; ++I) kfn[I][p] = rowfrag_nat<DK>(R, 16 * I + c, p);
#pragma unroll
    for (int I = 0; I < CNT; ++I) {
      vtn[I] = lds_read_tr4(&R.v[16 * I + 4 * g + (c >> 2)][16 * v + 4 * (c & 3)]);
      b4n[I] = *reinterpret_cast<const f32x4*>(&R.beta[16 * I + 4 * g]);
    }
#pragma unroll
    for (int A = 0; A < KTP; ++A)
#pragma unroll
      for (int p = 0; p < 2; ++p) ktn[A][p] = ktpack_lds<DK>(R, A, p);
  }

  // one chunk: S^T out, K S, Y, U' = T Y (out), state update.  LDS operands are
  // requested in two batches, each ahead of the phase before the one that needs it, so
  // that the reads overlap MFMA and VALU work instead of sitting between them.
  // Rn: the next chunk's inputs (already in LDS), whose K rows are read at the end of
  // this step, off the dependency chain of the next one
  __device__ __forceinline__ void step(const ChunkIn<DK>& R, const ChunkIn<DK>& Rn, const ChunkGates& GT,
                                       ChunkBuf<DK>& B, int v) {
    const int l = lane_id(), g = l >> 4, c = l & 15;
    // batch 1: e^G (K rows, V tiles and beta were read by the previous step)
    bf16x8 kf[CNT][NP];
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int I = 0; I < CNT; ++I) kf[I][p] = kfn[I][p];
    bf16x4 vt[CNT];
    f32x4 b4[CNT], e4[CNT];
#pragma unroll
    for (int I = 0; I < CNT; ++I) {
      vt[I] = vtn[I];
      b4[I] = b4n[I];
      e4[I] = *reinterpret_cast<const f32x4*>(&GT.eg[16 * I + 4 * g]);
    }
    const float egc = GT.egc;
    __builtin_amdgcn_sched_barrier(0);
    // S as bf16: column packs for K S here (slot t <-> d = 32p + 8g + t), which are
    // also S^T rows (8 consecutive d per lane) for the output waves
    bf16x8 cps[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      cps[p] = pack8(S[2 * p], S[2 * p + 1]);
      *reinterpret_cast<bf16x8*>(&B.st[v][c][32 * p + 8 * g]) = cps[p];
    }
    // K S (D-form), contraction over d_k, the four row tiles interleaved
    f32x4 ks[CNT];
#pragma unroll
    for (int I = 0; I < CNT; ++I) ks[I] = zero4();
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int I = 0; I < CNT; ++I) ks[I] = mma_bf16(kf[I][p], cps[p], ks[I]);
    // e^{G_C} S while the K S products run (S itself is free once packed)
#pragma unroll
    for (int A = 0; A < NA; ++A) S[A] = S[A] * egc;
    __builtin_amdgcn_sched_barrier(0);
    // batch 2: T row packs, e^{G_C - G}, e^{G_C}, K^T packs
    bf16x8 tf[CNT][2];
#pragma unroll
    for (int I = 0; I < CNT; ++I)
#pragma unroll
      for (int p = 0; p < 2; ++p)
        if (2 * p <= I && I - (2 * p + 1) <= MAXD) tf[I][p] = B.trp[I][p][l];
    f32x4 w4[CNT];
#pragma unroll
    for (int I = 0; I < CNT; ++I) w4[I] = *reinterpret_cast<const f32x4*>(&GT.egcg[16 * I + 4 * g]);
    bf16x8 kt[NA][2];
#pragma unroll
    for (int A = 0; A < NA; ++A)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        if (A < KTP)
          kt[A][p] = ktn[A][p];  // read at the end of the previous step
        else
          kt[A][p] = ktpack_lds<DK>(R, A, p);
      }
    __builtin_amdgcn_sched_barrier(0);
    // Y = diag(beta) (V - diag(e^G) K S), D-form rows 16I + 4g + r
    f32x4 y[CNT];
#pragma unroll
    for (int I = 0; I < CNT; ++I) y[I] = b4[I] * (unpack4(vt[I]) - e4[I] * ks[I]);
    // U' = T Y = Y + (T - I) Y (D-form): the identity part exactly in fp32, the rest
    // with Y rounded once to bf16
    const bf16x8 cy[2] = {pack8(y[0], y[1]), pack8(y[2], y[3])};
    f32x4 u[CNT];
#pragma unroll
    for (int I = 0; I < CNT; ++I) u[I] = y[I];
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int I = 0; I < CNT; ++I)
        if (2 * p <= I && I - (2 * p + 1) <= MAXD) u[I] = mma_bf16(tf[I][p], cy[p], u[I]);
    // S <- e^{G_C} S + K^T diag(e^{G_C - G}) U'
    f32x4 ut[CNT];
#pragma unroll
    for (int I = 0; I < CNT; ++I) ut[I] = u[I] * w4[I];
    bf16x8 cth[2], ctl[2];
    pack8_hilo(ut[0], ut[1], cth[0], ctl[0]);
    pack8_hilo(ut[2], ut[3], cth[1], ctl[1]);
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int A = 0; A < NA; ++A) S[A] = mma_bf16(kt[A][p], k ? ctl[p] : cth[p], S[A]);
    // U' (hi/lo) for the output waves, off the state's dependency chain
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      bf16x8 h, lw;
      pack8_hilo(u[2 * p], u[2 * p + 1], h, lw);
      B.uh[v][p][l] = h;
      B.ul[v][p][l] = lw;
    }
    read_inputs(Rn, v);
  }
};

// ---- output waves: P and O = scale (e^G Q S + P U') for NI row tiles I0 (, I1) --------
// q holds the chunk's Q rows of those tiles, kr its K rows of tiles 0 .. max(I0, I1)
// (natural d order).
template <int DK, int NI, int I0, int I1, bool OBF16>
__device__ __forceinline__ void emit_rows(const ChunkArgs& a, int64_t row0, int col0,
                                          const bf16x8 (&kr)[CNT][DK / 32], const ChunkGates& GT,
                                          const ChunkBuf<DK>& B, const bf16x8 (&q)[NI][DK / 32]) {
  constexpr int NP = DK / 32;
  constexpr int IS[2] = {I0, NI > 1 ? I1 : I0};
  constexpr int IMAX = IS[0] > IS[NI - 1] ? IS[0] : IS[NI - 1];
  const int l = lane_id(), g = l >> 4, c = l & 15;
  // Q S for both column halves (T-form: lane (g,c) reg r = row 16I + c, column 4g + r)
  f32x4 acc[NI][2];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) acc[i][h] = zero4();
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bf16x8 sf = *reinterpret_cast<const bf16x8*>(&B.st[h][c][32 * p + 8 * g]);
#pragma unroll
      for (int i = 0; i < NI; ++i) acc[i][h] = mma_bf16(sf, q[i][p], acc[i][h]);
    }
  // raw P tiles (I, J), J <= I, one K tile-row at a time
  f32x4 pt[NI][CNT];
#pragma unroll
  for (int J = 0; J < CNT; ++J) {
    if (J > IMAX) continue;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (J > IS[i]) continue;
      f32x4 t = zero4();
#pragma unroll
      for (int p = 0; p < NP; ++p) t = mma_bf16(kr[J][p], q[i][p], t);
      pt[i][J] = t;
    }
  }
  // decay and causal mask of P; e^G on Q S.  exp(-G) finite over the chunk: the decay
  // factor splits into a row and a column factor (uniform branch)
  const bool split = __builtin_amdgcn_readfirstlane(GT.split) != 0;
  const int lo_ = 4 * g - c;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int I = IS[i];
    const float rowf = GT.eg[16 * I + c];
#pragma unroll
    for (int h = 0; h < 2; ++h) acc[i][h] = acc[i][h] * rowf;
#pragma unroll
    for (int J = 0; J < CNT; ++J) {
      if (J > I) {
        pt[i][J] = zero4();
        continue;
      }
      f32x4 fac;
      if (split) {
        fac = *reinterpret_cast<const f32x4*>(&GT.eng[16 * J + 4 * g]) * rowf;
      } else {
        const float Gi = GT.G[16 * I + c];
        const f32x4 Gcol = *reinterpret_cast<const f32x4*>(&GT.G[16 * J + 4 * g]);
#pragma unroll
        for (int r = 0; r < 4; ++r) fac[r] = __expf(Gi - Gcol[r]);
      }
      if (J < I) {
        pt[i][J] = pt[i][J] * fac;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) pt[i][J][r] = (r + lo_ <= 0) ? pt[i][J][r] * fac[r] : 0.f;  // i >= j
      }
    }
  }
  // + P U' (T-form), U' and P as hi/lo pairs
  bf16x8 uh[2][2], ul[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
      uh[h][q2] = B.uh[h][q2][l];
      ul[h][q2] = B.ul[h][q2][l];
    }
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
      if (2 * q2 > IS[i]) continue;
      bf16x8 ph, pl;
      pack8_hilo(pt[i][2 * q2], pt[i][2 * q2 + 1], ph, pl);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        acc[i][h] = mma_bf16(uh[h][q2], ph, acc[i][h]);
        acc[i][h] = mma_bf16(ul[h][q2], ph, acc[i][h]);
        acc[i][h] = mma_bf16(uh[h][q2], pl, acc[i][h]);
      }
    }
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4 o = acc[i][h] * a.scale;
      const int64_t off = (row0 + 16 * IS[i] + c) * a.dv + col0 + 16 * h + 4 * g;
      if constexpr (OBF16)
        *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(a.O) + off) = pack4(o);
      else
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.O) + off) = o;
    }
}

// Slot `idx` of an LDS ring.  The byte offset goes through readfirstlane so that the
// compiler treats it as one opaque uniform value: each access is then a per-lane base
// plus a constant folded into the instruction's offset field, instead of a separately
// strength-reduced address per access.
template <class T>
__device__ __forceinline__ T& ring(T* base, int idx) {
  const uint32_t off = __builtin_amdgcn_readfirstlane((uint32_t)idx * (uint32_t)sizeof(T));
  return *reinterpret_cast<T*>(reinterpret_cast<char*>(base) + off);
}

// Hand-over of LDS buffers between the waves of the workgroup: wait for this wave's
// LDS accesses, then the barrier.  Global memory is never exchanged between waves
// here, so outstanding global loads (prefetches into registers) stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Schedule: iterations it = -1 .. nchunks with one barrier at the end of each, and one
// barrier before the loop.  Rings: raw inputs of chunk j in in[j % 4], gate factors in
// gr[j % 4], the other products of chunk j in buf[j % 2].
//   wave 4      it: stores chunk it+2 into in and its gate factors into gr (loaded at
//               it-1), loads chunk it+3
//   wave 5      it: T of chunk it+1         reads in, gr (or the packs) writes buf.trp
//   waves 0, 1  it: state step of chunk it  reads in, gr, buf.trp
//                                           writes buf.st, buf.uh/ul
//   waves 2, 3, 6, 7 it: P, O of chunk it-1 reads in, gr, buf.{st, uh, ul}
// Every slot is written in one iteration and read only in later ones, and its next
// write comes after its last read: in[j] and gr[j] are written at j-2, read at
// j-1 .. j+1 and rewritten at j+2; buf[j].trp is read
// at j and rewritten at j+1, the other buf[j] fields are read at j+1 and rewritten at
// j+2.  In iteration it, the output waves read buf[(it-1) % 2] = buf[(it+1) % 2] while
// the T wave writes that buffer's trp, a field they do not touch.  Global loads are issued
// one iteration before their data is needed (register ping-pong, no loop-carried
// copies, no conditional loads), so their latency overlaps a whole iteration.
constexpr int W_STATE0 = 0, W_STATE1 = 1, W_T = 5, W_STAGE = 4;
// output wave of row tile 0..3
constexpr int W_OUT0 = 2, W_OUT1 = 3, W_OUT2 = 6, W_OUT3 = 7;

template <int DK, int MODE, int CMP, int MAXD, bool OBF16>
__global__ __launch_bounds__(NWAVES * WAVE, 1) void chunk_fwd_kernel(ChunkArgs a) {
  __shared__ ChunkIn<DK> in[4];
  __shared__ ChunkGates gr[4];
  __shared__ ChunkBuf<DK> buf[2];
  __shared__ float xr[CH][XR_LD];  // Gram band rows (band mode, T wave only)
  // wave index as a uniform (scalar) value: role branches and loop counters stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  const int l = lane_id(), g = l >> 4, c = l & 15;
  // workgroup -> (head, slice): the slices of one head are consecutive workgroup
  // indices inside one XCD (workgroups are dealt round-robin over the 8 XCDs), so they
  // share that XCD's L2 for the rows they all read
  const int n_slices = a.dv / DVS;
  const int total = a.BH * n_slices;
  const int wg = blockIdx.x;
  const int idx = (total % 8 == 0) ? (wg % 8) * (total / 8) + wg / 8 : wg;
  const int bh = idx / n_slices, slice = idx % n_slices;
  const int nchunks = (int)(a.T / CH);
  const int64_t head_row0 = (int64_t)bh * a.T;
  const int last = nchunks - 1;  // >= 0: the launcher is never called with T = 0

  if (wave == W_STAGE) {
    __builtin_amdgcn_s_setprio(1);
    // K: the chunk's rows are contiguous, 16 bytes per lane and instruction; V: this
    // workgroup's 32 columns (64 bytes) of each row, 4 lanes per row
    constexpr int SEG = DK / 8;
    constexpr int NK = CH * SEG / WAVE;
    constexpr int NV = CH * (DVS / 8) / WAVE;
    struct Regs {
      bf16x8 k[NK];
      bf16x8 v[NV];
      float g, b;
    };
    const __bf16* vlane = a.V + (head_row0 + (l >> 2)) * a.dv + slice * DVS + 8 * (l & 3);
    auto load = [&](int ch, Regs& r) {
      const __bf16* kc = a.K + (head_row0 + (int64_t)ch * CH) * DK;
#pragma unroll
      for (int i = 0; i < NK; ++i) r.k[i] = *reinterpret_cast<const bf16x8*>(kc + 8 * (i * WAVE + l));
      const __bf16* vc = vlane + (int64_t)ch * CH * a.dv;
#pragma unroll
      for (int i = 0; i < NV; ++i) r.v[i] = *reinterpret_cast<const bf16x8*>(vc + (int64_t)(16 * i) * a.dv);
      r.g = a.g[head_row0 + (int64_t)ch * CH + l];
      r.b = a.beta[head_row0 + (int64_t)ch * CH + l];
    };
    auto store = [&](const Regs& r, ChunkIn<DK>& S) {
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        const int e = i * WAVE + l;
        *reinterpret_cast<bf16x8*>(&S.k[e / SEG][8 * (e % SEG)]) = r.k[i];
      }
#pragma unroll
      for (int i = 0; i < NV; ++i) *reinterpret_cast<bf16x8*>(&S.v[16 * i + (l >> 2)][8 * (l & 3)]) = r.v[i];
      S.g[l] = r.g;
      S.beta[l] = r.b;
    };
    // chunk c sits in r0 for even c and in r1 for odd c.  Every load is issued
    // unconditionally (chunk index clamped into range; loads past the end re-read the
    // last chunk and are never stored) so that the wait before each store covers only
    // the loads of that chunk, not the ones issued after it.
    auto clampc = [&](int ch) { return ch < last ? ch : last; };
    Regs r0, r1;
    load(0, r0);
    load(clampc(1), r1);
    store(r0, in[0]);
    write_gates(r0.g, r0.b, gr[0]);
    lds_barrier();
    for (int it = -1; it <= nchunks; it += 2) {
      // iteration it (odd): chunk it+3 (even) -> r0, chunk it+2 (odd) r1 -> LDS
      load(clampc(it + 3), r0);
      if (it + 2 < nchunks) {
        store(r1, ring(in, (it + 2) & 3));
        write_gates(r1.g, r1.b, ring(gr, (it + 2) & 3));
      }
      lds_barrier();
      if (it + 1 > nchunks) break;
      // iteration it+1 (even): chunk it+4 (odd) -> r1, chunk it+3 (even) r0 -> LDS
      load(clampc(it + 4), r1);
      if (it + 3 < nchunks) {
        store(r0, ring(in, (it + 3) & 3));
        write_gates(r0.g, r0.b, ring(gr, (it + 3) & 3));
      }
      lds_barrier();
    }
    return;
  }
  if (wave == W_T) {
    // issue priority on the shared SIMDs: the T wave level with state wave 1, the
    // stager one level below state wave 0 (it mostly waits on its loads)
    __builtin_amdgcn_s_setprio(2);
    if constexpr (MODE == MODE_BAND) {
      const bf16x8 z = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int I = 0; I < CNT; ++I)
#pragma unroll
          for (int p = 0; p < 2; ++p) buf[b].trp[I][p][l] = z;
      lds_barrier();
      for (int it = -1; it <= nchunks; ++it) {
        const int ch = it + 1;
        if (ch < nchunks) produce_T_band<DK>(a, ring(in, ch & 3), ring(buf, ch & 1).trp, ring(gr, ch & 3), xr);
        lds_barrier();
      }
    } else if constexpr (MODE == MODE_LOADBAND) {
      // the band pre-pass's rows of chunk ch sit at band[(bh * nchunks + ch) * 64]; loaded one
      // iteration earlier (register ping-pong, chunk index clamped) and put into the band
      // slots of the row packs, whose other slots were cleared once
      const bf16x8 z = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int I = 0; I < CNT; ++I)
#pragma unroll
          for (int p = 0; p < 2; ++p) buf[b].trp[I][p][l] = z;
      const bf16x4* hb = a.band + (size_t)bh * nchunks * CH + l;
      auto clampc = [&](int ch) { return ch < last ? ch : last; };
      auto put = [&](const bf16x4& r, bf16x8 (&trp)[CNT][2][WAVE]) {
        const float t[4] = {0.f, (float)r[1], (float)r[2], (float)r[3]};
        scatter_band(t, trp);
      };
      bf16x4 r0 = hb[0], r1;
      lds_barrier();
      for (int it = -1; it <= nchunks; it += 2) {
        r1 = hb[(size_t)clampc(it + 2) * CH];
        if (it + 1 < nchunks) put(r0, ring(buf, (it + 1) & 1).trp);
        lds_barrier();
        if (it + 1 > nchunks) break;
        r0 = hb[(size_t)clampc(it + 3) * CH];
        if (it + 2 < nchunks) put(r1, ring(buf, (it + 2) & 1).trp);
        lds_barrier();
      }
    } else {
      // the pre-pass's packs of chunk ch sit at packs[(bh * nchunks + ch) * 6 * 64]; chunk
      // it + 1 goes to LDS in iteration it, loaded one iteration earlier (register
      // ping-pong, every load unconditional with the chunk index clamped, as the stager)
      const bf16x8* hp = a.packs + (size_t)bh * nchunks * T_PACKS * WAVE + l;
      auto clampc = [&](int ch) { return ch < last ? ch : last; };
      auto load = [&](int ch, bf16x8 (&r)[T_PACKS]) {
#pragma unroll
        for (int k = 0; k < T_PACKS; ++k) r[k] = hp[((size_t)ch * T_PACKS + k) * WAVE];
      };
      auto store = [&](const bf16x8 (&r)[T_PACKS], bf16x8 (&trp)[CNT][2][WAVE]) {
#pragma unroll
        for (int I = 0; I < CNT; ++I)
#pragma unroll
          for (int p = 0; p < 2; ++p)
            if (2 * p <= I) trp[I][p][l] = r[t_pack_index(I, p)];
      };
      bf16x8 r0[T_PACKS], r1[T_PACKS];
      load(0, r0);
      lds_barrier();
      for (int it = -1; it <= nchunks; it += 2) {
        // iteration it: chunk it + 1 (even) from r0, chunk it + 2 (odd) -> r1
        load(clampc(it + 2), r1);
        if (it + 1 < nchunks) store(r0, ring(buf, (it + 1) & 1).trp);
        lds_barrier();
        if (it + 1 > nchunks) break;
        // iteration it + 1: chunk it + 2 (odd) from r1, chunk it + 3 (even) -> r0
        load(clampc(it + 3), r0);
        if (it + 2 < nchunks) store(r1, ring(buf, (it + 2) & 1).trp);
        lds_barrier();
      }
    }
    return;
  }
  if (wave == W_OUT0 || wave == W_OUT1 || wave == W_OUT2 || wave == W_OUT3) {
    // chunk ch = it - 1 in iteration it; that iteration also loads chunk ch + 1's Q rows
    auto out_loop = [&](auto i0) {
      constexpr int I0 = decltype(i0)::value;
      auto clampc = [&](int ch) { return ch < 0 ? 0 : (ch < last ? ch : last); };
      bf16x8 q0[1][DK / 32], q1[1][DK / 32];
      // K rows of tiles 0..I0 of the chunk worked on next: read right after the
      // current chunk's work (that chunk is already in LDS), off the next work's chain
      bf16x8 kr[CNT][DK / 32];
      auto read_k = [&](int ch) {
        const ChunkIn<DK>& R = ring(in, ch & 3);
#pragma unroll
        for (int J = 0; J <= I0; ++J)
#pragma unroll
          for (int p = 0; p < DK / 32; ++p) kr[J][p] = rowfrag_nat<DK>(R, 16 * J + c, p);
      };
      auto work = [&](int ch, const bf16x8 (&q)[1][DK / 32]) {
        emit_rows<DK, 1, I0, I0, OBF16>(a, head_row0 + (int64_t)ch * CH, slice * DVS, kr, ring(gr, ch & 3),
                                        ring(buf, ch & 1), q);
      };
      lds_barrier();
      read_k(0);
      for (int it = -1; it <= nchunks; it += 2) {
        int ch = it - 1;  // even
        load_q_nat<DK, 1, I0, I0>(a, head_row0 + (int64_t)clampc(ch + 1) * CH, q1);
        if (ch >= 0 && ch < nchunks) {
          work(ch, q0);
          read_k(ch + 1);
        }
        lds_barrier();
        if (it + 1 > nchunks) break;
        ch += 1;  // odd
        load_q_nat<DK, 1, I0, I0>(a, head_row0 + (int64_t)clampc(ch + 1) * CH, q0);
        if (ch >= 0 && ch < nchunks) {
          work(ch, q1);
          read_k(ch + 1);
        }
        lds_barrier();
      }
    };
    if (wave == W_OUT0) out_loop(std::integral_constant<int, 0>{});
    else if (wave == W_OUT1) out_loop(std::integral_constant<int, 1>{});
    else if (wave == W_OUT2) out_loop(std::integral_constant<int, 2>{});
    else out_loop(std::integral_constant<int, 3>{});
    return;
  }
  if (wave != W_STATE0 && wave != W_STATE1) {
    lds_barrier();
    for (int it = -1; it <= nchunks; ++it) lds_barrier();
    return;
  }
  // state waves
  __builtin_amdgcn_s_setprio(2);
  const int v = wave;
  const int col0 = slice * DVS + 16 * v;
  StateWave<DK, MAXD> sw;
#pragma unroll
  for (int A = 0; A < DK / 16; ++A)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      sw.S[A][r] = a.S0 ? a.S0[((size_t)bh * DK + sdim(A, g, r)) * a.dv + col0 + c] : 0.f;
  lds_barrier();
  sw.read_inputs(in[0], v);  // chunk 0 is in LDS after the first barrier
  for (int it = -1; it <= nchunks; ++it) {
    // the next chunk's slot: staged one iteration earlier, rewritten three later (past
    // the end it holds stale rows, read but never used)
    if (it >= 0 && it < nchunks)
      sw.step(ring(in, it & 3), ring(in, (it + 1) & 3), ring(gr, it & 3), ring(buf, it & 1), v);
    lds_barrier();
  }
#pragma unroll
  for (int A = 0; A < DK / 16; ++A)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      a.S_out[((size_t)bh * DK + sdim(A, g, r)) * a.dv + col0 + c] = sw.S[A][r];
}

bool chunk_fwd_band_path(int mode, int N, int mask, int cmp) {
  return mode == MODE_NEUMANN && mask && N <= 3 && cmp == CMP_BF16;
}

bool chunk_fwd_fp8_band(int mode, int N, int mask, int cmp) {
  return mode == MODE_NEUMANN && mask && N <= 3 && cmp == CMP_FP8;
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
  a.packs = p.band_rows ? nullptr : reinterpret_cast<const bf16x8*>(p.packs);
  a.band = p.band_rows ? reinterpret_cast<const bf16x4*>(p.packs) : nullptr;
  a.T = p.T;
  a.BH = p.B * p.H;
  a.dv = p.d_v;
  a.N = p.N;
  a.mask = p.mask;
  a.scale = p.scale;
  const dim3 grid((unsigned)(a.BH * (p.d_v / DVS)));
  const dim3 block(NWAVES * WAVE);
  // the pre-pass's packs, when given, are used (every variant but the band path, and the
  // band-masked sum when its Horner products were asked for)
  const bool band = p.packs == nullptr;
  if (band && !chunk_fwd_band_path(p.mode, p.N, p.mask, p.cmp)) return -1;
  // with the band mask and N <= 16 the packs below the first sub-tile-diagonal are zero
  const bool narrow = p.mode == MODE_NEUMANN && p.mask && p.N <= 16;
  auto go = [&](auto dk, auto mode, auto maxd) {
    if (p.o_bf16)
      hipLaunchKernelGGL((chunk_fwd_kernel<dk.value, mode.value, CMP_BF16, maxd.value, true>), grid, block,
                         0, s, a);
    else
      hipLaunchKernelGGL((chunk_fwd_kernel<dk.value, mode.value, CMP_BF16, maxd.value, false>), grid, block,
                         0, s, a);
    return 0;
  };
  using I1 = std::integral_constant<int, 1>;
  using I3 = std::integral_constant<int, 3>;
  using MB = std::integral_constant<int, MODE_BAND>;
  using ML = std::integral_constant<int, MODE_LOAD>;
  using MLB = std::integral_constant<int, MODE_LOADBAND>;
  auto with_dk = [&](auto dk) -> int {
    if (band) return go(dk, MB{}, I1{});
    if (p.band_rows) return go(dk, MLB{}, I1{});
    return narrow ? go(dk, ML{}, I1{}) : go(dk, ML{}, I3{});
  };
  switch (p.d_k) {
    case 64: return with_dk(std::integral_constant<int, 64>{});
    case 128: return with_dk(std::integral_constant<int, 128>{});
    default: return -1;
  }
}

}  // namespace gdn
