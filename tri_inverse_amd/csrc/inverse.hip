// inverse.hip -- batched per-block kernels: A build, the multiplication-only inverses of
// I - A (truncated / masked Neumann sum in fp32, bf16, fp8, int8 or int16 operands, exact
// doubling, residual correction) and forward substitution.  A wave (64 lanes) works on
// one C x C block at a time with the matrices in registers (the exact 64 x 64 doubling
// also passes each square through a per-wave LDS slice); the unmasked fp8 chain over
// many blocks walks several blocks per wave.
//
// [GEO] "When Good Enough Is Optimal: Multiplication-Only Matrix Inversion
// Approximation for Quantized Gated DeltaNet": problem statement (T = (I - A)^-1 per
// chunk, A strictly lower), Methodologie SS1 (truncated Neumann, Lemma 3.1), SS2
// (structural diagonal mask), "Adaptation a la Quantification" (low-bit operands).
#include "gdn_kernels.hpp"
#include "tri_block.hpp"

namespace gdn {

// input source of A for one block
enum : int { SRC_A = 0, SRC_K_BF16 = 1, SRC_K_F32 = 2 };

// Raw inputs of one block (what the prefetch holds): K fragments + lane gate values,
// or A's lower tiles.
template <int NT, int SRC, int DK>
struct BlockIn;
template <int NT, int DK>
struct BlockIn<NT, SRC_K_BF16, DK> {
  KBlock<NT, DK> k;
  // GF: load the gate inputs first and form the gate factors (they need only those two
  // loads) while the key rows arrive, before any Gram product waits for the keys.
  // Measured faster where the block's work after A is long (exact doubling, quantised
  // chains: 8-10 %; residual correction: 2-3 %) and slower for the light bf16 / fp32
  // truncated sums (3-4 %), which keep the compiler's own order.
  // STREAM: streaming (non-temporal) key loads.  Each load instruction covers half of
  // 16 rows' 128-byte lines and the next one the other half; over 8192 and more blocks
  // (the chunk forward's pre-pass) streaming loads fetched lines twice (1.12-1.15x the
  // key bytes) and plain loads are faster (bf16 products pre-pass 40 -> 34 us at 8192
  // blocks), while the 2048-block inverses read exactly their bytes either way.
  template <bool GF = false, bool STREAM = true, bool ORDERED = false>
  __device__ __forceinline__ void load(const BlocksArgs& a, int64_t blk) {
    constexpr int C = 16 * NT;
    load_kblock<NT, DK, STREAM, GF, ORDERED>(reinterpret_cast<const __bf16*>(a.K) + (size_t)blk * C * DK,
                                  a.beta + (size_t)blk * C, a.g + (size_t)blk * C, k);
  }
  template <int MAXD, bool BANDED, bool GF = false>
  __device__ __forceinline__ void to_A(const BlocksArgs& a, int band, Mat<NT>& AD, Mat<NT>& AT) const {
    Gates<NT> gt;
    gates_from_lanes<NT>(k.gl, k.bl, a.g_cumulative != 0, gt);
    if constexpr (GF) __builtin_amdgcn_sched_barrier(0);
    Mat<NT> S;
    gram_from_frags<NT, DK, MAXD>(k, S);
    gram_to_A<NT, MAXD, BANDED>(S, gt, band, AD, AT);
  }
};
template <int NT, int DK>
struct BlockIn<NT, SRC_A, DK> {
  ABlock<NT> ab;
  template <bool GF = false, bool STREAM = true, bool ORDERED = false>
  __device__ __forceinline__ void load(const BlocksArgs& a, int64_t blk) {
    constexpr int C = 16 * NT;
    load_ablock<NT>(a.A + (size_t)blk * C * C, ab);
  }
  template <int MAXD, bool BANDED, bool GF = false>
  __device__ __forceinline__ void to_A(const BlocksArgs&, int band, Mat<NT>& AD, Mat<NT>& AT) const {
    ablock_to_A<NT, MAXD, BANDED>(ab, band, AD, AT);
  }
};

// A alone (gdn_build_A): one block per wave, fp32 or bf16 keys.
template <int NT, int SRC, int DK>
__global__ __launch_bounds__(256) void build_A_kernel(BlocksArgs a, float* __restrict__ A_out) {
  constexpr int C = 16 * NT;
  const int64_t blk = (int64_t)blockIdx.x * (blockDim.x / WAVE) + (threadIdx.x / WAVE);
  if (blk >= a.n_blocks) return;
  Gates<NT> gt;
  load_gates<NT>(a.beta + (size_t)blk * C, a.g + (size_t)blk * C, a.g_cumulative != 0, gt);
  Mat<NT> S, AD, AT;  // every tile is formed: A is an output here
  if constexpr (SRC == SRC_K_BF16)
    gram_bf16<NT, DK>(reinterpret_cast<const __bf16*>(a.K) + (size_t)blk * C * DK, S);
  else
    gram_f32<NT, DK>(reinterpret_cast<const float*>(a.K) + (size_t)blk * C * DK, S);
  gram_to_A<NT>(S, gt, -1, AD, AT);
  if constexpr (NT >= 2)
    store_T_rows_f32<NT, NT - 1>(A_out + (size_t)blk * C * C, AT);
  else
    store_T_f32<NT>(A_out + (size_t)blk * C * C, AT);
}

// long work after A: the gate factors are formed first, while the keys arrive (BlockIn)
template <int CMP, int MODE>
constexpr bool gates_first() {
  return MODE == MODE_EXACT || MODE == MODE_RESIDUAL ||
         (MODE == MODE_NEUMANN && (CMP == CMP_FP8 || CMP == CMP_INT8 || CMP == CMP_INT16));
}

// The inverse of one block by the current wave.  MAXD is the largest tile distance
// I - J kept (NT - 1 in general, 1 for the band-masked sum with N <= 16).
// PK: write T - I as the chunk forward's row packs (store_T_packs) instead of T.
template <int NT, int SRC, int DK, int CMP, int MODE, int MAXD, bool PK, int WPG>
__device__ __forceinline__ void inverse_block(const BlocksArgs& a, int64_t blk, const BlockIn<NT, SRC, DK>& in,
                                              int N, int mask, void* T_out, int t_bf16, Fp8Counts& cnt,
                                              bool count, int S, int wave) {
  constexpr int C = 16 * NT;
  // fp8 and int8 mask A and every intermediate (the band sets the quantisation
  // scales); bf16 / fp32 mask only the final sum (identical result, see neumann_T)
  const int band = (MODE == MODE_NEUMANN && mask) ? N : -1;
  constexpr bool BANDED = (MODE == MODE_NEUMANN && (CMP == CMP_FP8 || CMP == CMP_INT8 || CMP == CMP_INT16));
  Mat<NT> AD, AT, TT;
  in.template to_A<MAXD, BANDED, gates_first<CMP, MODE>()>(a, BANDED ? band : -1, AD, AT);
  if constexpr (MODE == MODE_EXACT && NT == 4 && CMP == CMP_BF16) {
    __shared__ __bf16 xt[WPG][64][XT_LD];  // per wave: X^T for the transpose read
    doubling_T_lds<SRC == SRC_K_BF16>(AD, AT, TT, xt[wave]);
  } else if constexpr (MODE == MODE_EXACT)
    doubling_T<NT, CMP>(AD, AT, TT);
  else if constexpr (MODE == MODE_RESIDUAL)
    residual_T<NT>(AD, AT, N, mask != 0, S, TT);
  else if constexpr (CMP == CMP_INT8)
    neumann_T_i8<NT, MAXD>(AD, AT, N, mask != 0, TT);
  else if constexpr (CMP == CMP_INT16)
    neumann_T_i16<NT, MAXD>(AD, AT, N, mask != 0, TT);
  else
    neumann_T<NT, CMP, MAXD>(AD, AT, N, mask != 0, TT, cnt, count);
  if constexpr (PK) {
    static_assert(NT == 4, "row packs of 64 x 64 blocks");
    store_T_packs(reinterpret_cast<bf16x8*>(T_out) + (size_t)blk * T_PACKS * WAVE, TT);
  } else if (t_bf16) {
    if constexpr (NT >= 2)
      store_T_rows_bf16<NT, MAXD>(reinterpret_cast<__bf16*>(T_out) + (size_t)blk * C * C, TT);
    else
      store_T_bf16<NT, MAXD>(reinterpret_cast<__bf16*>(T_out) + (size_t)blk * C * C, TT);
  } else {
    if constexpr (NT >= 2)
      store_T_rows_f32<NT, MAXD>(reinterpret_cast<float*>(T_out) + (size_t)blk * C * C, TT);
    else
      store_T_f32<NT, MAXD>(reinterpret_cast<float*>(T_out) + (size_t)blk * C * C, TT);
  }
}

// The band-masked sum with N = 2 or 3 of a 64 x 64 block from bf16 keys, T in bf16, in
// two halves of rows.  With the mask (N <= 16) A, every Horner iterate and T reach one
// tile-diagonal below the main one, so their tile rows 0-1 need only the key rows 0-31:
// that half is formed and its T rows stored while the key rows 32-63 still arrive (the
// gate inputs and the keys load in that order, and loads complete in order).  Rows 2-3
// follow and read the first half's tile row 1 of each iterate.  Every tile is formed by
// the same MFMAs on the same operands as in neumann_T, so T is bit-identical.
template <int DK>
__device__ __forceinline__ void neumann_rows_in_halves(const BlocksArgs& a, int64_t blk,
                                                       const BlockIn<4, SRC_K_BF16, DK>& in, int N,
                                                       void* T_out) {
  constexpr int C = 64, MAXD = 1;
  Gates<4> gt;
  gates_from_lanes<4>(in.k.gl, in.k.bl, a.g_cumulative != 0, gt);
  Mat<4> S, AD, AT, H1, H2, TT;
  const f32x4 eye = eye_tile();
  auto half = [&](auto lo) {
    constexpr int ILO = decltype(lo)::value, IHI = ILO + 1;
    gram_from_frags<4, DK, MAXD, ILO, IHI>(in.k, S);
    gram_to_A<4, MAXD, false, ILO, IHI>(S, gt, -1, AD, AT);
#pragma unroll
    for (int I = ILO; I <= IHI; ++I)
#pragma unroll
      for (int J = 0; J <= I; ++J) H1.t[I][J] = (I == J) ? AD.t[I][J] + eye : AD.t[I][J];  // H_1 = I + A
    if (N == 3) {
      lmul_bf16<4, false, MAXD, true, ILO, IHI>(AT, H1, H2);  // H_2 = I + A H_1
      lmul_bf16<4, true, MAXD, true, ILO, IHI>(AT, H2, TT);   // T = I + A H_2
    } else {
      lmul_bf16<4, true, MAXD, true, ILO, IHI>(AT, H1, TT);   // T = I + A H_1
    }
    mask_T<4, ILO, IHI>(TT, N);
    store_T_rows_bf16<4, MAXD, ILO, IHI>(reinterpret_cast<__bf16*>(T_out) + (size_t)blk * C * C, TT);
  };
  half(std::integral_constant<int, 0>{});
  __builtin_amdgcn_sched_barrier(0);  // keep the second half's work behind the first's stores
  half(std::integral_constant<int, 2>{});
}

// The batched inverse.  WPG: waves per workgroup (the launch's block size, 2 or 4).
// PF = false: one wave per block.  PF = true: fewer waves than
// blocks, each walking the blocks with the grid's stride; while it forms and stores T
// of one block, the next block's raw inputs are already on their way into registers
// (the index is clamped, so the load is unconditional and the wait before the next
// block covers only those loads).  That overlap pays where the per-block work is long
// next to its loads (the unmasked fp8 chain over many blocks); with fewer blocks or
// lighter work, independent waves hide the loads better, so PF stays off there.
template <int NT, int SRC, int DK, int CMP, int MODE, int MAXD, bool PK = false, bool PF = false, int WPG = 4>
__global__ __launch_bounds__(256) void inverse_kernel(BlocksArgs a, int N, int mask, void* T_out,
                                                      int t_bf16, unsigned long long* stats, int S) {
  Fp8Counts cnt{0, 0, 0, 0};
  const bool count = (CMP == CMP_FP8) && stats != nullptr;
  if constexpr (!PF) {
    const int64_t blk = (int64_t)blockIdx.x * WPG + (threadIdx.x / WAVE);
    if (blk >= a.n_blocks) return;
    BlockIn<NT, SRC, DK> in;
    if constexpr (NT == 4 && SRC == SRC_K_BF16 && CMP == CMP_BF16 && MODE == MODE_NEUMANN && MAXD == 1 && !PK) {
      // bf16 T only: with fp32 T (twice the store bytes) the first half's stores, mixed
      // into the second half's key reads, made the launch slower (13.2 -> 14.2 us),
      // while bf16 T gained (12.7 -> 12.2 us)
      if ((N == 2 || N == 3) && t_bf16) {
        in.template load<true, true, true>(a, blk);
        neumann_rows_in_halves<DK>(a, blk, in, N, T_out);
        return;
      }
    }
    // loads issued in program order (gates as gates_first says, then key row tiles 0..3),
    // so the Gram products of the first row tiles start while the last ones arrive; the
    // compiler's own interleaving of the loads made most of them wait for nearly all
    // keys.  Measured 3-9 % faster on the 2048-block inverses and 3-4 % on the chunk
    // forward's pre-passes.
    in.template load<gates_first<CMP, MODE>(), !PK, true>(a, blk);
    inverse_block<NT, SRC, DK, CMP, MODE, MAXD, PK, WPG>(a, blk, in, N, mask, T_out, t_bf16, cnt, count, S,
                                                         threadIdx.x / WAVE);
  } else {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
    const int64_t first = (int64_t)blockIdx.x * WPG + wave;
    if (first >= a.n_blocks) return;
    const int64_t stride = (int64_t)gridDim.x * WPG;
    BlockIn<NT, SRC, DK> in;
    in.template load<gates_first<CMP, MODE>(), !PK>(a, first);
    for (int64_t blk = first; blk < a.n_blocks; blk += stride) {
      BlockIn<NT, SRC, DK> nxt;
      nxt.template load<gates_first<CMP, MODE>(), !PK>(a, blk + stride < a.n_blocks ? blk + stride : a.n_blocks - 1);
      inverse_block<NT, SRC, DK, CMP, MODE, MAXD, PK, WPG>(a, blk, in, N, mask, T_out, t_bf16, cnt, count, S, wave);
      in = nxt;
    }
  }
  if constexpr (CMP == CMP_FP8) {
    if (count) flush_counts(cnt, stats);
  }
}

// Forward substitution, the sequential baseline of [GEO]'s problem statement:
// T = I + A T row by row, T[i][.] = e_i + sum_{m<i} A[i][m] T[m][.], in fp32.  One wave
// per block; lane j holds column j of T in registers (Tc[i] = T[i][j]); each A[i][m] is
// broadcast with one readlane straight from the T-form tiles of A (lane (g,c) reg r of
// tile (I,J) holds A[16I + c][16J + 4g + r]).  C (C - 1) / 2 dependent-row FMAs.
template <int NT, int SRC, int DK>
__global__ __launch_bounds__(256) void fs_kernel(BlocksArgs a, void* T_out, int t_bf16) {
  constexpr int C = 16 * NT;
  const int64_t blk = (int64_t)blockIdx.x * (blockDim.x / WAVE) + (threadIdx.x / WAVE);
  if (blk >= a.n_blocks) return;
  BlockIn<NT, SRC, DK> in;
  in.load(a, blk);
  Mat<NT> AD, AT;
  in.template to_A<NT - 1, false>(a, -1, AD, AT);
  const int j = lane_id();
  float Tc[C];
#pragma unroll
  for (int i = 0; i < C; ++i) {
    float acc = (j == i) ? 1.f : 0.f;
#pragma unroll
    for (int m = 0; m < i; ++m) {
      // copy the element out first: a bit cast applied to a vector-element expression
      // directly reads the vector's first element
      const float e = AT.t[i / 16][m / 16][m % 4];
      const float aim = __builtin_bit_cast(
          float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, e), 16 * ((m % 16) / 4) + (i % 16)));
      acc = fmaf(aim, Tc[m], acc);
    }
    Tc[i] = acc;
  }
  if (j < C) {
#pragma unroll
    for (int i = 0; i < C; ++i) {
      const size_t o = (size_t)blk * C * C + (size_t)i * C + j;
      if (t_bf16)
        reinterpret_cast<__bf16*>(T_out)[o] = (__bf16)Tc[i];
      else
        reinterpret_cast<float*>(T_out)[o] = Tc[i];
    }
  }
}

__global__ void zero_u64_kernel(unsigned long long* p, int n) {
  int i = threadIdx.x;
  if (i < n) p[i] = 0ull;
}

// ---- host-side dispatch ------------------------------------------------------

static constexpr int WAVES_PER_WG = 4;

static dim3 grid_for(int64_t n_blocks, int wpg = WAVES_PER_WG) {
  return dim3((unsigned)((n_blocks + wpg - 1) / wpg));
}

// One launch of the batched inverse (T out, one wave per block).  The truncated sums on
// blocks of 32 x 32 and 64 x 64 go two waves to a workgroup: twice as many workgroups
// spread over the CUs more evenly.  Same-box A/Bs over 2048 blocks of 64 x 64, two boxes:
// unmasked N = 3 12.41-12.61 -> 11.98-12.20 us, int8 12.9 -> 12.4 us, int16 17.45 ->
// 16.9 us, masked N = 3 with T fp32 12.26-12.31 -> 11.86-12.32 us (a gain on one box,
// level on the other).  The exact product (T bf16 11.24 -> 11.64 us on one box), the
// residual correction (level) and the masked sum with bf16 T in two halves of rows
// (11.28-11.33 against 11.43 us) keep four waves.
template <int NT, int SRC, int DK, int CMP, int MODE, int MAXD>
static void launch_inverse(const BlocksArgs& a, int N, int mask, void* T_out, int t_bf16,
                           unsigned long long* stats, int S, hipStream_t s) {
  const bool halves = NT == 4 && SRC == SRC_K_BF16 && CMP == CMP_BF16 && MODE == MODE_NEUMANN && MAXD == 1 &&
                      t_bf16 && (N == 2 || N == 3);
  if constexpr (NT >= 2 && MODE == MODE_NEUMANN) {
    if (!halves) {
      hipLaunchKernelGGL((inverse_kernel<NT, SRC, DK, CMP, MODE, MAXD, false, false, 2>), grid_for(a.n_blocks, 2),
                         dim3(WAVE * 2), 0, s, a, N, mask, T_out, t_bf16, stats, S);
      return;
    }
  }
  hipLaunchKernelGGL((inverse_kernel<NT, SRC, DK, CMP, MODE, MAXD>), grid_for(a.n_blocks),
                     dim3(WAVE * WAVES_PER_WG), 0, s, a, N, mask, T_out, t_bf16, stats, S);
}

// Waves of the persistent fp8 pre-pass: two per SIMD of the 256 CUs.  It is used for the
// unmasked chain (all ten lower tiles per power) from four blocks per wave on: measured
// on one box at 32768 chunks, 633 -> 453 us.  The band-masked chain has a third of the
// tiles and is faster with one wave per chunk (228 against 271 us), as are fewer blocks.
static constexpr int64_t PF_WAVES = 2048;

// dispatch helpers over (NT, SRC, DK); `F` is a generic lambda taking the three
// integral constants and launching the right instantiation.
template <typename F>
static int dispatch_nt_src_dk(int C, int src, int dk, F&& f) {
  auto with_dk = [&](auto nt, auto s) -> int {
    if constexpr (decltype(s)::value == SRC_A) {
      return f(nt, s, std::integral_constant<int, 32>{});
    } else {
    switch (dk) {
      case 32: return f(nt, s, std::integral_constant<int, 32>{});
      case 64: return f(nt, s, std::integral_constant<int, 64>{});
      case 128: return f(nt, s, std::integral_constant<int, 128>{});
      case 256: return f(nt, s, std::integral_constant<int, 256>{});
      default: return -1;
    }
    }
  };
  auto with_src = [&](auto nt) -> int {
    switch (src) {
      case SRC_A: return with_dk(nt, std::integral_constant<int, SRC_A>{});
      case SRC_K_BF16: return with_dk(nt, std::integral_constant<int, SRC_K_BF16>{});
      default: return -1;
    }
  };
  switch (C) {
    case 16: return with_src(std::integral_constant<int, 1>{});
    case 32: return with_src(std::integral_constant<int, 2>{});
    case 64: return with_src(std::integral_constant<int, 4>{});
    default: return -1;
  }
}

int launch_build_A(const BlocksArgs& a, int src, float* A_out, hipStream_t s) {
  auto go = [&](auto nt, auto sc, auto dk) -> int {
    hipLaunchKernelGGL((build_A_kernel<nt.value, sc.value, dk.value>), grid_for(a.n_blocks),
                       dim3(WAVE * WAVES_PER_WG), 0, s, a, A_out);
    return 0;
  };
  auto with_dk = [&](auto nt, auto sc) -> int {
    switch (a.d_k) {
      case 32: return go(nt, sc, std::integral_constant<int, 32>{});
      case 64: return go(nt, sc, std::integral_constant<int, 64>{});
      case 128: return go(nt, sc, std::integral_constant<int, 128>{});
      case 256: return go(nt, sc, std::integral_constant<int, 256>{});
      default: return -1;
    }
  };
  auto with_src = [&](auto nt) -> int {
    if (src == SRC_K_BF16) return with_dk(nt, std::integral_constant<int, SRC_K_BF16>{});
    if (src == SRC_K_F32) return with_dk(nt, std::integral_constant<int, SRC_K_F32>{});
    return -1;
  };
  switch (a.C) {
    case 16: return with_src(std::integral_constant<int, 1>{});
    case 32: return with_src(std::integral_constant<int, 2>{});
    case 64: return with_src(std::integral_constant<int, 4>{});
    default: return -1;
  }
}

void launch_zero_stats(unsigned long long* stats, hipStream_t s) {
  hipLaunchKernelGGL(zero_u64_kernel, dim3(1), dim3(64), 0, s, stats, 4);
}

int launch_neumann(const BlocksArgs& a, int src, int N, int mask, int cmp, void* T_out, int t_bf16,
                   unsigned long long* stats, hipStream_t s) {
  return dispatch_nt_src_dk(a.C, src, a.d_k, [&](auto nt, auto sc, auto dk) -> int {
    auto go = [&](auto cm) {
      constexpr int NTv = nt.value;
      // band-masked with N <= 16: tiles two or more tile-diagonals down stay zero
      if (mask && N <= 16 && NTv > 2) {
        launch_inverse<NTv, sc.value, dk.value, cm.value, MODE_NEUMANN, 1>(a, N, mask, T_out, t_bf16, stats, 0, s);
      } else {
        launch_inverse<NTv, sc.value, dk.value, cm.value, MODE_NEUMANN, NTv - 1>(a, N, mask, T_out, t_bf16, stats,
                                                                                 0, s);
      }
      return 0;
    };
    switch (cmp) {
      case CMP_F32: return go(std::integral_constant<int, CMP_F32>{});
      case CMP_BF16: return go(std::integral_constant<int, CMP_BF16>{});
      case CMP_FP8: return go(std::integral_constant<int, CMP_FP8>{});
      case CMP_INT8: return go(std::integral_constant<int, CMP_INT8>{});
      case CMP_INT16: return go(std::integral_constant<int, CMP_INT16>{});
      default: return -1;
    }
  });
}

int launch_exact(const BlocksArgs& a, int src, int cmp, void* T_out, int t_bf16, hipStream_t s) {
  return dispatch_nt_src_dk(a.C, src, a.d_k, [&](auto nt, auto sc, auto dk) -> int {
    auto go = [&](auto cm) {
      launch_inverse<nt.value, sc.value, dk.value, cm.value, MODE_EXACT, nt.value - 1>(
          a, 0, 0, T_out, t_bf16, (unsigned long long*)nullptr, 0, s);
      return 0;
    };
    switch (cmp) {
      case CMP_F32: return go(std::integral_constant<int, CMP_F32>{});
      case CMP_BF16: return go(std::integral_constant<int, CMP_BF16>{});
      default: return -1;
    }
  });
}

// T - I of every 64 x 64 block as row packs (the chunk forward's pre-pass): bf16 keys,
// d_k 64 or 128; mode 0 (Neumann, bf16 or fp8 products) or 1 (exact doubling, bf16)
int launch_T_packs(const BlocksArgs& a, int mode, int N, int mask, int cmp, void* packs,
                   unsigned long long* stats, hipStream_t s) {
  if (a.C != 64) return -1;
  auto go = [&](auto dk, auto cm, auto md, auto maxd) {
    if (cm.value == CMP_FP8 && maxd.value == 3 && a.n_blocks >= 4 * PF_WAVES)
      hipLaunchKernelGGL((inverse_kernel<4, SRC_K_BF16, dk.value, cm.value, md.value, maxd.value, true, true>),
                         grid_for(PF_WAVES), dim3(WAVE * WAVES_PER_WG), 0, s, a, N, mask, packs, 0, stats, 0);
    else
      hipLaunchKernelGGL((inverse_kernel<4, SRC_K_BF16, dk.value, cm.value, md.value, maxd.value, true>),
                         grid_for(a.n_blocks), dim3(WAVE * WAVES_PER_WG), 0, s, a, N, mask, packs, 0,
                         stats, 0);
    return 0;
  };
  using M1 = std::integral_constant<int, 1>;
  using M3 = std::integral_constant<int, 3>;
  auto with_dk = [&](auto dk) -> int {
    if (mode == 1) {
      if (cmp != CMP_BF16) return -1;
      return go(dk, std::integral_constant<int, CMP_BF16>{}, std::integral_constant<int, MODE_EXACT>{}, M3{});
    }
    const bool narrow = mask && N <= 16;
    using MN = std::integral_constant<int, MODE_NEUMANN>;
    if (cmp == CMP_BF16) {
      using CB = std::integral_constant<int, CMP_BF16>;
      return narrow ? go(dk, CB{}, MN{}, M1{}) : go(dk, CB{}, MN{}, M3{});
    }
    if (cmp == CMP_FP8) {
      using CF = std::integral_constant<int, CMP_FP8>;
      return narrow ? go(dk, CF{}, MN{}, M1{}) : go(dk, CF{}, MN{}, M3{});
    }
    return -1;
  };
  switch (a.d_k) {
    case 64: return with_dk(std::integral_constant<int, 64>{});
    case 128: return with_dk(std::integral_constant<int, 128>{});
    default: return -1;
  }
}

// parallel residual correction on the Neumann sum: fp32 products throughout
int launch_residual(const BlocksArgs& a, int src, int N, int mask, int S, void* T_out, int t_bf16,
                    hipStream_t s) {
  return dispatch_nt_src_dk(a.C, src, a.d_k, [&](auto nt, auto sc, auto dk) -> int {
    launch_inverse<nt.value, sc.value, dk.value, CMP_F32, MODE_RESIDUAL, nt.value - 1>(
        a, N, mask, T_out, t_bf16, (unsigned long long*)nullptr, S, s);
    return 0;
  });
}

// forward substitution (fp32), the sequential baseline
int launch_fs(const BlocksArgs& a, int src, void* T_out, int t_bf16, hipStream_t s) {
  return dispatch_nt_src_dk(a.C, src, a.d_k, [&](auto nt, auto sc, auto dk) -> int {
    hipLaunchKernelGGL((fs_kernel<nt.value, sc.value, dk.value>), grid_for(a.n_blocks),
                       dim3(WAVE * WAVES_PER_WG), 0, s, a, T_out, t_bf16);
    return 0;
  });
}

}  // namespace gdn
