// inverse.hip -- batched per-block kernels: A build and the two multiplication-only
// inverses of I - A, one wave (64 lanes) per C x C block, everything in registers.
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
  __device__ __forceinline__ void load(const BlocksArgs& a, int64_t blk) {
    constexpr int C = 16 * NT;
    load_kblock<NT, DK, true>(reinterpret_cast<const __bf16*>(a.K) + (size_t)blk * C * DK,
                        a.beta + (size_t)blk * C, a.g + (size_t)blk * C, k);
  }
  template <int MAXD, bool BANDED>
  __device__ __forceinline__ void to_A(const BlocksArgs& a, int band, Mat<NT>& AD, Mat<NT>& AT) const {
    Gates<NT> gt;
    gates_from_lanes<NT>(k.gl, k.bl, a.g_cumulative != 0, gt);
    Mat<NT> S;
    gram_from_frags<NT, DK, MAXD>(k, S);
    gram_to_A<NT, MAXD, BANDED>(S, gt, band, AD, AT);
  }
};
template <int NT, int DK>
struct BlockIn<NT, SRC_A, DK> {
  ABlock<NT> ab;
  __device__ __forceinline__ void load(const BlocksArgs& a, int64_t blk) {
    constexpr int C = 16 * NT;
    load_ablock<NT>(a.A + (size_t)blk * C * C, ab);
  }
  template <int MAXD, bool BANDED>
  __device__ __forceinline__ void to_A(const BlocksArgs&, int band, Mat<NT>& AD, Mat<NT>& AT) const {
    ablock_to_A<NT, MAXD, BANDED>(ab, band, AD, AT);
  }
};

__device__ __forceinline__ void flush_counts(Fp8Counts& cnt, unsigned long long* stats) {
  uint32_t v0 = wave_sum_u32(cnt.nonfinite), v1 = wave_sum_u32(cnt.sat_dyn);
  uint32_t v2 = wave_sum_u32(cnt.sat_static), v3 = wave_sum_u32(cnt.underflow);
  if (lane_id() == 0) {
    if (v0) atomicAdd(stats + 0, (unsigned long long)v0);
    if (v1) atomicAdd(stats + 1, (unsigned long long)v1);
    if (v2) atomicAdd(stats + 2, (unsigned long long)v2);
    if (v3) atomicAdd(stats + 3, (unsigned long long)v3);
  }
}

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
  store_T_f32<NT>(A_out + (size_t)blk * C * C, AT);
}

// The inverse: one wave per block.  MAXD is the largest tile distance I - J kept
// (NT - 1 in general, 1 for the band-masked sum with N <= 16).
template <int NT, int SRC, int DK, int CMP, int MODE, int MAXD>
__global__ __launch_bounds__(256) void inverse_kernel(BlocksArgs a, int N, int mask, void* T_out,
                                                      int t_bf16, unsigned long long* stats, int S) {
  constexpr int C = 16 * NT;
  const int64_t blk = (int64_t)blockIdx.x * (blockDim.x / WAVE) + (threadIdx.x / WAVE);
  if (blk >= a.n_blocks) return;
  // fp8 and int8 mask A and every intermediate (the band sets the quantisation
  // scales); bf16 / fp32 mask only the final sum (identical result, see neumann_T)
  const int band = (MODE == MODE_NEUMANN && mask) ? N : -1;
  constexpr bool BANDED = (MODE == MODE_NEUMANN && (CMP == CMP_FP8 || CMP == CMP_INT8));
  Fp8Counts cnt{0, 0, 0, 0};
  const bool count = (CMP == CMP_FP8) && stats != nullptr;
  BlockIn<NT, SRC, DK> in;
  in.load(a, blk);
  Mat<NT> AD, AT, TT;
  in.template to_A<MAXD, BANDED>(a, BANDED ? band : -1, AD, AT);
  if constexpr (MODE == MODE_EXACT)
    doubling_T<NT, CMP>(AD, AT, TT);
  else if constexpr (MODE == MODE_RESIDUAL)
    residual_T<NT>(AD, AT, N, mask != 0, S, TT);
  else if constexpr (CMP == CMP_INT8)
    neumann_T_i8<NT, MAXD>(AD, AT, N, mask != 0, TT);
  else
    neumann_T<NT, CMP, MAXD>(AD, AT, N, mask != 0, TT, cnt, count);
  if (t_bf16)
    store_T_bf16<NT, MAXD>(reinterpret_cast<__bf16*>(T_out) + (size_t)blk * C * C, TT);
  else
    store_T_f32<NT, MAXD>(reinterpret_cast<float*>(T_out) + (size_t)blk * C * C, TT);
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

static dim3 grid_for(int64_t n_blocks) {
  return dim3((unsigned)((n_blocks + WAVES_PER_WG - 1) / WAVES_PER_WG));
}

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
        hipLaunchKernelGGL((inverse_kernel<NTv, sc.value, dk.value, cm.value, MODE_NEUMANN, 1>),
                           grid_for(a.n_blocks), dim3(WAVE * WAVES_PER_WG), 0, s, a, N, mask,
                           T_out, t_bf16, stats, 0);
      } else {
        hipLaunchKernelGGL((inverse_kernel<NTv, sc.value, dk.value, cm.value, MODE_NEUMANN, NTv - 1>),
                           grid_for(a.n_blocks), dim3(WAVE * WAVES_PER_WG), 0, s, a, N, mask,
                           T_out, t_bf16, stats, 0);
      }
      return 0;
    };
    switch (cmp) {
      case CMP_F32: return go(std::integral_constant<int, CMP_F32>{});
      case CMP_BF16: return go(std::integral_constant<int, CMP_BF16>{});
      case CMP_FP8: return go(std::integral_constant<int, CMP_FP8>{});
      case CMP_INT8: return go(std::integral_constant<int, CMP_INT8>{});
      default: return -1;
    }
  });
}

int launch_exact(const BlocksArgs& a, int src, int cmp, void* T_out, int t_bf16, hipStream_t s) {
  return dispatch_nt_src_dk(a.C, src, a.d_k, [&](auto nt, auto sc, auto dk) -> int {
    auto go = [&](auto cm) {
      hipLaunchKernelGGL((inverse_kernel<nt.value, sc.value, dk.value, cm.value, MODE_EXACT,
                                         nt.value - 1>),
                         grid_for(a.n_blocks), dim3(WAVE * WAVES_PER_WG), 0, s, a, 0, 0,
                         T_out, t_bf16, (unsigned long long*)nullptr, 0);
      return 0;
    };
    switch (cmp) {
      case CMP_F32: return go(std::integral_constant<int, CMP_F32>{});
      case CMP_BF16: return go(std::integral_constant<int, CMP_BF16>{});
      default: return -1;
    }
  });
}

// parallel residual correction on the Neumann sum: fp32 products throughout
int launch_residual(const BlocksArgs& a, int src, int N, int mask, int S, void* T_out, int t_bf16,
                    hipStream_t s) {
  return dispatch_nt_src_dk(a.C, src, a.d_k, [&](auto nt, auto sc, auto dk) -> int {
    hipLaunchKernelGGL((inverse_kernel<nt.value, sc.value, dk.value, CMP_F32, MODE_RESIDUAL, nt.value - 1>),
                       grid_for(a.n_blocks), dim3(WAVE * WAVES_PER_WG), 0, s, a, N, mask, T_out, t_bf16,
                       (unsigned long long*)nullptr, S);
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
