// fs.hip -- forward substitution at C = 128, the sequential baseline of [GEO] "When
// Good Enough Is Optimal: Multiplication-Only Matrix Inversion Approximation for
// Quantized Gated DeltaNet", problem statement: T = (I - A)^-1 from T = I + A T, row
// after row, T[i][.] = e_i + sum_{m<i} A[i][m] T[m][.], in fp32.
//
// One workgroup of two waves per 128 x 128 block.  A goes to LDS first: given (fp32),
// or built from bf16 keys with 16x16x32 MFMA Gram tiles (the two waves take
// alternate lower tiles) and the gate and beta factors,
//   A_ij = -beta_i (k_i . k_j) exp(G_i - G_j)  (i > j),  G = in-block cumsum of gamma.
// Then thread j (0..127) carries column j of T in 128 registers through the fully
// unrolled substitution; each A[i][4q .. 4q+3] is one 16-byte LDS broadcast read, and
// four partial sums per row break the dependent chain.  C (C - 1) / 2 multiply-adds per
// thread, in row order.
#include "gdn_kernels.hpp"
#include "tri_block.hpp"

namespace gdn {

constexpr int FS_C = 128;
enum : int { FS_SRC_A = 0, FS_SRC_K_BF16 = 1 };  // the launchers' src codes
constexpr int FS_LD = FS_C + 4;  // padded LDS row (floats)

template <int SRC, int DK>
__global__ __launch_bounds__(128) void fs128_kernel(BlocksArgs a, void* T_out, int t_bf16) {
  __shared__ float As[FS_C][FS_LD];
  __shared__ float Gs[FS_C], Bs[FS_C];
  __shared__ float wave0_total;
  const int64_t blk = blockIdx.x;
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t / WAVE);
  const int l = lane_id(), g = l >> 4, c = l & 15;

  if constexpr (SRC == FS_SRC_A) {
    // rows 0..127 of A, 16 bytes per thread and step (strict lower part only is read)
    const float* src = a.A + (size_t)blk * FS_C * FS_C;
#pragma unroll 4
    for (int e = t; e < FS_C * FS_C / 4; e += FS_C) {
      const int row = e / (FS_C / 4), col = 4 * (e % (FS_C / 4));
      *reinterpret_cast<f32x4*>(&As[row][col]) = *reinterpret_cast<const f32x4*>(src + (size_t)row * FS_C + col);
    }
    __syncthreads();
  } else {
    // gates: G = inclusive cumsum of gamma over the block (one wave per half)
    const float gl = a.g[(size_t)blk * FS_C + t];
    const float bl = a.beta[(size_t)blk * FS_C + t];
    float G = a.g_cumulative ? gl : wave_inclusive_scan(gl);
    if (!a.g_cumulative && wave == 0 && l == WAVE - 1) wave0_total = G;
    __syncthreads();
    if (!a.g_cumulative && wave == 1) G += wave0_total;
    Gs[t] = G;
    Bs[t] = bl;
    __syncthreads();
    // Gram tiles (I >= J), alternating between the waves; D-form: lane (g,c) reg r holds
    // (K K^T)[16I + 4g + r][16J + c]
    const __bf16* K = reinterpret_cast<const __bf16*>(a.K) + (size_t)blk * FS_C * DK;
    constexpr int NTL = FS_C / 16;
    for (int idx = wave; idx < NTL * (NTL + 1) / 2; idx += 2) {
      int I = 0;
      while ((I + 1) * (I + 2) / 2 <= idx) ++I;
      const int J = idx - I * (I + 1) / 2;
      f32x4 acc = zero4();
#pragma unroll
      for (int s = 0; s < DK / 32; ++s) {
        const bf16x8 ki = *reinterpret_cast<const bf16x8*>(K + (size_t)(16 * I + c) * DK + 32 * s + 8 * g);
        const bf16x8 kj = *reinterpret_cast<const bf16x8*>(K + (size_t)(16 * J + c) * DK + 32 * s + 8 * g);
        acc = mma_bf16(ki, kj, acc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * I + 4 * g + r, j = 16 * J + c;
        As[i][j] = (i > j) ? -Bs[i] * acc[r] * __expf(Gs[i] - Gs[j]) : 0.f;
      }
    }
    __syncthreads();
  }

  // forward substitution, thread t = column t
  float Tc[FS_C];
#pragma unroll
  for (int i = 0; i < FS_C; ++i) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < (i + 3) / 4; ++q) {
      const f32x4 a4 = *reinterpret_cast<const f32x4*>(&As[i][4 * q]);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (4 * q + k < i) acc[k] = fmaf(a4[k], Tc[4 * q + k], acc[k]);
    }
    Tc[i] = ((t == i) ? 1.f : 0.f) + ((acc[0] + acc[1]) + (acc[2] + acc[3]));
    // Keep each row's LDS reads next to its multiply-adds: the empty asm consumes the
    // row's result and is ordered before the next row's reads (memory clobber), so the
    // compiler cannot gather the reads of all rows first and hold thousands of values.
    asm volatile("" : "+v"(Tc[i])::"memory");
  }
  // row-major store: row i is 128 consecutive values across the threads
#pragma unroll
  for (int i = 0; i < FS_C; ++i) {
    const size_t o = (size_t)blk * FS_C * FS_C + (size_t)i * FS_C + t;
    if (t_bf16)
      reinterpret_cast<__bf16*>(T_out)[o] = (__bf16)Tc[i];
    else
      reinterpret_cast<float*>(T_out)[o] = Tc[i];
  }
}

int launch_fs128(const BlocksArgs& a, int src, void* T_out, int t_bf16, hipStream_t s) {
  if (a.C != FS_C) return -1;
  const dim3 grid((unsigned)a.n_blocks), block(FS_C);
  if (src == FS_SRC_A) {
    hipLaunchKernelGGL((fs128_kernel<FS_SRC_A, 32>), grid, block, 0, s, a, T_out, t_bf16);
    return 0;
  }
  if (src != FS_SRC_K_BF16) return -1;
  switch (a.d_k) {
    case 64: hipLaunchKernelGGL((fs128_kernel<FS_SRC_K_BF16, 64>), grid, block, 0, s, a, T_out, t_bf16); return 0;
    case 128: hipLaunchKernelGGL((fs128_kernel<FS_SRC_K_BF16, 128>), grid, block, 0, s, a, T_out, t_bf16); return 0;
    default: return -1;
  }
}

}  // namespace gdn
