// gdn_kernels.hpp -- host-visible launch interface between the C-ABI layer (abi.cpp)
// and the kernel translation units.  Arguments are validated by abi.cpp before any
// launcher is called; launchers return 0 on success, -1 for a configuration they
// have no instantiation for (reported as GDN_ERR_UNSUPPORTED).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace gdn {

struct BlocksArgs {
  const float* A;
  const void* K;
  const float* beta;
  const float* g;
  int64_t n_blocks;
  int C;
  int d_k;
  int g_cumulative;
};

// src: 0 = A given, 1 = K bf16, 2 = K fp32.  cmp: 0 = f32, 1 = bf16, 2 = fp8.
int launch_build_A(const BlocksArgs& a, int src, float* A_out, hipStream_t s);
int launch_neumann(const BlocksArgs& a, int src, int N, int mask, int cmp, void* T_out, int t_bf16,
                   unsigned long long* stats, hipStream_t s);
int launch_exact(const BlocksArgs& a, int src, int cmp, void* T_out, int t_bf16, hipStream_t s);
void launch_zero_stats(unsigned long long* stats, hipStream_t s);
// truncated sum refined by the parallel residual correction (S Horner steps in E), fp32
int launch_residual(const BlocksArgs& a, int src, int N, int mask, int S, void* T_out, int t_bf16,
                    hipStream_t s);
// forward substitution (fp32), the sequential baseline, C <= 64
int launch_fs(const BlocksArgs& a, int src, void* T_out, int t_bf16, hipStream_t s);
// forward substitution at C = 128 (A given in fp32, or built from bf16 keys, d_k 64 or 128)
int launch_fs128(const BlocksArgs& a, int src, void* T_out, int t_bf16, hipStream_t s);

// WY products; T given (t_bf16 selects its dtype) or formed with (mode, N, mask);
// C in {32, 64}, d_k and d_v in {64, 128}
int launch_wy(const BlocksArgs& a, const void* T, int t_bf16, int mode, int N, int mask,
              const void* V, int d_v, int gate_k, void* W_out, void* U_out, int out_bf16,
              hipStream_t s);

// masked truncated Neumann with band N <= 16 for C a multiple of 64 (d_k in {64, 128}):
// T (T_out non-NULL, row-major [C][C]) or the WY products (d_v in {64, 128}); one
// wave per 16-row tile, each on its own 32-row window
int launch_band(const BlocksArgs& a, const void* V, int d_v, int N, int gate_k, void* T_out, int t_bf16,
                void* W_out, void* U_out, int out_bf16, hipStream_t s);

// full lower triangle at C in {128, 256} (d_k in {64, 128}): Neumann (any N, masked or
// not) or exact doubling, as T (T_out) or as the WY products (d_v in {64, 128}); WY
// of a given T (T_in, fp32 or bf16) too.  One workgroup of C/32 waves per block.
int launch_dense(const BlocksArgs& a, const void* T_in, int t_in_bf16, int mode, int N, int mask,
                 const void* V, int d_v, int gate_k, void* T_out, int t_bf16, void* W_out, void* U_out,
                 int out_bf16, hipStream_t s);

// T - I of every 64 x 64 block as the chunk forward's row packs (6 x 64 x 16 bytes per
// block, store_T_packs): the pre-pass of every chunk-forward variant but the band path
int launch_T_packs(const BlocksArgs& a, int mode, int N, int mask, int cmp, void* packs,
                   unsigned long long* stats, hipStream_t s);
constexpr size_t T_PACK_BYTES = 6 * 64 * 16;

struct ChunkLaunch {
  const void* Q;
  const void* K;
  const void* V;
  const float* beta;
  const float* g;
  const float* S0;
  void* O;
  float* S_out;
  const void* packs;  // T - I from the pre-pass (NULL on the band path): row packs, or
                      // with band_rows the fp8 band pre-pass's rows
  int band_rows;
  int64_t T;
  int B, H, d_k, d_v;
  int o_bf16;
  int mode, N, mask, cmp;
  float scale;
};
// chunk-wise forward, C = 64; d_k in {64, 128}; d_v a multiple of 32.  The band path
// (Neumann, mask, N <= 3, bf16) forms T - I itself; the masked fp8 chain with N <= 3 reads
// the band rows of launch_band_fp8 (p.packs, p.band_rows); every other variant reads the
// row packs of launch_T_packs (p.packs).
bool chunk_fwd_band_path(int mode, int N, int mask, int cmp);
bool chunk_fwd_fp8_band(int mode, int N, int mask, int cmp);
// the band of T - I of every 64-row chunk for the masked fp8 chain, N <= 3 (bf16 keys,
// d_k 64 or 128, raw log-gates): 64 rows x 8 bytes per chunk; stats: its counters (or NULL)
int launch_band_fp8(const BlocksArgs& a, int N, void* out, unsigned long long* stats, hipStream_t s);
constexpr size_t BAND_ROW_BYTES = 64 * 8;
int launch_chunk_fwd(const ChunkLaunch& p, hipStream_t s);
}  // namespace gdn

#include "gdn.h"
namespace gdn {
// gdn_chunk_fwd's validation and launches.  With workspace_of_device == NULL the
// workspace arguments are the caller's; otherwise workspace_bytes is the most the
// resolver can supply and the resolver returns device memory of at least `need` bytes
// for the current device (NULL if the HIP runtime failed).
gdn_status chunk_fwd_impl(const void* Q, const void* K, const void* V, int32_t qkv_dtype,
                          const float* beta, const float* g, const float* S0, void* O,
                          int32_t o_dtype, float* S_out, int32_t B, int32_t H, int64_t T,
                          int32_t d_k, int32_t d_v, int32_t C, float scale,
                          const gdn_inverse_cfg* inv, void* workspace, size_t workspace_bytes,
                          void* (*workspace_of_device)(size_t need), gdn_fp8_stats* stats, void* stream);

struct DecodeLaunch {
  const void* Q;
  const void* K;
  const void* V;
  const float* beta;
  const float* g;
  const float* S_in;  // NULL = zeros; may equal S_out
  float* S_out;
  void* O;
  int B, H, n, d_k, d_v;
  int in_bf16, o_bf16;
  float scale;
};
// gated delta rule token by token with the state resident on chip for all n tokens;
// d_k in {64, 128}, d_v a multiple of 32 up to 256
int launch_decode(const DecodeLaunch& p, hipStream_t s);
}  // namespace gdn
