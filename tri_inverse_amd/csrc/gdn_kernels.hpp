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

}  // namespace gdn
