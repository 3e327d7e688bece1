// abi.cpp -- the C ABI of libgdn (declared in include/gdn.h): argument validation,
// status codes, and the hand-off to the kernel launchers on the caller's stream.
// Validation happens entirely on the host and returns before any HIP call, so every
// error path can be exercised without a GPU.
#include "gdn.h"

#include <hip/hip_runtime.h>

#include "gdn_kernels.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool chunk_ok(int C) { return C == 16 || C == 32 || C == 64 || C == 128 || C == 256; }
bool chunk_small(int C) { return C == 16 || C == 32 || C == 64; }
bool head_dim_ok(int d) { return d == 32 || d == 64 || d == 128 || d == 256; }

gdn_status launch_result(int rc) {
  if (rc < 0) return GDN_ERR_UNSUPPORTED;
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

// validates a gdn_blocks descriptor; src_out: 0 = A given, 1 = K bf16, 2 = K fp32.
// An empty batch (n_blocks == 0) only needs valid sizes: its pointers may be NULL.
gdn_status check_blocks(const gdn_blocks* in, bool allow_A, bool allow_k_f32, int* src_out) {
  if (!in) return GDN_ERR_NULL_POINTER;
  if (in->n_blocks < 0 || in->C <= 0) return GDN_ERR_BAD_SHAPE;
  if (!chunk_ok(in->C)) return GDN_ERR_UNSUPPORTED;
  const bool empty = in->n_blocks == 0;
  if (in->A) {
    if (!allow_A) return GDN_ERR_UNSUPPORTED;
    if (!aligned16(in->A)) return GDN_ERR_BAD_ALIGNMENT;
    *src_out = 0;
    return GDN_OK;
  }
  if (in->d_k <= 0) {
    if (empty && !in->K) {  // empty batch given as A == NULL, K == NULL
      *src_out = 0;
      return GDN_OK;
    }
    return GDN_ERR_BAD_SHAPE;
  }
  if (!head_dim_ok(in->d_k)) return GDN_ERR_UNSUPPORTED;
  if (in->k_dtype == GDN_BF16) {
    *src_out = 1;
  } else if (in->k_dtype == GDN_F32) {
    if (!allow_k_f32) return GDN_ERR_UNSUPPORTED;
    *src_out = 2;
  } else {
    return GDN_ERR_BAD_DTYPE;
  }
  if (empty) return GDN_OK;
  if (!in->K || !in->beta || !in->g) return GDN_ERR_NULL_POINTER;
  if (!aligned16(in->K) || !aligned16(in->beta) || !aligned16(in->g)) return GDN_ERR_BAD_ALIGNMENT;
  return GDN_OK;
}

gdn::BlocksArgs to_args(const gdn_blocks* in) {
  gdn::BlocksArgs a;
  a.A = in->A;
  a.K = in->K;
  a.beta = in->beta;
  a.g = in->g;
  a.n_blocks = in->n_blocks;
  a.C = in->C;
  a.d_k = in->d_k;
  a.g_cumulative = in->g_cumulative;
  return a;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_status_string(int32_t s) {
  switch (s) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_NULL_POINTER: return "GDN_ERR_NULL_POINTER: a required pointer is NULL";
    case GDN_ERR_BAD_SHAPE: return "GDN_ERR_BAD_SHAPE: a size or order argument is out of range";
    case GDN_ERR_BAD_DTYPE: return "GDN_ERR_BAD_DTYPE: dtype code not accepted for this argument";
    case GDN_ERR_BAD_ALIGNMENT: return "GDN_ERR_BAD_ALIGNMENT: a tensor pointer is not 16-byte aligned";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: configuration not implemented by this build";
    case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE: workspace missing or smaller than the query returned";
    case GDN_ERR_HIP: return "GDN_ERR_HIP: the HIP runtime reported an error at launch";
    default: return "unknown gdn_status";
  }
}

gdn_status gdn_build_A(const gdn_blocks* in, float* A_out, void* stream) {
  int src = 0;
  if (in && in->A) return GDN_ERR_UNSUPPORTED;  // A is the output here
  gdn_status st = check_blocks(in, false, true, &src);
  if (st != GDN_OK) return st;
  if (!chunk_small(in->C)) return GDN_ERR_UNSUPPORTED;
  if (in->n_blocks == 0) return GDN_OK;
  if (!A_out) return GDN_ERR_NULL_POINTER;
  if (!aligned16(A_out)) return GDN_ERR_BAD_ALIGNMENT;
  return launch_result(gdn::launch_build_A(to_args(in), src, A_out, as_stream(stream)));
}

gdn_status gdn_tri_inverse_neumann(const gdn_blocks* in, int32_t N, int32_t mask, int32_t compute,
                                   void* T_out, int32_t t_dtype, gdn_fp8_stats* stats, void* stream) {
  int src = 0;
  gdn_status st = check_blocks(in, true, false, &src);
  if (st != GDN_OK) return st;
  if (N < 1 || N >= in->C) return GDN_ERR_BAD_SHAPE;
  if (mask != 0 && mask != 1) return GDN_ERR_BAD_SHAPE;
  if (compute != GDN_F32 && compute != GDN_BF16 && compute != GDN_FP8_E4M3 && compute != GDN_INT8 &&
      compute != GDN_INT16)
    return GDN_ERR_BAD_DTYPE;
  if (t_dtype != GDN_F32 && t_dtype != GDN_BF16) return GDN_ERR_BAD_DTYPE;
  // C >= 128 (bf16 keys and products): the band kernel for the masked sum with N <= 16,
  // the full-triangle kernel otherwise
  const bool large = !chunk_small(in->C);
  if (large && (src != 1 || compute != GDN_BF16)) return GDN_ERR_UNSUPPORTED;
  const bool band = large && mask && N <= 16;
  if (stats && !aligned16(stats)) return GDN_ERR_BAD_ALIGNMENT;
  if (in->n_blocks > 0) {
    if (!T_out) return GDN_ERR_NULL_POINTER;
    if (!aligned16(T_out)) return GDN_ERR_BAD_ALIGNMENT;
  }
  hipStream_t s = as_stream(stream);
  auto* st64 = reinterpret_cast<unsigned long long*>(stats);
  if (st64) {
    gdn::launch_zero_stats(st64, s);
    if (hipGetLastError() != hipSuccess) return GDN_ERR_HIP;
  }
  if (in->n_blocks == 0) return GDN_OK;
  if (band)
    return launch_result(gdn::launch_band(to_args(in), nullptr, 0, N, 0, T_out, t_dtype == GDN_BF16,
                                          nullptr, nullptr, 0, s));
  if (large)
    return launch_result(gdn::launch_dense(to_args(in), nullptr, 0, 0, N, mask, nullptr, 0, 0, T_out,
                                           t_dtype == GDN_BF16, nullptr, nullptr, 0, s));
  return launch_result(gdn::launch_neumann(to_args(in), src, N, mask, compute, T_out,
                                           t_dtype == GDN_BF16, st64, s));
}

gdn_status gdn_tri_inverse_exact(const gdn_blocks* in, int32_t compute, void* T_out,
                                 int32_t t_dtype, void* stream) {
  int src = 0;
  gdn_status st = check_blocks(in, true, false, &src);
  if (st != GDN_OK) return st;
  if (compute == GDN_FP8_E4M3 || compute == GDN_INT8 || compute == GDN_INT16) return GDN_ERR_UNSUPPORTED;
  if (compute != GDN_F32 && compute != GDN_BF16) return GDN_ERR_BAD_DTYPE;
  if (t_dtype != GDN_F32 && t_dtype != GDN_BF16) return GDN_ERR_BAD_DTYPE;
  const bool large = !chunk_small(in->C);
  if (large && (src != 1 || compute != GDN_BF16)) return GDN_ERR_UNSUPPORTED;
  if (in->n_blocks == 0) return GDN_OK;
  if (!T_out) return GDN_ERR_NULL_POINTER;
  if (!aligned16(T_out)) return GDN_ERR_BAD_ALIGNMENT;
  if (large)
    return launch_result(gdn::launch_dense(to_args(in), nullptr, 0, 1, 0, 0, nullptr, 0, 0, T_out,
                                           t_dtype == GDN_BF16, nullptr, nullptr, 0, as_stream(stream)));
  return launch_result(gdn::launch_exact(to_args(in), src, compute, T_out, t_dtype == GDN_BF16,
                                         as_stream(stream)));
}

gdn_status gdn_tri_inverse_residual(const gdn_blocks* in, int32_t N, int32_t mask, int32_t S,
                                    int32_t compute, void* T_out, int32_t t_dtype, void* stream) {
  int src = 0;
  gdn_status st = check_blocks(in, true, false, &src);
  if (st != GDN_OK) return st;
  if (N < 1 || N >= in->C) return GDN_ERR_BAD_SHAPE;
  if (mask != 0 && mask != 1) return GDN_ERR_BAD_SHAPE;
  if (S < 0 || S > 64) return GDN_ERR_BAD_SHAPE;
  if (compute != GDN_F32 && compute != GDN_BF16 && compute != GDN_FP8_E4M3 && compute != GDN_INT8 &&
      compute != GDN_INT16)
    return GDN_ERR_BAD_DTYPE;
  if (t_dtype != GDN_F32 && t_dtype != GDN_BF16) return GDN_ERR_BAD_DTYPE;
  if (compute != GDN_F32) return GDN_ERR_UNSUPPORTED;
  if (!chunk_small(in->C)) return GDN_ERR_UNSUPPORTED;
  if (in->n_blocks == 0) return GDN_OK;
  if (!T_out) return GDN_ERR_NULL_POINTER;
  if (!aligned16(T_out)) return GDN_ERR_BAD_ALIGNMENT;
  return launch_result(gdn::launch_residual(to_args(in), src, N, mask, S, T_out, t_dtype == GDN_BF16,
                                            as_stream(stream)));
}

gdn_status gdn_tri_inverse_fs(const gdn_blocks* in, void* T_out, int32_t t_dtype, void* stream) {
  int src = 0;
  gdn_status st = check_blocks(in, true, false, &src);
  if (st != GDN_OK) return st;
  if (t_dtype != GDN_F32 && t_dtype != GDN_BF16) return GDN_ERR_BAD_DTYPE;
  const bool c128 = in->C == 128;
  if (!chunk_small(in->C) && !c128) return GDN_ERR_UNSUPPORTED;
  if (c128 && src == 2) return GDN_ERR_UNSUPPORTED;  // fp32 keys: C <= 64 only
  if (c128 && src == 1 && !(in->d_k == 64 || in->d_k == 128)) return GDN_ERR_UNSUPPORTED;
  if (in->n_blocks == 0) return GDN_OK;
  if (!T_out) return GDN_ERR_NULL_POINTER;
  if (!aligned16(T_out)) return GDN_ERR_BAD_ALIGNMENT;
  if (c128)
    return launch_result(gdn::launch_fs128(to_args(in), src, T_out, t_dtype == GDN_BF16, as_stream(stream)));
  return launch_result(gdn::launch_fs(to_args(in), src, T_out, t_dtype == GDN_BF16, as_stream(stream)));
}

gdn_status gdn_wy(const gdn_blocks* in, const void* T, int32_t t_dtype, const gdn_inverse_cfg* inv,
                  const void* V, int32_t d_v, int32_t gate_k, void* W_out, void* U_out,
                  int32_t out_dtype, void* stream) {
  int src = 0;
  if (in && in->A) return GDN_ERR_UNSUPPORTED;  // the products need K itself
  gdn_status st = check_blocks(in, false, false, &src);
  if (st != GDN_OK) return st;
  if (T) {
    if (t_dtype != GDN_F32 && t_dtype != GDN_BF16) return GDN_ERR_BAD_DTYPE;
  } else {
    if (!inv) return GDN_ERR_NULL_POINTER;
    if (inv->mode != GDN_INV_NEUMANN && inv->mode != GDN_INV_EXACT) return GDN_ERR_BAD_SHAPE;
    if (inv->mode == GDN_INV_NEUMANN && (inv->N < 1 || inv->N >= in->C)) return GDN_ERR_BAD_SHAPE;
    if (inv->mask != 0 && inv->mask != 1) return GDN_ERR_BAD_SHAPE;
    if (inv->compute != GDN_BF16) {
      if (inv->compute == GDN_F32 || inv->compute == GDN_FP8_E4M3 || inv->compute == GDN_INT8 ||
          inv->compute == GDN_INT16)
        return GDN_ERR_UNSUPPORTED;
      return GDN_ERR_BAD_DTYPE;
    }
  }
  if (d_v <= 0) return GDN_ERR_BAD_SHAPE;
  if (gate_k != 0 && gate_k != 1) return GDN_ERR_BAD_SHAPE;
  if (out_dtype != GDN_F32 && out_dtype != GDN_BF16) return GDN_ERR_BAD_DTYPE;
  // C >= 128: the band kernel when T is formed as the masked sum with N <= 16, the
  // full-triangle kernel otherwise (T formed, or given)
  const bool large = in->C == 128 || in->C == 256;
  const bool band = large && !T && inv->mode == GDN_INV_NEUMANN && inv->mask && inv->N <= 16;
  if (!(large || in->C == 32 || in->C == 64)) return GDN_ERR_UNSUPPORTED;
  if (!(in->d_k == 64 || in->d_k == 128) || !(d_v == 64 || d_v == 128)) return GDN_ERR_UNSUPPORTED;
  if (in->n_blocks == 0) return GDN_OK;
  if (!V || !W_out || !U_out) return GDN_ERR_NULL_POINTER;
  if (!aligned16(V) || !aligned16(W_out) || !aligned16(U_out) || (T && !aligned16(T)))
    return GDN_ERR_BAD_ALIGNMENT;
  const int mode = T ? 0 : inv->mode, N = T ? 0 : inv->N, mask = T ? 0 : inv->mask;
  if (band)
    return launch_result(gdn::launch_band(to_args(in), V, d_v, N, gate_k, nullptr, 0, W_out, U_out,
                                          out_dtype == GDN_BF16, as_stream(stream)));
  if (large)
    return launch_result(gdn::launch_dense(to_args(in), T, t_dtype == GDN_BF16, mode, N, mask, V, d_v,
                                           gate_k, nullptr, 0, W_out, U_out, out_dtype == GDN_BF16,
                                           as_stream(stream)));
  return launch_result(gdn::launch_wy(to_args(in), T, t_dtype == GDN_BF16, mode, N, mask, V, d_v,
                                      gate_k, W_out, U_out, out_dtype == GDN_BF16,
                                      as_stream(stream)));
}

// argument checks of gdn_chunk_fwd that need no pointer (shared with the workspace query)
static gdn_status check_chunk_args(int32_t qkv_dtype, int32_t o_dtype, int32_t B, int32_t H, int64_t T, int32_t d_k,
                            int32_t d_v, int32_t C, const gdn_inverse_cfg* inv) {
  if (!inv) return GDN_ERR_NULL_POINTER;
  if (B < 0 || H < 0 || T < 0 || d_k <= 0 || d_v <= 0 || C <= 0) return GDN_ERR_BAD_SHAPE;
  if (qkv_dtype != GDN_BF16) return (qkv_dtype == GDN_F32) ? GDN_ERR_UNSUPPORTED : GDN_ERR_BAD_DTYPE;
  if (o_dtype != GDN_F32 && o_dtype != GDN_BF16) return GDN_ERR_BAD_DTYPE;
  if (!chunk_ok(C)) return GDN_ERR_UNSUPPORTED;
  if (T % C != 0) return GDN_ERR_BAD_SHAPE;
  if (inv->mode != GDN_INV_NEUMANN && inv->mode != GDN_INV_EXACT && inv->mode != GDN_INV_NEUMANN_PRODUCTS)
    return GDN_ERR_BAD_SHAPE;
  if (inv->mode != GDN_INV_EXACT && (inv->N < 1 || inv->N >= C)) return GDN_ERR_BAD_SHAPE;
  if (inv->mask != 0 && inv->mask != 1) return GDN_ERR_BAD_SHAPE;
  if (inv->compute != GDN_BF16 && inv->compute != GDN_FP8_E4M3 && inv->compute != GDN_F32 &&
      inv->compute != GDN_INT8 && inv->compute != GDN_INT16)
    return GDN_ERR_BAD_DTYPE;
  if (inv->compute == GDN_F32 || inv->compute == GDN_INT8 || inv->compute == GDN_INT16) return GDN_ERR_UNSUPPORTED;
  if (inv->compute == GDN_FP8_E4M3 && inv->mode == GDN_INV_EXACT) return GDN_ERR_UNSUPPORTED;
  if (C != 64) return GDN_ERR_UNSUPPORTED;
  if (!(d_k == 64 || d_k == 128)) return GDN_ERR_UNSUPPORTED;
  if (d_v % 32 != 0 || d_v > 256) return GDN_ERR_UNSUPPORTED;
  return GDN_OK;
}

static size_t chunk_workspace(int32_t B, int32_t H, int64_t T, int32_t C, const gdn_inverse_cfg* inv) {
  if (inv->mode == GDN_INV_NEUMANN && gdn::chunk_fwd_band_path(inv->mode, inv->N, inv->mask, inv->compute))
    return 0;
  const size_t chunks = (size_t)B * (size_t)H * (size_t)(T / C);
  if (inv->mode == GDN_INV_NEUMANN && gdn::chunk_fwd_fp8_band(inv->mode, inv->N, inv->mask, inv->compute))
    return chunks * gdn::BAND_ROW_BYTES;
  return chunks * gdn::T_PACK_BYTES;
}

size_t gdn_chunk_fwd_workspace_bytes(int32_t B, int32_t H, int64_t T, int32_t d_k, int32_t d_v,
                                     int32_t C, const gdn_inverse_cfg* inv) {
  if (check_chunk_args(GDN_BF16, GDN_BF16, B, H, T, d_k, d_v, C, inv) != GDN_OK) return 0;
  return chunk_workspace(B, H, T, C, inv);
}

gdn_status gdn_chunk_fwd(const void* Q, const void* K, const void* V, int32_t qkv_dtype,
                         const float* beta, const float* g, const float* S0, void* O,
                         int32_t o_dtype, float* S_out, int32_t B, int32_t H, int64_t T,
                         int32_t d_k, int32_t d_v, int32_t C, float scale,
                         const gdn_inverse_cfg* inv, void* workspace, size_t workspace_bytes,
                         gdn_fp8_stats* stats, void* stream) {
  return gdn::chunk_fwd_impl(Q, K, V, qkv_dtype, beta, g, S0, O, o_dtype, S_out, B, H, T, d_k, d_v, C,
                             scale, inv, workspace, workspace_bytes, nullptr, stats, stream);
}

gdn_status gdn_decode(const void* Q, const void* K, const void* V, int32_t qkv_dtype,
                      const float* beta, const float* g, const float* S_in, float* S_out,
                      void* O, int32_t o_dtype, int32_t B, int32_t H, int32_t n,
                      int32_t d_k, int32_t d_v, float scale, void* stream) {
  if (B < 0 || H < 0 || n < 0 || d_k <= 0 || d_v <= 0) return GDN_ERR_BAD_SHAPE;
  if (qkv_dtype != GDN_BF16 && qkv_dtype != GDN_F32) return GDN_ERR_BAD_DTYPE;
  if (o_dtype != GDN_F32 && o_dtype != GDN_BF16) return GDN_ERR_BAD_DTYPE;
  if (!(d_k == 64 || d_k == 128)) return GDN_ERR_UNSUPPORTED;
  if (d_v % 32 != 0 || d_v > 256) return GDN_ERR_UNSUPPORTED;
  if ((int64_t)B * H == 0) return GDN_OK;
  if (!S_out) return GDN_ERR_NULL_POINTER;
  if (n > 0 && (!Q || !K || !V || !beta || !g || !O)) return GDN_ERR_NULL_POINTER;
  for (const void* p : {Q, K, V, (const void*)beta, (const void*)g, (const void*)S_in,
                        (const void*)S_out, (const void*)O})
    if (p && !aligned16(p)) return GDN_ERR_BAD_ALIGNMENT;
  gdn::DecodeLaunch p;
  p.Q = Q;
  p.K = K;
  p.V = V;
  p.beta = beta;
  p.g = g;
  p.S_in = S_in;
  p.S_out = S_out;
  p.O = O;
  p.B = B;
  p.H = H;
  p.n = n;
  p.d_k = d_k;
  p.d_v = d_v;
  p.in_bf16 = qkv_dtype == GDN_BF16;
  p.o_bf16 = o_dtype == GDN_BF16;
  p.scale = scale;
  return launch_result(gdn::launch_decode(p, as_stream(stream)));
}

}  // extern "C"

namespace gdn {

gdn_status chunk_fwd_impl(const void* Q, const void* K, const void* V, int32_t qkv_dtype,
                          const float* beta, const float* g, const float* S0, void* O,
                          int32_t o_dtype, float* S_out, int32_t B, int32_t H, int64_t T,
                          int32_t d_k, int32_t d_v, int32_t C, float scale,
                          const gdn_inverse_cfg* inv, void* workspace, size_t workspace_bytes,
                          void* (*workspace_of_device)(size_t need), gdn_fp8_stats* stats, void* stream) {
  gdn_status st = check_chunk_args(qkv_dtype, o_dtype, B, H, T, d_k, d_v, C, inv);
  if (st != GDN_OK) return st;
  if (stats && !aligned16(stats)) return GDN_ERR_BAD_ALIGNMENT;
  hipStream_t s = as_stream(stream);
  auto* st64 = reinterpret_cast<unsigned long long*>(stats);
  const bool empty = (int64_t)B * H == 0 || T == 0;
  const size_t need = empty ? 0 : chunk_workspace(B, H, T, C, inv);
  // the masked fp8 chain with N <= 3: its band pre-pass instead of the row packs
  const bool fp8_band =
      inv->mode == GDN_INV_NEUMANN && gdn::chunk_fwd_fp8_band(inv->mode, inv->N, inv->mask, inv->compute);
  if (!empty) {
    if (!Q || !K || !V || !beta || !g || !O || !S_out) return GDN_ERR_NULL_POINTER;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(beta) || !aligned16(g) ||
        !aligned16(O) || !aligned16(S_out) || (S0 && !aligned16(S0)))
      return GDN_ERR_BAD_ALIGNMENT;
    if (need > 0) {
      if (workspace_of_device) {
        // no workspace argument: the caller's resolver supplies it (NULL if need exceeds
        // what it holds, or if the HIP runtime failed; it reports which)
        if (need > workspace_bytes) return GDN_ERR_WORKSPACE;
        workspace = workspace_of_device(need);
        if (!workspace) return GDN_ERR_HIP;
      } else if (!workspace || workspace_bytes < need) {
        return GDN_ERR_WORKSPACE;
      }
      if (!aligned16(workspace)) return GDN_ERR_BAD_ALIGNMENT;
    }
  }
  if (st64) {
    gdn::launch_zero_stats(st64, s);
    if (hipGetLastError() != hipSuccess) return GDN_ERR_HIP;
  }
  if (empty) return GDN_OK;
  if (need > 0) {
    // pre-pass: T - I of every chunk as row packs, each chunk a block of the keys
    gdn::BlocksArgs ba;
    ba.A = nullptr;
    ba.K = K;
    ba.beta = beta;
    ba.g = g;
    ba.n_blocks = (int64_t)B * H * (T / C);
    ba.C = C;
    ba.d_k = d_k;
    ba.g_cumulative = 0;
    const int mode = inv->mode == GDN_INV_EXACT ? 1 : 0;  // the products of either Neumann mode
    const gdn_status pre =
        launch_result(fp8_band ? gdn::launch_band_fp8(ba, inv->N, workspace, st64, s)
                               : gdn::launch_T_packs(ba, mode, inv->N, inv->mask, inv->compute, workspace, st64, s));
    if (pre != GDN_OK) return pre;
  }
  gdn::ChunkLaunch p;
  p.Q = Q;
  p.K = K;
  p.V = V;
  p.beta = beta;
  p.g = g;
  p.S0 = S0;
  p.O = O;
  p.S_out = S_out;
  p.packs = need > 0 ? workspace : nullptr;
  p.band_rows = fp8_band ? 1 : 0;
  p.T = T;
  p.B = B;
  p.H = H;
  p.d_k = d_k;
  p.d_v = d_v;
  p.o_bf16 = o_dtype == GDN_BF16;
  p.mode = inv->mode == GDN_INV_EXACT ? 1 : 0;
  p.N = inv->N;
  p.mask = inv->mask;
  p.cmp = inv->compute;
  p.scale = scale;
  return launch_result(gdn::launch_chunk_fwd(p, s));
}

}  // namespace gdn
