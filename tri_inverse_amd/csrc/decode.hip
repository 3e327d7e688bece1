// decode.hip -- the gated delta rule one token at a time (decode), with each head's
// state held on chip from its first token to its last.
//
// Per (b, h) and token t, with a = exp(gamma_t) and the state S [d_k][d_v] fp32:
//   r = S^T k,  p = S^T q                (one read of S for both retrievals)
//   u = beta (v - a r)                   (delta correction)
//   S <- a S + k u^T                     (state write)
//   o = scale (a p + (k . q) u)          (output, corrected without a second read of S)
// This is the read / correct / write split of one recurrence step that [PSDA] section
// 2.B describes, with the state read once and written once per launch: the GPU
// analogue of [PSDA] section 2.A's persistent on-chip state is the register file,
// which keeps S across all n tokens of a launch.  n = 1 is one decode step.
//
// Layout: one wave per (b, h, 32 columns of d_v); a workgroup holds the d_v/32 waves of
// one head, so they share the head's k and q lines in L1.  Lane l = 8 rg + cg holds
// columns 4cg..4cg+3 of the wave's slice for rows RPL rg .. RPL rg + RPL - 1 of d_k
// (RPL = d_k / 8), RPL x 4 fp32 values.  Every load of S moves 8 rows x 128 B with
// 16-byte accesses; S is read and written with non-temporal accesses (streamed once
// per call).  k and q are read as the lane's RPL contiguous elements (the 8 lanes of
// a row group read the same bytes).  The retrieval sums reduce over the 8 row groups
// with a butterfly across lanes.
#include "gdn_device.hpp"
#include "gdn_kernels.hpp"

namespace gdn {

namespace {

template <bool BF16>
struct In;
template <>
struct In<true> {
  typedef __bf16 T;
};
template <>
struct In<false> {
  typedef float T;
};

// N contiguous elements starting at p (16-byte aligned), widened to fp32
template <int N>
__device__ __forceinline__ void load_row(const __bf16* p, float (&x)[N]) {
  static_assert(N % 8 == 0, "bf16 rows load in 16-byte pieces");
#pragma unroll
  for (int i = 0; i < N / 8; ++i) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(p + 8 * i);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[8 * i + e] = (float)v[e];
  }
}
template <int N>
__device__ __forceinline__ void load_row(const float* p, float (&x)[N]) {
  static_assert(N % 4 == 0, "fp32 rows load in 16-byte pieces");
#pragma unroll
  for (int i = 0; i < N / 4; ++i) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(p + 4 * i);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[4 * i + e] = v[e];
  }
}

// Sum over the 8 row groups (lanes l ^ 8m, m = 0..7); every lane gets the same total.
// All three steps stay in the VALU:
//   x + x[l ^ 8]  : DPP row rotate by 8 within each 16-lane row;
//   x + x[l ^ 16] : v_permlane16_swap of x with itself swaps the odd rows of the first
//                   copy with the even rows of the second, so the two results hold rows
//                   (0,0,2,2) and (1,1,3,3) and their sum is row-pair total everywhere;
//   x + x[l ^ 32] : v_permlane32_swap likewise pairs rows (0,1) with (2,3).
__device__ __forceinline__ float sum_row_groups(float x) {
  const int r8 = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128 /* row_ror:8 */,
                                             0xf, 0xf, false);
  x += __builtin_bit_cast(float, r8);
  // (vector elements are copied to scalars before the bit casts: a bit cast applied to
  // a vector-element expression reads the vector's first element)
  const unsigned ux = __builtin_bit_cast(unsigned, x);
  const auto p16 = __builtin_amdgcn_permlane16_swap(ux, ux, false, false);
  const unsigned a0 = p16[0], a1 = p16[1];
  x = __builtin_bit_cast(float, a0) + __builtin_bit_cast(float, a1);
  const unsigned uy = __builtin_bit_cast(unsigned, x);
  const auto p32 = __builtin_amdgcn_permlane32_swap(uy, uy, false, false);
  const unsigned b0 = p32[0], b1 = p32[1];
  return __builtin_bit_cast(float, b0) + __builtin_bit_cast(float, b1);
}

// one token's inputs for one lane
template <int RPL>
struct Tok {
  float k[RPL], q[RPL], v[4];
  float beta, gam;
};

}  // namespace

struct DecodeArgs {
  const void* Q;
  const void* K;
  const void* V;
  const float* beta;
  const float* g;
  const float* S_in;  // may equal S_out: each element is read and written by one lane
  float* S_out;
  void* O;
  int n;  // tokens per (b, h)
  int n_heads;  // B * H
  int d_v;
  float scale;
};

template <int DK, bool IN_BF16, bool O_BF16>
__global__ __launch_bounds__(512) void decode_kernel(DecodeArgs a) {
  constexpr int RPL = DK / 8;
  typedef typename In<IN_BF16>::T TI;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  const int64_t bh = blockIdx.x;
  const int l = lane_id(), rg = l >> 3, cg = l & 7;
  const int dv = a.d_v;
  const int col = 32 * wave + 4 * cg;  // first of this lane's four columns
  const int row0 = RPL * rg;           // first of this lane's RPL rows

  const TI* __restrict__ Qp = reinterpret_cast<const TI*>(a.Q) + bh * a.n * DK + row0;
  const TI* __restrict__ Kp = reinterpret_cast<const TI*>(a.K) + bh * a.n * DK + row0;
  const TI* __restrict__ Vp = reinterpret_cast<const TI*>(a.V) + bh * a.n * dv + col;
  const float* __restrict__ bp = a.beta + bh * a.n;
  const float* __restrict__ gp = a.g + bh * a.n;

  // the lane's part of S: S[row0 + i][col + c] = s[i][c]
  float s[RPL][4];
  const size_t sbase = (size_t)bh * DK * dv + (size_t)row0 * dv + col;
  if (a.S_in) {
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.S_in + sbase + (size_t)i * dv));
#pragma unroll
      for (int c = 0; c < 4; ++c) s[i][c] = v[c];
    }
  } else {
#pragma unroll
    for (int i = 0; i < RPL; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) s[i][c] = 0.f;
  }

  auto load_tok = [&](int t, Tok<RPL>& x) {
    load_row<RPL>(Kp + (size_t)t * DK, x.k);
    load_row<RPL>(Qp + (size_t)t * DK, x.q);
    if constexpr (IN_BF16) {
      const bf16x4 v = *reinterpret_cast<const bf16x4*>(Vp + (size_t)t * dv);
#pragma unroll
      for (int c = 0; c < 4; ++c) x.v[c] = (float)v[c];
    } else {
      const f32x4 v = *reinterpret_cast<const f32x4*>(Vp + (size_t)t * dv);
#pragma unroll
      for (int c = 0; c < 4; ++c) x.v[c] = v[c];
    }
    x.beta = bp[t];
    x.gam = gp[t];
  };

  if (a.n > 0) {  // n == 0 leaves S as given (S_out = S_in, or zeros)
  Tok<RPL> cur;
  load_tok(0, cur);
  for (int t = 0; t < a.n; ++t) {
    // next token's inputs in flight while this one is processed (index clamped so
    // the load is unconditional)
    Tok<RPL> nxt;
    load_tok(t + 1 < a.n ? t + 1 : t, nxt);

    const float av = __expf(cur.gam);
    float r[4] = {0.f, 0.f, 0.f, 0.f}, p[4] = {0.f, 0.f, 0.f, 0.f}, kq = 0.f;
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      kq = fmaf(cur.k[i], cur.q[i], kq);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        r[c] = fmaf(s[i][c], cur.k[i], r[c]);
        p[c] = fmaf(s[i][c], cur.q[i], p[c]);
      }
    }
    kq = sum_row_groups(kq);
    float u[4], o[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      r[c] = sum_row_groups(r[c]);
      p[c] = sum_row_groups(p[c]);
      u[c] = cur.beta * (cur.v[c] - av * r[c]);
      o[c] = a.scale * fmaf(av, p[c], kq * u[c]);
    }
#pragma unroll
    for (int i = 0; i < RPL; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) s[i][c] = fmaf(av, s[i][c], cur.k[i] * u[c]);

    if (rg == 0) {
      const size_t oo = (size_t)(bh * a.n + t) * dv + col;
      if constexpr (O_BF16) {
        bf16x4 w;
#pragma unroll
        for (int c = 0; c < 4; ++c) w[c] = (__bf16)o[c];
        *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(a.O) + oo) = w;
      } else {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.O) + oo) =
            f32x4{o[0], o[1], o[2], o[3]};
      }
    }
    cur = nxt;
  }
  }

#pragma unroll
  for (int i = 0; i < RPL; ++i)
    __builtin_nontemporal_store(f32x4{s[i][0], s[i][1], s[i][2], s[i][3]},
                                reinterpret_cast<f32x4*>(a.S_out + sbase + (size_t)i * dv));
}

int launch_decode(const DecodeLaunch& p, hipStream_t s) {
  DecodeArgs a;
  a.Q = p.Q;
  a.K = p.K;
  a.V = p.V;
  a.beta = p.beta;
  a.g = p.g;
  a.S_in = p.S_in;
  a.S_out = p.S_out;
  a.O = p.O;
  a.n = p.n;
  a.n_heads = p.B * p.H;
  a.d_v = p.d_v;
  a.scale = p.scale;
  if (p.d_v % 32 != 0 || p.d_v > 256 || p.d_v <= 0) return -1;
  const dim3 grid((unsigned)a.n_heads), block((unsigned)(WAVE * (p.d_v / 32)));
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, s, a);
    return 0;
  };
  const bool ib = p.in_bf16 != 0, ob = p.o_bf16 != 0;
  switch (p.d_k) {
    case 64:
      if (ib) return ob ? go(decode_kernel<64, true, true>) : go(decode_kernel<64, true, false>);
      return ob ? go(decode_kernel<64, false, true>) : go(decode_kernel<64, false, false>);
    case 128:
      if (ib) return ob ? go(decode_kernel<128, true, true>) : go(decode_kernel<128, true, false>);
      return ob ? go(decode_kernel<128, false, true>) : go(decode_kernel<128, false, false>);
    default:
      return -1;
  }
}

}  // namespace gdn
