"""The chunk forward's bf16 rounding points, emulated on the CPU (test helper).

This is not the oracle: it is a model of where the GPU chunk forward rounds to bf16, used
to explain (and bound) its error on inputs where that error exceeds the usual bar.  Per
chunk, with T from the oracle (same inverse variant) and everything else in fp64:
  S_b = bf16(S)                  the state enters K S and Q S as bf16
  Y   = diag(beta)(V - diag(e^G) K S_b)
  U'  = Y + bf16(T - I) bf16(Y)  the identity part exact, the rest on bf16 operands
  O   = scale (diag(e^G) Q S_b + P U')   P, U' enter as hi/lo pairs (taken exact here)
  S  <- e^{G_C} S + K^T diag(e^{G_C - G}) U'   (hi/lo, taken exact)
Q, K, V are bf16 inputs and exact in fp64.
"""
import numpy as np
import torch

import oracle


def bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def chunk_fwd_bf16_model(Q, K, V, beta, g, C, scale, N=3, mask=True):
    """Q, K [B,H,T,dk], V [B,H,T,dv], beta, g [B,H,T] (fp64 arrays) -> (O, S)."""
    B, H, Tn, dk = K.shape
    dv = V.shape[-1]
    O = np.zeros((B, H, Tn, dv))
    S_all = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv))
            for c in range(Tn // C):
                sl = slice(c * C, (c + 1) * C)
                Kc, Qc, Vc, bc = K[b, h, sl], Q[b, h, sl], V[b, h, sl], beta[b, h, sl]
                G = np.cumsum(g[b, h, sl])
                A = oracle.build_A(Kc[None], bc[None], g[b, h, sl][None])
                TmI = oracle.neumann(A, N, mask)[0] - np.eye(C)
                Sb = bf16(S)
                Y = bc[:, None] * (Vc - np.exp(G)[:, None] * (Kc @ Sb))
                U = Y + bf16(TmI) @ bf16(Y)
                P = np.tril((Qc @ Kc.T) * np.exp(G[:, None] - G[None, :]))
                O[b, h, sl] = scale * (np.exp(G)[:, None] * (Qc @ Sb) + P @ U)
                S = np.exp(G[-1]) * S + Kc.T @ (np.exp(G[-1] - G)[:, None] * U)
            S_all[b, h] = S
    return O, S_all
