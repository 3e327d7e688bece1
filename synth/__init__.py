"""Seeded synthetic inputs shaped like one Gated DeltaNet layer.

This module draws random numbers and shapes them; it holds none of the method's
arithmetic (no A, no inverse, no products, no gate cumsum).  Both the GPU tests and
the oracle consume exactly the tensors produced here, so input rounding is never
counted as kernel error.

Recipe (numpy PCG64 ``default_rng(seed)``; draw order K, V, Q, beta, gate):
  * keys / queries: rows ~ N(0, 1) (float32 draws), L2-normalised per row in float64,
    then rounded to bf16 with round-to-nearest-even (torch's CPU cast);
  * values: N(0, 1), rounded to bf16;
  * beta: U(0, 1) ("uniform" family) or sigmoid(N(0, 1)) ("sigmoid" family), float32;
  * per-token log-gates gamma: log sigmoid(N(0, 1) + shift), float32 (shift 0 for the
    block workloads, +2 for the prefill workload).  The gate cumsum inside a chunk is
    the method's step and is left to the consumers.
"""
from __future__ import annotations

import numpy as np
import torch


def _log_sigmoid(x: np.ndarray) -> np.ndarray:
    # log(1 / (1 + e^-x)) = -log1p(e^-x), stable for both signs
    return np.where(x >= 0, -np.log1p(np.exp(-x)), x - np.log1p(np.exp(x)))


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def _unit_rows(rng: np.random.Generator, shape) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32).astype(np.float64)
    x /= np.linalg.norm(x, axis=-1, keepdims=True)
    return x


def _bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def blocks(seed: int, n_blocks: int, C: int = 64, d_k: int = 128, k_dtype: str = "bf16",
           d_v: int = 0):
    """Independent C x C blocks: K [n_blocks, C, d_k], beta, gamma [n_blocks, C].

    k_dtype: "bf16" (torch.bfloat16), "f32" (torch.float32) or "f64" (numpy float64,
    unrounded: the fp32-A correctness workload builds A from these in fp64).
    beta ~ U(0,1); gamma = log sigmoid(N(0,1)).  With d_v > 0 also V ~ N(0,1) bf16.
    """
    rng = np.random.default_rng(seed)
    K = _unit_rows(rng, (n_blocks, C, d_k))
    V = None
    if d_v:
        V = _bf16(rng.standard_normal(size=(n_blocks, C, d_v), dtype=np.float32))
    beta = rng.random(size=(n_blocks, C)).astype(np.float32)
    gamma = _log_sigmoid(rng.standard_normal(size=(n_blocks, C))).astype(np.float32)
    if k_dtype == "bf16":
        Kt = _bf16(K)
    elif k_dtype == "f32":
        Kt = torch.from_numpy(K.astype(np.float32))
    elif k_dtype == "f64":
        Kt = K
    else:
        raise ValueError(k_dtype)
    out = {"K": Kt, "beta": torch.from_numpy(beta), "g": torch.from_numpy(gamma)}
    if V is not None:
        out["V"] = V
    return out


def prefill(seed: int, B: int, H: int, T: int, d_k: int = 128, d_v: int = 128,
            family: str = "sigmoid"):
    """One GDN layer's prefill inputs, layout [B, H, T, d] (tokens of a head contiguous).

    family "sigmoid": beta = sigmoid(N(0,1)), gamma = log sigmoid(N(0,1) + 2)
    family "uniform": beta ~ U(0,1),          gamma = log sigmoid(N(0,1))
    Q, K unit rows (bf16), V ~ N(0,1) (bf16); beta, gamma float32.
    """
    rng = np.random.default_rng(seed)
    K = _bf16(_unit_rows(rng, (B, H, T, d_k)))
    V = _bf16(rng.standard_normal(size=(B, H, T, d_v), dtype=np.float32))
    Q = _bf16(_unit_rows(rng, (B, H, T, d_k)))
    if family == "sigmoid":
        beta = _sigmoid(rng.standard_normal(size=(B, H, T)))
        gamma = _log_sigmoid(rng.standard_normal(size=(B, H, T)) + 2.0)
    elif family == "uniform":
        beta = rng.random(size=(B, H, T))
        gamma = _log_sigmoid(rng.standard_normal(size=(B, H, T)))
    else:
        raise ValueError(family)
    return {"Q": Q, "K": K, "V": V,
            "beta": torch.from_numpy(beta.astype(np.float32)),
            "g": torch.from_numpy(gamma.astype(np.float32))}


def correlated_keys(n_blocks: int, C: int, d_k: int, rho: float):
    """Deterministic stress keys: k_i = sqrt(rho) e_0 + sqrt(1 - rho) e_{i+1}.

    Every pair of distinct keys has k_i . k_j = rho and |k_i| = 1 (needs d_k >= C + 1).
    beta = 1, gamma = 0.  Returned as float64 numpy (exact) and bf16 torch.
    """
    if d_k < C + 1:
        raise ValueError("correlated keys need d_k >= C + 1")
    K = np.zeros((n_blocks, C, d_k))
    K[:, :, 0] = np.sqrt(rho)
    for i in range(C):
        K[:, i, i + 1] = np.sqrt(1.0 - rho)
    beta = np.ones((n_blocks, C), dtype=np.float32)
    gamma = np.zeros((n_blocks, C), dtype=np.float32)
    return {"K64": K, "K": _bf16(K), "beta": torch.from_numpy(beta), "g": torch.from_numpy(gamma)}


def dyadic_keys(n_blocks: int, C: int, d_k: int, a: float, b: float, beta: float):
    """Deterministic keys exact in bf16: k_i = a e_0 + b e_{i+1} (a, b dyadic), so
    k_i . k_j = a^2 for i != j; beta constant, gamma = 0.  Needs d_k >= C + 1."""
    if d_k < C + 1:
        raise ValueError("dyadic keys need d_k >= C + 1")
    K = np.zeros((n_blocks, C, d_k), dtype=np.float32)
    K[:, :, 0] = a
    for i in range(C):
        K[:, i, i + 1] = b
    return {"K": _bf16(K), "beta": torch.full((n_blocks, C), float(beta)),
            "g": torch.zeros((n_blocks, C))}


def dyadic_prefill(seed: int, B: int, H: int, T: int, C: int, d_k: int, d_v: int,
                   a: float, b: float, beta: float):
    """Prefill inputs whose keys repeat the dyadic pattern of dyadic_keys in every chunk
    (position r of a chunk: a e_0 + b e_{r+1}), beta constant, gamma = 0; Q unit rows
    and V ~ N(0, 1) drawn as in prefill (bf16)."""
    rng = np.random.default_rng(seed)
    kb = dyadic_keys(1, C, d_k, a, b, beta)["K"][0]
    K = kb.repeat(T // C, 1).expand(B, H, T, d_k).contiguous()
    V = _bf16(rng.standard_normal(size=(B, H, T, d_v), dtype=np.float32))
    Q = _bf16(_unit_rows(rng, (B, H, T, d_k)))
    return {"Q": Q, "K": K, "V": V, "beta": torch.full((B, H, T), float(beta)),
            "g": torch.zeros((B, H, T))}
