"""Seeded synthetic workloads for the EFLA chunked forward and decode step.

This module draws inputs only: it holds none of the operator's arithmetic, and both the HIP
path and the CPU oracle are fed from it.  Every tensor is drawn in float64 with numpy's PCG64
seeded by ``SeedSequence([config_id, tensor_id, step, salt])``, stored as float32, and -- for
bfloat16 workloads -- rounded to bfloat16 with round-to-nearest-even before either side sees
it, so that both sides read exactly the same values.

Tensor ids: 0=q, 1=k, 2=v, 3=beta, 4=key scale / mask, 5=value noise, 6=initial state, 7=packed lengths,
8=output gradient, 9=final-state gradient.

The five workloads (sizes, distributions) follow the targets this library is measured on:
  1 "tiny"          B1 H1 L256 d16 fp32, q,k,v ~ N(0,1), beta = sigmoid(N(0,1)), S0 = 0, chunk 16
  2 "stiff"         B4 H8 L2048 d64 fp32, q,v ~ N(0,1), k = u*s with u uniform on the unit sphere
                    and s log-uniform in [1e-3, 30], beta = sigmoid(1.5 N(0,1)), S0 = 0.1 N(0,1), chunk 64
  3 "lm_layer"      B8 H16 L4096 d128 bf16, q,v ~ N(0,1), k = z*s with s = exp(0.5 N(0,1)) per token,
                    beta = sigmoid(N(0,1)) fp32, S0 = 0, chunk 64
  4 "long_context"  B1 H16 L65536 d128 bf16, q ~ N(0,1), k = N(0,1) times 8 on a Bernoulli(0.1) mask
                    per (b, t) shared by all heads, v = N(0,1) + 0.5 N(0,1), beta = sigmoid(N(0,1)), chunk 64
  5 "decode"        256 sequences x 32 heads, d128, fp32 state S0 = 0.1 N(0,1); per step s: q,k,v bf16
                    N(0,1), beta = sigmoid(N(0,1)); 64 steps
  6 "gates"         B2 H2 L300 d64 fp32 (or bf16), q,v ~ N(0,1), k = u*s with u uniform on the unit sphere
                    and s uniform in [0.2, 1.3], beta = sigmoid(N(0,1)), S0 = 0.1 N(0,1), chunk 32: keys of
                    moderate norm (beta ||k||^2 < 1.7), where the explicit Runge-Kutta gates are stable

"N(0, s)" is read as a normal with standard deviation s.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

T_Q, T_K, T_V, T_BETA, T_SCALE, T_NOISE, T_S0, T_LEN, T_DO, T_DSF = range(10)


@dataclass(frozen=True)
class Workload:
    cfg_id: int
    name: str
    B: int
    H: int
    L: int
    d_k: int
    d_v: int
    dtype: str          # "f32" or "bf16": storage type of q, k, v and o
    chunk: int
    steps: int = 0      # decode workloads: number of steps (one token per sequence per step)

    @property
    def NH(self) -> int:
        return self.B * self.H


WORKLOADS = {
    1: Workload(1, "tiny", 1, 1, 256, 16, 16, "f32", 16),
    2: Workload(2, "stiff", 4, 8, 2048, 64, 64, "f32", 64),
    3: Workload(3, "lm_layer", 8, 16, 4096, 128, 128, "bf16", 64),
    4: Workload(4, "long_context", 1, 16, 65536, 128, 128, "bf16", 64),
    5: Workload(5, "decode", 256, 32, 1, 128, 128, "bf16", 64, steps=64),
    6: Workload(6, "gates", 2, 2, 300, 64, 64, "f32", 32),
}


def workload(cfg_id: int, **overrides) -> Workload:
    """The named workload, optionally with some sizes replaced (same distributions)."""
    return replace(WORKLOADS[cfg_id], **overrides)


def _rng(cfg_id: int, tensor_id: int, step: int = 0, salt: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg_id, tensor_id, step, salt])))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16 (ties to even), returned as float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) & np.uint32(0xFFFF0000)).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bfloat16-representable (as int16)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u >> 16).astype(np.uint16).view(np.int16)


def _sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z))


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    x = x.astype(np.float32)
    return round_bf16(x) if dtype == "bf16" else x


def make_fwd_inputs(w: Workload, salt: int = 0) -> dict:
    """Inputs of a chunked-forward workload: float32 numpy arrays (bf16-exact when dtype is bf16).

    Returns dict(q, k, v [B,H,L,d], beta [B,H,L], initial_state [B,H,d_k,d_v] or None).
    """
    B, H, L, dk, dv = w.B, w.H, w.L, w.d_k, w.d_v
    c = w.cfg_id
    q = _rng(c, T_Q, 0, salt).standard_normal((B, H, L, dk))
    beta_z = _rng(c, T_BETA, 0, salt).standard_normal((B, H, L))
    s0 = None
    if c == 2:
        g = _rng(c, T_K, 0, salt).standard_normal((B, H, L, dk))
        u = g / np.linalg.norm(g, axis=-1, keepdims=True)
        s = np.exp(_rng(c, T_SCALE, 0, salt).uniform(np.log(1e-3), np.log(30.0), (B, H, L, 1)))
        k = u * s
        v = _rng(c, T_V, 0, salt).standard_normal((B, H, L, dv))
        beta = _sigmoid(1.5 * beta_z)
        s0 = 0.1 * _rng(c, T_S0, 0, salt).standard_normal((B, H, dk, dv))
    elif c == 3:
        z = _rng(c, T_K, 0, salt).standard_normal((B, H, L, dk))
        s = np.exp(0.5 * _rng(c, T_SCALE, 0, salt).standard_normal((B, H, L, 1)))
        k = z * s
        v = _rng(c, T_V, 0, salt).standard_normal((B, H, L, dv))
        beta = _sigmoid(beta_z)
    elif c == 4:
        z = _rng(c, T_K, 0, salt).standard_normal((B, H, L, dk))
        m = _rng(c, T_SCALE, 0, salt).random((B, 1, L, 1)) < 0.1
        k = z * np.where(m, 8.0, 1.0)
        v = _rng(c, T_V, 0, salt).standard_normal((B, H, L, dv)) + \
            0.5 * _rng(c, T_NOISE, 0, salt).standard_normal((B, H, L, dv))
        beta = _sigmoid(beta_z)
    elif c == 6:
        g = _rng(c, T_K, 0, salt).standard_normal((B, H, L, dk))
        u = g / np.linalg.norm(g, axis=-1, keepdims=True)
        k = u * _rng(c, T_SCALE, 0, salt).uniform(0.2, 1.3, (B, H, L, 1))
        v = _rng(c, T_V, 0, salt).standard_normal((B, H, L, dv))
        beta = _sigmoid(beta_z)
        s0 = 0.1 * _rng(c, T_S0, 0, salt).standard_normal((B, H, dk, dv))
    else:  # 1 and any plain workload
        k = _rng(c, T_K, 0, salt).standard_normal((B, H, L, dk))
        v = _rng(c, T_V, 0, salt).standard_normal((B, H, L, dv))
        beta = _sigmoid(beta_z)
    return dict(q=_store(q, w.dtype), k=_store(k, w.dtype), v=_store(v, w.dtype),
                beta=beta.astype(np.float32),
                initial_state=None if s0 is None else s0.astype(np.float32))


def packed_lengths(cfg_id: int, n: int, mean: float, salt: int = 0) -> list:
    """n sequence lengths of a packed batch: round(exp(N(log(mean) - 1/2, 1))), a log-normal mix of mean
    about `mean` with many short and a few long sequences (zero lengths included when mean is small)."""
    z = _rng(cfg_id, T_LEN, 0, salt).standard_normal(n)
    return [int(x) for x in np.rint(np.exp(np.log(mean) - 0.5 + z))]


def make_packed_inputs(w: Workload, lengths, salt: int = 0) -> dict:
    """Packed sequences of workload w's distributions: q, k, v [1,H,T,d], beta [1,H,T] for T = sum(lengths)
    tokens drawn as one sequence of w, cu_seqlens [N+1] int32, and per-sequence initial states
    [N,H,d_k,d_v] = 0.1 N(0,1) (or None when w has none)."""
    lengths = [int(n) for n in lengths]
    T = int(sum(lengths))
    x = make_fwd_inputs(replace(w, B=1, L=T), salt)
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    s0 = None
    if x["initial_state"] is not None:
        s0 = (0.1 * _rng(w.cfg_id, T_S0, 1, salt).standard_normal((len(lengths), w.H, w.d_k, w.d_v))).astype(np.float32)
    x["initial_state"] = s0
    x["cu_seqlens"] = cu
    return x


def make_grads(w: Workload, salt: int = 0) -> dict:
    """Incoming gradients of a backward pass: d_o [B,H,L,d_v] ~ N(0,1) in w's storage type and d_final
    [B,H,d_k,d_v] ~ 0.1 N(0,1) fp32."""
    d_o = _rng(w.cfg_id, T_DO, 0, salt).standard_normal((w.B, w.H, w.L, w.d_v))
    dsf = 0.1 * _rng(w.cfg_id, T_DSF, 0, salt).standard_normal((w.B, w.H, w.d_k, w.d_v))
    return dict(d_o=_store(d_o, w.dtype), d_final=dsf.astype(np.float32))


def make_decode_state(w: Workload, salt: int = 0) -> np.ndarray:
    """Initial decode state [NH, d_k, d_v] float32, 0.1 N(0,1)."""
    return (0.1 * _rng(w.cfg_id, T_S0, 0, salt).standard_normal((w.NH, w.d_k, w.d_v))).astype(np.float32)


def make_decode_token(w: Workload, step: int, salt: int = 0) -> dict:
    """Inputs of decode step ``step``: q, k [NH,d_k], v [NH,d_v] (bf16-exact float32), beta [NH]."""
    c = w.cfg_id
    q = _rng(c, T_Q, step, salt).standard_normal((w.NH, w.d_k))
    k = _rng(c, T_K, step, salt).standard_normal((w.NH, w.d_k))
    v = _rng(c, T_V, step, salt).standard_normal((w.NH, w.d_v))
    beta = _sigmoid(_rng(c, T_BETA, step, salt).standard_normal(w.NH))
    return dict(q=_store(q, w.dtype), k=_store(k, w.dtype), v=_store(v, w.dtype),
                beta=beta.astype(np.float32))


def rel_max_err(x, ref) -> float:
    """max|x - ref| / max|ref| over a whole tensor (0 when both are empty or ref is all zero and x == ref)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    den = np.max(np.abs(ref))
    num = np.max(np.abs(x - ref))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)
