"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle, element by element on the
same seeded inputs.  Gate: relative max error max|x - ref| / max|ref| per tensor, 1e-5 for fp32
inputs and 2e-2 for bf16 inputs, on the outputs and on the final state separately."""
import os
import sys

import numpy as np
import pytest
import torch

import exact_flow_delta_amd as efla
import oracle
from exact_flow_delta_amd import workloads as W

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from gpu_helpers import TOL, dev, errs, fwd_inputs_dev, host  # noqa: E402

pytestmark = pytest.mark.gpu


METHODS = ["split", "fused"]


def _run_fwd(x, dtype, chunk, dv_slab=0, poison=True, method="split"):
    d = fwd_inputs_dev(x, dtype)
    B, H, L, d_k = d["k"].shape
    d_v = d["v"].shape[-1]
    out = torch.empty((B, H, L, d_v), dtype=d["v"].dtype, device="cuda")
    # NaN-filled outputs: every element of o and of the final state must be written
    sf = torch.empty((B, H, d_k, d_v), dtype=torch.float32, device="cuda")
    if poison:
        out.fill_(float("nan"))
        sf.fill_(float("nan"))
    ws = None
    if method == "split":
        # a NaN-filled workspace: every block the state pass reads must have been written by the UT launch
        ws = torch.full((max(1, efla.split_workspace_size(B, H, L, chunk, d["v"].dtype)),), 0xFF, dtype=torch.uint8,
                        device="cuda")
    elif method == "scan":
        need = efla.scan_plan(B, H, L, d_k, d_v, chunk, d["v"].dtype)[3]
        ws = torch.full((max(1, need),), 0xFF, dtype=torch.uint8, device="cuda")
    elif method == "auto":
        ws = torch.full((max(256, efla.fwd_workspace_size(B, H, L, d_k, d_v, chunk, d["v"].dtype)),), 0xFF,
                        dtype=torch.uint8, device="cuda")
    o, S = efla.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], initial_state=d["initial_state"], chunk_size=chunk,
                          dv_slab=dv_slab, out=out, final_state=sf, method=method, workspace=ws)
    torch.cuda.synchronize()
    return o, S


_ORACLE_CACHE = {}


def _oracle_full(cfg):
    """The oracle's outputs and final states of a whole workload (computed once per test session)."""
    if cfg not in _ORACLE_CACHE:
        w = W.workload(cfg)
        x = W.make_fwd_inputs(w)
        _ORACLE_CACHE.clear()
        _ORACLE_CACHE[cfg] = (w, x) + _oracle_fwd(x)
    return _ORACLE_CACHE[cfg]


def _oracle_fwd(x):
    ro, rS, _ = oracle.fwd(x["q"], x["k"], x["v"], x["beta"], x["initial_state"])
    return ro, rS


# ------------------------------------------------------------------------------------------------
# alpha
# ------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d_k", [16, 32, 64, 128])
def test_alpha(dtype, d_k):
    rng = np.random.default_rng(100 + d_k)
    n = 3001
    g = rng.standard_normal((n, d_k))
    scale = np.exp(rng.uniform(np.log(1e-4), np.log(40.0), (n, 1)))
    k = (g / np.linalg.norm(g, axis=-1, keepdims=True) * scale).astype(np.float32)
    k[:7] = 0.0                                  # lambda = 0 -> alpha = beta
    if dtype == "bf16":
        k = W.round_bf16(k)
    beta = rng.uniform(0, 1, n).astype(np.float32)
    beta[3] = 0.0
    a = host(efla.alpha(dev(k, dtype), torch.from_numpy(beta).cuda()))
    ref = oracle.alpha(k, beta)
    np.testing.assert_array_equal(a[:7], beta[:7].astype(np.float64))
    rel = np.abs(a - ref) / np.maximum(np.abs(ref), 1e-30)
    assert rel.max() < 2e-6, rel.max()


# ------------------------------------------------------------------------------------------------
# decode step
# ------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d_k,d_v", [(16, 16), (64, 32), (32, 128), (128, 128), (128, 16)])
def test_recurrent_step_multi(dtype, d_k, d_v):
    w = W.workload(5, B=7, H=3, d_k=d_k, d_v=d_v, dtype=dtype)
    S0 = W.make_decode_state(w)
    S = torch.from_numpy(S0.copy()).cuda()
    rS = S0.astype(np.float64)
    for step in range(6):
        t = W.make_decode_token(w, step, salt=d_k * 1000 + d_v)
        out = torch.full((w.NH, d_v), float("nan"), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32,
                         device="cuda")
        o = efla.recurrent_step(dev(t["q"], dtype), dev(t["k"], dtype), dev(t["v"], dtype),
                                torch.from_numpy(t["beta"]).cuda(), S, out=out)
        ro, rS, _ = oracle.step(t["q"], t["k"], t["v"], t["beta"], rS)
        torch.cuda.synchronize()
        eo = W.rel_max_err(host(o), ro)
        assert eo < TOL[dtype], (step, eo)
        eS = W.rel_max_err(host(S), rS)      # the state is fp32 in both paths
        assert eS < 1e-5, (step, eS)


def test_recurrent_step_headline_all_states():
    """256 sequences x 32 heads, d 128, 64 steps (the decode workload): every state and every step's output
    against the oracle; the output buffer is NaN-filled before each step."""
    w = W.workload(5)
    S0 = W.make_decode_state(w)
    S = torch.from_numpy(S0).cuda()
    rS = S0.astype(np.float64)
    o = torch.empty((w.NH, w.d_v), dtype=torch.bfloat16, device="cuda")
    for step in range(w.steps):
        t = W.make_decode_token(w, step)
        o.fill_(float("nan"))
        efla.recurrent_step(dev(t["q"], "bf16"), dev(t["k"], "bf16"), dev(t["v"], "bf16"),
                            torch.from_numpy(t["beta"]).cuda(), S, out=o)
        ro, rS, _ = oracle.step(t["q"], t["k"], t["v"], t["beta"], rS)
        eo = W.rel_max_err(host(o), ro)
        assert eo < TOL["bf16"], (step, eo)
    torch.cuda.synchronize()
    Sh = host(S)
    eS = W.rel_max_err(Sh, rS)
    assert eS < TOL["bf16"], eS
    # per state too: no state may hide behind the largest one
    per = np.abs(Sh - rS).reshape(w.NH, -1).max(axis=1) / np.abs(rS).reshape(w.NH, -1).max(axis=1)
    assert per.max() < TOL["bf16"], (int(per.argmax()), per.max())


# ------------------------------------------------------------------------------------------------
# chunked forward: the small workloads at full size
# ------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("method", METHODS)
def test_chunk_fwd_tiny_workload(method):
    w = W.workload(1)
    x = W.make_fwd_inputs(w)
    o, S = _run_fwd(x, w.dtype, w.chunk, method=method)
    eo, eS = errs(o, S, *_oracle_fwd(x))
    assert eo < TOL["f32"] and eS < TOL["f32"], (eo, eS)


@pytest.mark.parametrize("method", METHODS + ["scan", "auto"])
def test_chunk_fwd_stiff_workload(method):
    w = W.workload(2)
    x = W.make_fwd_inputs(w)
    o, S = _run_fwd(x, w.dtype, w.chunk, method=method)
    eo, eS = errs(o, S, *_oracle_fwd(x))
    assert eo < TOL["f32"] and eS < TOL["f32"], (eo, eS)


# ------------------------------------------------------------------------------------------------
# chunked forward: every (d_k, d_v, chunk, dtype) at sizes spanning several chunks and a ragged tail
# ------------------------------------------------------------------------------------------------
SWEEP = [(dk, dv, c, dt) for dt in ("f32", "bf16") for dk in (16, 32, 64, 128) for dv in (16, 64, 128)
         for c in (16, 32, 64)]


@pytest.mark.parametrize("method", METHODS)
@pytest.mark.parametrize("d_k,d_v,chunk,dtype", SWEEP)
def test_chunk_fwd_sweep(d_k, d_v, chunk, dtype, method):
    cfg = 2 if dtype == "f32" else 3
    w = W.workload(cfg, B=2, H=3, L=3 * chunk + 5, d_k=d_k, d_v=d_v, dtype=dtype)
    x = W.make_fwd_inputs(w, salt=d_k + 7 * d_v + 31 * chunk)
    if x["initial_state"] is None:
        x["initial_state"] = (0.1 * np.random.default_rng(d_k + d_v).standard_normal((2, 3, d_k, d_v))).astype(
            np.float32)
    else:
        x["initial_state"] = x["initial_state"][:, :, :d_k, :d_v].copy()
    o, S = _run_fwd(x, dtype, chunk, method=method)
    eo, eS = errs(o, S, *_oracle_fwd(x))
    assert eo < TOL[dtype] and eS < TOL[dtype], (eo, eS)


@pytest.mark.parametrize("method", METHODS)
@pytest.mark.parametrize("L", [1, 15, 16, 17, 63, 64, 65, 784])
def test_chunk_fwd_ragged_lengths(L, method):
    """Short and ragged sequences, including the 784-token d=64 shape of the pixel-sequence workload."""
    w = W.workload(2, B=1, H=9, L=L)
    x = W.make_fwd_inputs(w, salt=L)
    o, S = _run_fwd(x, "f32", 64, method=method)
    eo, eS = errs(o, S, *_oracle_fwd(x))
    assert eo < TOL["f32"] and eS < TOL["f32"], (eo, eS)


@pytest.mark.parametrize("method", METHODS)
@pytest.mark.parametrize("d_k,d_v", [(128, 128), (32, 64), (64, 16)])
@pytest.mark.parametrize("L", [1, 31, 32, 33, 63, 64, 65, 129, 200])
def test_chunk_fwd_ragged_lengths_bf16(L, d_k, d_v, method):
    """bf16 inputs with 64-token chunks at short and ragged lengths (with "fused" this is the one-launch kernel
    whose UT waves transform each 32-token half of a chunk: halves that are partly or wholly past the end), with
    an initial state."""
    w = W.workload(3, B=1, H=3, L=L, d_k=d_k, d_v=d_v)
    x = W.make_fwd_inputs(w, salt=L + d_k)
    x["initial_state"] = (0.1 * np.random.default_rng(L).standard_normal((1, 3, d_k, d_v))).astype(np.float32)
    o, S = _run_fwd(x, "bf16", 64, method=method)
    eo, eS = errs(o, S, *_oracle_fwd(x))
    assert eo < TOL["bf16"] and eS < TOL["bf16"], (eo, eS)


@pytest.mark.parametrize("method", METHODS)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])   # bf16, d_k 64, chunk 64: the one-launch kernel
def test_chunk_fwd_empty_sequence_copies_state(method, dtype):
    rng = np.random.default_rng(5)
    s0 = torch.from_numpy(rng.standard_normal((2, 3, 64, 32)).astype(np.float32)).cuda()
    e = torch.empty((2, 3, 0, 64), device="cuda", dtype=dtype)
    ev = torch.empty((2, 3, 0, 32), device="cuda", dtype=dtype)
    b = torch.empty((2, 3, 0), device="cuda")
    o, S = efla.chunk_fwd(e, e, ev, b, initial_state=s0, method=method)
    torch.cuda.synchronize()
    assert o.shape == (2, 3, 0, 32)
    assert torch.equal(S, s0)
    o, S = efla.chunk_fwd(e, e, ev, b, method=method)
    torch.cuda.synchronize()
    assert torch.count_nonzero(S) == 0


# ------------------------------------------------------------------------------------------------
# metamorphic properties
# ------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("method", METHODS)
def test_slab_split_is_bitwise_identical(method):
    """State columns are independent: every d_v split gives bit-identical results."""
    w = W.workload(3, B=1, H=5, L=300)
    x = W.make_fwd_inputs(w)
    res = [_run_fwd(x, "bf16", 64, dv_slab=s, method=method) for s in (16, 32, 64)]
    for o, S in res[1:]:
        assert torch.equal(o, res[0][0]) and torch.equal(S, res[0][1])


@pytest.mark.parametrize("method", METHODS)
def test_deterministic(method):
    w = W.workload(3, B=2, H=4, L=500)
    x = W.make_fwd_inputs(w)
    o1, S1 = _run_fwd(x, "bf16", 64, method=method)
    o2, S2 = _run_fwd(x, "bf16", 64, method=method)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


@pytest.mark.parametrize("method", METHODS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk_size_independence(dtype, method):
    w = W.workload(2 if dtype == "f32" else 3, B=1, H=4, L=200, d_k=64, d_v=64, dtype=dtype)
    x = W.make_fwd_inputs(w)
    ro, rS = _oracle_fwd(x)
    for c in (16, 32, 64):
        o, S = _run_fwd(x, dtype, c, method=method)
        eo, eS = errs(o, S, ro, rS)
        assert eo < TOL[dtype] and eS < TOL[dtype], (c, eo, eS)


@pytest.mark.parametrize("method", METHODS)
def test_state_chaining_bitwise_at_chunk_boundary(method):
    """fwd over [0, L) == fwd over [0, L1) then [L1, L) from its final state, when L1 is a chunk multiple."""
    w = W.workload(3, B=2, H=3, L=320)
    x = W.make_fwd_inputs(w)
    d = fwd_inputs_dev(x, "bf16")
    o, S = efla.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], method=method)
    L1 = 192
    o1, S1 = efla.chunk_fwd(d["q"][:, :, :L1].contiguous(), d["k"][:, :, :L1].contiguous(),
                            d["v"][:, :, :L1].contiguous(), d["beta"][:, :, :L1].contiguous(), method=method)
    o2, S2 = efla.chunk_fwd(d["q"][:, :, L1:].contiguous(), d["k"][:, :, L1:].contiguous(),
                            d["v"][:, :, L1:].contiguous(), d["beta"][:, :, L1:].contiguous(),
                            initial_state=S1, final_state=S1, method=method)      # in place
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([o1, o2], dim=2), o)
    assert torch.equal(S2, S)


def test_prefill_then_decode_matches_oracle():
    w = W.workload(3, B=2, H=4, L=150)
    x = W.make_fwd_inputs(w)
    d = fwd_inputs_dev(x, "bf16")
    Lp = 130
    o, S = efla.chunk_fwd(d["q"][:, :, :Lp].contiguous(), d["k"][:, :, :Lp].contiguous(),
                          d["v"][:, :, :Lp].contiguous(), d["beta"][:, :, :Lp].contiguous())
    outs = [o]
    for t in range(Lp, w.L):
        ot = efla.recurrent_step(d["q"][:, :, t].contiguous(), d["k"][:, :, t].contiguous(),
                                 d["v"][:, :, t].contiguous(), d["beta"][:, :, t].contiguous(), S)
        outs.append(ot.unsqueeze(2))
    torch.cuda.synchronize()
    ro, rS = _oracle_fwd(x)
    eo, eS = errs(torch.cat(outs, dim=2), S, ro, rS)
    assert eo < TOL["bf16"] and eS < TOL["bf16"], (eo, eS)


# ------------------------------------------------------------------------------------------------
# the headline workloads at full size, in the launch configuration the benchmark times
# ------------------------------------------------------------------------------------------------
def _sampled_heads(w, x, o, S, heads):
    B, H = w.B, w.H
    for (b, h) in heads:
        sl = lambda a: a[b:b + 1, h:h + 1]  # noqa: E731
        xs = dict(q=sl(x["q"]), k=sl(x["k"]), v=sl(x["v"]), beta=sl(x["beta"]),
                  initial_state=None if x["initial_state"] is None else sl(x["initial_state"]))
        ro, rS = _oracle_fwd(xs)
        eo = W.rel_max_err(host(o[b, h]), ro[0, 0])
        eS = W.rel_max_err(host(S[b, h]), rS[0, 0])
        assert eo < TOL[w.dtype] and eS < TOL[w.dtype], ((b, h), eo, eS)


def _all_heads(w, o, S, ro, rS):
    """Every (batch, head) of a full-size run against the oracle, gated per head and over the whole tensor."""
    oh, Sh = host(o), host(S)
    assert not np.isnan(oh).any() and not np.isnan(Sh).any()
    worst = 0.0
    for b in range(w.B):
        for h in range(w.H):
            eo = W.rel_max_err(oh[b, h], ro[b, h])
            eS = W.rel_max_err(Sh[b, h], rS[b, h])
            worst = max(worst, eo, eS)
            assert eo < TOL[w.dtype] and eS < TOL[w.dtype], ((b, h), eo, eS)
    assert W.rel_max_err(oh, ro) < TOL[w.dtype] and W.rel_max_err(Sh, rS) < TOL[w.dtype]
    return worst


@pytest.mark.parametrize("method", METHODS + ["auto"])
def test_lm_layer_workload_full_size_all_heads(method):
    w, x, ro, rS = _oracle_full(3)
    o, S = _run_fwd(x, "bf16", w.chunk, method=method)
    _all_heads(w, o, S, ro, rS)


@pytest.mark.parametrize("method", METHODS + ["scan", "auto"])
def test_long_context_workload_full_size_all_heads(method):
    w, x, ro, rS = _oracle_full(4)
    o, S = _run_fwd(x, "bf16", w.chunk, method=method)
    _all_heads(w, o, S, ro, rS)


def test_c_entry_picks_the_scan_on_long_context():
    """efla_chunk_fwd (the library's own choice) on the long-context shape is the segment-parallel form, bit for
    bit."""
    w = W.workload(4)
    assert efla.fwd_form(w.B, w.H, w.L, w.d_k, w.d_v, w.chunk, torch.bfloat16)[0] == "scan"
    x = W.make_fwd_inputs(w)
    o0, S0 = _run_fwd(x, "bf16", w.chunk, method="auto")
    o1, S1 = _run_fwd(x, "bf16", w.chunk, method="scan")
    assert torch.equal(o0, o1) and torch.equal(S0, S1)
