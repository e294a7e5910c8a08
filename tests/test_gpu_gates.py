"""Parity of the gate variants with the fp64 oracle, through the C ABI: the delta rule's alpha = beta
(gate 1) and the p-th order Runge-Kutta coefficients, on the same kernels as the exact gate.

The oracle's gated coefficient is pinned on the CPU against one step of textbook Runge-Kutta methods
applied to the ODE itself (tests/test_oracle_pins.py, check_gate_rk_tableaus).  Inputs: workload 6
(keys of moderate norm, so that the explicit schemes are stable).  Gates as for the exact coefficient:
max |x - ref| / max |ref| per tensor below 1e-5 (fp32 inputs) or 2e-2 (bf16 inputs); alpha itself
elementwise relative 4e-6 (an fp32 Horner evaluation of at most 16 terms)."""
import os
import sys

import numpy as np
import pytest
import torch

import exact_flow_delta_amd as efla
import oracle
from exact_flow_delta_amd import workloads as W

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from gpu_helpers import TOL, dev, errs, fwd_inputs_dev, host, ut_dense  # noqa: E402

pytestmark = pytest.mark.gpu

GATES = [1, 2, 3, 4, 16]


def _inputs(dtype, **kw):
    w = W.workload(6, dtype=dtype, **kw)
    return w, W.make_fwd_inputs(w)


@pytest.mark.parametrize("gate", [0] + GATES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_alpha_gates(dtype, gate):
    w, x = _inputs(dtype)
    k = x["k"].reshape(-1, w.d_k).copy()
    beta = x["beta"].reshape(-1).copy()
    k[:7] = 0.0                                       # zero keys: every gate gives beta
    a = efla.alpha(dev(k, dtype), torch.from_numpy(beta).cuda(), gate=gate)
    torch.cuda.synchronize()
    ref = oracle.alpha(k, beta, gate=gate)
    got = host(a)
    assert np.all(np.abs(got - ref) <= 4e-6 * np.abs(ref) + 1e-30), (dtype, gate)
    if gate == 1:
        np.testing.assert_array_equal(got, beta.astype(np.float64))


@pytest.mark.parametrize("method", ["split", "fused"])
@pytest.mark.parametrize("gate", GATES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk_fwd_gates(dtype, gate, method):
    w, x = _inputs(dtype)
    ro, rS, _ = oracle.fwd(x["q"], x["k"], x["v"], x["beta"], x["initial_state"], gate=gate)
    a = fwd_inputs_dev(x, dtype)
    o, S = efla.chunk_fwd(a["q"], a["k"], a["v"], a["beta"], initial_state=a["initial_state"],
                          chunk_size=w.chunk, method=method, gate=gate)
    torch.cuda.synchronize()
    eo, eS = errs(o, S, ro, rS)
    assert eo < TOL[dtype] and eS < TOL[dtype], (dtype, gate, method, eo, eS)


@pytest.mark.parametrize("method", ["auto", "split", "fused"])
@pytest.mark.parametrize("gate", GATES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk_fwd_gate_headline_shape(dtype, gate, method):
    """d_k = d_v = 128, chunk 64, a ragged length: for bf16 the one-launch kernel ("auto" and "fused"), whose UT
    waves form every gate's alpha, and the diagonal-block UT launch of the split form; for fp32 the split form."""
    w, x = _inputs(dtype, B=1, H=3, L=200, d_k=128, d_v=128, chunk=64)
    if dtype == "bf16" and method != "split":
        assert efla.fwd_form(w.B, w.H, w.L, 128, 128, 64, torch.bfloat16)[0] == "fused"
    ro, rS, _ = oracle.fwd(x["q"], x["k"], x["v"], x["beta"], x["initial_state"], gate=gate)
    a = fwd_inputs_dev(x, dtype)
    sf = torch.full((w.B, w.H, 128, 128), float("nan"), device="cuda")
    o, S = efla.chunk_fwd(a["q"], a["k"], a["v"], a["beta"], initial_state=a["initial_state"], chunk_size=64,
                          gate=gate, method=method, final_state=sf)
    torch.cuda.synchronize()
    eo, eS = errs(o, S, ro, rS)
    assert eo < TOL[dtype] and eS < TOL[dtype], (dtype, gate, method, eo, eS)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ut_transform_gate(dtype):
    w, x = _inputs(dtype, L=130)
    k = dev(x["k"], dtype)
    beta = torch.from_numpy(x["beta"]).cuda()
    for gate in (1, 3):
        t = efla.ut_transform(k, beta, chunk_size=w.chunk, gate=gate)
        torch.cuda.synchronize()
        got = ut_dense(t, w.chunk)
        ref = oracle.ut(x["k"], x["beta"], w.chunk, gate=gate)
        err = np.abs(got - ref).max() / np.abs(ref).max()
        assert err < TOL[dtype], (dtype, gate, err)


@pytest.mark.parametrize("gate", [1, 3])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_recurrent_step_gates(dtype, gate):
    """Eight decode steps per (batch, head) with the gate, from the workload's S0."""
    w, x = _inputs(dtype, L=8)
    NH = w.B * w.H
    S_ref = x["initial_state"].reshape(NH, w.d_k, w.d_v).astype(np.float64)
    S = torch.from_numpy(x["initial_state"].reshape(NH, w.d_k, w.d_v).copy()).cuda()
    for t in range(w.L):
        q, k, v = (x[n][:, :, t].reshape(NH, -1) for n in ("q", "k", "v"))
        b = x["beta"][:, :, t].reshape(NH)
        o = efla.recurrent_step(dev(q, dtype), dev(k, dtype), dev(v, dtype), torch.from_numpy(b.copy()).cuda(), S,
                                gate=gate)
        torch.cuda.synchronize()
        ro, S_ref, _ = oracle.step(q, k, v, b, S_ref, gate=gate)
        assert W.rel_max_err(host(o), ro) < TOL[dtype], (dtype, gate, t)
    assert W.rel_max_err(host(S), S_ref) < TOL[dtype]


@pytest.mark.parametrize("method", ["split", "fused"])
def test_exact_gate_is_the_default(method):
    w, x = _inputs("bf16", L=100)
    a = fwd_inputs_dev(x, "bf16")
    o0, S0 = efla.chunk_fwd(a["q"], a["k"], a["v"], a["beta"], initial_state=a["initial_state"], chunk_size=32,
                            method=method)
    o1, S1 = efla.chunk_fwd(a["q"], a["k"], a["v"], a["beta"], initial_state=a["initial_state"], chunk_size=32,
                            method=method, gate=efla.GATE_EXACT)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(S0, S1)
