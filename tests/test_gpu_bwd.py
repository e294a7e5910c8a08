"""Parity of the backward pass (efla_chunk_bwd, through the C ABI) with the fp64 oracle's gradients.

The oracle's gradients are the adjoint of the token recurrence, pinned by finite differences of the pinned
forward (tests/test_oracle_pins.py).  Each gradient -- dq, dk, dv, dbeta and the initial state's -- is gated
separately by max |x - ref| / max |ref| over the tensor, at the forward's bar: below 1e-5 for fp32 inputs and
2e-2 for bf16 inputs (the bf16 path also reads the forward's bf16 T diag(alpha) workspace).
Cases: every d_k path and chunk size, ragged last chunks, with and without the initial state and the
final-state gradient, stiff keys, the Runge-Kutta gates, and the full LM-layer shape checked on every head and
for determinism: a second call gives the same bits (no kernel accumulates with
atomics, so the sums' order never depends on timing).  Also the autograd wrapper against direct calls, over
[B,L,H,d] views (bit-identical to contiguous tensors) and over packed sequences (bit-identical to one call per
sequence)."""
import os
import sys
from dataclasses import replace

import numpy as np
import pytest
import torch

import exact_flow_delta_amd as efla
import oracle
from exact_flow_delta_amd import workloads as W

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from gpu_helpers import TOL, dev, host  # noqa: E402

pytestmark = pytest.mark.gpu


def _run(w, gate=0, with_s0=True, with_dsf=True, salt=0):
    x = W.make_fwd_inputs(w, salt)
    g = W.make_grads(w, salt)
    s0 = x["initial_state"] if with_s0 else None
    dsf = g["d_final"] if with_dsf else None
    q, k, v, d_o = (dev(a, w.dtype) for a in (x["q"], x["k"], x["v"], g["d_o"]))
    beta = torch.from_numpy(x["beta"]).cuda()
    s0_d = None if s0 is None else torch.from_numpy(s0).cuda()
    dsf_d = None if dsf is None else torch.from_numpy(dsf).cuda()
    dq, dk, dv, db, ds0 = efla.chunk_bwd(q, k, v, beta, d_o, initial_state=s0_d, d_final=dsf_d, chunk_size=w.chunk,
                                         gate=gate)
    torch.cuda.synchronize()
    ref = oracle.bwd(x["q"], x["k"], x["v"], x["beta"], s0, g["d_o"], dsf, gate=gate)
    return (dq, dk, dv, db, ds0), ref


def _check(got, ref, dtype):
    for name, a, r in zip(("dq", "dk", "dv", "dbeta", "d_initial"), got, ref):
        h = host(a)
        assert np.isfinite(h).all(), name
        e = W.rel_max_err(h, r)
        assert e < TOL[dtype], (name, e)


@pytest.mark.parametrize("cfg,dtype,d_k,d_v,chunk,L", [
    (1, "f32", 16, 16, 16, 77), (2, "f32", 64, 64, 64, 300), (2, "f32", 32, 64, 32, 130), (6, "f32", 64, 16, 16, 99),
    (2, "f32", 128, 32, 64, 200), (3, "bf16", 128, 128, 64, 300), (2, "bf16", 64, 64, 32, 257),
    (6, "bf16", 32, 128, 16, 150), (3, "bf16", 128, 32, 64, 203), (2, "bf16", 32, 32, 32, 161)])
def test_bwd_shapes(cfg, dtype, d_k, d_v, chunk, L):
    w = W.workload(cfg, B=1, H=2, L=L, d_k=d_k, d_v=d_v, chunk=chunk, dtype=dtype)
    got, ref = _run(w)
    _check(got, ref, dtype)


@pytest.mark.parametrize("with_s0,with_dsf", [(False, False), (False, True), (True, False)])
def test_bwd_optional_states(with_s0, with_dsf):
    w = W.workload(2, B=2, H=1, L=150, d_k=64, d_v=64, chunk=64, dtype="f32")
    got, ref = _run(w, with_s0=with_s0, with_dsf=with_dsf)
    _check(got, ref, "f32")


@pytest.mark.parametrize("gate", [1, 2, 3, 5])
def test_bwd_gates(gate):
    w = W.workload(6, B=1, H=2, L=300, d_k=64, d_v=64, chunk=32, dtype="f32")
    got, ref = _run(w, gate=gate)
    _check(got, ref, "f32")


def test_bwd_lm_layer_full_size_all_heads():
    # the full LM-layer shape (B8 H16 L4096 d128 bf16, the matrix-core kernels), every head against the oracle, and a
    # second call for determinism
    w = W.workload(3)
    x = W.make_fwd_inputs(w)
    g = W.make_grads(w)
    q, k, v, d_o = (dev(a, "bf16") for a in (x["q"], x["k"], x["v"], g["d_o"]))
    beta = torch.from_numpy(x["beta"]).cuda()
    dsf = torch.from_numpy(g["d_final"]).cuda()
    got = efla.chunk_bwd(q, k, v, beta, d_o, d_final=dsf, chunk_size=64)
    again = efla.chunk_bwd(q, k, v, beta, d_o, d_final=dsf, chunk_size=64)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv", "dbeta", "d_initial"), got, again):
        assert torch.equal(a, b), name
    del again, q, k, v, d_o
    ref = oracle.bwd(x["q"], x["k"], x["v"], x["beta"], None, g["d_o"], g["d_final"])
    _check(got, ref, "bf16")


def test_autograd_wrapper_matches_direct_calls():
    w = W.workload(2, B=1, H=2, L=200, d_k=64, d_v=64, chunk=64, dtype="f32")
    x = W.make_fwd_inputs(w)
    g = W.make_grads(w)
    q, k, v = (dev(a, "f32").requires_grad_() for a in (x["q"], x["k"], x["v"]))
    beta = torch.from_numpy(x["beta"]).cuda().requires_grad_()
    s0 = torch.from_numpy(x["initial_state"]).cuda().requires_grad_()
    d_o, dsf = dev(g["d_o"], "f32"), torch.from_numpy(g["d_final"]).cuda()
    o, sf = efla.efla_attention(q, k, v, beta, initial_state=s0)
    ((o * d_o).sum() + (sf * dsf).sum()).backward()
    dq, dk, dv, db, ds0 = efla.chunk_bwd(q.detach(), k.detach(), v.detach(), beta.detach(), d_o,
                                         initial_state=s0.detach(), d_final=dsf)
    torch.cuda.synchronize()
    for a, b in ((q.grad, dq), (k.grad, dk), (v.grad, dv), (beta.grad, db), (s0.grad, ds0)):
        assert torch.equal(a, b)


def test_autograd_wrapper_over_bthd_views():
    # q, k, v as [B,H,L,d] views of [B,L,H,d] leaves (a model layer's projections), beta of [B,L,H]: no copies, o
    # laid out like v, and every output and gradient bit-identical to the same op on contiguous tensors
    w = W.workload(3, B=2, H=4, L=300)
    x = W.make_fwd_inputs(w)
    g = W.make_grads(w)

    def leaves(bthd):
        ts = []
        for a in (x["q"], x["k"], x["v"]):
            t = dev(np.ascontiguousarray(a.transpose(0, 2, 1, 3)) if bthd else a, "bf16")
            ts.append(t.requires_grad_())
        b = x["beta"].transpose(0, 2, 1) if bthd else x["beta"]
        ts.append(torch.from_numpy(np.ascontiguousarray(b)).cuda().requires_grad_())
        return ts

    d_o, dsf = dev(g["d_o"], "bf16"), torch.from_numpy(g["d_final"]).cuda()
    lv = leaves(True)
    views = [t.transpose(1, 2) for t in lv]
    o, sf = efla.efla_attention(*views)
    assert o.stride() == views[2].stride()
    ((o.float() * d_o.float()).sum() + (sf * dsf).sum()).backward()
    lc = leaves(False)
    o2, sf2 = efla.efla_attention(*lc)
    ((o2.float() * d_o.float()).sum() + (sf2 * dsf).sum()).backward()
    torch.cuda.synchronize()
    assert torch.equal(o.contiguous(), o2) and torch.equal(sf, sf2)
    for a, b in zip(lv, lc):
        assert torch.equal(a.grad.transpose(1, 2).contiguous(), b.grad)


def test_autograd_wrapper_packed_sequences():
    # three packed sequences (one empty) with their own initial states: outputs, final states and gradients equal
    # those of one call per sequence
    lengths = [130, 0, 77]
    w = W.workload(2, H=2, d_k=64, d_v=64, chunk=64, dtype="bf16")
    x = W.make_packed_inputs(w, lengths)
    cu = torch.from_numpy(x["cu_seqlens"]).cuda()
    T = sum(lengths)
    d_o = dev(W.make_grads(replace(w, B=1, L=T))["d_o"], "bf16")

    def inputs(sl):
        ts = [dev(np.ascontiguousarray(x[n][:, :, sl]), "bf16").requires_grad_() for n in ("q", "k", "v")]
        ts.append(torch.from_numpy(np.ascontiguousarray(x["beta"][:, :, sl])).cuda().requires_grad_())
        return ts

    full = inputs(slice(0, T))
    s0 = torch.from_numpy(x["initial_state"]).cuda().requires_grad_()
    o, sf = efla.efla_attention(*full, initial_state=s0, cu_seqlens=cu)
    ((o.float() * d_o.float()).sum() + sf.sum()).backward()
    torch.cuda.synchronize()
    for n in range(len(lengths)):
        t0, t1 = int(x["cu_seqlens"][n]), int(x["cu_seqlens"][n + 1])
        part = inputs(slice(t0, t1))
        s0n = torch.from_numpy(np.ascontiguousarray(x["initial_state"][n:n + 1])).cuda().requires_grad_()
        if t1 > t0:
            on, sfn = efla.efla_attention(*part, initial_state=s0n)
            ((on.float() * d_o[:, :, t0:t1].float()).sum() + sfn.sum()).backward()
            torch.cuda.synchronize()
            assert torch.equal(o[:, :, t0:t1], on) and torch.equal(sf[n:n + 1], sfn)
            for a, b in zip(full, part):
                assert torch.equal(a.grad[:, :, t0:t1], b.grad)
            assert torch.equal(s0.grad[n:n + 1], s0n.grad)
        else:   # an empty sequence passes its state through: S_L = S_0, so dS_0 = dS_L = 1
            assert torch.equal(sf[n:n + 1], s0[n:n + 1].detach())
            assert torch.equal(s0.grad[n:n + 1], torch.ones_like(s0n))
