"""The backward pass over strided views and packed sequences (efla_chunk_bwd_layout, through the C ABI).

A layout changes only where the kernels read and write, so over [B,L,H,d] views and slices of a fused
projection the gradients must equal efla_chunk_bwd's on contiguous copies bit for bit (that entry point is
held to the fp64 oracle in test_gpu_bwd.py; one case here is also checked against the oracle directly).
Packed sequences are checked one sequence at a time: against the oracle's gradients of that sequence alone
(max |x - ref| / max |ref| per tensor below 1e-5 for fp32 inputs, 2e-2 for bf16), and against a separate
efla_chunk_bwd call on that sequence, bit for bit.  Gradients of tokens outside every sequence stay unwritten,
and nothing outside a strided gradient's own elements is written.  Cases cover every backward kernel family:
the bf16 matrix-core state, state-gradient and per-chunk kernels (d_k >= 32, 64-token chunks), the bf16
per-chunk kernel with the generic state passes (32-token chunks), and the generic kernels (fp32, 16-token
chunks); packed batches with empty, one-token, chunk-edge and long sequences, a long mixed-length batch,
offsets that need clamping, and a Runge-Kutta gate."""
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

NAMES = ("dq", "dk", "dv", "dbeta", "d_initial")


def _bthd(x: np.ndarray, dtype: str) -> torch.Tensor:
    """[B,H,L,d] values stored as a [B,L,H,d] tensor; returns the [B,H,L,d] view of it."""
    return dev(np.ascontiguousarray(x.transpose(0, 2, 1, 3)), dtype).transpose(1, 2)


def _beta_bth(b: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(b.transpose(0, 2, 1))).cuda().transpose(1, 2)


def _cuda(a):
    return None if a is None else torch.from_numpy(a).cuda()


def _equal(got, ref):
    for name, a, r in zip(NAMES, got, ref):
        if r is None:
            assert a is None, name
            continue
        assert a.shape == r.shape, name
        assert torch.equal(a.contiguous(), r.contiguous()), (name, (a.float() - r.float()).abs().max().item())


def _oracle_check(got, ref, dtype):
    for name, a, r in zip(NAMES, got, ref):
        h = host(a)
        assert np.isfinite(h).all(), name
        e = W.rel_max_err(h, r)
        assert e < TOL[dtype], (name, e)


@pytest.mark.parametrize("cfg,dtype,d_k,d_v,chunk,L", [
    (3, "bf16", 128, 128, 64, 300), (2, "bf16", 64, 64, 32, 257), (6, "bf16", 32, 128, 16, 150),
    (2, "f32", 64, 32, 64, 130), (1, "f32", 16, 16, 16, 77)])
def test_bthd_views_equal_contiguous(cfg, dtype, d_k, d_v, chunk, L):
    w = W.workload(cfg, B=2, H=3, L=L, d_k=d_k, d_v=d_v, chunk=chunk, dtype=dtype)
    x = W.make_fwd_inputs(w)
    g = W.make_grads(w)
    s0, dsf = _cuda(x["initial_state"]), _cuda(g["d_final"])
    q, k, v, d_o = (_bthd(x[n] if n != "d_o" else g["d_o"], dtype) for n in ("q", "k", "v", "d_o"))
    beta = _beta_bth(x["beta"])
    got = efla.chunk_bwd_layout(q, k, v, beta, d_o, initial_state=s0, d_final=dsf, chunk_size=chunk)
    torch.cuda.synchronize()
    assert got[0].stride() == q.stride() and got[3].stride() == beta.stride()
    ref = efla.chunk_bwd(*(t.contiguous() for t in (q, k, v, beta, d_o)), initial_state=s0, d_final=dsf,
                         chunk_size=chunk)
    torch.cuda.synchronize()
    _equal(got, ref)
    if cfg == 3:
        _oracle_check(got, oracle.bwd(x["q"], x["k"], x["v"], x["beta"], x["initial_state"], g["d_o"],
                                      g["d_final"]), dtype)


def test_fused_projection_slices_write_only_their_elements():
    # q, k, v slices of one [B,L,3,H,d] projection; their gradients slices of a NaN-filled [B,L,3,H,d] buffer;
    # beta and dbeta slices of [B,L,H,2] buffers; d_o a [B,L,H,d] view
    B, H, L, d = 2, 4, 333, 128
    w = W.workload(3, B=B, H=H, L=L)
    x = W.make_fwd_inputs(w)
    g = W.make_grads(w)
    qkv = np.stack([x["q"], x["k"], x["v"]], axis=2)                       # [B,H,3,L,d]
    t = dev(np.ascontiguousarray(qkv.transpose(0, 3, 2, 1, 4)), "bf16")   # [B,L,3,H,d]
    q, k, v = (t[:, :, i].transpose(1, 2) for i in range(3))
    bb = np.zeros((B, L, H, 2), dtype=np.float32)
    bb[..., 1] = x["beta"].transpose(0, 2, 1)
    beta = torch.from_numpy(bb).cuda()[..., 1].transpose(1, 2)
    d_o = _bthd(g["d_o"], "bf16")
    gbuf = torch.full((B, L, 3, H, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    bbuf = torch.full((B, L, H, 2), float("nan"), dtype=torch.float32, device="cuda")
    grads = tuple(gbuf[:, :, i].transpose(1, 2) for i in range(3)) + (bbuf[..., 1].transpose(1, 2),)
    s0, dsf = _cuda(x["initial_state"]), _cuda(g["d_final"])
    got = efla.chunk_bwd_layout(q, k, v, beta, d_o, initial_state=s0, d_final=dsf, chunk_size=64, grads=grads)
    torch.cuda.synchronize()
    assert all(a.data_ptr() == b.data_ptr() for a, b in zip(got[:4], grads))
    ref = efla.chunk_bwd(*(a.contiguous() for a in (q, k, v, beta, d_o)), initial_state=s0, d_final=dsf,
                         chunk_size=64)
    torch.cuda.synchronize()
    _equal(got, ref)
    assert not torch.isnan(gbuf).any()              # dq, dk, dv fill the three slices exactly
    assert torch.isnan(bbuf[..., 0]).all()          # the other half of the beta buffer is untouched


def _sanitised(cu, T):
    """The offsets as efla.h defines their reading: each clamped to [0, T], then a running maximum."""
    out, m = [], 0
    for c in cu:
        m = max(m, min(max(int(c), 0), T))
        out.append(m)
    return out


def _packed_bwd(x, g, dtype, chunk, gate=0, bthd=False, cu_override=None):
    """efla_chunk_bwd_layout over the packed batch, gradients NaN-filled before the call."""
    if bthd:
        q, k, v, d_o = _bthd(x["q"], dtype), _bthd(x["k"], dtype), _bthd(x["v"], dtype), _bthd(g["d_o"], dtype)
        beta = _beta_bth(x["beta"])
    else:
        q, k, v, d_o = dev(x["q"], dtype), dev(x["k"], dtype), dev(x["v"], dtype), dev(g["d_o"], dtype)
        beta = torch.from_numpy(x["beta"]).cuda()
    cu = torch.from_numpy(x["cu_seqlens"] if cu_override is None else cu_override).cuda()
    grads = tuple(torch.empty_strided(t.shape, t.stride(), dtype=t.dtype, device="cuda").fill_(float("nan"))
                  for t in (q, k, v, beta))
    got = efla.chunk_bwd_layout(q, k, v, beta, d_o, cu_seqlens=cu, initial_state=_cuda(x["initial_state"]),
                                d_final=_cuda(g["d_final"]), chunk_size=chunk, gate=gate, grads=grads)
    torch.cuda.synchronize()
    return got


def _check_packed(x, g, dtype, chunk, got, cu, gate=0):
    """Each sequence against the oracle on that sequence alone and against a separate contiguous efla_chunk_bwd
    call, bit for bit; tokens outside every sequence stay NaN."""
    T = x["q"].shape[2]
    s0, dsf = x["initial_state"], g["d_final"]
    tok = _sanitised(cu, T)
    inside = np.zeros(T, dtype=bool)
    dq, dk, dv, db, ds0 = got
    for n in range(len(cu) - 1):
        t0, t1 = tok[n], tok[n + 1]
        sl = slice(t0, t1)
        inside[sl] = True
        init = None if s0 is None else s0[n:n + 1]
        fin = None if dsf is None else dsf[n:n + 1]
        seq = (dq[:, :, sl], dk[:, :, sl], dv[:, :, sl], db[:, :, sl], None if ds0 is None else ds0[n:n + 1])
        if t1 > t0:
            ref = efla.chunk_bwd(dev(x["q"][:, :, sl], dtype), dev(x["k"][:, :, sl], dtype),
                                 dev(x["v"][:, :, sl], dtype), torch.from_numpy(np.ascontiguousarray(
                                     x["beta"][:, :, sl])).cuda(), dev(g["d_o"][:, :, sl], dtype),
                                 initial_state=_cuda(init), d_final=_cuda(fin), chunk_size=chunk, gate=gate,
                                 want_initial_grad=ds0 is not None)
            torch.cuda.synchronize()
            _equal(seq, ref)
        r = oracle.bwd(x["q"][:, :, sl], x["k"][:, :, sl], x["v"][:, :, sl], x["beta"][:, :, sl], init,
                       g["d_o"][:, :, sl], fin, gate=gate)
        for name, a, rr in zip(NAMES, seq, r):
            if a is None or (t1 == t0 and name != "d_initial"):
                continue
            e = W.rel_max_err(host(a), rr)
            assert e < TOL[dtype], (n, t0, t1, name, e)
    out = ~inside
    for name, a in zip(NAMES[:4], got[:4]):
        h = host(a)
        assert np.isfinite(h[:, :, inside]).all(), name
        assert np.isnan(h[:, :, out]).all(), name


def _packed_case(cfg, H, d_k, d_v, chunk, dtype, lengths, with_s0=True, with_dsf=True):
    w = W.workload(cfg, H=H, d_k=d_k, d_v=d_v, chunk=chunk, dtype=dtype)
    x = W.make_packed_inputs(w, lengths)
    if not with_s0:
        x["initial_state"] = None
    T, N = int(sum(lengths)), len(lengths)
    g = dict(d_o=W.make_grads(replace(w, B=1, L=T))["d_o"],
             d_final=W.make_grads(replace(w, B=N, L=1))["d_final"] if with_dsf else None)
    return x, g


@pytest.mark.parametrize("dtype,d_k,chunk", [("bf16", 128, 64), ("bf16", 64, 32), ("f32", 64, 32), ("f32", 16, 16)])
def test_packed_edge_lengths(dtype, d_k, chunk):
    lengths = [0, 1, chunk - 1, chunk, chunk + 1, 0, 3 * chunk + 5, 2, 0]
    x, g = _packed_case(2, 3, d_k, d_k, chunk, dtype, lengths)
    got = _packed_bwd(x, g, dtype, chunk)
    _check_packed(x, g, dtype, chunk, got, x["cu_seqlens"])


def test_packed_lm_mix_bthd():
    # 40 sequences of a log-normal length mix (mean 300 tokens) as [1,T,H,d] views with per-sequence states
    lengths = W.packed_lengths(3, 40, 300.0)
    x, g = _packed_case(2, 4, 128, 128, 64, "bf16", lengths)
    got = _packed_bwd(x, g, "bf16", 64, bthd=True)
    _check_packed(x, g, "bf16", 64, got, x["cu_seqlens"])


def test_packed_gate_without_states():
    # keys of moderate norm (the "gates" workload), where the explicit Runge-Kutta gates are stable; no initial
    # state (no d_initial) and no final-state gradient
    x, g = _packed_case(6, 2, 64, 64, 64, "bf16", [130, 0, 64, 1, 250], with_s0=False, with_dsf=False)
    got = _packed_bwd(x, g, "bf16", 64, gate=3)
    assert got[4] is not None
    _check_packed(x, g, "bf16", 64, got, x["cu_seqlens"], gate=3)


@pytest.mark.parametrize("dtype,chunk", [("f32", 32), ("bf16", 64)])
@pytest.mark.parametrize("cu", [[-5, 120, 90, 400], [0, 200, 0, 200], [50, 10, 70, 70]])
def test_packed_offsets_are_sanitised(cu, dtype, chunk):
    # offsets out of order and out of range: [-5,120,90,400] -> [0,120,120,200]; [0,200,0,200] -> one full
    # sequence and two empty ones; [50,10,70,70] -> [50,50,70,70], tokens 0..49 and 70..199 in no sequence
    x, g = _packed_case(2, 2, 64, 64, chunk, dtype, [100, 40, 60])
    cu = np.array(cu, dtype=np.int32)
    got = _packed_bwd(x, g, dtype, chunk, cu_override=cu)
    _check_packed(x, g, dtype, chunk, got, cu)
