"""Parity of the forward over strided views and packed sequences (efla_chunk_fwd_layout, through the C ABI)
with the fp64 oracle.

The layouts change only where the kernels read and write, so the results must match the token recurrence to
the same bar as the contiguous forward: max |x - ref| / max |ref| per tensor below 1e-5 (fp32 inputs) or 2e-2
(bf16 inputs); with a contiguous layout they must equal efla_chunk_fwd's form for the sizes bit for bit.  Packed sequences are
checked one sequence at a time against the oracle run on that sequence alone from its own initial state.
Cases: [B,L,H,d] views, slices of a fused projection (token stride 3 H d, beta with a token stride),
segment-parallel runs over strided views, packed batches with empty, one-token, chunk-edge and long
sequences, a long mixed-length batch, offsets that need clamping, and each state-pass kernel (the swizzled
bf16 one for d_k >= 32, the generic one for fp32); bf16 with d_k >= 32 and 64-token chunks runs the one-launch
kernel (the UT transform inside the state pass's workgroups), whose strided and packed results must equal its
contiguous ones bit for bit."""
import os
import sys

import numpy as np
import pytest
import torch

import exact_flow_delta_amd as efla
import oracle
from exact_flow_delta_amd import workloads as W

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from gpu_helpers import TOL, dev, errs, host  # noqa: E402

pytestmark = pytest.mark.gpu


def _bthd(x: np.ndarray, dtype: str) -> torch.Tensor:
    """[B,H,L,d] values stored as a [B,L,H,d] tensor; returns the [B,H,L,d] view of it."""
    return dev(np.ascontiguousarray(x.transpose(0, 2, 1, 3)), dtype).transpose(1, 2)


def _beta_bth(b: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(b.transpose(0, 2, 1))).cuda().transpose(1, 2)


def _check(x, dtype, o, S, gate=0):
    ro, rS, _ = oracle.fwd(x["q"], x["k"], x["v"], x["beta"], x["initial_state"], gate=gate)
    assert not torch.isnan(o).any()
    eo, eS = errs(o, S, ro, rS)
    assert eo < TOL[dtype] and eS < TOL[dtype], (eo, eS)


def _s0(x):
    return None if x["initial_state"] is None else torch.from_numpy(x["initial_state"]).cuda()


@pytest.mark.parametrize("cfg,dtype,d_k,d_v,chunk,L", [
    (3, "bf16", 128, 128, 64, 1000), (2, "bf16", 64, 64, 32, 517), (2, "f32", 64, 32, 64, 300),
    (1, "f32", 16, 16, 16, 77), (6, "bf16", 32, 64, 16, 200)])
def test_bthd_views(cfg, dtype, d_k, d_v, chunk, L):
    w = W.workload(cfg, B=2, H=3, L=L, d_k=d_k, d_v=d_v, chunk=chunk, dtype=dtype)
    x = W.make_fwd_inputs(w)
    q, k, v = _bthd(x["q"], dtype), _bthd(x["k"], dtype), _bthd(x["v"], dtype)
    beta = _beta_bth(x["beta"])
    o, S = efla.chunk_fwd_layout(q, k, v, beta, initial_state=_s0(x), chunk_size=chunk)
    torch.cuda.synchronize()
    assert o.stride() == v.stride()          # o laid out like v: [B,L,H,d]
    _check(x, dtype, o, S)


def test_fused_projection_slices():
    # q, k, v as slices of one [B,L,3,H,d] projection; beta a slice of [B,L,H,2]; o into a [B,L,H,d] buffer
    w = W.workload(3, B=2, H=4, L=333)
    x = W.make_fwd_inputs(w)
    B, H, L, d = 2, 4, 333, 128
    qkv = np.stack([x["q"], x["k"], x["v"]], axis=2)            # [B,H,3,L,d]
    t = dev(np.ascontiguousarray(qkv.transpose(0, 3, 2, 1, 4)), "bf16")   # [B,L,3,H,d]
    q, k, v = (t[:, :, i].transpose(1, 2) for i in range(3))
    bb = np.zeros((B, L, H, 2), dtype=np.float32)
    bb[..., 1] = x["beta"].transpose(0, 2, 1)
    beta = torch.from_numpy(bb).cuda()[..., 1].transpose(1, 2)
    assert q.stride(2) == 3 * H * d and beta.stride(2) == 2 * H
    out = torch.full((B, L, H, d), float("nan"), dtype=torch.bfloat16, device="cuda").transpose(1, 2)
    o, S = efla.chunk_fwd_layout(q, k, v, beta, out=out, chunk_size=64)
    torch.cuda.synchronize()
    assert o.data_ptr() == out.data_ptr()
    _check(x, "bf16", o, S)


@pytest.mark.parametrize("dtype,d_k,chunk", [("bf16", 128, 64), ("f32", 64, 32)])
def test_strided_segments(dtype, d_k, chunk):
    w = W.workload(2, B=1, H=2, L=41 * chunk + 9, d_k=d_k, d_v=d_k, chunk=chunk, dtype=dtype)
    x = W.make_fwd_inputs(w)
    q, k, v = _bthd(x["q"], dtype), _bthd(x["k"], dtype), _bthd(x["v"], dtype)
    beta = _beta_bth(x["beta"])
    ns, need = efla.layout_plan(1, 2, w.L, d_k, d_k, chunk, q.dtype, segments=5)
    assert ns == 5
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    o, S = efla.chunk_fwd_layout(q, k, v, beta, initial_state=_s0(x), chunk_size=chunk, segments=5, workspace=ws)
    torch.cuda.synchronize()
    _check(x, dtype, o, S)


@pytest.mark.parametrize("chunk,method", [(64, "fused"), (32, "split")])
def test_contiguous_layout_equals_default(chunk, method):
    """With a contiguous layout the layout entry is efla_chunk_fwd's form for the sizes, bit for bit: the one-launch
    kernel for bf16 with 64-token chunks, the split form otherwise."""
    w = W.workload(3, B=2, H=4, L=700)
    x = W.make_fwd_inputs(w)
    d = {n: dev(x[n], "bf16") for n in ("q", "k", "v")}
    beta = torch.from_numpy(x["beta"]).cuda()
    o1, S1 = efla.chunk_fwd(d["q"], d["k"], d["v"], beta, method=method, chunk_size=chunk)
    o2, S2 = efla.chunk_fwd_layout(d["q"], d["k"], d["v"], beta, chunk_size=chunk)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


@pytest.mark.parametrize("gate", [0, 3])
def test_one_launch_bthd_equals_contiguous(gate):
    """[B,L,H,d] views through the one-launch kernel (bf16, d_k 128, 64-token chunks, a ragged length, an initial
    state): the same arithmetic as on contiguous copies, so the same bits; and the oracle's result."""
    w = W.workload(6 if gate else 3, B=2, H=3, L=333, d_k=128, d_v=128, chunk=64, dtype="bf16")
    x = W.make_fwd_inputs(w)
    if x["initial_state"] is None:
        x["initial_state"] = (0.1 * np.random.default_rng(5).standard_normal((2, 3, 128, 128))).astype(np.float32)
    q, k, v = _bthd(x["q"], "bf16"), _bthd(x["k"], "bf16"), _bthd(x["v"], "bf16")
    beta = _beta_bth(x["beta"])
    out = torch.full_like(v, float("nan"))
    sf = torch.full((2, 3, 128, 128), float("nan"), device="cuda")
    o1, S1 = efla.chunk_fwd_layout(q, k, v, beta, initial_state=_s0(x), chunk_size=64, gate=gate, out=out,
                                   final_state=sf)
    o2, S2 = efla.chunk_fwd(q.contiguous(), k.contiguous(), v.contiguous(), beta.contiguous(), initial_state=_s0(x),
                            chunk_size=64, gate=gate, method="fused")
    torch.cuda.synchronize()
    assert torch.equal(o1.contiguous(), o2) and torch.equal(S1, S2)
    _check(x, "bf16", o1, S1, gate=gate)


def test_one_launch_packed_gate_no_initial_state():
    # packed sequences through the one-launch kernel with a Runge-Kutta gate and no initial state
    lengths = [130, 0, 64, 1, 250, 63]
    w = W.workload(6, H=2, d_k=128, d_v=128, chunk=64, dtype="bf16")
    x = W.make_packed_inputs(w, lengths)
    x["initial_state"] = None
    o, S = _packed(x, "bf16", 64, gate=3)
    _check_packed(x, "bf16", o, S, x["cu_seqlens"], gate=3)


def _packed(x, dtype, chunk, gate=0, bthd=False, cu_override=None, out_nan=True):
    if bthd:
        q, k, v = _bthd(x["q"], dtype), _bthd(x["k"], dtype), _bthd(x["v"], dtype)
        beta = _beta_bth(x["beta"])
    else:
        q, k, v = dev(x["q"], dtype), dev(x["k"], dtype), dev(x["v"], dtype)
        beta = torch.from_numpy(x["beta"]).cuda()
    cu = torch.from_numpy(x["cu_seqlens"] if cu_override is None else cu_override).cuda()
    out = torch.empty_like(v)
    if out_nan:
        out.fill_(float("nan"))
    o, S = efla.chunk_fwd_layout(q, k, v, beta, cu_seqlens=cu, initial_state=_s0(x), chunk_size=chunk, gate=gate,
                                 out=out)
    torch.cuda.synchronize()
    return host(o), host(S)


def _sanitised(cu, T):
    """The offsets as efla.h defines their reading: each clamped to [0, T], then a running maximum."""
    out, m = [], 0
    for c in cu:
        m = max(m, min(max(int(c), 0), T))
        out.append(m)
    return out


def _check_packed(x, dtype, o, S, cu, gate=0):
    """Each sequence (offsets read as efla.h defines) against the oracle run on that sequence alone."""
    T = x["q"].shape[2]
    s0 = x["initial_state"]
    tok = _sanitised(cu, T)
    written = np.zeros(T, dtype=bool)
    for n in range(len(cu) - 1):
        t0, t1 = tok[n], tok[n + 1]
        sl = slice(t0, t1)
        init = None if s0 is None else s0[n:n + 1]
        ro, rS, _ = oracle.fwd(x["q"][:, :, sl], x["k"][:, :, sl], x["v"][:, :, sl], x["beta"][:, :, sl], init,
                               gate=gate)
        if t1 > t0:
            eo = W.rel_max_err(o[:, :, sl], ro)
            assert eo < TOL[dtype], (n, t0, t1, eo)
        eS = W.rel_max_err(S[n:n + 1], rS)
        assert eS < TOL[dtype], (n, t0, t1, eS)
        written[sl] = True
    return written


@pytest.mark.parametrize("dtype,d_k,chunk", [("bf16", 128, 64), ("bf16", 64, 32), ("f32", 64, 32), ("f32", 16, 16)])
def test_packed_edge_lengths(dtype, d_k, chunk):
    lengths = [0, 1, chunk - 1, chunk, chunk + 1, 0, 3 * chunk + 5, 2, 0]
    w = W.workload(2, H=3, d_k=d_k, d_v=d_k, chunk=chunk, dtype=dtype)
    x = W.make_packed_inputs(w, lengths)
    o, S = _packed(x, dtype, chunk)
    written = _check_packed(x, dtype, o, S, x["cu_seqlens"])
    assert written.all() and not np.isnan(o).any()


def test_packed_lm_mix_bthd():
    # 40 sequences of a log-normal length mix (mean 300 tokens) as a [1,T,H,d] tensor with per-sequence states
    lengths = W.packed_lengths(3, 40, 300.0)
    w = W.workload(2, H=4, d_k=128, d_v=128, chunk=64, dtype="bf16")
    x = W.make_packed_inputs(w, lengths)
    o, S = _packed(x, "bf16", 64, bthd=True)
    _check_packed(x, "bf16", o, S, x["cu_seqlens"])


def test_packed_gate_and_no_initial_state():
    # keys of moderate norm (the "gates" workload), where the explicit Runge-Kutta gates are stable
    lengths = [130, 0, 64, 1, 250]
    w = W.workload(6, H=2, d_k=64, d_v=64, chunk=32, dtype="bf16")
    x = W.make_packed_inputs(w, lengths)
    x["initial_state"] = None
    o, S = _packed(x, "bf16", 32, gate=2)
    _check_packed(x, "bf16", o, S, x["cu_seqlens"], gate=2)


@pytest.mark.parametrize("dtype,chunk", [("f32", 32), ("bf16", 64)])
@pytest.mark.parametrize("cu", [[-5, 120, 90, 400], [0, 200, 0, 200], [50, 10, 70, 70]])
def test_packed_offsets_are_sanitised(cu, dtype, chunk):
    # offsets out of order and out of range: [-5,120,90,400] -> [0,120,120,200]; [0,200,0,200] -> one full
    # sequence and two empty ones; [50,10,70,70] -> [50,50,70,70] (bf16 with 64-token chunks: the one-launch kernel)
    w = W.workload(2, H=2, d_k=64, d_v=64, chunk=chunk, dtype=dtype)
    x = W.make_packed_inputs(w, [100, 40, 60])
    cu = np.array(cu, dtype=np.int32)
    o, S = _packed(x, dtype, chunk, cu_override=cu, out_nan=False)
    _check_packed(x, dtype, o, S, cu)
