"""Parity of the stand-alone UT transform (efla_ut_transform, through the C ABI) with the fp64 oracle's
T diag(alpha), T = (I + strict_lower(diag(alpha) K K^T))^{-1}, per chunk, and of the workspace the
two-launch forward leaves behind.

Gate per chunk: max |x - ref| / max |ref| over the chunk's C x C block (the largest entry of T diag(alpha)
in a chunk sets its scale), below 1e-5 for fp32 inputs and 2e-2 for bf16 inputs (the bf16 build rounds
A's off-diagonal blocks and the output to bf16, relative step 2^-8)."""
import os
import sys

import numpy as np
import pytest
import torch

import exact_flow_delta_amd as efla
import oracle
from exact_flow_delta_amd import workloads as W

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from gpu_helpers import TOL, dev, fwd_inputs_dev, host, ut_dense  # noqa: E402

pytestmark = pytest.mark.gpu


def _chunk_err(got, ref):
    num = np.abs(got - ref).reshape(*got.shape[:3], -1).max(-1)
    den = np.abs(ref).reshape(*ref.shape[:3], -1).max(-1)
    return float((num / np.maximum(den, 1e-300)).max())


def _ut_gpu(x, dtype, chunk):
    k = dev(x["k"], dtype)
    beta = torch.from_numpy(x["beta"]).cuda()
    B, H, L, _ = k.shape
    nb = (chunk // 16) * (chunk // 16 + 1) // 2
    out = torch.full((B, H, (L + chunk - 1) // chunk, nb, 64, 4), float("nan"), dtype=k.dtype, device="cuda")
    t = efla.ut_transform(k, beta, chunk_size=chunk, out=out)
    torch.cuda.synchronize()
    return t


@pytest.mark.parametrize("cfg", [1, 2])
def test_ut_transform_fp32_workloads(cfg):
    w = W.workload(cfg)
    x = W.make_fwd_inputs(w)
    got = ut_dense(_ut_gpu(x, "f32", w.chunk), w.chunk)
    ref = oracle.ut(x["k"], x["beta"], w.chunk)
    e = _chunk_err(got, ref)
    assert e < TOL["f32"], e


def test_ut_transform_lm_layer_full_size():
    w = W.workload(3)
    x = W.make_fwd_inputs(w)
    got = ut_dense(_ut_gpu(x, "bf16", w.chunk), w.chunk)
    ref = oracle.ut(x["k"], x["beta"], w.chunk)
    e = _chunk_err(got, ref)
    assert e < TOL["bf16"], e


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("d_k", [16, 32, 64, 128])
def test_ut_transform_sweep(d_k, chunk, dtype):
    w = W.workload(2 if dtype == "f32" else 3, B=2, H=3, L=3 * chunk + 7, d_k=d_k, d_v=16, dtype=dtype)
    x = W.make_fwd_inputs(w, salt=3 * d_k + chunk)
    got = ut_dense(_ut_gpu(x, dtype, chunk), chunk)
    ref = oracle.ut(x["k"], x["beta"], chunk)
    e = _chunk_err(got, ref)
    assert e < TOL[dtype], e
    # the padded rows and columns of the short last chunk are exactly zero
    n = w.L - (w.L // chunk) * chunk
    assert np.all(got[:, :, -1, n:, :] == 0) and np.all(got[:, :, -1, :, n:] == 0)


def test_ut_transform_zero_keys_and_zero_beta():
    """k = 0 gives alpha = beta and no coupling; beta = 0 gives a zero column (alpha = 0)."""
    w = W.workload(3, B=1, H=2, L=64)
    x = W.make_fwd_inputs(w)
    x["k"][0, 0, 5] = 0.0
    x["beta"][0, 1, 9] = 0.0
    got = ut_dense(_ut_gpu(x, "bf16", 64), 64)
    ref = oracle.ut(x["k"], x["beta"], 64)
    assert _chunk_err(got, ref) < TOL["bf16"]
    assert got[0, 0, 0, 5, 5] == pytest.approx(float(x["beta"][0, 0, 5]), rel=1e-2)
    assert np.all(got[0, 1, 0, :, 9] == 0)


# quads (row block, column block) of a 64-token chunk's Ta inside its two diagonal 32 x 32 blocks:
# (0,0) (1,0) (1,1) (2,2) (3,2) (3,3) at qi = rb (rb + 1) / 2 + kb
DIAG32_QUADS = [0, 1, 2, 5, 8, 9]


@pytest.mark.parametrize("dtype,d_k,chunk,diag_only", [("bf16", 128, 64, True), ("bf16", 64, 32, False),
                                                       ("bf16", 16, 64, False), ("f32", 64, 64, False)])
def test_split_workspace_holds_ut_output(dtype, d_k, chunk, diag_only):
    """The two-launch forward leaves the stand-alone UT output in its workspace, bit for bit.  With bf16
    inputs, d_k >= 32 and 64-token chunks the state pass steps each chunk as two 32-token halves and reads
    only the diagonal 32 x 32 blocks of Ta, so the forward forms only those (the other quads are unwritten)."""
    w = W.workload(3, B=2, H=3, L=200, d_k=d_k, d_v=d_k)
    x = W.make_fwd_inputs(w)
    d = fwd_inputs_dev(x, dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    nbytes = efla.split_workspace_size(2, 3, 200, chunk, tdt)
    ws = torch.zeros((nbytes,), dtype=torch.uint8, device="cuda")
    efla.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], workspace=ws, chunk_size=chunk, method="split")
    t = efla.ut_transform(d["k"], d["beta"], chunk_size=chunk)
    torch.cuda.synchronize()
    got = ws.view(tdt)[: t.numel()].view(t.shape)
    if diag_only:
        assert torch.equal(got[:, :, :, DIAG32_QUADS], t[:, :, :, DIAG32_QUADS])
        off = [qi for qi in range(t.shape[3]) if qi not in DIAG32_QUADS]
        assert torch.all(got[:, :, :, off] == 0)   # left as the zeros the test filled in
    else:
        assert torch.equal(got, t)


def test_split_equals_fused_closely():
    """Both forms round the same products to bf16 in different places; they agree to the bf16 gate."""
    w = W.workload(3, B=2, H=4, L=777)
    x = W.make_fwd_inputs(w)
    d = fwd_inputs_dev(x, "bf16")
    o1, S1 = efla.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], method="split")
    o2, S2 = efla.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], method="fused")
    torch.cuda.synchronize()
    assert W.rel_max_err(host(o1), host(o2)) < TOL["bf16"]
    assert W.rel_max_err(host(S1), host(S2)) < TOL["bf16"]


def test_state_pass_after_ut_transform_equals_split():
    """efla_ut_transform then efla_chunk_state_pass is bit-identical to the two-launch forward."""
    w = W.workload(3, B=2, H=3, L=333)
    x = W.make_fwd_inputs(w)
    d = fwd_inputs_dev(x, "bf16")
    s0 = torch.from_numpy((0.1 * np.random.default_rng(4).standard_normal((2, 3, 128, 128))).astype(np.float32)).cuda()
    o1, S1 = efla.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], initial_state=s0, method="split")
    t = efla.ut_transform(d["k"], d["beta"])
    o2, S2 = efla.state_pass(d["q"], d["k"], d["v"], t, initial_state=s0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


@pytest.mark.parametrize("dtype,d_k,chunk,L,expect", [
    ("bf16", 128, 64, 300, "fused"),    # the one-launch kernel's shapes
    ("bf16", 32, 64, 130, "fused"),
    ("bf16", 128, 32, 300, "split"),    # other chunk sizes: two launches
    ("bf16", 16, 64, 130, "split"),
    ("f32", 64, 64, 300, "split"),
])
def test_default_method_dispatch(dtype, d_k, chunk, L, expect):
    """efla_chunk_fwd (chunk_fwd with no method) picks the one-launch forward for bf16, d_k >= 32 and 64-token
    chunks and the two-launch one otherwise (many heads: no segments); the outputs are bit-identical to that
    method's."""
    w = W.workload(3, B=2, H=8, L=L, d_k=d_k, d_v=64, chunk=chunk, dtype=dtype)
    x = W.make_fwd_inputs(w)
    d = fwd_inputs_dev(x, dtype)
    assert efla.scan_plan(w.B, w.H, w.L, d_k, 64, chunk, d["v"].dtype)[0] == 1
    assert efla.fwd_form(w.B, w.H, w.L, d_k, 64, chunk, d["v"].dtype)[0] == expect
    o0, S0 = efla.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], initial_state=d["initial_state"], chunk_size=chunk)
    o1, S1 = efla.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], initial_state=d["initial_state"], chunk_size=chunk,
                            method=expect)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(S0, S1)
