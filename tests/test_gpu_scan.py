"""Parity of the segment-parallel forward (efla_chunk_fwd_scan, through the C ABI) with the fp64 oracle.

The method regroups the same recurrence (the state pass is affine in the state: over a segment
S_out = M S_in + S_out(0)), so its outputs and final state must match the token recurrence to the same
tolerance as the other forms: max |x - ref| / max |ref| per tensor below 1e-5 (fp32 inputs) or 2e-2 (bf16
inputs).  Cases cover segment counts that leave a short last segment, a ragged last chunk, initial states,
in-place state passing, every d_k path (the swizzled bf16 state pass for d_k >= 32, the generic one for fp32
and d_k = 16), the 128-column first pass of d_k = d_v = 128, and a Runge-Kutta gate.  The full-size long-context workload runs in test_gpu_parity.py."""
import os
import sys

import numpy as np
import pytest
import torch

import exact_flow_delta_amd as efla
import oracle
from exact_flow_delta_amd import workloads as W

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from gpu_helpers import TOL, errs, fwd_inputs_dev  # noqa: E402

pytestmark = pytest.mark.gpu


def _scan(x, dtype, chunk, segments, gate=0, inplace=False):
    d = fwd_inputs_dev(x, dtype)
    B, H, L, d_k = d["k"].shape
    d_v = d["v"].shape[-1]
    nseg, sc, sw, need = efla.scan_plan(B, H, L, d_k, d_v, chunk, d["v"].dtype, segments)
    ws = torch.full((max(1, need),), 0xFF, dtype=torch.uint8, device="cuda")   # NaN-filled: all of it is written first
    out = torch.full((B, H, L, d_v), float("nan"), dtype=d["v"].dtype, device="cuda")
    s0 = d["initial_state"]
    fs = s0 if (inplace and s0 is not None) else None
    o, S = efla.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], initial_state=s0, final_state=fs, chunk_size=chunk,
                          out=out, method="scan", segments=segments, workspace=ws, gate=gate)
    torch.cuda.synchronize()
    return o, S, nseg


def _check(x, dtype, o, S, gate=0):
    ro, rS, _ = oracle.fwd(x["q"], x["k"], x["v"], x["beta"], x["initial_state"], gate=gate)
    assert not torch.isnan(o).any()
    eo, eS = errs(o, S, ro, rS)
    assert eo < TOL[dtype] and eS < TOL[dtype], (eo, eS)


@pytest.mark.parametrize("segments", [2, 3, 5, 16])
def test_scan_tiny_fp32(segments):
    w = W.workload(1)
    x = W.make_fwd_inputs(w)
    o, S, nseg = _scan(x, "f32", w.chunk, segments)
    per = -(-16 // segments)            # 16 chunks: ceil(16 / segments) per segment, no empty segment
    assert nseg == -(-16 // per)
    _check(x, "f32", o, S)


@pytest.mark.parametrize("inplace", [False, True])
def test_scan_stiff_fp32_with_initial_state(inplace):
    w = W.workload(2, B=1, H=3, L=700)
    x = W.make_fwd_inputs(w)
    o, S, nseg = _scan(x, "f32", w.chunk, 4, inplace=inplace)
    assert nseg == 4
    _check(x, "f32", o, S)


@pytest.mark.parametrize("d_k,d_v,chunk", [(128, 128, 64), (64, 64, 32), (32, 64, 16), (16, 32, 32), (128, 64, 64)])
def test_scan_bf16_shapes(d_k, d_v, chunk):
    w = W.workload(2, B=1, H=3, L=17 * chunk + 5, d_k=d_k, d_v=d_v, chunk=chunk, dtype="bf16")
    x = W.make_fwd_inputs(w)
    o, S, nseg = _scan(x, "bf16", chunk, 4)
    assert nseg == 4
    _check(x, "bf16", o, S)


def test_scan_lm_heads_with_gate():
    w = W.workload(6, B=1, H=4, L=1500, d_k=128, d_v=128, chunk=64, dtype="bf16")
    x = W.make_fwd_inputs(w)
    o, S, nseg = _scan(x, "bf16", 64, 6, gate=3)
    assert nseg == 6
    _check(x, "bf16", o, S, gate=3)


def test_scan_wide_first_pass():
    # 16 heads x 8 segments of 3 chunks (the last chunk ragged): at d_k = d_v = 128 the first pass then takes
    # 128-column slabs (eight compute waves sharing each chunk's K and Ta), the second 64-column ones
    w = W.workload(4, H=16, L=24 * 64 - 27)
    x = W.make_fwd_inputs(w)
    o, S, nseg = _scan(x, "bf16", 64, 8)
    assert nseg == 8
    _check(x, "bf16", o, S)


def test_scan_automatic_segments_long_heads():
    w = W.workload(4, H=2, L=8192)
    x = W.make_fwd_inputs(w)
    o, S, nseg = _scan(x, "bf16", 64, 0)
    assert nseg > 1
    _check(x, "bf16", o, S)


def test_scan_one_segment_is_the_split_forward():
    w = W.workload(3, B=1, H=2, L=300)
    x = W.make_fwd_inputs(w)
    d = fwd_inputs_dev(x, "bf16")
    o1, S1 = efla.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], chunk_size=64, method="split")
    o2, S2, nseg = _scan(x, "bf16", 64, 1)
    assert nseg == 1
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_scan_empty_sequence_copies_state():
    w = W.workload(2, B=1, H=2, L=0)
    x = W.make_fwd_inputs(w)
    d = fwd_inputs_dev(x, "f32")
    S = torch.full((1, 2, 64, 64), float("nan"), device="cuda")
    efla.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], initial_state=d["initial_state"], final_state=S, chunk_size=64,
                   method="scan", segments=4)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(S.cpu().numpy(), x["initial_state"])
