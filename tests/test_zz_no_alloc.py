"""efla_chunk_fwd_noalloc through the C ABI: the forward for callers that cannot allocate, whose workspace is the
library's fixed scratch array.  Its outputs must equal efla_chunk_fwd's (same forms and kernels, a workspace of
the caller's own) bit for bit, and the oracle's within the parity bar, on two calls in a row with the second one
smaller (the scratch keeps the first call's contents)."""
import ctypes
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

LIMIT = 128 << 20


def _lib():
    lib = efla.load_library()
    lib.efla_chunk_fwd_noalloc.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int] + [ctypes.c_void_p] * 3 + \
        [ctypes.c_int] * 7 + [ctypes.c_void_p]
    lib.efla_chunk_fwd_noalloc.restype = ctypes.c_int
    return lib


def _outputs(d):
    B, H, L, d_k = d["k"].shape
    d_v = d["v"].shape[-1]
    o = torch.full((B, H, L, d_v), float("nan"), dtype=d["v"].dtype, device="cuda")
    S = torch.full((B, H, d_k, d_v), float("nan"), dtype=torch.float32, device="cuda")
    return o, S


def _noalloc(lib, d, chunk, gate=0):
    B, H, L, d_k = d["k"].shape
    d_v = d["v"].shape[-1]
    o, S = _outputs(d)
    dt = efla.EFLA_BF16 if d["v"].dtype == torch.bfloat16 else efla.EFLA_F32
    s0 = d["initial_state"]
    before = torch.cuda.memory_allocated()
    st = lib.efla_chunk_fwd_noalloc(d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(), d["beta"].data_ptr(),
                                    dt, o.data_ptr(), None if s0 is None else s0.data_ptr(), S.data_ptr(),
                                    B, H, L, d_k, d_v, chunk, gate, torch.cuda.current_stream().cuda_stream)
    assert st == efla.EFLA_OK, lib.efla_status_string(st)
    assert torch.cuda.memory_allocated() == before
    torch.cuda.synchronize()
    return o, S


def _reference(d, chunk, gate=0):
    """efla_chunk_fwd (the library's choice of form) with a workspace of its own, NaN-filled."""
    B, H, L, d_k = d["k"].shape
    d_v = d["v"].shape[-1]
    o, S = _outputs(d)
    need = efla.fwd_workspace_size(B, H, L, d_k, d_v, chunk, d["v"].dtype)
    ws = torch.full((max(need, 256),), 0xFF, dtype=torch.uint8, device="cuda")
    efla.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], initial_state=d["initial_state"], chunk_size=chunk, out=o,
                   final_state=S, workspace=ws, gate=gate)
    torch.cuda.synchronize()
    return o, S, need


def _case(lib, w, sample_heads=None):
    x = W.make_fwd_inputs(w)
    d = fwd_inputs_dev(x, w.dtype)
    o, S = _noalloc(lib, d, w.chunk)
    ro_, rS_, need = _reference(d, w.chunk)
    assert 0 < need <= LIMIT or need == 0
    assert torch.equal(o, ro_) and torch.equal(S, rS_)
    if sample_heads is None:
        ro, rS, _ = oracle.fwd(x["q"], x["k"], x["v"], x["beta"], x["initial_state"])
        eo, eS = errs(o, S, ro, rS)
    else:
        eo = eS = 0.0
        for b, h in sample_heads:
            sl = lambda a: None if a is None else a[b:b + 1, h:h + 1]  # noqa: E731
            ro, rS, _ = oracle.fwd(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["beta"]), sl(x["initial_state"]))
            e1, e2 = errs(o[b:b + 1, h:h + 1], S[b:b + 1, h:h + 1], ro, rS)
            eo, eS = max(eo, e1), max(eS, e2)
    assert eo < TOL[w.dtype] and eS < TOL[w.dtype], (w, eo, eS)
    return need


def test_noalloc_fp32_scan_then_smaller_split():
    lib = _lib()
    w1 = W.workload(2)                                              # stiff fp32: the segment-parallel form
    assert efla.fwd_form(w1.B, w1.H, w1.L, w1.d_k, w1.d_v, w1.chunk, torch.float32)[0] == "scan"
    n1 = _case(lib, w1)
    w2 = W.workload(2, B=1, H=3, L=300, chunk=32)                   # smaller, the split form
    assert efla.fwd_form(w2.B, w2.H, w2.L, w2.d_k, w2.d_v, w2.chunk, torch.float32)[0] == "split"
    n2 = _case(lib, w2)
    assert 0 < n2 < n1


def test_noalloc_bf16_long_context_then_smaller():
    lib = _lib()
    w1 = W.workload(4)                                              # 16 heads x 65,536 tokens: the scan form
    assert efla.fwd_form(w1.B, w1.H, w1.L, w1.d_k, w1.d_v, w1.chunk, torch.bfloat16)[0] == "scan"
    n1 = _case(lib, w1, sample_heads=[(0, 0), (0, 9)])
    w2 = W.workload(3, B=2, H=4, L=333, chunk=32)                   # bf16, chunk 32: the split form
    n2 = _case(lib, w2)
    assert 0 < n2 < n1
    w3 = W.workload(3, B=2, H=4, L=333)                             # the one-launch form: no scratch
    assert _case(lib, w3) == 0
