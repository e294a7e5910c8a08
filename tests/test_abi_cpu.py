"""The C ABI on the host: the library loads, exports every declared symbol, and rejects bad arguments
before touching any device (no GPU needed).  Nothing here launches a kernel: calls either fail
argument checks, or -- only on a machine with no GPU -- reach the device check and report
EFLA_ERR_NO_DEVICE."""
import ctypes
import os
import re

import pytest
import torch

import exact_flow_delta_amd as efla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "efla.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, NO_DEVICE, HIP = range(6)
F32, BF16 = 0, 1

pytestmark = pytest.mark.skipif(not os.path.exists(efla.library_path()), reason="libefla.so not built")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:efla_status|const char\*|int|size_t)\s+(efla_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    return efla.load_library()


def _no_gpu():
    return torch.cuda.device_count() == 0


# fake, 16-byte-aligned, non-overlapping device addresses (never dereferenced by these tests)
def P(i):
    return ctypes.c_void_p(0x7F0000000000 + i * (1 << 32))


def test_exports_match_header(lib):
    names = _declared()
    assert {"efla_alpha", "efla_chunk_fwd", "efla_recurrent_step"} <= set(names)
    for n in names:
        assert hasattr(lib, n), "missing export " + n


def test_status_values_match_header(lib):
    # the numeric values are part of the ABI: read them from the header and from the library's strings
    text = open(HEADER).read()
    vals = dict((m.group(1), int(m.group(2))) for m in re.finditer(r"(EFLA_(?:OK|ERR_\w+))\s*=\s*(\d+)", text))
    assert vals == {"EFLA_OK": 0, "EFLA_ERR_INVALID_ARG": 1, "EFLA_ERR_UNSUPPORTED": 2, "EFLA_ERR_WORKSPACE": 3,
                    "EFLA_ERR_NO_DEVICE": 4, "EFLA_ERR_HIP": 5}
    for name, v in vals.items():
        assert lib.efla_status_string(v).decode().startswith(name)
    assert (efla.EFLA_OK, efla.EFLA_ERR_INVALID_ARG, efla.EFLA_ERR_UNSUPPORTED, efla.EFLA_ERR_WORKSPACE,
            efla.EFLA_ERR_NO_DEVICE, efla.EFLA_ERR_HIP) == (0, 1, 2, 3, 4, 5)


def test_status_strings_and_version(lib):
    for s in range(6):
        assert lib.efla_status_string(s).decode().startswith("EFLA")
    assert b"WORKSPACE" in lib.efla_status_string(WORKSPACE)
    assert lib.efla_status_string(99).decode().startswith("EFLA")
    assert lib.efla_version() >= 10000
    assert isinstance(lib.efla_last_error(), bytes)


def test_plan_default_slabs(lib):
    # headline forward: 128 heads x 2 slabs of 64 columns, 4 waves each
    wg, sw, lds = efla.chunk_plan(8, 16, 4096, 128, 128, 64, torch.bfloat16)
    assert (wg, sw) == (256, 64) and 0 < lds <= 160 * 1024
    # few heads: narrower slabs give more workgroups
    wg, sw, _ = efla.chunk_plan(1, 16, 65536, 128, 128, 64, torch.bfloat16)
    assert sw == 16 and wg == 128
    # explicit slab, grid padded to whole groups of 8 heads
    wg, sw, _ = efla.chunk_plan(1, 1, 256, 16, 16, 16, torch.float32, 16)
    assert (wg, sw) == (8, 16)
    # the fused kernel plans the same grid
    assert efla.chunk_plan(8, 16, 4096, 128, 128, 64, torch.bfloat16, method="fused")[:2] == (256, 64)
    # state pass: Q, K, V-slab rows padded by 4 fp32 elements, two buffers when they fit in 160 KiB
    wg, sw, lds = efla.chunk_plan(1, 2, 256, 128, 128, 64, torch.float32)
    assert sw == 16 and lds == 2 * 64 * (2 * 132 + 20) * 4
    wg, sw, lds = efla.chunk_plan(1, 2, 256, 128, 128, 64, torch.float32, dv_slab=64)
    assert sw == 64 and lds == 64 * (2 * 132 + 68) * 4


def test_plan_rejects_unsupported(lib):
    wg = ctypes.c_int()
    for args in [(1, 1, 8, 48, 64, 64, BF16, 0), (1, 1, 8, 64, 256, 64, BF16, 0), (1, 1, 8, 64, 64, 128, BF16, 0),
                 (1, 1, 8, 64, 64, 64, BF16, 48), (1, 1, 8, 64, 32, 64, BF16, 64)]:
        assert lib.efla_chunk_fwd_plan(*args, ctypes.byref(wg), None, None) == UNSUPPORTED, args
    assert lib.efla_chunk_fwd_plan(-1, 1, 8, 64, 64, 64, BF16, 0, None, None, None) == INVALID
    assert lib.efla_chunk_fwd_plan(1, 1, 8, 64, 64, 64, 7, 0, None, None, None) == INVALID
    assert lib.efla_chunk_fwd_plan(1, 1, 8, 128, 128, 64, F32, 0, None, None, None) == OK
    for sizes in [(16, 16, 16), (128, 128, 64), (64, 64, 64)]:
        for dt in (F32, BF16):
            assert lib.efla_chunk_fwd_plan(1, 1, 8, sizes[0], sizes[1], sizes[2], dt, 0, None, None, None) == OK


def _chunk(lib, **kw):
    a = dict(q=P(1), k=P(2), v=P(3), beta=P(4), dt=BF16, o=P(5), s0=None, sf=P(6), B=2, H=3, L=100, dk=64, dv=64,
             C=64, slab=0)
    a.update(kw)
    return lib.efla_chunk_fwd_slab(a["q"], a["k"], a["v"], a["beta"], a["dt"], a["o"], a["s0"], a["sf"], a["B"],
                                   a["H"], a["L"], a["dk"], a["dv"], a["C"], a["slab"], None)


def test_chunk_fwd_argument_errors(lib):
    assert _chunk(lib, q=None) == INVALID
    assert _chunk(lib, o=None) == INVALID
    assert _chunk(lib, beta=None) == INVALID
    assert _chunk(lib, k=ctypes.c_void_p(0x7F0000000008)) == INVALID      # misaligned
    assert _chunk(lib, sf=ctypes.c_void_p(0x7F0600000004)) == INVALID     # misaligned state
    assert _chunk(lib, L=-1) == INVALID
    assert _chunk(lib, dt=5) == INVALID
    assert _chunk(lib, dk=96) == UNSUPPORTED
    assert _chunk(lib, C=8) == UNSUPPORTED
    assert _chunk(lib, slab=32, dv=16) == UNSUPPORTED
    # o overlapping an input, the final state overlapping an input, partially overlapping states
    assert _chunk(lib, o=ctypes.c_void_p(0x7F0100000000 + 256)) == INVALID
    assert _chunk(lib, sf=P(3)) == INVALID
    assert _chunk(lib, s0=P(6), sf=ctypes.c_void_p(0x7F0600000000 + 1024)) == INVALID
    # empty problems are no-ops that need no device
    assert _chunk(lib, B=0) == OK
    assert _chunk(lib, L=0, sf=None, q=None, k=None, v=None, beta=None, o=None) == OK


@pytest.mark.skipif(not _no_gpu(), reason="needs a machine without a GPU")
def test_no_device_reported_after_valid_arguments(lib):
    assert _chunk(lib) == NO_DEVICE
    assert _chunk(lib, s0=P(6)) == NO_DEVICE           # in-place state passing is allowed
    assert lib.efla_recurrent_step(P(1), P(2), P(3), P(4), BF16, P(5), P(6), 8192, 128, 128, None) == NO_DEVICE
    assert lib.efla_alpha(P(1), BF16, P(2), P(3), 1000, 128, None) == NO_DEVICE
    assert b"no HIP device" in lib.efla_last_error()


def test_recurrent_step_argument_errors(lib):
    f = lib.efla_recurrent_step
    assert f(P(1), P(2), P(3), P(4), BF16, P(5), P(6), 0, 128, 128, None) == OK    # empty
    assert f(P(1), P(2), P(3), P(4), BF16, P(5), P(6), -1, 128, 128, None) == INVALID
    assert f(P(1), P(2), P(3), P(4), BF16, None, P(6), 8, 128, 128, None) == INVALID
    assert f(P(1), P(2), P(3), P(4), BF16, P(5), P(5), 8, 128, 128, None) == INVALID  # o aliases state
    assert f(P(1), P(2), P(3), P(4), BF16, P(5), P(6), 8, 100, 128, None) == UNSUPPORTED
    assert f(P(1), P(2), P(3), P(4), 3, P(5), P(6), 8, 128, 128, None) == INVALID
    assert f(P(1), P(2), P(3), P(4), BF16, ctypes.c_void_p(0x7F0500000008), P(6), 8, 128, 128, None) == INVALID


def test_alpha_argument_errors(lib):
    f = lib.efla_alpha
    assert f(P(1), BF16, P(2), P(3), 0, 128, None) == OK
    assert f(P(1), BF16, P(2), P(3), -5, 128, None) == INVALID
    assert f(None, BF16, P(2), P(3), 5, 128, None) == INVALID
    assert f(P(1), BF16, P(2), P(1), 5, 128, None) == INVALID     # alpha overlaps k
    assert f(P(1), BF16, P(2), P(3), 5, 20, None) == UNSUPPORTED


def test_binding_refuses_cpu_tensors():
    x = torch.zeros(1, 1, 16, 16)
    b = torch.zeros(1, 1, 16)
    with pytest.raises(ValueError, match="GPU tensor"):
        efla.chunk_fwd(x, x, x, b)
    with pytest.raises(ValueError, match="GPU tensor"):
        efla.recurrent_step(x[0, 0], x[0, 0], x[0, 0], b[0, 0], torch.zeros(16, 16, 16))
    with pytest.raises(ValueError, match="GPU tensor"):
        efla.alpha(x, b)


def test_workspace_size(lib):
    # per (batch, head) and chunk: (C/16)(C/16+1)/2 blocks of 256 elements
    assert efla.split_workspace_size(2, 3, 100, 64, torch.bfloat16) == 6 * 2 * 10 * 256 * 2
    assert efla.split_workspace_size(2, 3, 100, 16, torch.float32) == 6 * 7 * 1 * 256 * 4
    assert efla.split_workspace_size(8, 16, 4096, 64, torch.bfloat16) == 128 * 64 * 10 * 512
    assert efla.split_workspace_size(1, 1, 0, 32, torch.bfloat16) == 0
    n = ctypes.c_size_t()
    assert lib.efla_chunk_split_workspace_size(1, 1, 8, 48, BF16, ctypes.byref(n)) == UNSUPPORTED
    assert lib.efla_chunk_split_workspace_size(1, -1, 8, 64, BF16, ctypes.byref(n)) == INVALID
    assert lib.efla_chunk_split_workspace_size(1, 1, 8, 64, BF16, None) == INVALID


def _split(lib, **kw):
    a = dict(q=P(1), k=P(2), v=P(3), beta=P(4), dt=BF16, o=P(5), s0=None, sf=P(6), B=2, H=3, L=100, dk=64, dv=64,
             C=64, slab=0, ws=P(7), wsb=6 * 2 * 10 * 256 * 2)
    a.update(kw)
    return lib.efla_chunk_fwd_split(a["q"], a["k"], a["v"], a["beta"], a["dt"], a["o"], a["s0"], a["sf"], a["B"],
                                    a["H"], a["L"], a["dk"], a["dv"], a["C"], a["slab"], a["ws"], a["wsb"], None)


def test_split_argument_errors(lib):
    assert _split(lib, ws=None) == WORKSPACE
    assert _split(lib, wsb=6 * 2 * 10 * 256 * 2 - 1) == WORKSPACE
    assert _split(lib, ws=ctypes.c_void_p(0x7F0700000008)) == WORKSPACE           # misaligned
    assert _split(lib, ws=ctypes.c_void_p(0x7F0500000000 + 4096)) == INVALID     # inside o
    assert _split(lib, ws=P(6)) == INVALID                                        # is the final state
    assert _split(lib, q=None) == INVALID
    assert _split(lib, dk=96) == UNSUPPORTED
    assert _split(lib, slab=32, dv=16) == UNSUPPORTED
    assert _split(lib, B=0, ws=None, wsb=0) == OK
    assert _split(lib, L=0, sf=None, q=None, k=None, v=None, beta=None, o=None, ws=None, wsb=0) == OK


def test_ut_transform_argument_errors(lib):
    f = lib.efla_ut_transform
    need = 6 * 2 * 10 * 256 * 2
    assert f(P(1), P(2), BF16, P(3), need, 2, 3, 0, 64, 64, None) == OK          # empty
    assert f(P(1), P(2), BF16, P(3), need - 2, 2, 3, 100, 64, 64, None) == WORKSPACE
    assert f(P(1), P(2), BF16, None, need, 2, 3, 100, 64, 64, None) == WORKSPACE
    assert f(None, P(2), BF16, P(3), need, 2, 3, 100, 64, 64, None) == INVALID
    assert f(P(1), P(2), BF16, P(1), need, 2, 3, 100, 64, 64, None) == INVALID    # output overlaps k
    assert f(P(1), P(2), BF16, P(3), need, 2, 3, 100, 64, 48, None) == UNSUPPORTED
    assert f(P(1), P(2), BF16, P(3), need, 2, 3, 100, 20, 64, None) == UNSUPPORTED
    assert f(P(1), P(2), 9, P(3), need, 2, 3, 100, 64, 64, None) == INVALID


def test_state_pass_argument_errors(lib):
    f = lib.efla_chunk_state_pass
    need = 6 * 2 * 10 * 256 * 2

    def call(**kw):
        a = dict(q=P(1), k=P(2), v=P(3), t=P(7), tb=need, dt=BF16, o=P(5), s0=None, sf=P(6), L=100)
        a.update(kw)
        return f(a["q"], a["k"], a["v"], a["t"], a["tb"], a["dt"], a["o"], a["s0"], a["sf"], 2, 3, a["L"], 64, 64, 64,
                 0, None)

    assert call(t=None) == WORKSPACE
    assert call(tb=need - 1) == WORKSPACE
    assert call(t=P(5)) == INVALID                 # t overlaps o
    assert call(v=None) == INVALID
    assert call(dt=4) == INVALID
    assert call(L=0, q=None, k=None, v=None, o=None, t=None, tb=0, sf=None) == OK
    if _no_gpu():
        assert call() == NO_DEVICE


@pytest.mark.skipif(not _no_gpu(), reason="needs a machine without a GPU")
def test_split_no_device_after_valid_arguments(lib):
    assert _split(lib) == NO_DEVICE
    assert lib.efla_ut_transform(P(1), P(2), BF16, P(3), 6 * 2 * 10 * 256 * 2, 2, 3, 100, 64, 64, None) == NO_DEVICE


def _gated_calls(lib, gate):
    """Every *_gate entry point, with arguments that are valid apart from (possibly) the gate."""
    need = 6 * 2 * 10 * 256 * 2
    return {
        "alpha": lib.efla_alpha_gate(P(1), BF16, P(2), P(3), 5, 128, gate, None),
        "recurrent_step": lib.efla_recurrent_step_gate(P(1), P(2), P(3), P(4), BF16, P(5), P(6), 8, 128, 128, gate,
                                                       None),
        "ut_transform": lib.efla_ut_transform_gate(P(1), P(2), BF16, P(3), need, 2, 3, 100, 64, 64, gate, None),
        "chunk_fwd_split": lib.efla_chunk_fwd_split_gate(P(1), P(2), P(3), P(4), BF16, P(5), None, P(6), 2, 3, 100,
                                                         64, 64, 64, 0, gate, P(7), need, None),
        "chunk_fwd_slab": lib.efla_chunk_fwd_slab_gate(P(1), P(2), P(3), P(4), BF16, P(5), None, P(6), 2, 3, 100,
                                                       64, 64, 64, 0, gate, None),
    }


def test_gate_argument_errors(lib):
    for gate in (-1, efla.GATE_MAX_ORDER + 1, 1000):
        for name, st in _gated_calls(lib, gate).items():
            assert st == INVALID, (name, gate)


@pytest.mark.skipif(not _no_gpu(), reason="needs a machine without a GPU")
def test_every_gate_passes_argument_checks(lib):
    for gate in (efla.GATE_EXACT, efla.GATE_DELTANET, 2, 4, efla.GATE_MAX_ORDER):
        for name, st in _gated_calls(lib, gate).items():
            assert st == NO_DEVICE, (name, gate)


def test_scan_plan(lib):
    # long-context shape: 16 heads x 2 slabs per segment, eight segments of 128 chunks fill 256 workgroups
    assert efla.scan_plan(1, 16, 65536, 128, 128, 64, torch.bfloat16) == (8, 128, 64, 109051904)
    # many heads: one segment, i.e. the split forward and its workspace
    assert efla.scan_plan(8, 16, 4096, 128, 128, 64, torch.bfloat16) == (1, 64, 64, 41943040)
    # segments only while one segment's grid fills at most a quarter of the chip (64 workgroups): 32 heads x 2
    # slabs -> 4 segments; 64 heads x 2 slabs (128 workgroups) -> none, however long the sequences
    assert efla.scan_plan(2, 16, 16384, 128, 128, 64, torch.bfloat16)[:2] == (4, 64)
    assert efla.scan_plan(1, 32, 32768, 128, 128, 64, torch.bfloat16)[:2] == (4, 128)
    assert efla.scan_plan(4, 16, 8192, 128, 128, 64, torch.bfloat16)[:2] == (1, 128)
    assert efla.scan_plan(4, 16, 65536, 128, 128, 64, torch.bfloat16)[0] == 1
    # explicit counts: no empty segment; at most one per chunk; d_k = 16 narrows the slab
    assert efla.scan_plan(1, 1, 256, 16, 16, 16, torch.float32, 5)[:3] == (4, 4, 16)
    assert efla.scan_plan(1, 1, 100, 64, 64, 64, torch.float32, 9)[:2] == (2, 1)
    ns, sc, sw, nb = efla.scan_plan(2, 3, 1000, 64, 32, 32, torch.bfloat16, 4)
    assert (ns, sc, sw) == (4, 8, 32)
    ut = 6 * 32 * 3 * 256 * 2
    assert nb == ut + 6 * 4 * 64 * (32 + 64) * 4 + 6 * 4 * 64 * 32 * 4
    n = ctypes.c_int()
    assert lib.efla_chunk_scan_plan(1, 1, 8, 64, 64, 48, BF16, 0, ctypes.byref(n), None, None, None) == UNSUPPORTED
    assert lib.efla_chunk_scan_plan(1, 1, 8, 64, 64, 64, BF16, -1, ctypes.byref(n), None, None, None) == INVALID


def _scan_call(lib, **kw):
    a = dict(q=P(1), k=P(2), v=P(3), beta=P(4), dt=BF16, o=P(5), s0=None, sf=P(6), B=1, H=2, L=4096, dk=128, dv=128,
             C=64, seg=4, gate=0, ws=P(7), wsb=1 << 30)
    a.update(kw)
    return lib.efla_chunk_fwd_scan(a["q"], a["k"], a["v"], a["beta"], a["dt"], a["o"], a["s0"], a["sf"], a["B"], a["H"],
                                   a["L"], a["dk"], a["dv"], a["C"], a["seg"], a["gate"], a["ws"], a["wsb"], None)


def test_scan_argument_errors(lib):
    need = efla.scan_plan(1, 2, 4096, 128, 128, 64, torch.bfloat16, 4)[3]
    assert _scan_call(lib, ws=None) == WORKSPACE
    assert _scan_call(lib, wsb=need - 1) == WORKSPACE
    assert _scan_call(lib, ws=ctypes.c_void_p(0x7F0700000000 + 128)) == WORKSPACE   # not 256-byte aligned
    assert _scan_call(lib, ws=ctypes.c_void_p(0x7F0500000000 + 4096)) == INVALID    # inside o
    assert _scan_call(lib, seg=-2) == INVALID
    assert _scan_call(lib, gate=17) == INVALID
    assert _scan_call(lib, dk=96) == UNSUPPORTED
    assert _scan_call(lib, q=None) == INVALID
    assert _scan_call(lib, B=0, ws=None, wsb=0) == OK
    assert _scan_call(lib, L=0, sf=None, q=None, k=None, v=None, beta=None, o=None, ws=None, wsb=0) == OK


@pytest.mark.skipif(not _no_gpu(), reason="needs a machine without a GPU")
def test_scan_reaches_the_device_check(lib):
    assert _scan_call(lib) == NO_DEVICE
    assert _scan_call(lib, seg=0, s0=P(6)) == NO_DEVICE      # in-place state passing


def test_layout_plan(lib):
    # fixed-length sequences: the scan plan (split workspace and one segment when heads are many)
    assert efla.layout_plan(8, 16, 4096, 128, 128, 64, torch.bfloat16) == (1, 41943040)
    assert efla.layout_plan(1, 16, 65536, 128, 128, 64, torch.bfloat16) == (8, 109051904)
    assert efla.layout_plan(1, 16, 65536, 128, 128, 64, torch.bfloat16, segments=1) == (1, 16 * 1024 * 10 * 512)
    # packed sequences: 256-byte-rounded chunk offsets, then H * (ceil(T / C) + N) chunks of UT output
    ns, nb = efla.layout_plan(5, 3, 1000, 64, 64, 32, torch.float32, varlen=True)
    assert ns == 1
    assert nb == 256 + 3 * (32 + 5) * 3 * 256 * 4   # 2 x 6 offsets fit in 256 bytes
    n, b = ctypes.c_int(), ctypes.c_size_t()
    assert lib.efla_chunk_layout_plan(5, 3, 1000, 64, 64, 32, F32, 1, 2, ctypes.byref(n), ctypes.byref(b)) == UNSUPPORTED
    assert lib.efla_chunk_layout_plan(5, 3, 1000, 64, 64, 32, F32, 1, -1, ctypes.byref(n), ctypes.byref(b)) == INVALID
    assert lib.efla_chunk_layout_plan(5, 3, 1000, 96, 64, 32, F32, 0, 0, ctypes.byref(n), ctypes.byref(b)) == UNSUPPORTED


def _bthd(B, H, L, dk, dv):
    """efla_layout of [B,L,H,d] tensors (beta [B,L,H])."""
    lay = efla.Layout()
    lay.q[:] = [L * H * dk, dk, H * dk]
    lay.k[:] = [L * H * dk, dk, H * dk]
    lay.v[:] = [L * H * dv, dv, H * dv]
    lay.o[:] = [L * H * dv, dv, H * dv]
    lay.beta[:] = [L * H, 1, H]
    return lay


def _layout_call(lib, lay, **kw):
    a = dict(q=P(1), k=P(2), v=P(3), beta=P(4), dt=BF16, o=P(5), s0=None, sf=P(6), B=2, H=4, L=1000, dk=64, dv=64,
             C=64, seg=0, gate=0, ws=P(7), wsb=1 << 30)
    a.update(kw)
    return lib.efla_chunk_fwd_layout(a["q"], a["k"], a["v"], a["beta"], a["dt"], a["o"], a["s0"], a["sf"], a["B"],
                                     a["H"], a["L"], a["dk"], a["dv"], a["C"], a["seg"], a["gate"],
                                     None if lay is None else ctypes.byref(lay), a["ws"], a["wsb"], None)


def test_layout_argument_errors(lib):
    lay = _bthd(2, 4, 1000, 64, 64)
    assert _layout_call(lib, lay, ws=None) == WORKSPACE
    assert _layout_call(lib, lay, gate=-1) == INVALID
    bad = _bthd(2, 4, 1000, 64, 64)
    bad.q[2] = 4 * 64 + 4            # rows not 16-byte aligned in bf16
    assert _layout_call(lib, bad) == INVALID
    bad = _bthd(2, 4, 1000, 64, 64)
    bad.k[1] = -64
    assert _layout_call(lib, bad) == INVALID
    bad = _bthd(2, 4, 1000, 64, 64)
    bad.k[2] = 0                     # every token of k on one row: rows past a sequence's end would not read 0
    assert _layout_call(lib, bad) == INVALID
    bad = _bthd(2, 4, 1000, 64, 64)
    bad.beta[2] = 0
    assert _layout_call(lib, bad) == INVALID
    bad = _bthd(2, 4, 1000, 64, 64)
    bad.o[2] = 32                    # rows of o overlap one another
    assert _layout_call(lib, bad) == INVALID
    bad = _bthd(2, 4, 1000, 64, 64)
    bad.o[:] = [1000 * 4 * 64, 64, 64 * 2]   # heads and tokens interleave onto the same rows
    assert _layout_call(lib, bad) == INVALID
    bad = _bthd(2, 4, 1000, 64, 64)
    bad.v[2] = 1 << 28               # token stride beyond the 32-bit in-chunk offsets
    assert _layout_call(lib, bad) == INVALID
    # o inside q's extent (q spans 2 * 1000 * 4 * 64 bf16 elements)
    assert _layout_call(lib, lay, o=ctypes.c_void_p(0x7F0100000000 + 4096)) == INVALID
    # packed sequences: more than one segment is not built; cu_seqlens inside o
    cu = _bthd(1, 4, 1000, 64, 64)
    cu.cu_seqlens = 0x7F0800000000
    assert _layout_call(lib, cu, seg=2) == UNSUPPORTED
    cu.cu_seqlens = 0x7F0500000000 + 64
    assert _layout_call(lib, cu) == INVALID
    # nothing to do
    assert _layout_call(lib, lay, B=0, ws=None, wsb=0) == OK
    assert _layout_call(lib, lay, L=0, sf=None, q=None, k=None, v=None, beta=None, o=None, ws=None, wsb=0) == OK


@pytest.mark.skipif(not _no_gpu(), reason="needs a machine without a GPU")
def test_layout_reaches_the_device_check(lib):
    assert _layout_call(lib, _bthd(2, 4, 1000, 64, 64)) == NO_DEVICE
    assert _layout_call(lib, None) == NO_DEVICE
    cu = _bthd(1, 4, 1000, 64, 64)
    cu.cu_seqlens = 0x7F0800000000
    assert _layout_call(lib, cu, B=7) == NO_DEVICE
    # an empty packed batch still writes the final states (from the initial ones)
    assert _layout_call(lib, cu, B=7, L=0, q=None, k=None, v=None, beta=None, o=None) == NO_DEVICE


def test_bwd_workspace_size(lib):
    # UT output, then two blocks of B H ceil(L/C) d_k d_v states (each 256-byte rounded), then (bf16 with d_k >= 32,
    # chunk >= 32, d_v a multiple of 32: the matrix-core per-chunk kernel) T^T of every chunk in bf16; the states
    # are bf16 when all three passes run on the matrix cores (those sizes with 64-token chunks), else fp32
    nb = efla.chunk_bwd_workspace_size(8, 16, 4096, 128, 128, 64, torch.bfloat16)
    assert nb == 41943040 + 2 * 128 * 64 * 128 * 128 * 2 + 128 * 64 * 64 * 64 * 2
    nb = efla.chunk_bwd_workspace_size(8, 16, 4096, 128, 128, 32, torch.bfloat16)
    assert nb == 128 * 128 * 3 * 256 * 2 + 2 * 128 * 128 * 128 * 128 * 4 + 128 * 128 * 32 * 32 * 2
    nb = efla.chunk_bwd_workspace_size(1, 2, 64, 128, 16, 64, torch.bfloat16)   # d_v 16: generic per-chunk kernel
    assert nb == 2 * 10 * 256 * 2 + 2 * 256 * (-(-(2 * 128 * 16 * 4) // 256))
    nb = efla.chunk_bwd_workspace_size(1, 3, 100, 32, 16, 32, torch.float32)
    ut = 3 * 4 * 3 * 256 * 4
    st = -(-(3 * 4 * 32 * 16 * 4) // 256) * 256
    assert nb == ut + 2 * st
    n = ctypes.c_size_t()
    assert lib.efla_chunk_bwd_workspace_size(1, 1, 8, 96, 64, 64, BF16, ctypes.byref(n)) == UNSUPPORTED
    assert lib.efla_chunk_bwd_workspace_size(1, 1, 8, 64, 64, 48, BF16, ctypes.byref(n)) == UNSUPPORTED
    assert lib.efla_chunk_bwd_workspace_size(-1, 1, 8, 64, 64, 64, BF16, ctypes.byref(n)) == INVALID


def _bwd_call(lib, **kw):
    a = dict(q=P(1), k=P(2), v=P(3), beta=P(4), dt=BF16, s0=None, do=P(5), dsf=None, dq=P(6), dk=P(7), dv=P(8),
             db=P(9), ds0=P(10), B=1, H=2, L=1000, dk_=64, dv_=64, C=64, gate=0, ws=P(11), wsb=1 << 30)
    a.update(kw)
    return lib.efla_chunk_bwd(a["q"], a["k"], a["v"], a["beta"], a["dt"], a["s0"], a["do"], a["dsf"], a["dq"], a["dk"],
                              a["dv"], a["db"], a["ds0"], a["B"], a["H"], a["L"], a["dk_"], a["dv_"], a["C"], a["gate"],
                              a["ws"], a["wsb"], None)


def test_bwd_argument_errors(lib):
    need = efla.chunk_bwd_workspace_size(1, 2, 1000, 64, 64, 64, torch.bfloat16)
    assert _bwd_call(lib, ws=None) == WORKSPACE
    assert _bwd_call(lib, wsb=need - 1) == WORKSPACE
    assert _bwd_call(lib, ws=ctypes.c_void_p(0x7F0B00000000 + 128)) == WORKSPACE
    assert _bwd_call(lib, gate=17) == INVALID
    assert _bwd_call(lib, dk_=96) == UNSUPPORTED
    assert _bwd_call(lib, do=None) == INVALID
    assert _bwd_call(lib, dq=None) == INVALID
    assert _bwd_call(lib, dq=ctypes.c_void_p(0x7F0100000000 + 64)) == INVALID    # dq inside q
    assert _bwd_call(lib, dv=ctypes.c_void_p(0x7F0600000000 + 64)) == INVALID    # dv inside dq
    assert _bwd_call(lib, ws=ctypes.c_void_p(0x7F0300000000)) == INVALID         # workspace on v
    assert _bwd_call(lib, B=0, ws=None, wsb=0) == OK
    assert _bwd_call(lib, L=0, ds0=None, q=None, k=None, v=None, beta=None, do=None, dq=None, dk=None, dv=None,
                     db=None, ws=None, wsb=0) == OK


@pytest.mark.skipif(not _no_gpu(), reason="needs a machine without a GPU")
def test_bwd_reaches_the_device_check(lib):
    assert _bwd_call(lib) == NO_DEVICE
    assert _bwd_call(lib, s0=P(12), dsf=P(13), gate=3) == NO_DEVICE


def test_bwd_layout_workspace_size(lib):
    # without packed sequences the same bytes as efla_chunk_bwd's; with them the offsets ((B + 1) x 2 int32, then
    # ceil(L/C) + B int32, 256-byte rounded) first and H (ceil(L/C) + B) chunks in every later part
    for args in ((8, 16, 4096, 128, 128, 64, torch.bfloat16), (1, 3, 100, 32, 16, 32, torch.float32)):
        assert efla.chunk_bwd_layout_workspace_size(*args) == efla.chunk_bwd_workspace_size(*args)
    B, H, L, dk, dv, C = 5, 4, 1000, 128, 64, 64
    nu = H * (-(-L // C) + B)
    r = lambda n: -(-n // 256) * 256  # noqa: E731
    want = r((B + 1) * 8 + (-(-L // C) + B) * 4) + r(nu * 10 * 256 * 2) + 2 * r(nu * dk * dv * 2) + r(nu * C * C * 2)
    assert efla.chunk_bwd_layout_workspace_size(B, H, L, dk, dv, C, torch.bfloat16, varlen=True) == want
    n = ctypes.c_size_t()
    assert lib.efla_chunk_bwd_layout_workspace_size(1, 1, 8, 96, 64, 64, BF16, 1, ctypes.byref(n)) == UNSUPPORTED
    assert lib.efla_chunk_bwd_layout_workspace_size(1, -1, 8, 64, 64, 64, BF16, 1, ctypes.byref(n)) == INVALID
    assert lib.efla_chunk_bwd_layout_workspace_size(1, 1, 8, 64, 64, 64, BF16, 1, None) == INVALID


def _bwd_layout_call(lib, lay, **kw):
    a = dict(q=P(1), k=P(2), v=P(3), beta=P(4), dt=BF16, s0=None, do=P(5), dsf=None, dq=P(6), dk=P(7), dv=P(8),
             db=P(9), ds0=P(10), B=2, H=4, L=1000, dk_=64, dv_=64, C=64, gate=0, ws=P(11), wsb=1 << 30)
    a.update(kw)
    return lib.efla_chunk_bwd_layout(a["q"], a["k"], a["v"], a["beta"], a["dt"], a["s0"], a["do"], a["dsf"], a["dq"],
                                     a["dk"], a["dv"], a["db"], a["ds0"], a["B"], a["H"], a["L"], a["dk_"], a["dv_"],
                                     a["C"], a["gate"], None if lay is None else ctypes.byref(lay), a["ws"], a["wsb"],
                                     None)


def _fused(B, H, L, d):
    """efla_layout of q, k, v as slices of a [B,L,3,H,d] buffer, beta a slice of [B,L,H,2], d_o [B,L,H,d]."""
    lay = _bthd(B, H, L, d, d)
    for f in ("q", "k", "v"):
        getattr(lay, f)[:] = [L * 3 * H * d, d, 3 * H * d]
    lay.beta[:] = [L * H * 2, 2, 2 * H]
    return lay, 0x7F2000000000


def _fused_grads(base, step, shift=0):
    """dq, dk, dv at base + {0, 1, 2} * step (+ shift for dk) bytes; dbeta element 1 of each pair in its buffer."""
    return dict(dq=ctypes.c_void_p(base), dk=ctypes.c_void_p(base + step + shift), dv=ctypes.c_void_p(base + 2 * step),
                db=ctypes.c_void_p(0x7F3000000000 + 4))


def test_bwd_layout_argument_errors(lib):
    lay = _bthd(2, 4, 1000, 64, 64)
    need = efla.chunk_bwd_layout_workspace_size(2, 4, 1000, 64, 64, 64, torch.bfloat16)
    assert _bwd_layout_call(lib, lay, ws=None) == WORKSPACE
    assert _bwd_layout_call(lib, lay, wsb=need - 1) == WORKSPACE
    assert _bwd_layout_call(lib, lay, gate=17) == INVALID
    assert _bwd_layout_call(lib, lay, dk_=96) == UNSUPPORTED
    bad = _bthd(2, 4, 1000, 64, 64)
    bad.q[2] = 4 * 64 + 4            # rows not 16-byte aligned in bf16
    assert _bwd_layout_call(lib, bad) == INVALID
    bad = _bthd(2, 4, 1000, 64, 64)
    bad.v[2] = 32                    # rows of v, hence of dv, overlap one another
    assert _bwd_layout_call(lib, bad) == INVALID
    bad = _bthd(2, 4, 1000, 64, 64)
    bad.k[:] = [1000 * 4 * 64, 64, 64 * 2]   # heads and tokens of k (and dk) interleave onto the same rows
    assert _bwd_layout_call(lib, bad) == INVALID
    bad = _bthd(2, 4, 1000, 64, 64)
    bad.beta[:] = [1000 * 4, 1, 1]           # dbeta elements shared between heads and tokens
    assert _bwd_layout_call(lib, bad) == INVALID
    bad = _bthd(2, 4, 1000, 64, 64)
    bad.o[2] = 1 << 28               # d_o's token stride beyond the 32-bit in-chunk offsets
    assert _bwd_layout_call(lib, bad) == INVALID
    # d_o's rows may overlap (it is only read); a [B,L,H,d] q's extent is 2 * 1000 * 4 * 64 bf16 elements
    ok = _bthd(2, 4, 1000, 64, 64)
    ok.o[2] = 0
    assert _bwd_layout_call(lib, ok, ws=None) == WORKSPACE
    assert _bwd_layout_call(lib, lay, dq=ctypes.c_void_p(0x7F0100000000 + 4096)) == INVALID   # dq inside q
    assert _bwd_layout_call(lib, lay, dv=ctypes.c_void_p(0x7F0500000000 + 4096)) == INVALID   # dv inside d_o
    cu = _bthd(1, 4, 1000, 64, 64)
    cu.cu_seqlens = 0x7F0600000000 + 64                                                    # offsets inside dq
    assert _bwd_layout_call(lib, cu, B=3) == INVALID
    # gradients as slices of one fused [B,L,3,H,d] buffer (H d elements apart) interleave; dk shifted by one row
    # (d elements) overlaps dq's heads
    fz, base = _fused(2, 4, 1000, 64)
    assert _bwd_layout_call(lib, fz, **_fused_grads(base, 4 * 64 * 2), ws=None) == WORKSPACE
    assert _bwd_layout_call(lib, fz, **_fused_grads(base, 4 * 64 * 2, shift=64 * 2)) == INVALID
    assert _bwd_layout_call(lib, fz, **_fused_grads(base, 4 * 64 * 2, shift=3)) == INVALID   # not element-aligned
    assert _bwd_layout_call(lib, lay, B=0, ws=None, wsb=0) == OK
    assert _bwd_layout_call(lib, lay, L=0, ds0=None, q=None, k=None, v=None, beta=None, do=None, dq=None, dk=None,
                            dv=None, db=None, ws=None, wsb=0) == OK


@pytest.mark.skipif(not _no_gpu(), reason="needs a machine without a GPU")
def test_bwd_layout_reaches_the_device_check(lib):
    assert _bwd_layout_call(lib, _bthd(2, 4, 1000, 64, 64)) == NO_DEVICE
    assert _bwd_layout_call(lib, None) == NO_DEVICE
    cu = _bthd(1, 4, 1000, 64, 64)
    cu.cu_seqlens = 0x7F0C00000000
    assert _bwd_layout_call(lib, cu, B=7, s0=P(12), dsf=P(13), gate=3) == NO_DEVICE
    fz, base = _fused(2, 4, 1000, 64)
    assert _bwd_layout_call(lib, fz, **_fused_grads(base, 4 * 64 * 2)) == NO_DEVICE
    # an empty packed batch still writes d_initial (from d_final)
    assert _bwd_layout_call(lib, cu, B=7, L=0, q=None, k=None, v=None, beta=None, do=None, dq=None, dk=None, dv=None,
                            db=None) == NO_DEVICE


def _form(lib, B, H, L, dk, dv, C, dt):
    f, ns, nb = ctypes.c_int(-1), ctypes.c_int(-1), ctypes.c_size_t(7)
    st = lib.efla_chunk_fwd_form(B, H, L, dk, dv, C, dt, ctypes.byref(f), ctypes.byref(ns), ctypes.byref(nb))
    return st, f.value, ns.value, nb.value


def test_fwd_form_policy(lib):
    # the LM-layer shape: the one-launch kernel, no workspace
    assert _form(lib, 8, 16, 4096, 128, 128, 64, BF16) == (OK, efla.FWD_ONE_LAUNCH, 1, 0)
    assert lib.efla_chunk_fwd_workspace_size(8, 16, 4096, 128, 128, 64, BF16) == 0
    # 16 heads x 65,536 tokens: the segment-parallel form, with the scan plan's segments and workspace
    st, form, ns, nb = _form(lib, 1, 16, 65536, 128, 128, 64, BF16)
    assert (st, form) == (OK, efla.FWD_SCAN) and ns > 1
    n, b = ctypes.c_int(), ctypes.c_size_t()
    assert lib.efla_chunk_scan_plan(1, 16, 65536, 128, 128, 64, BF16, 0, ctypes.byref(n), None, None,
                                    ctypes.byref(b)) == OK
    assert (ns, nb) == (n.value, b.value)
    assert lib.efla_chunk_fwd_workspace_size(1, 16, 65536, 128, 128, 64, BF16) == b.value
    # fp32, and bf16 with chunks below 64 or d_k = 16: the split form, whose workspace is the UT output
    for args in [(1, 1, 256, 16, 16, 16, F32), (2, 3, 100, 64, 64, 32, BF16), (2, 3, 100, 16, 64, 64, BF16),
                 (8, 16, 300, 64, 64, 64, F32)]:
        B, H, L, dk, dv, C, dt = args
        st, form, ns, nb = _form(lib, *args)
        assert (st, form, ns) == (OK, efla.FWD_SPLIT, 1), args
        m = ctypes.c_size_t()
        assert lib.efla_chunk_split_workspace_size(B, H, L, C, dt, ctypes.byref(m)) == OK
        assert nb == m.value == lib.efla_chunk_fwd_workspace_size(*args), args
    # invalid sizes: the call's error, and a size of 0
    assert _form(lib, 1, 1, 8, 48, 64, 64, BF16)[0] == UNSUPPORTED
    assert _form(lib, 1, 1, 8, 64, 64, 8, BF16)[0] == UNSUPPORTED
    assert _form(lib, -1, 1, 8, 64, 64, 64, BF16)[0] == INVALID
    assert _form(lib, 1, 1, 8, 64, 64, 64, 9)[0] == INVALID
    assert lib.efla_chunk_fwd_workspace_size(1, 1, 8, 48, 64, 64, BF16) == 0
    assert lib.efla_chunk_fwd_form(8, 16, 4096, 128, 128, 64, BF16, None, None, None) == OK
    # the binding reports the same
    assert efla.fwd_form(8, 16, 4096, 128, 128, 64, torch.bfloat16) == ("fused", 1, 0)
    assert efla.fwd_form(1, 16, 65536, 128, 128, 64, torch.bfloat16)[0] == "scan"
    assert efla.fwd_workspace_size(4, 8, 2048, 64, 64, 64, torch.float32) == \
        efla.fwd_form(4, 8, 2048, 64, 64, 64, torch.float32)[2]


def _fwd(lib, **kw):
    a = dict(q=P(1), k=P(2), v=P(3), beta=P(4), dt=BF16, o=P(5), s0=None, sf=P(6), B=2, H=3, L=100, dk=64, dv=64,
             C=32, ws=P(7), wsb=6 * 4 * 3 * 256 * 2, gate=0)
    a.update(kw)
    return lib.efla_chunk_fwd_gate(a["q"], a["k"], a["v"], a["beta"], a["dt"], a["o"], a["s0"], a["sf"], a["B"],
                                   a["H"], a["L"], a["dk"], a["dv"], a["C"], a["gate"], a["ws"], a["wsb"], None)


def test_chunk_fwd_workspace_errors(lib):
    need = lib.efla_chunk_fwd_workspace_size(2, 3, 100, 64, 64, 32, BF16)
    assert need == 6 * 4 * 3 * 256 * 2            # split form: 4 chunks of 32 tokens, 3 blocks each
    assert _fwd(lib, ws=None) == WORKSPACE
    assert _fwd(lib, wsb=need - 1) == WORKSPACE
    assert _fwd(lib, ws=ctypes.c_void_p(0x7F0700000000 + 16)) == WORKSPACE     # not 256-byte aligned
    assert _fwd(lib, ws=P(6)) == INVALID                                      # is the final state
    assert _fwd(lib, gate=17) == INVALID
    assert _fwd(lib, dk=96) == UNSUPPORTED
    assert _fwd(lib, B=0, ws=None, wsb=0) == OK
    # the one-launch form takes no workspace: NULL is fine
    assert _fwd(lib, C=64, ws=None, wsb=0, dk=128, dv=128, B=0) == OK
    # the plain entry is the exact gate
    assert lib.efla_chunk_fwd(P(1), P(2), P(3), P(4), BF16, P(5), None, P(6), 2, 3, 100, 64, 64, 32, None, 0,
                              None) == WORKSPACE


@pytest.mark.skipif(not _no_gpu(), reason="needs a machine without a GPU")
def test_chunk_fwd_reaches_device_check(lib):
    assert _fwd(lib) == NO_DEVICE
    assert _fwd(lib, C=64, dk=128, dv=128, ws=None, wsb=0) == NO_DEVICE                      # one launch
    need = lib.efla_chunk_fwd_workspace_size(1, 16, 65536, 128, 128, 64, BF16)
    assert _fwd(lib, B=1, H=16, L=65536, dk=128, dv=128, C=64, ws=P(8), wsb=need) == NO_DEVICE  # scan


def _noalloc(lib, **kw):
    a = dict(q=P(1), k=P(2), v=P(3), beta=P(4), dt=F32, o=P(5), s0=None, sf=P(6), B=2, H=3, L=100, dk=64, dv=64,
             C=32, gate=0)
    a.update(kw)
    return lib.efla_chunk_fwd_noalloc(a["q"], a["k"], a["v"], a["beta"], a["dt"], a["o"], a["s0"], a["sf"], a["B"],
                                      a["H"], a["L"], a["dk"], a["dv"], a["C"], a["gate"], None)


def test_noalloc_limit_and_argument_errors(lib):
    limit = 128 << 20
    text = open(HEADER).read()
    assert re.search(r"#define EFLA_NOALLOC_SCRATCH_BYTES \(\(size_t\)128 << 20\)", text)
    # fp32, 16 x 16 heads of 8192 tokens, d 128: the split form's UT output alone is 335 MB
    need = lib.efla_chunk_fwd_workspace_size(16, 16, 8192, 128, 128, 64, F32)
    assert need > limit
    assert _noalloc(lib, B=16, H=16, L=8192, dk=128, dv=128, C=64) == WORKSPACE
    assert b"above the library" in lib.efla_last_error()
    assert _noalloc(lib, gate=-1) == INVALID
    assert _noalloc(lib, dk=96) == UNSUPPORTED
    assert _noalloc(lib, q=None) == INVALID
    assert _noalloc(lib, o=P(1)) == INVALID                 # o overlaps q
    assert _noalloc(lib, B=0) == OK                         # empty: nothing to do, no device touched
    assert _noalloc(lib, L=0, sf=None, q=None, k=None, v=None, beta=None, o=None) == OK


@pytest.mark.skipif(not _no_gpu(), reason="needs a machine without a GPU")
def test_noalloc_reaches_device_check(lib):
    assert _noalloc(lib) == NO_DEVICE                                           # split form: needs the scratch
    assert _noalloc(lib, dt=BF16, C=64, dk=128, dv=128) == NO_DEVICE             # one launch: no scratch
