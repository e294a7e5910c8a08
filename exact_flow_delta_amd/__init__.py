"""Error-Free Linear Attention (EFLA) on AMD Instinct MI355X -- Python binding of libefla.so.

Argument marshalling only: every step of the operator runs in the HIP kernels of ``libefla.so``
(built in-tree by ``python -m exact_flow_delta_amd.build``).  PyTorch supplies device memory and
the current stream; nothing here computes on the CPU, and there is no fallback path: if the
library is missing, every call raises.

    o, S = chunk_fwd(q, k, v, beta, initial_state=None, output_final_state=True, chunk_size=64)
    o    = recurrent_step(q, k, v, beta, state)          # state updated in place
    a    = alpha(k, beta)
    t    = ut_transform(k, beta, chunk_size=64)          # T diag(alpha) per chunk (operand layout)

    o, S = chunk_fwd_layout(q, k, v, beta, cu_seqlens=None)   # strided [B,H,L,d] views, packed sequences
    dq, dk, dv, dbeta, dS0 = chunk_bwd(q, k, v, beta, d_o, initial_state=None, d_final=None)
    dq, dk, dv, dbeta, dS0 = chunk_bwd_layout(q, k, v, beta, d_o, cu_seqlens=None)   # gradients in the inputs' strides
    o, S = efla_attention(q, k, v, beta, initial_state=None, cu_seqlens=None)   # differentiable (torch.autograd)

chunk_fwd calls efla_chunk_fwd by default, where the library picks the form for the sizes (fwd_form): the
segment-parallel one for few heads and long sequences (method="scan"), else for bf16, d_k >= 32 and 64-token
chunks the single kernel (method="fused": the chunks' UT transform runs in the same workgroups as the state
pass, no workspace), else the two-launch form (method="split": UT transform of all chunks into a workspace,
then the state pass).

Every call that forms alpha takes ``gate``: GATE_EXACT (0, the default) for the exact coefficient, or
p in 1 .. GATE_MAX_ORDER for the coefficient of a p-th order Runge-Kutta step of the same dynamics
(GATE_DELTANET = 1 is the delta rule's alpha = beta); see efla.h, "Gates".

The operator ("Exact Flow Linear Attention" (gist.science), Metodologia items 1-3; "Error-Free
Linear Attention is a Free Lunch" (howistudyai.com), Steps 1-4):
    alpha_t = (1 - exp(-beta_t ||k_t||^2)) / ||k_t||^2
    S_t     = (I - alpha_t k_t k_t^T) S_{t-1} + alpha_t k_t v_t^T
    o_t     = S_t^T q_t
Layouts: q, k [B,H,L,d_k]; v, o [B,H,L,d_v]; beta [B,H,L] fp32; state [B,H,d_k,d_v] fp32.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["EflaError", "alpha", "chunk_fwd", "chunk_fwd_layout", "layout_plan", "chunk_bwd", "chunk_bwd_workspace_size",
           "chunk_bwd_layout", "chunk_bwd_layout_workspace_size", "efla_attention", "recurrent_step", "chunk_plan",
           "split_workspace_size", "fwd_workspace_size", "fwd_form", "ut_transform", "state_pass", "scan_plan", "library_path", "load_library"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libefla.so")
_lib = None

EFLA_OK, EFLA_ERR_INVALID_ARG, EFLA_ERR_UNSUPPORTED, EFLA_ERR_WORKSPACE, EFLA_ERR_NO_DEVICE, EFLA_ERR_HIP = range(6)
FWD_ONE_LAUNCH, FWD_SPLIT, FWD_SCAN = 0, 1, 2
FORM_NAMES = {FWD_ONE_LAUNCH: "fused", FWD_SPLIT: "split", FWD_SCAN: "scan"}
EFLA_F32, EFLA_BF16 = 0, 1
GATE_EXACT, GATE_DELTANET, GATE_MAX_ORDER = 0, 1, 16

_vp = ctypes.c_void_p
_i32 = ctypes.c_int
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t


class Layout(ctypes.Structure):
    """efla_layout: element strides (batch, head, token) of q, k, v, o and beta, and packed-sequence offsets."""
    _fields_ = [("q", _i64 * 3), ("k", _i64 * 3), ("v", _i64 * 3), ("o", _i64 * 3), ("beta", _i64 * 3),
                ("cu_seqlens", _vp)]


class EflaError(RuntimeError):
    """A non-OK status from libefla.so."""

    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        msg = "%s failed: %s" % (where, _status_string(status))
        if detail:
            msg += " -- " + detail
        super().__init__(msg)


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libefla.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError("libefla.so is not built (%s); run `python -m exact_flow_delta_amd.build`" % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    lib.efla_alpha.argtypes = [_vp, _i32, _vp, _vp, _i64, _i32, _vp]
    lib.efla_chunk_fwd.argtypes = [_vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                   _vp, _sz, _vp]
    lib.efla_chunk_fwd_gate.argtypes = [_vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                        _i32, _vp, _sz, _vp]
    lib.efla_chunk_fwd_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i32]
    lib.efla_chunk_fwd_workspace_size.restype = _sz
    lib.efla_chunk_fwd_form.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_i32),
                                        ctypes.POINTER(_i32), ctypes.POINTER(_sz)]
    lib.efla_chunk_fwd_slab.argtypes = [_vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp,
                                        _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp]
    lib.efla_recurrent_step.argtypes = [_vp, _vp, _vp, _vp, _i32, _vp, _vp, _i64, _i32, _i32, _vp]
    lib.efla_chunk_fwd_plan.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                        ctypes.POINTER(_i32), ctypes.POINTER(_i32), ctypes.POINTER(_i32)]
    lib.efla_chunk_fwd_split_plan.argtypes = lib.efla_chunk_fwd_plan.argtypes
    lib.efla_chunk_split_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_sz)]
    lib.efla_ut_transform.argtypes = [_vp, _vp, _i32, _vp, _sz, _i32, _i32, _i32, _i32, _i32, _vp]
    lib.efla_chunk_fwd_split.argtypes = [_vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp,
                                         _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _sz, _vp]
    lib.efla_alpha_gate.argtypes = [_vp, _i32, _vp, _vp, _i64, _i32, _i32, _vp]
    lib.efla_chunk_fwd_slab_gate.argtypes = [_vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp,
                                             _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp]
    lib.efla_recurrent_step_gate.argtypes = [_vp, _vp, _vp, _vp, _i32, _vp, _vp, _i64, _i32, _i32, _i32, _vp]
    lib.efla_ut_transform_gate.argtypes = [_vp, _vp, _i32, _vp, _sz, _i32, _i32, _i32, _i32, _i32, _i32, _vp]
    lib.efla_chunk_fwd_split_gate.argtypes = [_vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                              _i32, _i32, _i32, _i32, _vp, _sz, _vp]
    lib.efla_chunk_fwd_scan.argtypes = [_vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                        _i32, _i32, _i32, _vp, _sz, _vp]
    lib.efla_chunk_scan_plan.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_i32),
                                         ctypes.POINTER(_i32), ctypes.POINTER(_i32), ctypes.POINTER(_sz)]
    lib.efla_chunk_fwd_layout.argtypes = [_vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                          _i32, _i32, _i32, ctypes.POINTER(Layout), _vp, _sz, _vp]
    lib.efla_chunk_layout_plan.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                           ctypes.POINTER(_i32), ctypes.POINTER(_sz)]
    lib.efla_chunk_bwd.argtypes = [_vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                   _i32, _i32, _i32, _i32, _vp, _sz, _vp]
    lib.efla_chunk_bwd_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_sz)]
    lib.efla_chunk_bwd_layout.argtypes = [_vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                          _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(Layout), _vp, _sz, _vp]
    lib.efla_chunk_bwd_layout_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                                         ctypes.POINTER(_sz)]
    lib.efla_chunk_state_pass.argtypes = [_vp, _vp, _vp, _vp, _sz, _i32, _vp, _vp, _vp,
                                          _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp]
    for fn in ("efla_alpha", "efla_chunk_fwd", "efla_chunk_fwd_gate", "efla_chunk_fwd_form", "efla_chunk_fwd_slab", "efla_recurrent_step", "efla_chunk_fwd_plan",
               "efla_chunk_fwd_split_plan", "efla_chunk_split_workspace_size", "efla_ut_transform", "efla_chunk_fwd_split",
               "efla_chunk_state_pass"):
        getattr(lib, fn).restype = _i32
    lib.efla_status_string.argtypes = [_i32]
    lib.efla_status_string.restype = ctypes.c_char_p
    lib.efla_last_error.argtypes = []
    lib.efla_last_error.restype = ctypes.c_char_p
    lib.efla_version.argtypes = []
    lib.efla_version.restype = _i32
    _lib = lib
    return lib


def _status_string(status: int) -> str:
    try:
        return load_library().efla_status_string(status).decode()
    except Exception:  # pragma: no cover - library missing
        return "status %d" % status


def _check(status: int, where: str):
    if status != EFLA_OK:
        detail = load_library().efla_last_error().decode() if status == EFLA_ERR_HIP else ""
        raise EflaError(status, where, detail)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return EFLA_BF16
    if t.dtype == torch.float32:
        return EFLA_F32
    raise TypeError("q, k, v must be float32 or bfloat16, got %s" % t.dtype)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dev_tensor(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor (got %s); libefla has no CPU path" % (name, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _stream(device: torch.device):
    return torch.cuda.current_stream(device).cuda_stream


def alpha(k: torch.Tensor, beta: torch.Tensor, out: torch.Tensor | None = None, gate: int = GATE_EXACT) -> torch.Tensor:
    """Gate alpha for keys k [..., d_k] (fp32/bf16) and steps beta [...] (fp32); returns fp32 [...]."""
    lib = load_library()
    _dev_tensor(k, "k")
    _dev_tensor(beta, "beta")
    if beta.dtype != torch.float32 or tuple(beta.shape) != tuple(k.shape[:-1]):
        raise ValueError("beta must be float32 with shape k.shape[:-1]")
    if out is None:
        out = torch.empty(beta.shape, dtype=torch.float32, device=k.device)
    _dev_tensor(out, "out")
    _check(lib.efla_alpha_gate(_ptr(k), _dtype_code(k), _ptr(beta), _ptr(out), beta.numel(), k.shape[-1], int(gate),
                               _stream(k.device)), "efla_alpha")
    return out


def _dtype_of(dtype) -> int:
    return EFLA_BF16 if dtype == torch.bfloat16 else EFLA_F32


def split_workspace_size(B, H, L, chunk=64, dtype=torch.bfloat16) -> int:
    """Bytes of workspace the two-launch chunked forward needs (= size of the UT transform output)."""
    lib = load_library()
    n = _sz()
    _check(lib.efla_chunk_split_workspace_size(B, H, L, chunk, _dtype_of(dtype), ctypes.byref(n)),
           "efla_chunk_split_workspace_size")
    return n.value


def fwd_workspace_size(B, H, L, d_k, d_v, chunk=64, dtype=torch.bfloat16) -> int:
    """Bytes of workspace efla_chunk_fwd needs for these sizes (0 for the one-launch form)."""
    return int(load_library().efla_chunk_fwd_workspace_size(B, H, L, d_k, d_v, chunk, _dtype_of(dtype)))


def fwd_form(B, H, L, d_k, d_v, chunk=64, dtype=torch.bfloat16):
    """(form name, segments, workspace bytes) efla_chunk_fwd picks for these sizes: "fused" (the one-launch
    kernel), "split" or "scan"."""
    lib = load_library()
    f, ns, nb = _i32(), _i32(), _sz()
    _check(lib.efla_chunk_fwd_form(B, H, L, d_k, d_v, chunk, _dtype_of(dtype), ctypes.byref(f), ctypes.byref(ns),
                                   ctypes.byref(nb)), "efla_chunk_fwd_form")
    return FORM_NAMES[f.value], ns.value, nb.value


def ut_transform(k, beta, chunk_size=64, out=None, gate=GATE_EXACT):
    """T diag(alpha) of every chunk, T = (I + strict_lower(diag(alpha) K K^T))^{-1}, in the library's
    operand layout: a tensor [B, H, ceil(L/chunk), nblocks, 64, 4] of k's dtype, where block
    rb (rb+1)/2 + kb (kb <= rb < chunk/16) holds at [lane = 16 g + r][j] the entry
    (T diag(alpha))[16 rb + r][16 kb + 4 g + j] of that chunk.
    """
    lib = load_library()
    _dev_tensor(k, "k")
    _dev_tensor(beta, "beta")
    B, H, L, d_k = k.shape
    if beta.dtype != torch.float32 or tuple(beta.shape) != (B, H, L):
        raise ValueError("beta must be float32 [B,H,L]")
    nb = (chunk_size // 16) * (chunk_size // 16 + 1) // 2
    nc = (L + chunk_size - 1) // chunk_size
    if out is None:
        out = torch.empty((B, H, nc, nb, 64, 4), dtype=k.dtype, device=k.device)
    _dev_tensor(out, "out")
    _check(lib.efla_ut_transform_gate(_ptr(k), _ptr(beta), _dtype_code(k), _ptr(out), out.numel() * out.element_size(),
                                      B, H, L, d_k, int(chunk_size), int(gate), _stream(k.device)), "efla_ut_transform")
    return out


def chunk_fwd(q, k, v, beta, initial_state=None, output_final_state=True, chunk_size=64, dv_slab=0,
              out=None, final_state=None, method="auto", workspace=None, gate=GATE_EXACT, segments=0):
    """Chunkwise-parallel EFLA forward over [B,H,L,*] inputs.

    Returns (o [B,H,L,d_v] in the input dtype, final state [B,H,d_k,d_v] fp32 or None).
    ``final_state`` may be passed (and may be ``initial_state`` itself) to receive the state in place.
    ``method`` is "auto" (the default: efla_chunk_fwd, where the library picks the form for the sizes, see
    fwd_form; ``workspace``: a device tensor of at least fwd_workspace_size(...) bytes, allocated here when
    not given), "split" (UT transform launch + state-pass launch, efla_chunk_fwd_split; workspace of
    split_workspace_size(...) bytes), "fused" (one kernel, no workspace: efla_chunk_fwd_slab) or "scan"
    (segment-parallel: ``segments`` segments per sequence, 0 = the library's choice; workspace of
    scan_plan(...)[3] bytes).
    """
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("beta", beta)):
        _dev_tensor(t, name)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    B, H, L, d_k = k.shape
    d_v = v.shape[-1]
    if tuple(q.shape) != (B, H, L, d_k) or tuple(v.shape[:3]) != (B, H, L):
        raise ValueError("q, k, v shapes disagree: %s %s %s" % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    if beta.dtype != torch.float32 or tuple(beta.shape) != (B, H, L):
        raise ValueError("beta must be float32 [B,H,L]")
    if initial_state is not None:
        _dev_tensor(initial_state, "initial_state")
        if initial_state.dtype != torch.float32 or tuple(initial_state.shape) != (B, H, d_k, d_v):
            raise ValueError("initial_state must be float32 [B,H,d_k,d_v]")
    if out is None:
        out = torch.empty((B, H, L, d_v), dtype=v.dtype, device=v.device)
    _dev_tensor(out, "out")
    if final_state is None and output_final_state:
        final_state = torch.empty((B, H, d_k, d_v), dtype=torch.float32, device=v.device)
    if final_state is not None:
        _dev_tensor(final_state, "final_state")
        if final_state.dtype != torch.float32 or tuple(final_state.shape) != (B, H, d_k, d_v):
            raise ValueError("final_state must be float32 [B,H,d_k,d_v]")
    if method == "auto":
        need = fwd_workspace_size(B, H, L, d_k, d_v, int(chunk_size), v.dtype)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=v.device)
        if workspace is not None:
            _dev_tensor(workspace, "workspace")
        _check(lib.efla_chunk_fwd_gate(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _dtype_code(v), _ptr(out),
                                       _ptr(initial_state), _ptr(final_state), B, H, L, d_k, d_v, int(chunk_size),
                                       int(gate), _ptr(workspace),
                                       0 if workspace is None else workspace.numel() * workspace.element_size(),
                                       _stream(v.device)), "efla_chunk_fwd")
        return out, final_state
    if method == "fused":
        _check(lib.efla_chunk_fwd_slab_gate(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _dtype_code(v), _ptr(out),
                                            _ptr(initial_state), _ptr(final_state), B, H, L, d_k, d_v,
                                            int(chunk_size), int(dv_slab), int(gate), _stream(v.device)),
               "efla_chunk_fwd_slab")
    elif method == "split":
        need = split_workspace_size(B, H, L, int(chunk_size), v.dtype)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=v.device)
        _dev_tensor(workspace, "workspace")
        _check(lib.efla_chunk_fwd_split_gate(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _dtype_code(v), _ptr(out),
                                             _ptr(initial_state), _ptr(final_state), B, H, L, d_k, d_v,
                                             int(chunk_size), int(dv_slab), int(gate), _ptr(workspace),
                                             workspace.numel() * workspace.element_size(), _stream(v.device)),
               "efla_chunk_fwd_split")
    elif method == "scan":
        need = scan_plan(B, H, L, d_k, d_v, int(chunk_size), v.dtype, int(segments))[3]
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=v.device)
        _dev_tensor(workspace, "workspace")
        _check(lib.efla_chunk_fwd_scan(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _dtype_code(v), _ptr(out),
                                       _ptr(initial_state), _ptr(final_state), B, H, L, d_k, d_v, int(chunk_size),
                                       int(segments), int(gate), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream(v.device)),
               "efla_chunk_fwd_scan")
    else:
        raise ValueError("method must be 'split', 'fused' or 'scan'")
    return out, final_state


def _dev_view(t: torch.Tensor, name: str, ndim: int):
    """A GPU tensor of `ndim` dims whose last dimension is contiguous (other strides free)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor (got %s); libefla has no CPU path" % (name, t.device))
    if t.dim() != ndim:
        raise ValueError("%s must have %d dimensions, got shape %s" % (name, ndim, tuple(t.shape)))
    if ndim == 4 and t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError("%s: the feature dimension must be contiguous" % name)


def layout_plan(B, H, L, d_k, d_v, chunk=64, dtype=torch.bfloat16, varlen=False, segments=0):
    """(segments, workspace bytes) of chunk_fwd_layout; host only."""
    lib = load_library()
    ns, nb = _i32(), _sz()
    _check(lib.efla_chunk_layout_plan(B, H, L, d_k, d_v, chunk, _dtype_of(dtype), int(bool(varlen)), segments,
                                      ctypes.byref(ns), ctypes.byref(nb)), "efla_chunk_layout_plan")
    return ns.value, nb.value


def chunk_fwd_layout(q, k, v, beta, cu_seqlens=None, initial_state=None, output_final_state=True, chunk_size=64,
                     segments=0, gate=GATE_EXACT, out=None, final_state=None, workspace=None):
    """The chunked forward over strided views, or over packed sequences (efla_chunk_fwd_layout).

    q, k [B,H,L,d_k], v [B,H,L,d_v], beta [B,H,L] are views with any strides (the feature dimension
    contiguous): e.g. ``x.transpose(1, 2)`` of a [B,L,H,d] tensor, or slices of a fused projection.  With
    ``cu_seqlens`` (int32 GPU tensor of N + 1 offsets) the views are [1,H,T,d] and [1,H,T] holding N packed
    sequences, sequence n being tokens cu_seqlens[n] .. cu_seqlens[n+1]-1; states are then [N,H,d_k,d_v].
    ``out`` (default: like ``v``, keeping its strides when it is dense) receives o.  ``segments`` as
    chunk_fwd(method="scan"); with packed sequences one segment.  Returns (o, final state or None).
    """
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev_view(t, name, 4)
    _dev_view(beta, "beta", 3)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    B, H, L, d_k = k.shape
    d_v = v.shape[-1]
    if tuple(q.shape) != (B, H, L, d_k) or tuple(v.shape[:3]) != (B, H, L):
        raise ValueError("q, k, v shapes disagree: %s %s %s" % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    if beta.dtype != torch.float32 or tuple(beta.shape) != (B, H, L):
        raise ValueError("beta must be float32 [B,H,L]")
    N = B
    if cu_seqlens is not None:
        _dev_tensor(cu_seqlens, "cu_seqlens")
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
            raise ValueError("cu_seqlens must be a 1-D int32 tensor of N + 1 offsets")
        if B != 1:
            raise ValueError("packed sequences are given as [1,H,T,d] views")
        N = cu_seqlens.numel() - 1
    if initial_state is not None:
        _dev_tensor(initial_state, "initial_state")
        if initial_state.dtype != torch.float32 or tuple(initial_state.shape) != (N, H, d_k, d_v):
            raise ValueError("initial_state must be float32 [%d,H,d_k,d_v]" % N)
    if out is None:
        out = torch.empty_like(v)
    _dev_view(out, "out", 4)
    if tuple(out.shape) != (B, H, L, d_v) or out.dtype != v.dtype:
        raise ValueError("out must be %s [B,H,L,d_v]" % v.dtype)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, d_k, d_v), dtype=torch.float32, device=v.device)
    if final_state is not None:
        _dev_tensor(final_state, "final_state")
        if final_state.dtype != torch.float32 or tuple(final_state.shape) != (N, H, d_k, d_v):
            raise ValueError("final_state must be float32 [%d,H,d_k,d_v]" % N)
    lay = Layout()
    for f, t in (("q", q), ("k", k), ("v", v), ("o", out)):
        getattr(lay, f)[:] = [t.stride(0), t.stride(1), t.stride(2)]
    lay.beta[:] = [beta.stride(0), beta.stride(1), beta.stride(2)]
    lay.cu_seqlens = _ptr(cu_seqlens)
    need = layout_plan(N, H, L, d_k, d_v, int(chunk_size), v.dtype, cu_seqlens is not None, int(segments))[1]
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=v.device)
    _dev_tensor(workspace, "workspace")
    _check(lib.efla_chunk_fwd_layout(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _dtype_code(v), _ptr(out),
                                     _ptr(initial_state), _ptr(final_state), N, H, L, d_k, d_v, int(chunk_size),
                                     int(segments), int(gate), ctypes.byref(lay), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(v.device)),
           "efla_chunk_fwd_layout")
    return out, final_state


def chunk_bwd_workspace_size(B, H, L, d_k, d_v, chunk=64, dtype=torch.bfloat16) -> int:
    """Bytes of workspace chunk_bwd needs (host only)."""
    lib = load_library()
    n = _sz()
    _check(lib.efla_chunk_bwd_workspace_size(B, H, L, d_k, d_v, chunk, _dtype_of(dtype), ctypes.byref(n)),
           "efla_chunk_bwd_workspace_size")
    return n.value


def chunk_bwd(q, k, v, beta, d_o, initial_state=None, d_final=None, chunk_size=64, gate=GATE_EXACT,
              want_initial_grad=True, workspace=None):
    """Gradients of the chunked forward (efla_chunk_bwd): given d_o [B,H,L,d_v] (dLoss/do) and d_final
    [B,H,d_k,d_v] (dLoss/dS_L, None = 0), returns (dq, dk, dv in the input dtype, dbeta fp32, d_initial fp32
    [B,H,d_k,d_v] or None)."""
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("beta", beta), ("d_o", d_o)):
        _dev_tensor(t, name)
    if not (q.dtype == k.dtype == v.dtype == d_o.dtype):
        raise TypeError("q, k, v, d_o must share a dtype")
    B, H, L, d_k = k.shape
    d_v = v.shape[-1]
    if tuple(q.shape) != (B, H, L, d_k) or tuple(v.shape[:3]) != (B, H, L) or d_o.shape != v.shape:
        raise ValueError("q, k, v, d_o shapes disagree")
    if beta.dtype != torch.float32 or tuple(beta.shape) != (B, H, L):
        raise ValueError("beta must be float32 [B,H,L]")
    for name, x in (("initial_state", initial_state), ("d_final", d_final)):
        if x is not None:
            _dev_tensor(x, name)
            if x.dtype != torch.float32 or tuple(x.shape) != (B, H, d_k, d_v):
                raise ValueError("%s must be float32 [B,H,d_k,d_v]" % name)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dbeta = torch.empty_like(beta)
    d_init = torch.empty((B, H, d_k, d_v), dtype=torch.float32, device=v.device) if want_initial_grad else None
    need = chunk_bwd_workspace_size(B, H, L, d_k, d_v, int(chunk_size), v.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=v.device)
    _dev_tensor(workspace, "workspace")
    _check(lib.efla_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _dtype_code(v), _ptr(initial_state), _ptr(d_o),
                              _ptr(d_final), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbeta), _ptr(d_init), B, H, L, d_k, d_v,
                              int(chunk_size), int(gate), _ptr(workspace), workspace.numel() * workspace.element_size(),
                              _stream(v.device)), "efla_chunk_bwd")
    return dq, dk, dv, dbeta, d_init


def chunk_bwd_layout_workspace_size(B, H, L, d_k, d_v, chunk=64, dtype=torch.bfloat16, varlen=False) -> int:
    """Bytes of workspace chunk_bwd_layout needs (host only); varlen: packed sequences."""
    lib = load_library()
    n = _sz()
    _check(lib.efla_chunk_bwd_layout_workspace_size(B, H, L, d_k, d_v, chunk, _dtype_of(dtype), int(bool(varlen)),
                                                    ctypes.byref(n)), "efla_chunk_bwd_layout_workspace_size")
    return n.value


def chunk_bwd_layout(q, k, v, beta, d_o, cu_seqlens=None, initial_state=None, d_final=None, chunk_size=64,
                     gate=GATE_EXACT, want_initial_grad=True, grads=None, workspace=None):
    """Gradients of chunk_fwd_layout's operator over strided views or packed sequences (efla_chunk_bwd_layout).

    q, k, v, beta, d_o and cu_seqlens as chunk_fwd_layout's q, k, v, beta, o and cu_seqlens (any strides, the
    feature dimension contiguous).  The gradients are written with the strides of their inputs: ``grads`` =
    (dq, dk, dv, dbeta) views of exactly those strides (e.g. slices of a fused gradient buffer when q, k, v are
    slices of a fused projection), or None to allocate them.  Returns (dq, dk, dv, dbeta, d_initial or None);
    states are [N,H,d_k,d_v] for N packed sequences.
    """
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("d_o", d_o)):
        _dev_view(t, name, 4)
    _dev_view(beta, "beta", 3)
    if not (q.dtype == k.dtype == v.dtype == d_o.dtype):
        raise TypeError("q, k, v, d_o must share a dtype")
    B, H, L, d_k = k.shape
    d_v = v.shape[-1]
    if tuple(q.shape) != (B, H, L, d_k) or tuple(v.shape[:3]) != (B, H, L) or d_o.shape != v.shape:
        raise ValueError("q, k, v, d_o shapes disagree")
    if beta.dtype != torch.float32 or tuple(beta.shape) != (B, H, L):
        raise ValueError("beta must be float32 [B,H,L]")
    N = B
    if cu_seqlens is not None:
        _dev_tensor(cu_seqlens, "cu_seqlens")
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
            raise ValueError("cu_seqlens must be a 1-D int32 tensor of N + 1 offsets")
        if B != 1:
            raise ValueError("packed sequences are given as [1,H,T,d] views")
        N = cu_seqlens.numel() - 1
    for name, x in (("initial_state", initial_state), ("d_final", d_final)):
        if x is not None:
            _dev_tensor(x, name)
            if x.dtype != torch.float32 or tuple(x.shape) != (N, H, d_k, d_v):
                raise ValueError("%s must be float32 [%d,H,d_k,d_v]" % (name, N))
    if grads is None:
        grads = tuple(torch.empty_strided(t.shape, t.stride(), dtype=t.dtype, device=t.device) for t in (q, k, v, beta))
    dq, dk, dv, dbeta = grads
    for g, t, name in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv"), (dbeta, beta, "dbeta")):
        if not isinstance(g, torch.Tensor) or g.device != t.device or g.dtype != t.dtype or g.shape != t.shape or \
                g.stride() != t.stride():
            raise ValueError("%s must be a %s tensor of %s's shape and strides" % (name, t.dtype, name[1:]))
    d_init = torch.empty((N, H, d_k, d_v), dtype=torch.float32, device=v.device) if want_initial_grad else None
    lay = Layout()
    for f, t in (("q", q), ("k", k), ("v", v), ("o", d_o)):
        getattr(lay, f)[:] = [t.stride(0), t.stride(1), t.stride(2)]
    lay.beta[:] = [beta.stride(0), beta.stride(1), beta.stride(2)]
    lay.cu_seqlens = _ptr(cu_seqlens)
    need = chunk_bwd_layout_workspace_size(N, H, L, d_k, d_v, int(chunk_size), v.dtype, cu_seqlens is not None)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=v.device)
    _dev_tensor(workspace, "workspace")
    _check(lib.efla_chunk_bwd_layout(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _dtype_code(v), _ptr(initial_state),
                                     _ptr(d_o), _ptr(d_final), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbeta), _ptr(d_init),
                                     N, H, L, d_k, d_v, int(chunk_size), int(gate), ctypes.byref(lay),
                                     _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(v.device)), "efla_chunk_bwd_layout")
    return dq, dk, dv, dbeta, d_init


def _dense(t: torch.Tensor, feature_contiguous: bool) -> torch.Tensor:
    """t itself when its elements tile a block of memory without gaps or overlaps (a contiguous tensor, or a
    permutation of one such as the [B,H,L,d] view of a [B,L,H,d] tensor) and, for q, k, v, d_o, its feature
    dimension is contiguous; else a contiguous copy.  Gradients are then allocated with the same strides."""
    dims = sorted((d for d in range(t.dim()) if t.shape[d] > 1), key=lambda d: t.stride(d))
    expect = 1
    dense = True
    for d in dims:
        if t.stride(d) != expect:
            dense = False
            break
        expect *= t.shape[d]
    if feature_contiguous and t.shape[-1] > 1 and t.stride(-1) != 1:
        dense = False
    return t if dense else t.contiguous()


class _EflaFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, beta, initial_state, cu_seqlens, chunk_size, gate):
        q, k, v = (_dense(x, True) for x in (q, k, v))
        beta = _dense(beta, False)
        s0 = None if initial_state is None else initial_state.contiguous()
        o, sf = chunk_fwd_layout(q, k, v, beta, cu_seqlens=cu_seqlens, initial_state=s0, chunk_size=chunk_size,
                                 gate=gate)
        empty = torch.empty(0, device=v.device)
        ctx.save_for_backward(q, k, v, beta, s0 if s0 is not None else empty,
                              cu_seqlens if cu_seqlens is not None else empty)
        ctx.has_s0, ctx.has_cu = s0 is not None, cu_seqlens is not None
        ctx.chunk_size, ctx.gate = chunk_size, gate
        return o, sf

    @staticmethod
    def backward(ctx, d_o, d_final):
        q, k, v, beta, s0, cu = ctx.saved_tensors
        s0 = s0 if ctx.has_s0 else None
        cu = cu if ctx.has_cu else None
        d_o = torch.zeros_like(v) if d_o is None else _dense(d_o.to(v.dtype), True)
        d_final = None if d_final is None else d_final.contiguous().float()
        dq, dk, dv, dbeta, ds0 = chunk_bwd_layout(q, k, v, beta, d_o, cu_seqlens=cu, initial_state=s0,
                                                  d_final=d_final, chunk_size=ctx.chunk_size, gate=ctx.gate,
                                                  want_initial_grad=ctx.has_s0)
        return dq, dk, dv, dbeta, ds0, None, None, None


def efla_attention(q, k, v, beta, initial_state=None, chunk_size=64, gate=GATE_EXACT, cu_seqlens=None):
    """The chunked forward as a differentiable torch op: returns (o, final state); gradients flow to q, k, v,
    beta and initial_state through the backward pass.  q, k, v [B,H,L,d] and beta [B,H,L] may be views of
    another layout (e.g. ``x.transpose(1, 2)`` of [B,L,H,d] projections): dense views are used as they are, with
    o and the gradients laid out like them, other views are copied first.  ``cu_seqlens`` (int32 GPU tensor of
    N + 1 offsets) takes [1,H,T,d] packed sequences with per-sequence states [N,H,d_k,d_v], as chunk_fwd_layout."""
    return _EflaFunction.apply(q, k, v, beta, initial_state, cu_seqlens, int(chunk_size), int(gate))


def scan_plan(B, H, L, d_k, d_v, chunk=64, dtype=torch.bfloat16, segments=0):
    """(segments, chunks per segment, slab width, workspace bytes) of chunk_fwd(method="scan"); host only."""
    lib = load_library()
    ns, sc, sw, nb = _i32(), _i32(), _i32(), _sz()
    _check(lib.efla_chunk_scan_plan(B, H, L, d_k, d_v, chunk, _dtype_of(dtype), segments, ctypes.byref(ns),
                                    ctypes.byref(sc), ctypes.byref(sw), ctypes.byref(nb)), "efla_chunk_scan_plan")
    return ns.value, sc.value, sw.value, nb.value


def state_pass(q, k, v, t, initial_state=None, output_final_state=True, chunk_size=64, dv_slab=0, out=None,
               final_state=None):
    """Inter-chunk state pass alone, from ``t`` = ut_transform(k, beta, chunk_size).

    Returns (o, final state or None) exactly as chunk_fwd(method="split") would.
    """
    lib = load_library()
    for name, x in (("q", q), ("k", k), ("v", v), ("t", t)):
        _dev_tensor(x, name)
    B, H, L, d_k = k.shape
    d_v = v.shape[-1]
    if tuple(q.shape) != (B, H, L, d_k) or tuple(v.shape[:3]) != (B, H, L):
        raise ValueError("q, k, v shapes disagree")
    if out is None:
        out = torch.empty((B, H, L, d_v), dtype=v.dtype, device=v.device)
    _dev_tensor(out, "out")
    if final_state is None and output_final_state:
        final_state = torch.empty((B, H, d_k, d_v), dtype=torch.float32, device=v.device)
    for name, x in (("initial_state", initial_state), ("final_state", final_state)):
        if x is not None:
            _dev_tensor(x, name)
            if x.dtype != torch.float32 or tuple(x.shape) != (B, H, d_k, d_v):
                raise ValueError("%s must be float32 [B,H,d_k,d_v]" % name)
    _check(lib.efla_chunk_state_pass(_ptr(q), _ptr(k), _ptr(v), _ptr(t), t.numel() * t.element_size(),
                                     _dtype_code(v), _ptr(out), _ptr(initial_state), _ptr(final_state), B, H, L, d_k,
                                     d_v, int(chunk_size), int(dv_slab), _stream(v.device)), "efla_chunk_state_pass")
    return out, final_state


def recurrent_step(q, k, v, beta, state, out=None, gate=GATE_EXACT):
    """One decode token for [NH,*] inputs (or [N,H,*]); ``state`` [..., d_k, d_v] fp32 is updated in place.

    Returns o [..., d_v] in the input dtype.
    """
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("beta", beta), ("state", state)):
        _dev_tensor(t, name)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    d_k = k.shape[-1]
    d_v = v.shape[-1]
    lead = tuple(k.shape[:-1])
    NH = k.numel() // d_k
    if tuple(q.shape) != tuple(k.shape) or tuple(v.shape[:-1]) != lead or tuple(beta.shape) != lead:
        raise ValueError("q, k, v, beta leading shapes disagree")
    if state.dtype != torch.float32 or tuple(state.shape) != lead + (d_k, d_v):
        raise ValueError("state must be float32 %s" % (lead + (d_k, d_v),))
    if beta.dtype != torch.float32:
        raise ValueError("beta must be float32")
    if out is None:
        out = torch.empty(lead + (d_v,), dtype=v.dtype, device=v.device)
    _dev_tensor(out, "out")
    _check(lib.efla_recurrent_step_gate(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _dtype_code(v), _ptr(state),
                                        _ptr(out), NH, d_k, d_v, int(gate), _stream(v.device)), "efla_recurrent_step")
    return out


def chunk_plan(B, H, L, d_k, d_v, chunk=64, dtype=torch.bfloat16, dv_slab=0, method="split"):
    """(workgroups, slab width, LDS bytes) of the state-carrying launch chunk_fwd would make; host only."""
    lib = load_library()
    wg, sw, lds = _i32(), _i32(), _i32()
    fn = lib.efla_chunk_fwd_split_plan if method == "split" else lib.efla_chunk_fwd_plan
    _check(fn(B, H, L, d_k, d_v, chunk, _dtype_of(dtype), dv_slab, ctypes.byref(wg), ctypes.byref(sw),
              ctypes.byref(lds)), "chunk_plan")
    return wg.value, sw.value, lds.value
