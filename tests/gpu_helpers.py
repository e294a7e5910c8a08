"""Shared helpers of the GPU parity tests: seeded inputs to device tensors, oracle comparisons."""
import numpy as np
import torch

from exact_flow_delta_amd import workloads as W

TOL = {"f32": 1e-5, "bf16": 2e-2}


def dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    """float32 numpy (bf16-exact when dtype is bf16) -> contiguous GPU tensor of that storage type."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(W.bf16_bits(x))).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def fwd_inputs_dev(x: dict, dtype: str) -> dict:
    return dict(q=dev(x["q"], dtype), k=dev(x["k"], dtype), v=dev(x["v"], dtype),
                beta=torch.from_numpy(x["beta"]).cuda(),
                initial_state=None if x["initial_state"] is None else torch.from_numpy(x["initial_state"]).cuda())


def errs(o, S, ro, rS):
    return W.rel_max_err(host(o), ro), W.rel_max_err(host(S), rS)


def ut_dense(t: torch.Tensor, chunk: int) -> np.ndarray:
    """UT-transform output in the library's operand layout [B,H,NC,nblocks,64,4] -> dense float64
    [B,H,NC,chunk,chunk]: block rb (rb+1)/2 + kb holds at [16 g + r][j] the entry [16 rb + r][16 kb + 4 g + j]."""
    a = host(t)
    B, H, NC = a.shape[:3]
    out = np.zeros((B, H, NC, chunk, chunk))
    lane = np.arange(64)
    r, g = lane % 16, lane // 16
    qi = 0
    for rb in range(chunk // 16):
        for kb in range(rb + 1):
            for j in range(4):
                out[:, :, :, 16 * rb + r, 16 * kb + 4 * g + j] = a[:, :, :, qi, :, j]
            qi += 1
    return out
