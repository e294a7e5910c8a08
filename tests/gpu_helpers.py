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
