#!/usr/bin/env python3
"""Benchmark of the EFLA hot path on one MI355X.

One step = one chunked forward of the LM-layer workload (B8 H16 L4096 d_k = d_v = 128, bf16 q/k/v/o,
fp32 beta and state, chunk 64, zero initial state, final state returned), as the library's default form for
these sizes: the one-launch forward (efla_chunk_fwd), whose workgroups run the inter-chunk state pass and, on
waves of their own, the UT transform of their head's chunks (exact gate included), with no workspace.  The
roofline line is that kernel's: the forward's algorithmic bytes over its average launch duration (HIP events on
the stream it runs on).  The two-launch form (efla_chunk_fwd_split: the UT transform of all 8192 (head, chunk)
pairs into a workspace, then the state pass) is timed on the same inputs under "split", with its two launches
also timed one by one through the stand-alone UT and state-pass entry points (the same state-pass kernel; the
UT kernel in its all-blocks form, while the step's UT launch forms only the diagonal 32 x 32 blocks of each
chunk's T diag(alpha), all the state pass reads).
The batched decode workload (256 sequences x 32 heads, d 128, 512 MiB fp32 state, 64 dependent
one-token steps, one launch per step) is timed in the same run and reported under "decode"; the two small fp32
parity workloads (tiny single-head, stiff mixed-norm) are timed under "small_fp32".

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-decode] [--no-long] [--no-bwd]
                    [--only fwd|decode|copy|long|bwd]
    python bench.py --record-traffic DIR

--only runs one leg for profiling: the forward alone, the decode alone, a plain 512 MiB device-to-device
copy (the reference for scaling the HBM byte counters), the long-context forward, or the LM-layer backward.
--record-traffic (host only) reads the rocprofv3 counter CSVs of six runs under DIR -- fetch_fwd,
write_fwd, fetch_dec, write_dec, fetch_copy, write_copy, one FETCH_SIZE or WRITE_SIZE run each (the
commands are in profiles/hbm_counter_calibration_copy512MiB.md) -- and writes profiles/hbm_traffic.json.

Prints one JSON line.  Inputs are seeded synthetic tensors already resident in HBM when timing starts.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "EFLA chunked-fwd tokens/s at B8 H16 L4096 d128; % MFMA peak; decode HBM GB/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix, published
FP32_PEAK_TFLOPS = 157.3       # MI355X dense fp32 (matrix and vector), published


def chain_algorithmic(B, H, L, dk, dv, esize=2):
    """Bytes the state pass must move: q, k, v read and o written once per token-head, the fp32 final state."""
    return B * H * L * (2 * dk + 2 * dv) * esize + B * H * dk * dv * 4


def ut_algorithmic(B, H, L, dk, esize=2):
    """Bytes the UT transform must read: k and beta once per token-head."""
    return B * H * L * (dk * esize + 4)


def fwd_algorithmic(B, H, L, dk, dv, C, esize=2):
    """Bytes and flops one chunked forward must move / do, counted from the algorithm.

    Bytes: q, k (d_k each), v, o (d_v each) in the storage type and beta (fp32) once per token-head,
    plus the fp32 final state once per head.
    Flops per chunk (dense products counted 2 per multiply-add, triangular ones by their lower half):
    K S and Q S 2*(2 C dk dv), K^T Delta 2 C dk dv, lower(K K^T) and lower(Q K^T) 2*(C^2 dk),
    T diag(alpha) R and lower(Q K^T) Delta 2*(C^2 dv), T by substitution C^3/3.
    """
    tok = B * H * L
    nbytes = tok * ((2 * dk + 2 * dv) * esize + 4) + B * H * dk * dv * 4
    per_chunk = 6 * C * dk * dv + 2 * C * C * dk + 2 * C * C * dv + C ** 3 / 3.0
    flops = per_chunk * (tok / C)
    return nbytes, flops


def decode_algorithmic(NH, dk, dv, esize=2):
    """Bytes per decode step: the fp32 state read and written once, q, k, v, o in the storage type, beta."""
    return NH * (2 * dk * dv * 4 + (2 * dk + 2 * dv) * esize + 4)


PREWARM_S = 0.5   # wall-clock seconds of back-to-back calls before every timed loop


def prewarm(torch, fn, seconds=PREWARM_S, batch=20):
    """Back-to-back calls of fn for at least `seconds` of wall-clock time, so that the timed loop after it runs in
    the GPU's sustained state instead of the slower one after an idle period.  Synchronises after each batch
    except the last, so the GPU is still busy with it when the caller queues its next work.  Returns (seconds,
    calls)."""
    t0 = time.perf_counter()
    calls = 0
    while True:
        for _ in range(batch):
            fn()
        calls += batch
        if time.perf_counter() - t0 >= seconds:
            break
        torch.cuda.synchronize()
    return time.perf_counter() - t0, calls


# kernels whose HBM traffic bench.py reports: the names the profiler may list them under (mangled or
# demangled) and the sources they are built from (the recorded traffic is used only while these still
# hash to what was measured)
TRAFFIC_KERNELS = {
    "chain_bf16_kernel<128,64,64>": {
        "symbol": ["chain_bf16_kernelILi128ELi64ELi64ELb1ELi0E", "chain_bf16_kernel<128, 64, 64, true, 0>"],
        "sources": ["exact_flow_delta_amd/csrc/efla_chain_bf16.hpp", "exact_flow_delta_amd/csrc/efla_chunk_split.hpp",
                    "exact_flow_delta_amd/csrc/efla_common.hpp", "exact_flow_delta_amd/csrc/efla_launch.hpp",
                    "exact_flow_delta_amd/csrc/efla_split_bf16.hip"]},
    "ut_wave_kernel<128,64,diag32>": {
        "symbol": ["ut_wave_kernelILi128ELi64ELb0ELb1E", "ut_wave_kernel<128, 64, false, true>"],
        "sources": ["exact_flow_delta_amd/csrc/efla_ut_wave.hpp", "exact_flow_delta_amd/csrc/efla_chunk_split.hpp",
                    "exact_flow_delta_amd/csrc/efla_common.hpp", "exact_flow_delta_amd/csrc/efla_launch.hpp",
                    "exact_flow_delta_amd/csrc/efla_split_bf16.hip"]},
    "chain_bf16_kernel<128,64,64,utw>": {
        "symbol": ["chain_bf16_kernelILi128ELi64ELi64ELb1ELi2E", "chain_bf16_kernel<128, 64, 64, true, 2>"],
        "sources": ["exact_flow_delta_amd/csrc/efla_chain_bf16.hpp", "exact_flow_delta_amd/csrc/efla_chunk_split.hpp",
                    "exact_flow_delta_amd/csrc/efla_common.hpp", "exact_flow_delta_amd/csrc/efla_launch.hpp",
                    "exact_flow_delta_amd/csrc/efla_ut_wave.hpp", "exact_flow_delta_amd/csrc/efla_chunk_bf16.hip"]},
    "recurrent_step_kernel<bf16,128,128>": {
        "symbol": ["recurrent_step_kernelIDF16bLi128ELi128E", "recurrent_step_kernel<__bf16, 128, 128>"],
        "sources": ["exact_flow_delta_amd/csrc/efla_recurrent.hip", "exact_flow_delta_amd/csrc/efla_common.hpp"]},
}


def _sources_hash(sources):
    import hashlib

    h = hashlib.sha256()
    for src in sources:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def record_traffic(run_dir):
    """profiles/hbm_traffic.json from rocprofv3 FETCH_SIZE / WRITE_SIZE counter CSVs (host only)."""
    import csv
    import glob

    def per_dispatch(sub, counter, match):
        files = glob.glob(os.path.join(run_dir, sub, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit("no counter CSV under %s" % os.path.join(run_dir, sub))
        vals = {}
        with open(files[0]) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] == counter and match(row["Kernel_Name"]):
                    vals[row["Dispatch_Id"]] = vals.get(row["Dispatch_Id"], 0.0) + float(row["Counter_Value"])
        if not vals:
            raise SystemExit("no %s dispatch in %s" % (counter, sub))
        return statistics.mean(vals.values())

    copy_bytes = 512 * 1024 * 1024
    is_copy = lambda n: "copyBuffer" in n  # noqa: E731
    fetch_copy = per_dispatch("fetch_copy", "FETCH_SIZE", is_copy)
    write_copy = per_dispatch("write_copy", "WRITE_SIZE", is_copy)
    out = {
        "note": "HBM bytes per launch from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE (separate runs), each scaled "
                "by the reading of the same counter for a plain 512 MiB device copy; valid only while the kernel "
                "sources hash to 'sources_sha256_16'. Written by bench.py --record-traffic.",
        "copy_calibration": {"bytes": copy_bytes, "FETCH_SIZE_KiB": fetch_copy, "WRITE_SIZE_KiB": write_copy,
                             "read_factor": copy_bytes / (fetch_copy * 1024.0),
                             "write_factor": copy_bytes / (write_copy * 1024.0)},
    }
    rf, wf = out["copy_calibration"]["read_factor"], out["copy_calibration"]["write_factor"]
    for name, info in TRAFFIC_KERNELS.items():
        leg = "dec" if name.startswith("recurrent") else "fwd"
        match = lambda n, syms=info["symbol"]: any(x in n for x in syms)  # noqa: E731
        fk = per_dispatch("fetch_" + leg, "FETCH_SIZE", match)
        wk = per_dispatch("write_" + leg, "WRITE_SIZE", match)
        out[name] = {"sources": info["sources"], "sources_sha256_16": _sources_hash(info["sources"]),
                     "FETCH_SIZE_KiB": fk, "WRITE_SIZE_KiB": wk, "read_bytes": fk * 1024.0 * rf,
                     "write_bytes": wk * 1024.0 * wf, "traffic_bytes": (fk * rf + wk * wf) * 1024.0}
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps({k: (v["traffic_bytes"] if isinstance(v, dict) and "traffic_bytes" in v else None)
                      for k, v in out.items() if k not in ("note",)}))


def record_mfma(run_dir):
    """profiles/mfma_counters.json from one rocprofv3 --pmc run (host only): per dispatch of every kernel in
    TRAFFIC_KERNELS that the run holds, the matrix instructions executed (SQ_INSTS_MFMA), the bf16 matrix work in
    units of 512 flops (SQ_INSTS_VALU_MFMA_MOPS_BF16), the matrix-core busy cycles summed over all SIMDs
    (SQ_VALU_MFMA_BUSY_CYCLES) and the GPU's active cycles (GRBM_GUI_ACTIVE)."""
    import csv
    import glob

    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter CSV under %s" % run_dir)
    rows = []
    with open(files[0]) as f:
        rows = list(csv.DictReader(f))
    counters = ("SQ_INSTS_MFMA", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")
    out = {"note": "Matrix-core counters per launch from one rocprofv3 --pmc run (mean over the kernel's dispatches); "
                   "executed flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; SQ_VALU_MFMA_BUSY_CYCLES is summed over the "
                   "1,024 SIMDs, and bench.py divides it by 1,024 x the average launch time it measures x 2.4 GHz "
                   "(GRBM_GUI_ACTIVE is inflated by the counter run's serialised dispatches and is kept for reference "
                   "only); valid only while the kernel sources hash to 'sources_sha256_16'. Written by "
                   "bench.py --record-mfma."}
    for name, info in TRAFFIC_KERNELS.items():
        per = {}
        for row in rows:
            if any(x in row["Kernel_Name"] for x in info["symbol"]) and row["Counter_Name"] in counters:
                d = per.setdefault(row["Dispatch_Id"], {})
                d[row["Counter_Name"]] = d.get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
        if not per:
            continue
        mean = {c: statistics.mean(d.get(c, 0.0) for d in per.values()) for c in counters}
        out[name] = {"sources": info["sources"], "sources_sha256_16": _sources_hash(info["sources"]),
                     "dispatches": len(per), **mean,
                     "executed_flops": mean["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0}
    path = os.path.join(ROOT, "profiles", "mfma_counters.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps({k: v.get("executed_flops") for k, v in out.items() if isinstance(v, dict)}))


def measured_mfma(kernel):
    """The committed matrix-core counters of `kernel` (profiles/mfma_counters.json), or None when absent or when
    the kernel's sources no longer hash to what was measured."""
    path = os.path.join(ROOT, "profiles", "mfma_counters.json")
    try:
        with open(path) as f:
            entry = json.load(f)[kernel]
        return entry if _sources_hash(entry["sources"]) == entry["sources_sha256_16"] else None
    except (OSError, KeyError, ValueError):
        return None


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary (profiles/hbm_traffic.json),
    or None when the kernel's sources no longer hash to what was measured."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            entry = json.load(f)[kernel]
        return entry["traffic_bytes"] if _sources_hash(entry["sources"]) == entry["sources_sha256_16"] else None
    except (OSError, KeyError, ValueError):
        return None


def mfma_block(flops, tflops, launch_ms, kernel):
    """The matrix-core figures of the headline kernel: the algorithmic flops of a step against the dense bf16 peak,
    and -- from the committed rocprofv3 counters, while they match the kernel's sources -- the flops the matrix
    cores executed per launch over the average launch time measured here, and the matrix cores' busy cycles (summed
    over the 1,024 SIMDs) over that time at the 2.4 GHz peak clock."""
    m = {"algorithmic_tflops": round(tflops, 2), "peak_tflops": BF16_PEAK_TFLOPS,
         "frac": round(tflops / BF16_PEAK_TFLOPS, 4), "flops_per_launch": flops}
    c = measured_mfma(kernel)
    if c is None:
        m.update(executed_flops_per_launch=None, executed_frac=None, busy_frac=None)
    else:
        ex = c["executed_flops"] / (launch_ms * 1e-3) / 1e12
        busy = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * launch_ms * 1e-3 * 2.4e9)
        m.update(executed_flops_per_launch=c["executed_flops"], executed_tflops=round(ex, 2),
                 executed_frac=round(ex / BF16_PEAK_TFLOPS, 4), busy_frac=round(busy, 4),
                 counters="profiles/mfma_counters.json")
    return m


def run_forward(efla, W, torch, steps, warmup):
    w = W.workload(3)
    x = W.make_fwd_inputs(w)

    def dev(a):
        return torch.from_numpy(W.bf16_bits(a)).view(torch.bfloat16).cuda()

    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    beta = torch.from_numpy(x["beta"]).cuda()
    o = torch.empty((w.B, w.H, w.L, w.d_v), dtype=torch.bfloat16, device="cuda")
    S = torch.empty((w.B, w.H, w.d_k, w.d_v), dtype=torch.float32, device="cuda")
    del x
    nbytes = efla.split_workspace_size(w.B, w.H, w.L, w.chunk, torch.bfloat16)
    ws = torch.empty((nbytes,), dtype=torch.uint8, device="cuda")
    nc, nb = (w.L + w.chunk - 1) // w.chunk, (w.chunk // 16) * (w.chunk // 16 + 1) // 2
    t = ws.view(torch.bfloat16).view(w.B, w.H, nc, nb, 64, 4)

    # After an idle period the first ~150 forwards run up to 20 % slower than the steady state that sustained
    # back-to-back calls reach (a few tens of milliseconds in).  Every loop below is therefore preceded by a
    # pre-warm of back-to-back calls for a fixed wall-clock time (PREWARM_S, whatever --warmup says), and then
    # queues its own --warmup calls immediately before its timed calls, with no synchronisation between them:
    # the GPU is still busy when the first event is recorded, so no interval holds host time or an idle gap.
    def one_call(gate=efla.GATE_EXACT):
        # the library's default form for these sizes: the one-launch forward (efla_chunk_fwd)
        efla.chunk_fwd(q, k, v, beta, chunk_size=w.chunk, out=o, final_state=S, gate=gate)

    def split_call():
        efla.chunk_fwd(q, k, v, beta, chunk_size=w.chunk, out=o, final_state=S, workspace=ws, method="split")

    def timed(fn, do_prewarm=True):
        if do_prewarm:
            prewarm(torch, fn)
        for _ in range(warmup):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    def per_launch(fns):
        """Mean time of each of `fns` over `steps` rounds of calling them in turn, events between the calls."""
        prewarm(torch, lambda: [fn() for fn in fns])
        for _ in range(warmup):
            for fn in fns:
                fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(fns) * steps + 1)]
        ev[0].record()
        for i in range(steps):
            for j, fn in enumerate(fns):
                fn()
                ev[len(fns) * i + j + 1].record()
        torch.cuda.synchronize()
        return [[ev[len(fns) * i + j].elapsed_time(ev[len(fns) * i + j + 1]) for i in range(steps)]
                for j in range(len(fns))]

    torch.cuda.synchronize()
    head_prewarm = prewarm(torch, one_call)   # the headline's pre-warm, reported with the line
    ms = timed(one_call, do_prewarm=False)   # the headline: the whole forward, one efla_chunk_fwd call (one kernel) per step
    assert torch.isfinite(S).all().item(), "non-finite final state"
    # the same kernel between HIP events on torch's current stream -- the stream the library launches on -- for
    # its average launch duration
    fused_launch_ms = statistics.mean(per_launch([one_call])[0])

    # the two-launch form (efla_chunk_fwd_split), then its two launches through their own entry points
    # (efla_ut_transform, then efla_chunk_state_pass: bit-identical results) between events
    split_ms = timed(split_call)
    ut_t, chain_t = per_launch([lambda: efla.ut_transform(k, beta, chunk_size=w.chunk, out=t),
                                lambda: efla.state_pass(q, k, v, t, chunk_size=w.chunk, out=o, final_state=S)])
    ut_ms, chain_ms = statistics.mean(ut_t), statistics.mean(chain_t)

    # the delta rule's coefficient alpha = beta (gate 1) on the same kernel: steps of the two gates alternate, so
    # that both see the same clock, and each gate's median step is kept; the same for the one-launch and split
    # forms
    ex_t, dn_t = per_launch([lambda: one_call(efla.GATE_EXACT), lambda: one_call(efla.GATE_DELTANET)])
    alt_exact_ms, deltanet_ms = statistics.median(ex_t), statistics.median(dn_t)
    f_t, s_t = per_launch([one_call, split_call])
    alt_fused_ms, alt_split_ms = statistics.median(f_t), statistics.median(s_t)

    wg, slab, lds = efla.chunk_plan(w.B, w.H, w.L, w.d_k, w.d_v, w.chunk, torch.bfloat16, method="fused")
    return w, ms, dict(prewarm=head_prewarm, fused_launch_ms=fused_launch_ms, split_ms=split_ms, ut_ms=ut_ms, chain_ms=chain_ms,
                       workspace_bytes=nbytes, deltanet_ms=deltanet_ms, alt_exact_ms=alt_exact_ms,
                       alt_fused_ms=alt_fused_ms, alt_split_ms=alt_split_ms,
                       launch=dict(workgroups=wg, slab_width=slab, lds_bytes=lds))


def bwd_algorithmic(B, H, L, dk, dv, C):
    """Flops of one backward pass (efla_chunk_bwd), dense-counted per chunk of C tokens from the products the
    method needs once each: the state recomputation (K S, Ta R, K^T Delta), the state gradient (P = Q K^T,
    P^T dO, K dS', Ta^T dDelta, Q^T dO, K^T dR) and the per-chunk gradients (R, L = K K^T, T (D R), G = T^T
    dDelta, dO S^T, Delta dS'^T, dR S^T, dO Delta^T, G Delta^T, and the four C x C by C x d_k products of dQ
    and dK), 2 flops per multiply-add; the UT transform is counted as in the forward."""
    cdv, ccv, cck = C * dk * dv, C * C * dv, C * C * dk
    per_chunk = 2 * ((2 * cdv + ccv) + (cck + 2 * ccv + 3 * cdv) + (5 * cdv + 5 * ccv + 6 * cck))
    nc = -(-L // C)
    ut = C * C * dk + C ** 3 // 3
    return B * H * nc * (per_chunk + 2 * ut)


def run_backward(efla, W, torch, steps=5, warmup=5):
    """The LM-layer backward (B8 H16 L4096 d128 bf16): one efla_chunk_bwd call per step."""
    w = W.workload(3)
    x = W.make_fwd_inputs(w)
    g = W.make_grads(w)

    def dev(a):
        return torch.from_numpy(W.bf16_bits(a)).view(torch.bfloat16).cuda()

    q, k, v, d_o = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(g["d_o"])
    beta = torch.from_numpy(x["beta"]).cuda()
    dsf = torch.from_numpy(g["d_final"]).cuda()
    del x, g
    need = efla.chunk_bwd_workspace_size(w.B, w.H, w.L, w.d_k, w.d_v, w.chunk, torch.bfloat16)
    ws = torch.empty((need,), dtype=torch.uint8, device="cuda")

    def fn():
        return efla.chunk_bwd(q, k, v, beta, d_o, d_final=dsf, chunk_size=w.chunk, workspace=ws)
    prewarm(torch, fn, batch=2)
    for _ in range(warmup):     # queued right before the timed calls (no idle gap: see run_forward)
        out = fn()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        out = fn()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    assert all(torch.isfinite(t.float()).all().item() for t in out), "non-finite gradients"
    flops = bwd_algorithmic(w.B, w.H, w.L, w.d_k, w.d_v, w.chunk)
    tf = flops / (ms * 1e-3) / 1e12
    # every product of the bf16 backward runs on bf16 matrix cores with fp32 accumulation
    return {"workload": "lm_layer_bwd B8 H16 L4096 d128 bf16 chunk 64 (dq, dk, dv, dbeta, dS0)", "steps": steps,
            "ms_per_step": round(ms, 4), "tokens_per_s": round(w.B * w.L / (ms * 1e-3), 1),
            "workspace_bytes": need,
            "roofline": {"bound": "mfma", "dtype": "bf16", "achieved": round(tf, 2), "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4), "flops_per_call": flops,
                         "scope": "whole call (UT transform with T^T export + 3 launches), dense-counted flops"}}


def run_long_context(efla, W, torch, steps=20, warmup=30):
    """The long-context forward (16 heads x 65,536 tokens): the split forward, whose state pass runs 1,024
    chunks back to back per (head, slab), against the segment-parallel one."""
    w = W.workload(4)
    x = W.make_fwd_inputs(w)

    def dev(a):
        return torch.from_numpy(W.bf16_bits(a)).view(torch.bfloat16).cuda()

    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    beta = torch.from_numpy(x["beta"]).cuda()
    del x
    o = torch.empty((w.B, w.H, w.L, w.d_v), dtype=torch.bfloat16, device="cuda")
    S = torch.empty((w.B, w.H, w.d_k, w.d_v), dtype=torch.float32, device="cuda")
    nseg, seg_chunks, _, need = efla.scan_plan(w.B, w.H, w.L, w.d_k, w.d_v, w.chunk, torch.bfloat16)
    ws = torch.empty((max(need, efla.split_workspace_size(w.B, w.H, w.L, w.chunk, torch.bfloat16)),),
                     dtype=torch.uint8, device="cuda")
    res = {}
    for method in ("split", "scan"):
        def fn():
            efla.chunk_fwd(q, k, v, beta, chunk_size=w.chunk, out=o, final_state=S, workspace=ws, method=method)
        prewarm(torch, fn)
        for _ in range(warmup):     # queued right before the timed calls (no idle gap: see run_forward)
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        res[method] = a.elapsed_time(b) / steps
    assert torch.isfinite(S).all().item(), "non-finite long-context state"
    return {"workload": "long_context B1 H16 L65536 d128 bf16 chunk 64", "steps": steps,
            "split_ms_per_step": round(res["split"], 4), "scan_ms_per_step": round(res["scan"], 4),
            "segments": nseg, "chunks_per_segment": seg_chunks,
            "tokens_per_s_scan": round(w.B * w.L / (res["scan"] * 1e-3), 1),
            "scan_speedup": round(res["split"] / res["scan"], 3)}


def run_small(efla, W, torch, steps=50, warmup=100):
    """The two fp32 parity workloads, timed: the tiny single-head recurrence (B1 H1 L256 d16, chunk 16) and the
    stiff mixed-norm one (B4 H8 L2048 d64, chunk 64, initial state); one efla_chunk_fwd call per step (the form
    the library picks for the sizes, named in the result), median over `steps` HIP-event intervals.  Both are far
    too small to fill the GPU: launch latency and the length of the chunk chain set their times."""
    out = {}
    for cfg, name in ((1, "tiny B1 H1 L256 d16 f32 chunk 16"), (2, "stiff B4 H8 L2048 d64 f32 chunk 64")):
        w = W.workload(cfg)
        x = W.make_fwd_inputs(w)
        q, k, v = (torch.from_numpy(x[n]).cuda() for n in ("q", "k", "v"))
        beta = torch.from_numpy(x["beta"]).cuda()
        s0 = None if x["initial_state"] is None else torch.from_numpy(x["initial_state"]).cuda()
        o = torch.empty((w.B, w.H, w.L, w.d_v), dtype=torch.float32, device="cuda")
        S = torch.empty((w.B, w.H, w.d_k, w.d_v), dtype=torch.float32, device="cuda")
        form, nseg, need = efla.fwd_form(w.B, w.H, w.L, w.d_k, w.d_v, w.chunk, torch.float32)
        ws = torch.empty((max(need, 256),), dtype=torch.uint8, device="cuda")

        def fn():
            efla.chunk_fwd(q, k, v, beta, initial_state=s0, chunk_size=w.chunk, out=o, final_state=S, workspace=ws)
        prewarm(torch, fn)
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record()
        for i in range(steps):
            fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        med = statistics.median(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
        out["cfg%d" % cfg] = {"workload": name, "form": form, "segments": nseg, "median_ms_per_step": round(med, 5),
                              "tokens_per_s": round(w.B * w.L / (med * 1e-3), 1)}
    return out


def run_decode(efla, W, torch, warmup=100):
    w = W.workload(5)
    S = torch.from_numpy(W.make_decode_state(w)).cuda()
    toks = []
    for s in range(w.steps):
        t = W.make_decode_token(w, s)
        toks.append(tuple(torch.from_numpy(W.bf16_bits(t[n])).view(torch.bfloat16).cuda() for n in ("q", "k", "v"))
                    + (torch.from_numpy(t["beta"]).cuda(),))
    o = torch.empty((w.NH, w.d_v), dtype=torch.bfloat16, device="cuda")
    scratch = S.clone()
    torch.cuda.synchronize()
    # warm-up steps on a copy of the state, queued right before the timed steps (no idle gap: see run_forward)
    it = iter(range(1 << 30))
    prewarm(torch, lambda: efla.recurrent_step(*toks[next(it) % w.steps], scratch, out=o))
    for i in range(warmup):
        efla.recurrent_step(*toks[i % w.steps], scratch, out=o)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(w.steps + 1)]
    ev[0].record()
    for s in range(w.steps):
        efla.recurrent_step(*toks[s], S, out=o)
        ev[s + 1].record()
    torch.cuda.synchronize()
    step_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(w.steps)]
    assert torch.isfinite(S).all().item(), "non-finite decode state"
    return w, step_ms


def host_cpu():
    """(CPU model name, CPUs in this process's affinity mask, threads the oracle may use).  The thread count is the
    affinity mask's, lowered to OMP_NUM_THREADS when the environment sets it (the host's share of its cores)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    mask = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "").strip()
    threads = min(mask, int(env)) if env.isdigit() and int(env) > 0 else mask
    return model, mask, threads


def cpu_baseline(W):
    """The fp64 oracle, as it stands, on the host cores: the full LM-layer forward (all heads, full length) --
    the headline's rate --, the decode workload (all 8,192 states, its first 8 steps), and the two small fp32
    workloads on one thread."""
    import oracle

    model, mask, threads = host_cpu()
    w = W.workload(3)
    x = W.make_fwd_inputs(w)
    t0 = time.perf_counter()
    _, _, used = oracle.fwd(x["q"], x["k"], x["v"], x["beta"], None, n_threads=threads, want_o=True,
                            want_state=True)
    dt = time.perf_counter() - t0
    del x
    res = dict(value=w.B * w.L / dt, unit="tokens/s", cores=int(used), kind="oracle",
               sample="full LM-layer forward B8 H16 L4096 d128 (all 128 heads), fp64 token-by-token, %.1f s on %d "
                      "threads" % (dt, used),
               cpu_model=model, affinity_cpus=mask, omp_num_threads=os.environ.get("OMP_NUM_THREADS"))
    # the decode workload: its first 8 dependent steps of all 256 x 32 states (each step streams the 1 GiB fp64
    # state, so the whole 64 would take tens of seconds)
    dw = W.workload(5)
    S = W.make_decode_state(dw).astype("float64")
    nsteps = 8
    toks = [W.make_decode_token(dw, i) for i in range(nsteps)]
    t0 = time.perf_counter()
    for t in toks:
        _, S, dused = oracle.step(t["q"], t["k"], t["v"], t["beta"], S, n_threads=threads)
    ddt = time.perf_counter() - t0
    res["decode"] = {"tokens_per_s": round(dw.B * nsteps / ddt, 1), "seconds": round(ddt, 3), "threads": int(dused),
                     "sample": "decode 256 seq x 32 heads d128, steps 0-7 of 64, fp64"}
    # the small fp32 workloads on one thread (their whole size)
    single = {}
    for cfg in (1, 2):
        sw = W.workload(cfg)
        sx = W.make_fwd_inputs(sw)
        t0 = time.perf_counter()
        _, _, u1 = oracle.fwd(sx["q"], sx["k"], sx["v"], sx["beta"], sx["initial_state"], n_threads=1)
        sdt = time.perf_counter() - t0
        single["cfg%d" % cfg] = {"tokens_per_s": round(sw.B * sw.L / sdt, 1), "seconds": round(sdt, 4),
                                 "threads": int(u1)}
    res["single_thread"] = single
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode workload")
    ap.add_argument("--no-long", action="store_true", help="skip the long-context forward")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward pass")
    ap.add_argument("--only", choices=["fwd", "decode", "copy", "long", "bwd"], default=None,
                    help="run one leg only (for profiling); prints a short JSON line")
    ap.add_argument("--record-traffic", metavar="DIR", default=None,
                    help="write profiles/hbm_traffic.json from rocprofv3 counter CSVs under DIR (host only)")
    ap.add_argument("--record-mfma", metavar="DIR", default=None,
                    help="write profiles/mfma_counters.json from one rocprofv3 matrix-counter run under DIR (host only)")
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(args.record_traffic)
        return
    if args.record_mfma:
        record_mfma(args.record_mfma)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the forward and decode workloads shard across GPUs by independent "
              "heads with no communication, so a multi-GPU figure would be N independent copies; run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_flow_delta_amd as efla
    from exact_flow_delta_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    efla.load_library()

    if args.only == "copy":
        n = 512 * 1024 * 1024 // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"leg": "copy", "bytes_read_per_launch": 4 * n, "bytes_written_per_launch": 4 * n,
                          "launches": args.warmup + args.steps}), flush=True)
        return
    if args.only == "long":
        print(json.dumps({"leg": "long", **run_long_context(efla, W, torch)}), flush=True)
        return
    if args.only == "bwd":
        print(json.dumps({"leg": "bwd", **run_backward(efla, W, torch, steps=args.steps, warmup=args.warmup)}),
              flush=True)
        return
    if args.only == "decode":
        dw, step_ms = run_decode(efla, W, torch)
        print(json.dumps({"leg": "decode", "median_step_ms": statistics.median(step_ms)}), flush=True)
        return

    w, ms, info = run_forward(efla, W, torch, args.steps, args.warmup)
    if args.only == "fwd":
        print(json.dumps({"leg": "fwd", "ms_per_step": ms, **info}), flush=True)
        return
    tokens_per_s = w.B * w.L / (ms * 1e-3)
    nbytes, flops = fwd_algorithmic(w.B, w.H, w.L, w.d_k, w.d_v, w.chunk)
    chain_bytes = chain_algorithmic(w.B, w.H, w.L, w.d_k, w.d_v)
    ut_bytes = ut_algorithmic(w.B, w.H, w.L, w.d_k)
    # the timed region is bracketed by HIP events on the stream the library launches on, and each step is exactly
    # one kernel launch (efla_chunk_fwd's one-launch form), so the region's time per step is the kernel's average
    # launch duration (back to back, any gap between launches included); the average with an event recorded
    # between every two launches is reported beside it (those events add their own cost)
    launch_ms = ms
    fused_gbs = nbytes / (launch_ms * 1e-3) / 1e9
    chain_gbs = chain_bytes / (info["chain_ms"] * 1e-3) / 1e9
    split_ms = info["split_ms"]
    tflops = flops / (ms * 1e-3) / 1e12
    chain_kernel = "chain_bf16_kernel<128,64,64>"
    ut_kernel = "ut_wave_kernel<128,64,diag32>"
    fused_kernel = "chain_bf16_kernel<128,64,64,utw>"
    result = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "lm_layer_fwd", "B": w.B, "H": w.H, "L": w.L, "d_k": w.d_k, "d_v": w.d_v,
                   "chunk": w.chunk, "io": "bf16", "state": "fp32", "method": "fused (one launch)", **info["launch"]},
        # the step is one kernel: its algorithmic bytes (every input read and the outputs written once) over its
        # average launch duration
        "roofline": {"bound": "hbm", "achieved": round(fused_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(fused_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(fused_kernel),
                     "kernel": fused_kernel, "bytes_per_launch": nbytes,
                     "avg_launch_ms": round(launch_ms, 5),
                     "avg_launch_ms_events_between": round(info["fused_launch_ms"], 5)},
        # the two-launch form (efla_chunk_fwd_split) on the same inputs: the state pass's roofline, and the UT
        # launch, which forms only the diagonal 32 x 32 blocks of each chunk's T diag(alpha) (the stand-alone
        # efla_ut_transform entry, timed between events, is the same kernel on all blocks: an upper bound; the
        # split step minus the state pass estimates it)
        "split": {"entry": "efla_chunk_fwd_split (UT launch, then the state pass)", "ms_per_step": round(split_ms, 5),
                  "tokens_per_s": round(w.B * w.L / (split_ms * 1e-3), 1),
                  # steps of the two forms alternating, median of each
                  "alternating_median_ms": {"one_launch": round(info["alt_fused_ms"], 5),
                                            "split": round(info["alt_split_ms"], 5)},
                  "workspace_written_bytes": info["workspace_bytes"] * 6 // 10,
                  "state_pass": {"kernel": chain_kernel, "bytes_per_launch": chain_bytes,
                                 "avg_launch_ms": round(info["chain_ms"], 5), "achieved_gbs": round(chain_gbs, 1),
                                 "frac": round(chain_gbs / HBM_PEAK_GBS, 4),
                                 "traffic": measured_traffic(chain_kernel)},
                  "ut": {"kernel": ut_kernel, "entry_avg_launch_ms": round(info["ut_ms"], 5),
                         "in_step_est_ms": round(split_ms - info["chain_ms"], 5), "bytes_per_launch": ut_bytes,
                         "achieved_gbs_est": round(ut_bytes / (max(split_ms - info["chain_ms"], 1e-6) * 1e-3) / 1e9,
                                                   1),
                         "traffic": measured_traffic(ut_kernel)}},
        "deltanet_gate": {"median_ms_per_step": round(info["deltanet_ms"], 5),
                          "exact_median_ms_per_step": round(info["alt_exact_ms"], 5),
                          "exact_over_deltanet": round(info["alt_exact_ms"] / info["deltanet_ms"], 4)},
        "mfma": mfma_block(flops, tflops, launch_ms, fused_kernel),
        "prewarm": {"seconds": round(info["prewarm"][0], 3), "calls": info["prewarm"][1]},
    }
    if not args.no_decode:
        dw, step_ms = run_decode(efla, W, torch)
        med = statistics.median(step_ms)
        dbytes = decode_algorithmic(dw.NH, dw.d_k, dw.d_v)
        gbs = dbytes / (med * 1e-3) / 1e9
        result["decode"] = {
            "workload": "decode 256 seq x 32 heads d128, fp32 state, 64 steps",
            "median_step_ms": round(med, 5), "total_ms": round(sum(step_ms), 4),
            "tokens_per_s": round(dw.B / (med * 1e-3), 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("recurrent_step_kernel<bf16,128,128>"),
                         "kernel": "recurrent_step_kernel<bf16,128,128>", "bytes_per_launch": dbytes},
        }
    if not args.no_long:
        result["long_context"] = run_long_context(efla, W, torch)
    result["small_fp32"] = run_small(efla, W, torch)
    if not args.no_bwd:
        result["backward"] = run_backward(efla, W, torch)
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(W)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
