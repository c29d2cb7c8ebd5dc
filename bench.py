"""Benchmark of the gated delta-rule hot path on one MI355X.

One step = the whole path over one batch of synthetic input:
  * the chunked forward (prefill) of the Kaczmarz layer, B=1, H=16, T=65536,
    d_k = d_v = 128, bf16 q/k/v, fp32 gates and state, writing o and S_T;
  * 1024 single-token decode steps at batch 64 (16 heads), each a
    read-modify-write of the 64 x 16 x 128 x 128 fp32 state in HBM, each with
    its own pre-generated q, k, v, eta, alpha.

The JSON line reports whole-step throughput (prefill tokens + decode tokens per
second), the prefill and decode figures separately, a roofline entry for the
dominant kernel (decode: HBM-bound) timed with HIP events on the launch stream,
and the CPU oracle timed on a bounded sample of the same work.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--no-cpu]
    python bench.py --long-context [--steps 20] [--warmup 3]
    python bench.py --backward [--steps 10] [--warmup 2]
    python bench.py --routing [--steps 20] [--warmup 3]
    python bench.py --cold-decode [--steps 200] [--warmup 1]
    python bench.py --few-heads [--steps 20] [--warmup 3]

The second form measures the long-context shapes instead (131,072-token
prefill, single-sequence decode from position 32,768, Kaczmarz LA against Gated
DeltaNet) and prints its own JSON line.  The third measures the gradient of the
chunked forward on the same Kaczmarz prefill (upstream gradients for o and S_T
given) and prints its own JSON line.  The fourth measures what cross-layer
routing costs on the same Kaczmarz layer: the prefill and the batch-64 decode
step with a routed value added on load and the per-token written residual
stored, against the plain calls.  The fifth times single decode launches with
the state evicted from the last-level cache before each one, beside the same
launches warm, and measures the box's own copy bandwidth and GEMM rate.  The
sixth times only the prefills with few heads per device (the Kaczmarz layer at
4 and 2 heads), which the default run also reports as forward_few_heads, and
their gradients and saving forwards.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12          # B/s, MI355X HBM3E
PEAK_BF16 = 2.5e15         # FLOP/s, dense bf16 matrix cores
PEAK_FP32_MATRIX = 157.3e12  # FLOP/s, fp32 matrix cores
C = 64                     # chunk length


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def forward_flops_per_head_token(dk, dv, c=C):
    """Algorithmic FLOPs of the chunked method per head-token: the needed
    triangles of A, P, W, U~, P Delta, the three state products and the
    triangular solve."""
    return 2 * ((c - 1) / 2 * dk + (c + 1) / 2 * dk + (c + 1) / 2 * dk + (c + 1) / 2 * dv
                + (c + 1) / 2 * dv + 3 * dk * dv + c * c / 6)


def forward_bytes(B, T, H, dk, dv, in_bytes=2, channel_decay=False):
    """Algorithmic HBM bytes of one forward: q, k, v read and o written once,
    gates read once, S_0 absent (zeros), S_T written."""
    tok = B * T * H
    gates = 4 * (dk if channel_decay else 1) + 4  # alpha + eta
    return tok * (in_bytes * (2 * dk + 2 * dv) + gates) + B * H * dk * dv * 4


def forward_bytes_variant(variant, B, T, H, dk, dv, in_bytes):
    """Algorithmic HBM bytes of one forward of any variant: q, k, v read and o
    written once, each gate tensor the variant takes read once (alpha per
    token or per key channel, beta/eta per token, GDN-2's erase gate per key
    and write gate per value channel), S_0 absent, S_T written."""
    tok = B * T * H
    gates = {"deltanet": 4, "gated_deltanet": 8, "kla": 8, "kda": 4 * dk + 4,
             "gdn2": 4 * dk + 4 * dk + 4 * dv}[variant]
    return tok * (in_bytes * (2 * dk + 2 * dv) + gates) + B * H * dk * dv * 4


def decode_bytes(B, H, dk, dv, in_bytes=2):
    """Algorithmic HBM bytes of one decode step: state read + write, q, k, v
    read, o written, two scalar gates."""
    return B * H * (2 * dk * dv * 4 + in_bytes * (dk + dk + dv + dv) + 8)


def measured_traffic(kernel: str, source: str):
    """HBM bytes per dispatch of `kernel` from the committed counter summary,
    or None if the kernel source has changed since the counters were taken."""
    import glob
    import hashlib
    try:
        sha = hashlib.sha1(open(os.path.join(ROOT, source), "rb").read()).hexdigest()[:12]
    except OSError:
        return None
    for path in glob.glob(os.path.join(ROOT, "profiles", "hbm_counters_*.txt")):
        for line in open(path):
            parts = line.split()
            if len(parts) == 4 and parts[0] == "traffic" and parts[1] == kernel:
                kv = dict(x.split("=", 1) for x in parts[2:])
                if kv.get("source_sha1") == sha:
                    return int(kv["bytes_per_dispatch"])
    return None


def git_sha():
    try:
        return subprocess.run(["git", "rev-parse", "--short", "HEAD"], cwd=ROOT,
                              capture_output=True, text=True).stdout.strip() or None
    except Exception:
        return None


def cpu_baseline(wl, T_sample, decode_steps_sample, threads):
    """Time the oracle on a bounded sample: the first T_sample tokens of the
    prefill (all heads) and decode_steps_sample decode steps (all 64 x 16
    heads), then scale to one full step of the workload."""
    import numpy as np

    from gated_delta_rule_85_amd.inputs import make_decode_inputs, make_inputs
    from oracle import oracle

    oracle.load()
    inp = make_inputs(wl.variant, 1, T_sample, wl.H, wl.dk, wl.dv, wl.dtype, seed=wl.seed,
                      alpha_scale=wl.alpha_scale, eps=wl.eps,
                      unnormalised_keys=wl.unnormalised_keys)
    t0 = time.perf_counter()
    _, s_T = oracle.forward(wl.variant, inp["q"], inp["k"], inp["v"], alpha=inp["alpha"],
                            beta=inp["beta"], eps=inp["eps"], threads=threads)
    t_pre = time.perf_counter() - t0
    dec = make_decode_inputs(wl, steps=decode_steps_sample)
    Bd = wl.decode["B"]
    state = np.broadcast_to(s_T, (Bd,) + s_T.shape[1:]).copy()
    t0 = time.perf_counter()
    for s in range(decode_steps_sample):
        _, state = oracle.forward(wl.variant, dec["q"][s], dec["k"][s], dec["v"][s],
                                  alpha=dec["alpha"][s], beta=dec["beta"][s], eps=dec["eps"],
                                  state_in=state, threads=threads)
    t_dec = time.perf_counter() - t0
    t_step = t_pre * (wl.T / T_sample) + t_dec * (wl.decode["steps"] / decode_steps_sample)
    tokens = wl.B * wl.T + Bd * wl.decode["steps"]
    return dict(value=tokens / t_step, unit="tokens/s", cores=min(threads, Bd * wl.H),
                kind="oracle",
                sample=(f"float64 oracle: prefill of the first {T_sample} of {wl.T} tokens "
                        f"(16 heads, {min(threads, wl.H)} threads, {t_pre:.1f} s) and "
                        f"{decode_steps_sample} of {wl.decode['steps']} decode steps at batch "
                        f"{Bd} ({min(threads, Bd * wl.H)} threads, {t_dec:.1f} s), scaled "
                        f"linearly to one full step"),
                prefill_tokens_per_s=wl.B * T_sample / t_pre,
                decode_tokens_per_s=Bd * decode_steps_sample / t_dec)


def long_context(args):
    """The pages' efficiency comparison at kernel level: prefill latency of a
    131,072-token context and single-sequence decode throughput from the state
    at position 32,768, for the Kaczmarz layer and its Gated DeltaNet
    counterpart (same shapes; only the step size differs).  Prints one JSON
    line."""
    import torch

    from gated_delta_rule_85_amd import binding
    from gated_delta_rule_85_amd.inputs import WORKLOADS, make_decode_inputs, make_workload

    L = binding.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sh = torch.cuda.current_stream().cuda_stream
    ev = lambda: torch.cuda.Event(enable_timing=True)
    res = {}
    for wid in (6, 7):
        wl = WORKLOADS[wid]
        B, T, H, dk, dv = wl.B, wl.T, wl.H, wl.dk, wl.dv
        log(f"{wl.name}: generating the {T}-token prefill")
        d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v)
             for k, v in make_workload(wl).items()}
        o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
        s_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
        fa = binding.make_args(wl.variant, d["q"], d["k"], d["v"], o, d["alpha"], d["beta"],
                               None, None, d["eps"], None, s_T)
        binding.check(binding.gdr_check_args(fa, 0))
        nws = binding.gdr_forward_workspace_size(fa)
        ws = torch.empty(nws, dtype=torch.uint8, device=dev)
        for _ in range(args.warmup):
            binding.check(L.gdr_forward_chunked(ctypes.byref(fa), ws.data_ptr(), nws, sh))
        e0, e1 = ev(), ev()
        e0.record()
        for _ in range(args.steps):
            L.gdr_forward_chunked(ctypes.byref(fa), ws.data_ptr(), nws, sh)
        e1.record()
        torch.cuda.synchronize()
        pre_s = e0.elapsed_time(e1) / 1e3 / args.steps
        del d, o, ws

        pos, Bd, Sd = wl.decode["position"], wl.decode["B"], wl.decode["steps"]
        log(f"{wl.name}: prefill of {pos} tokens, then {Sd} decode steps at batch {Bd}")
        d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v)
             for k, v in make_workload(wl, T=pos).items()}
        _, s_pos = binding.forward(wl.variant, d["q"], d["k"], d["v"], alpha=d["alpha"],
                                   beta=d["beta"], eps=d["eps"])
        del d
        state = s_pos.expand(Bd, H, dk, dv).contiguous()
        dd = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v)
              for k, v in make_decode_inputs(wl).items()}
        o_dec = torch.empty((Sd, Bd, 1, H, dv), dtype=torch.bfloat16, device=dev)
        dargs = [binding.make_args(wl.variant, dd["q"][i], dd["k"][i], dd["v"][i], o_dec[i],
                                   dd["alpha"][i], dd["beta"][i], None, None, dd["eps"],
                                   state, state) for i in range(Sd)]
        for a in dargs:
            binding.check(binding.gdr_check_args(a, 1))
        refs = [ctypes.byref(a) for a in dargs]

        def block(handle):
            for r in refs:
                rc = L.gdr_decode_step(r, handle)
                if rc:
                    binding.check(rc)

        block(sh)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            block(torch.cuda.current_stream().cuda_stream)
        for _ in range(args.warmup):
            graph.replay()
        e0, e1 = ev(), ev()
        e0.record()
        for _ in range(args.steps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        dec_s = e0.elapsed_time(e1) / 1e3 / (args.steps * Sd)
        fl = forward_flops_per_head_token(dk, dv) * B * T * H
        fb = forward_bytes(B, T, H, dk, dv)
        res[wl.variant] = dict(
            workload=wl.name,
            prefill=dict(T=T, ms=pre_s * 1e3, tokens_per_s=B * T / pre_s,
                         tflops=fl / pre_s / 1e12, mfma_frac=fl / pre_s / PEAK_BF16,
                         hbm_frac=fb / pre_s / PEAK_HBM),
            decode=dict(position=pos, batch=Bd, steps=Sd, us_per_step=dec_s * 1e6,
                        tokens_per_s=Bd / dec_s,
                        hbm_frac=decode_bytes(Bd, H, dk, dv) / dec_s / PEAK_HBM))
        del state, dd, o_dec, graph
        torch.cuda.empty_cache()
    k, g = res["kla"], res["gated_deltanet"]
    out = {
        "metric": "131K-token prefill latency and decode throughput at position 32K, "
                  "Kaczmarz LA vs Gated DeltaNet (one layer, kernel level)",
        "value": k["prefill"]["ms"], "unit": "ms (Kaczmarz LA prefill, 131072 tokens)",
        "higher_is_better": False, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "B=1 H=16 d_k=d_v=128 bf16 layer; prefill T=131072; "
                               "decode at batch 1 from the state after 32768 tokens"},
        "kla": k, "gated_deltanet": g,
        "ratios": {"prefill_latency_kla_over_gdn": k["prefill"]["ms"] / g["prefill"]["ms"],
                   "decode_throughput_kla_over_gdn":
                       k["decode"]["tokens_per_s"] / g["decode"]["tokens_per_s"]},
        "git": git_sha(),
    }
    print(json.dumps(out))


def backward_flops_per_chunk_head(dk, dv, c=C, scalar_decay=True):
    """Algorithmic FLOPs of the per-chunk gradient step, counting only the
    needed triangles: the three C x dk products over dv (dQt, dW, dKbar), dP
    and dT_u over dv, the Gram products A (and P for a scalar decay), the
    triangular solve, dT += dW At^T, T^T dW, T^T dDelta, dA = -T^T dT T^T and
    the Gram backward (dA Xk, dP Xk, dA^T Xa, dP^T Xq)."""
    lo_inc, lo_str = c * (c + 1) / 2, c * (c - 1) / 2
    f = 3 * 2 * c * dv * dk                       # dQt, dW, dKbar
    f += 2 * lo_inc * dv + 2 * lo_str * dv        # dP, dT_u
    f += 2 * lo_str * dk + (2 * lo_inc * dk if scalar_decay else 0)   # A (, P)
    f += c ** 3 / 3                               # solve
    f += 2 * lo_str * dk + 2 * lo_inc * dk + 2 * lo_inc * dv   # dT, T^T dW, T^T dDelta
    f += 2 * c ** 3 / 3                           # dT T^T, T^T (.)
    f += 2 * (2 * lo_str * dk + 2 * lo_inc * dk)  # Gram backward
    return f


def backward(args):
    """Gradient of the chunked forward on the Kaczmarz prefill (B=1, H=16,
    T=65536, d=128, bf16): upstream gradients for o and S_T in, every input
    gradient out (fp32).  The forward on the same inputs is timed beside it,
    and so is the training pair that keeps the forward's records for the
    gradient (gdr_forward_chunked_save, then gdr_backward_chunked_saved in the
    same workspace) against forward + gradient.  Prints one JSON line."""
    import torch

    from gated_delta_rule_85_amd import binding
    from gated_delta_rule_85_amd.inputs import WORKLOADS, make_upstream_grads, make_workload

    L = binding.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sh = torch.cuda.current_stream().cuda_stream
    wl = WORKLOADS[5]
    B, T, H, dk, dv = wl.B, wl.T, wl.H, wl.dk, wl.dv
    log(f"{wl.name}: generating inputs and upstream gradients")
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in make_workload(wl).items()}
    up = {k: v.to(dev) for k, v in make_upstream_grads(B, T, H, dk, dv, wl.dtype,
                                                         seed=wl.seed + 1).items()}
    o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
    s_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    fa = binding.make_args(wl.variant, d["q"], d["k"], d["v"], o, d["alpha"], d["beta"], None,
                           None, d["eps"], None, s_T)
    binding.check(binding.gdr_check_args(fa, 0))
    nfw = binding.gdr_forward_workspace_size(fa)
    ba = binding.make_args(wl.variant, d["q"], d["k"], d["v"], None, d["alpha"], d["beta"], None,
                           None, d["eps"], None, None)
    nbw = binding.gdr_backward_workspace_size(ba)
    ws = torch.empty(max(nfw, nbw), dtype=torch.uint8, device=dev)
    f32 = torch.float32
    gr = {n: torch.empty(shape, dtype=f32, device=dev) for n, shape in
          (("q", (B, T, H, dk)), ("k", (B, T, H, dk)), ("v", (B, T, H, dv)), ("alpha", (B, T, H)),
           ("beta", (B, T, H)), ("s0", (B, H, dk, dv)))}
    ga = binding.GdrGrads(up["d_o"].data_ptr(), up["d_state_out"].data_ptr(), gr["q"].data_ptr(),
                          gr["k"].data_ptr(), gr["v"].data_ptr(), gr["alpha"].data_ptr(),
                          gr["beta"].data_ptr(), None, None, gr["s0"].data_ptr())
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / args.steps

    log(f"timing the forward and the gradient ({args.steps} steps each)")
    fw_s = timed(lambda: binding.check(L.gdr_forward_chunked(ctypes.byref(fa), ws.data_ptr(),
                                                             nfw, sh)))
    bw_s = timed(lambda: binding.check(L.gdr_backward_chunked(ctypes.byref(ba), ctypes.byref(ga),
                                                              ws.data_ptr(), nbw, sh)))
    fs_s = timed(lambda: binding.check(L.gdr_forward_chunked_save(ctypes.byref(fa), ws.data_ptr(),
                                                                  nbw, sh)))

    def pair():
        binding.check(L.gdr_forward_chunked_save(ctypes.byref(fa), ws.data_ptr(), nbw, sh))
        binding.check(L.gdr_backward_chunked_saved(ctypes.byref(ba), ctypes.byref(ga),
                                                   ws.data_ptr(), nbw, sh))

    pair_s = timed(pair)
    plain_pair_s = fw_s + bw_s
    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 268435456 bytes read and written")
        del src, dst
    finite = all(bool(torch.isfinite(t).all()) for t in gr.values())
    nch = B * H * ((T + C - 1) // C)
    out = {
        "metric": "gradient throughput of the chunked forward (tokens/s, one layer)",
        "value": B * T / bw_s, "unit": "tokens/s", "higher_is_better": True, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name.split("_decode")[0] + "; upstream gradients for o and "
                               "S_T; gradients w.r.t. q, k, v, eta, alpha and S_0 in fp32"},
        "backward_ms": bw_s * 1e3, "forward_ms": fw_s * 1e3,
        "backward_over_forward": bw_s / fw_s,
        "saved": {"note": "gdr_forward_chunked_save then gdr_backward_chunked_saved in one "
                          "workspace, timed as a pair; the saved gradient alone is the pair "
                          "minus the saving forward timed by itself",
                  "forward_save_ms": fs_s * 1e3, "pair_ms": pair_s * 1e3,
                  "backward_saved_ms": (pair_s - fs_s) * 1e3,
                  "forward_plus_backward_ms": plain_pair_s * 1e3,
                  "pair_speedup": plain_pair_s / pair_s},
        "chunk_grad_flops": backward_flops_per_chunk_head(dk, dv) * nch,
        "workspace_bytes": nbw, "outputs_finite": finite, "git": git_sha(),
    }
    print(json.dumps(out))


def routing(args):
    """Cost of cross-layer routing on the Kaczmarz layer: prefill (B=1, H=16,
    T=65536) and one decode step at batch 64, each plain, with the residual
    output, and with the routed value plus the residual output.  Prints one
    JSON line."""
    import torch

    from gated_delta_rule_85_amd import binding
    from gated_delta_rule_85_amd.inputs import (WORKLOADS, make_decode_inputs, make_routed_value,
                                                make_workload)

    L = binding.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sh = torch.cuda.current_stream().cuda_stream
    wl = WORKLOADS[5]
    B, T, H, dk, dv = wl.B, wl.T, wl.H, wl.dk, wl.dv
    log(f"{wl.name}: generating inputs and a routed value")
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in make_workload(wl).items()}
    vr = make_routed_value(B, T, H, dv, wl.dtype, seed=wl.seed + 2).to(dev)
    o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
    delta = torch.empty_like(o)
    s_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def timed(fn, reps):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / reps

    pre = {}
    for name, r, dl in (("plain", None, None), ("residual_out", None, delta),
                        ("routed_value_and_residual_out", vr, delta)):
        a = binding.make_args(wl.variant, d["q"], d["k"], d["v"], o, d["alpha"], d["beta"], None,
                              None, d["eps"], None, s_T, v_route=r, delta_out=dl)
        binding.check(binding.gdr_check_args(a, 0))
        n = binding.gdr_forward_workspace_size(a)
        ws = torch.empty(n, dtype=torch.uint8, device=dev)
        pre[name] = timed(lambda: binding.check(L.gdr_forward_chunked(ctypes.byref(a), ws.data_ptr(),
                                                                     n, sh)), args.steps) * 1e3
        del ws
    del d, vr, o, delta
    Bd = wl.decode["B"]
    dd = {k: (v[0].to(dev) if isinstance(v, torch.Tensor) else v)
          for k, v in make_decode_inputs(wl, steps=1).items()}
    state = torch.zeros((Bd, H, dk, dv), dtype=torch.float32, device=dev)
    od = torch.empty((Bd, 1, H, dv), dtype=torch.bfloat16, device=dev)
    vrd = make_routed_value(Bd, 1, H, dv, wl.dtype, seed=wl.seed + 3).to(dev)
    dld = torch.empty_like(od)
    dec = {}
    for name, r, dl in (("plain", None, None), ("residual_out", None, dld),
                        ("routed_value_and_residual_out", vrd, dld)):
        a = binding.make_args(wl.variant, dd["q"], dd["k"], dd["v"], od, dd["alpha"], dd["beta"],
                              None, None, dd["eps"], state, state, v_route=r, delta_out=dl)
        binding.check(binding.gdr_check_args(a, 1))
        dec[name] = timed(lambda: binding.check(L.gdr_decode_step(ctypes.byref(a), sh)),
                          args.steps * 20) * 1e6
    out = {
        "metric": "cost of cross-layer routing (routed value on load, per-token residual out)",
        "value": pre["routed_value_and_residual_out"] / pre["plain"], "unit": "prefill time ratio",
        "higher_is_better": False, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "Kaczmarz LA layer B=1 H=16 T=65536 d=128 bf16 prefill; decode "
                               "step at batch 64 (inputs of one step, repeated)"},
        "prefill_ms": pre, "decode_us": dec,
        "bytes_added": {"prefill_routed_value": B * T * H * dv * 2,
                        "prefill_residual_out": B * T * H * dv * 2,
                        "decode_routed_value": Bd * H * dv * 2, "decode_residual_out": Bd * H * dv * 2},
        "git": git_sha(),
    }
    print(json.dumps(out))


def state_rmw_reference(dev, stream, n_floats, n_cold, flush):
    """The plainest pass over memory of the decode state's size: torch's
    in-place multiply of an fp32 tensor of n_floats elements (read once,
    written once), back to back (warm: the tensor stays in the last-level
    cache) and as single launches after a read sweep of `flush` (cold).  The
    decode step is this read-modify-write plus its per-token inputs and
    arithmetic, so the ratio of the two rates is how close the decode comes
    to streaming its state."""
    import torch

    x = torch.full((n_floats,), 0.5, dtype=torch.float32, device=dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    for _ in range(5):
        x.mul_(1.0)
    e0, e1 = ev(), ev()
    e0.record(stream)
    for _ in range(100):
        x.mul_(1.0)
    e1.record(stream)
    torch.cuda.synchronize()
    warm_s = e0.elapsed_time(e1) / 1e3 / 100
    pairs = [(ev(), ev()) for _ in range(n_cold)]
    for s in range(n_cold):
        flush.sum()
        pairs[s][0].record(stream)
        x.mul_(1.0)
        pairs[s][1].record(stream)
    torch.cuda.synchronize()
    cold_s = sorted(a.elapsed_time(b) for a, b in pairs)[n_cold // 2] / 1e3
    nb = 2 * n_floats * 4
    del x
    return dict(note=f"torch in-place multiply of {n_floats * 4 >> 20} MiB fp32 (the batch "
                     "state's size), bytes read plus written; warm back to back, cold after "
                     "the same read sweep (median)",
                warm_us=warm_s * 1e6, cold_us=cold_s * 1e6, warm_GBps=nb / warm_s / 1e9,
                cold_GBps=nb / cold_s / 1e9)


def cold_decode(args):
    """Decode step of the Kaczmarz layer at batch 64 with the state cold: the
    64 MiB state fits in the 256 MiB last-level cache (MALL), so back-to-back
    steps find it there.  Here every step is preceded by a read sweep over a
    1 GiB buffer, which evicts the state to HBM, and each decode launch is timed
    on its own with HIP events on the launch stream; the same per-launch timing
    without the sweep gives the warm figure.  Also measures the box's own
    peaks: HBM copy and read bandwidth over buffers far larger than the MALL,
    and a large bf16 library GEMM.  Prints one JSON line."""
    import torch

    from gated_delta_rule_85_amd import binding
    from gated_delta_rule_85_amd.inputs import WORKLOADS, make_decode_inputs, make_workload

    L = binding.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    wl = WORKLOADS[5]
    B, T, H, dk, dv = wl.B, wl.T, wl.H, wl.dk, wl.dv
    Bd, n = wl.decode["B"], args.steps
    ev = lambda: torch.cuda.Event(enable_timing=True)

    # The decode starts from the prefill's final state, as in the main bench.
    log("prefill for the starting state")
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in make_workload(wl).items()}
    o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
    s_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    fa = binding.make_args(wl.variant, d["q"], d["k"], d["v"], o, d["alpha"], d["beta"], None,
                           None, d["eps"], None, s_T)
    nws = binding.gdr_forward_workspace_size(fa)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    binding.check(L.gdr_forward_chunked(ctypes.byref(fa), ws.data_ptr(), nws, sh))
    torch.cuda.synchronize()
    del d, o, ws
    dd = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v)
          for k, v in make_decode_inputs(wl, steps=n).items()}
    state = torch.empty((Bd, H, dk, dv), dtype=torch.float32, device=dev)
    state.copy_(s_T.expand(Bd, H, dk, dv))
    o_dec = torch.empty((n, Bd, 1, H, dv), dtype=torch.bfloat16, device=dev)
    dargs = [binding.make_args(wl.variant, dd["q"][s], dd["k"][s], dd["v"][s], o_dec[s],
                               dd["alpha"][s], dd["beta"][s], None, None, dd["eps"], state, state)
             for s in range(n)]
    for a in dargs:
        binding.check(binding.gdr_check_args(a, 1))
    flush = torch.ones(256 << 20, dtype=torch.float32, device=dev)   # 1 GiB

    def per_launch(cold):
        evs = [(ev(), ev()) for _ in range(n)]
        for s in range(n):
            if cold:
                flush.sum()
            evs[s][0].record(stream)
            binding.check(L.gdr_decode_step(ctypes.byref(dargs[s]), sh))
            evs[s][1].record(stream)
        torch.cuda.synchronize()
        us = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
        return dict(median_us=us[n // 2], mean_us=sum(us) / n, min_us=us[0], max_us=us[-1])

    for _ in range(args.warmup):
        per_launch(True)
    log(f"{n} decode launches each, warm and cold")
    warm = per_launch(False)
    cold = per_launch(True)
    db = decode_bytes(Bd, H, dk, dv)
    for r in (warm, cold):
        r["GBps_algorithmic"] = db / (r["median_us"] * 1e-6) / 1e9
        r["hbm_frac"] = db / (r["median_us"] * 1e-6) / PEAK_HBM

    # Box-measured peaks.
    def rate(fn, reps=20):
        fn()
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / reps

    rmw = state_rmw_reference(dev, stream, Bd * H * dk * dv, n, flush)
    del flush
    log("measuring HBM copy / read bandwidth and a bf16 GEMM")
    src = torch.ones(512 << 20, dtype=torch.float32, device=dev)   # 2 GiB
    dst = torch.empty_like(src)
    t_copy = rate(lambda: dst.copy_(src))
    t_read = rate(lambda: src.sum())
    del src, dst
    a = torch.randn(8192, 8192, dtype=torch.bfloat16, device=dev)
    bt = torch.randn(8192, 8192, dtype=torch.bfloat16, device=dev)
    t_mm = rate(lambda: torch.mm(a, bt), reps=10)
    peaks = dict(copy_GBps=2 * (2 << 30) / t_copy / 1e9, read_GBps=(2 << 30) / t_read / 1e9,
                 bf16_gemm_8192_TFLOPs=2 * 8192 ** 3 / t_mm / 1e12,
                 note="copy counts bytes read plus written over 2 GiB buffers; GEMM is "
                      "torch.mm (hipBLASLt) at 8192^3")
    out = {
        "metric": "decode step with the state evicted from the last-level cache",
        "value": cold["median_us"], "unit": "us per decode step (median, cold state)",
        "higher_is_better": False, "n_gpus": 1, "steps": n, "warmup": args.warmup,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "Kaczmarz LA decode step, batch 64, 16 heads, d=128, fp32 state "
                               "from the T=65536 prefill; a 1 GiB read sweep before each cold "
                               "launch"},
        "warm": warm, "cold": cold, "algorithmic_bytes": db, "state_rmw_reference": rmw,
        "frac_of_state_rmw": {"warm": warm["GBps_algorithmic"] / rmw["warm_GBps"],
                              "cold": cold["GBps_algorithmic"] / rmw["cold_GBps"]},
        "measured_peaks": peaks, "git": git_sha(),
    }
    print(json.dumps(out))


def _time_forward(L, dev, sh, variant, dtype, d, steps, warmup):
    """One forward configuration timed with HIP events on the launch stream: a
    HIP graph of `steps` calls replayed (device time per forward, the figure
    the rates use), and the same calls launched one by one from the host after
    `warmup` untimed ones (ms_eager)."""
    import torch

    from gated_delta_rule_85_amd import binding

    B, T, H, dk = d["q"].shape
    dv = d["v"].shape[-1]
    o = torch.empty((B, T, H, dv), dtype=d["q"].dtype, device=dev)
    s_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    a = binding.make_args(variant, d["q"], d["k"], d["v"], o, d["alpha"], d["beta"],
                          d["erase_b"], d["write_w"], d["eps"], None, s_T)
    binding.check(binding.gdr_check_args(a, 0))
    n = binding.gdr_forward_workspace_size(a)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    ref = ctypes.byref(a)
    for _ in range(warmup):
        binding.check(L.gdr_forward_chunked(ref, ws.data_ptr(), n, sh))
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        L.gdr_forward_chunked(ref, ws.data_ptr(), n, sh)
    e1.record()
    torch.cuda.synchronize()
    t_eager = e0.elapsed_time(e1) / 1e3 / steps
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gs = torch.cuda.current_stream().cuda_stream
        for _ in range(steps):
            binding.check(L.gdr_forward_chunked(ref, ws.data_ptr(), n, gs))
    graph.replay()
    torch.cuda.synchronize()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3 / steps
    del graph, o, s_T, ws
    in_bytes = 2 if dtype == "bf16" else 4
    fl = forward_flops_per_head_token(dk, dv) * B * T * H
    fb = forward_bytes_variant(variant, B, T, H, dk, dv, in_bytes)
    peak_mm = PEAK_BF16 if dtype == "bf16" else PEAK_FP32_MATRIX
    return dict(variant=variant, dtype=dtype, B=B, T=T, H=H, dk=dk, dv=dv,
                ms=t * 1e3, ms_eager=t_eager * 1e3, tokens_per_s=B * T / t,
                tflops=fl / t / 1e12, mfma_frac=fl / t / peak_mm,
                mfma_peak_TFLOPs=peak_mm / 1e12, hbm_GBps=fb / t / 1e9,
                hbm_frac=fb / t / PEAK_HBM, algorithmic_flop=fl, algorithmic_bytes=fb,
                workspace_bytes=n)


def other_workloads(L, dev, sh, steps, warmup):
    """The forward of workloads 1-4 (DeltaNet fp32, Gated DeltaNet, KDA,
    Gated DeltaNet-2), each timed by _time_forward (for the smallest workload
    the host's per-call cost exceeds the device time, hence ms_eager)."""
    import torch

    from gated_delta_rule_85_amd.inputs import WORKLOADS, make_workload

    res = {}
    for wid in (1, 2, 3, 4):
        wl = WORKLOADS[wid]
        d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v)
             for k, v in make_workload(wl).items()}
        r = _time_forward(L, dev, sh, wl.variant, wl.dtype, d, steps, warmup)
        res[wl.name] = r
        log(f"{wl.name}: {r['ms'] * 1e3:.1f} us (graph replay), {r['ms_eager'] * 1e3:.1f} us "
            "launched one by one")
        del d
    torch.cuda.empty_cache()
    return res


# Prefills with few heads per device (as when the heads are sharded over
# devices): the Kaczmarz layer of the benchmark at 4 and 2 of its 16 heads,
# which the library runs as segments whose chains run side by side.
FEW_HEAD_SHAPES = (("kla", 1, 65536, 8), ("kla", 1, 65536, 4), ("kla", 1, 131072, 2))


def _time_noalloc(L, dev, variant, d, steps):
    """gdr_forward_chunked_noalloc on the same call, as a replayed HIP graph of
    `steps` calls (ms per call)."""
    import torch

    from gated_delta_rule_85_amd import binding

    B, T, H, dk = d["q"].shape
    dv = d["v"].shape[-1]
    o = torch.empty((B, T, H, dv), dtype=d["q"].dtype, device=dev)
    s_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    a = binding.make_args(variant, d["q"], d["k"], d["v"], o, d["alpha"], d["beta"],
                          d["erase_b"], d["write_w"], d["eps"], None, s_T)
    ref = ctypes.byref(a)
    binding.check(L.gdr_forward_chunked_noalloc(ref, torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gs = torch.cuda.current_stream().cuda_stream
        for _ in range(steps):
            binding.check(L.gdr_forward_chunked_noalloc(ref, gs))
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    del graph, o, s_T
    return e0.elapsed_time(e1) / steps


def few_head_gradients(L, dev, sh, steps, warmup):
    """The gradient of FEW_HEAD_SHAPES' forwards (upstream gradients for o and
    S_T in, fp32 gradients of q, k, v, eta, alpha and S_0 out) and the saving
    forward, timed with HIP events on the launch stream after `warmup` calls
    (ms per call); with few heads both run their chains in segments."""
    import torch

    from gated_delta_rule_85_amd import binding
    from gated_delta_rule_85_amd.inputs import make_inputs, make_upstream_grads

    res = {}
    for variant, B, T, H in FEW_HEAD_SHAPES:
        dk = dv = 128
        d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v)
             for k, v in make_inputs(variant, B, T, H, dk, dv, "bf16", seed=85100 + H).items()}
        up = {k: v.to(dev) for k, v in make_upstream_grads(B, T, H, dk, dv, "bf16",
                                                             seed=85200 + H).items()}
        o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
        s_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
        fa = binding.make_args(variant, d["q"], d["k"], d["v"], o, d["alpha"], d["beta"], None,
                               None, d["eps"], None, s_T)
        ba = binding.make_args(variant, d["q"], d["k"], d["v"], None, d["alpha"], d["beta"], None,
                               None, d["eps"], None, None)
        binding.check(binding.gdr_check_args(fa, 0))
        nbw = binding.gdr_backward_workspace_size(ba)
        ws = torch.empty(nbw, dtype=torch.uint8, device=dev)
        gr = {n: torch.empty(shape, dtype=torch.float32, device=dev) for n, shape in
              (("q", (B, T, H, dk)), ("k", (B, T, H, dk)), ("v", (B, T, H, dv)),
               ("alpha", (B, T, H)), ("beta", (B, T, H)), ("s0", (B, H, dk, dv)))}
        ga = binding.GdrGrads(up["d_o"].data_ptr(), up["d_state_out"].data_ptr(),
                              gr["q"].data_ptr(), gr["k"].data_ptr(), gr["v"].data_ptr(),
                              gr["alpha"].data_ptr(), gr["beta"].data_ptr(), None, None,
                              gr["s0"].data_ptr())

        def timed(fn):
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / steps

        name = f"{variant}_bf16_B{B}_H{H}_T{T}_d128"
        bw = timed(lambda: binding.check(L.gdr_backward_chunked(ctypes.byref(ba), ctypes.byref(ga),
                                                                ws.data_ptr(), nbw, sh)))
        fs = timed(lambda: binding.check(L.gdr_forward_chunked_save(ctypes.byref(fa), ws.data_ptr(),
                                                                    nbw, sh)))
        res[name] = dict(backward_ms=bw, forward_save_ms=fs, tokens_per_s=B * T / (bw / 1e3),
                         outputs_finite=all(bool(torch.isfinite(t).all()) for t in gr.values()))
        log(f"{name}: gradient {bw * 1e3:.1f} us, saving forward {fs * 1e3:.1f} us")
        del d, up, ws, gr, o, s_T
        torch.cuda.empty_cache()
    return res


def few_head_workloads(L, dev, sh, steps, warmup):
    """The forward of FEW_HEAD_SHAPES (bf16, d = 128, synthetic inputs drawn
    as the Kaczmarz workload's), each timed by _time_forward.  Where the
    segmented plan's workspace exceeds the allocation-free entry point's
    static array, that entry point runs the same call as the blocked pipeline
    instead; its time is reported beside as ms_blocked_pipeline (same run,
    same inputs)."""
    import torch

    from gated_delta_rule_85_amd import binding
    from gated_delta_rule_85_amd.inputs import make_inputs

    res = {}
    for variant, B, T, H in FEW_HEAD_SHAPES:
        d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v)
             for k, v in make_inputs(variant, B, T, H, 128, 128, "bf16", seed=85100 + H).items()}
        name = f"{variant}_bf16_B{B}_H{H}_T{T}_d128"
        r = _time_forward(L, dev, sh, variant, "bf16", d, steps, warmup)
        if r["workspace_bytes"] > binding.NOALLOC_WORKSPACE_MAX:
            r["ms_blocked_pipeline"] = _time_noalloc(L, dev, variant, d, steps)
            r["speedup_over_blocked_pipeline"] = r["ms_blocked_pipeline"] / r["ms"]
        res[name] = r
        log(f"{name}: {r['ms'] * 1e3:.1f} us (graph replay)"
            + (f", {r['ms_blocked_pipeline'] * 1e3:.1f} us as the blocked pipeline"
               if "ms_blocked_pipeline" in r else ""))
        del d
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the cold-state decode and the forward of workloads 1-4 "
                         "(profiler runs of the main step)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 256 MiB device copy (calibrates HBM byte counters)")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch the decode steps one by one instead of replaying a HIP graph")
    ap.add_argument("--cpu-tokens", type=int, default=65536)
    ap.add_argument("--cpu-decode-steps", type=int, default=192)
    ap.add_argument("--long-context", action="store_true",
                    help="measure the long-context shapes (131K prefill, decode at 32K) instead")
    ap.add_argument("--backward", action="store_true",
                    help="measure the gradient of the chunked forward on the Kaczmarz prefill")
    ap.add_argument("--routing", action="store_true",
                    help="measure the cost of the cross-layer routing input and output")
    ap.add_argument("--few-heads", action="store_true",
                    help="time only the prefills with few heads per device (segmented path)")
    ap.add_argument("--cold-decode", action="store_true",
                    help="time decode launches one by one with the state evicted from the "
                         "last-level cache, and measure the box's copy / GEMM peaks")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path runs every (b, h) head on one "
              "device and has no multi-GPU mode; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.long_context:
        long_context(args)
        return
    if args.backward:
        backward(args)
        return
    if args.routing:
        routing(args)
        return
    if args.cold_decode:
        cold_decode(args)
        return
    if args.few_heads:
        import torch

        from gated_delta_rule_85_amd import binding

        dev = torch.device("cuda:0")
        torch.cuda.set_device(dev)
        L = binding.lib()
        sh = torch.cuda.current_stream().cuda_stream
        res = few_head_workloads(L, dev, sh, steps=args.steps, warmup=args.warmup)
        grads = few_head_gradients(L, dev, sh, steps=args.steps, warmup=args.warmup)
        print(json.dumps({"metric": "chunked-forward time with few heads per device (ms)",
                          "unit": "ms", "higher_is_better": False, "n_gpus": 1,
                          "steps": args.steps, "warmup": args.warmup, "dtype": "bf16",
                          "data": "synthetic", "forward_few_heads": res,
                          "gradient_few_heads": grads, "git": git_sha()}))
        return

    import torch

    from gated_delta_rule_85_amd import binding
    from gated_delta_rule_85_amd.inputs import WORKLOADS, make_decode_inputs, make_workload

    wl = WORKLOADS[5]
    L = binding.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    # ---- inputs (untimed), resident in HBM ----------------------------------
    log("generating prefill inputs")
    inp = make_workload(wl)
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    del inp
    B, T, H, dk, dv = wl.B, wl.T, wl.H, wl.dk, wl.dv
    o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
    s_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    fa = binding.make_args(wl.variant, d["q"], d["k"], d["v"], o, d["alpha"], d["beta"],
                           None, None, d["eps"], None, s_T)
    binding.check(binding.gdr_check_args(fa, 0))
    ws_bytes = binding.gdr_forward_workspace_size(fa)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    log(f"prefill workspace {ws_bytes / 2**20:.1f} MiB")

    log("generating decode inputs")
    Sd = wl.decode["steps"]
    Bd = wl.decode["B"]
    dec = make_decode_inputs(wl)
    dd = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in dec.items()}
    del dec
    state = torch.empty((Bd, H, dk, dv), dtype=torch.float32, device=dev)
    o_dec = torch.empty((Sd, Bd, 1, H, dv), dtype=torch.bfloat16, device=dev)
    dargs = [binding.make_args(wl.variant, dd["q"][s], dd["k"][s], dd["v"][s], o_dec[s],
                               dd["alpha"][s], dd["beta"][s], None, None, dd["eps"],
                               state, state) for s in range(Sd)]
    for a in dargs:
        binding.check(binding.gdr_check_args(a, 1))
    fa_ref = ctypes.byref(fa)
    dargs_ref = [ctypes.byref(a) for a in dargs]
    fwd_fn, dec_fn = L.gdr_forward_chunked, L.gdr_decode_step
    ws_ptr = ws.data_ptr()

    # Decode starts from the prefill's final state, broadcast over the batch.
    binding.check(fwd_fn(fa_ref, ws_ptr, ws_bytes, sh))
    state.copy_(s_T.expand(Bd, H, dk, dv))
    torch.cuda.synchronize()

    ev = lambda: torch.cuda.Event(enable_timing=True)

    def decode_block(handle):
        for s in range(Sd):
            rc = dec_fn(dargs_ref[s], handle)
            if rc:
                binding.check(rc)

    graph = None
    if not args.no_graph:
        # The 1024 decode launches are captured once into a HIP graph and
        # replayed each step, as a serving loop would.
        decode_block(sh)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            decode_block(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()

    def step(timers=None):
        if timers is not None:
            timers["f0"].record(stream)
        rc = fwd_fn(fa_ref, ws_ptr, ws_bytes, sh)
        if rc:
            binding.check(rc)
        if timers is not None:
            timers["f1"].record(stream)
        if graph is not None:
            graph.replay()
        else:
            decode_block(sh)
        if timers is not None:
            timers["d1"].record(stream)

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    timers = [dict(f0=ev(), f1=ev(), d1=ev()) for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(timers[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log("timed region done")

    if args.copy_calibration:
        # A plain copy of known size: its FETCH_SIZE / WRITE_SIZE counters give
        # the factor that turns those counters into bytes.
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 268435456 bytes read and written")
        del src, dst

    # ---- after the timed region: the decode with its state in HBM ----------
    # Back to back, the 64 MiB batch state stays in the 256 MiB last-level
    # cache (MALL) between steps, so the timed figure above is a cache-resident
    # one.  Here each launch follows a 1 GiB read sweep that evicts the state,
    # and is timed on its own on the launch stream; the box's device-copy rate
    # over 2 GiB buffers is measured beside it.
    n_cold = 0 if args.no_extras else 64
    if n_cold:
        log("cold-state decode launches and the box's copy rate")
        flush = torch.ones(256 << 20, dtype=torch.float32, device=dev)
        pairs = [(ev(), ev()) for _ in range(n_cold)]
        for s_ in range(n_cold):
            flush.sum()
            pairs[s_][0].record(stream)
            binding.check(dec_fn(dargs_ref[s_], sh))
            pairs[s_][1].record(stream)
        torch.cuda.synchronize()
        cold_us = sorted(a_.elapsed_time(b_) * 1e3 for a_, b_ in pairs)
        rmw = state_rmw_reference(dev, stream, Bd * H * dk * dv, n_cold, flush)
        del flush
        src = torch.ones(512 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        c0, c1 = ev(), ev()
        c0.record(stream)
        for _ in range(10):
            dst.copy_(src)
        c1.record(stream)
        torch.cuda.synchronize()
        copy_Bps = 2 * src.numel() * 4 / (c0.elapsed_time(c1) / 1e3 / 10)
        del src, dst
        torch.cuda.empty_cache()

    others = few = None
    if not args.no_extras:
        log("forward of workloads 1-4")
        others = other_workloads(L, dev, sh, steps=20, warmup=3)
        log("forward with few heads per device")
        few = few_head_workloads(L, dev, sh, steps=20, warmup=3)

    fwd_ms = [t["f0"].elapsed_time(t["f1"]) for t in timers]
    dec_ms = [t["f1"].elapsed_time(t["d1"]) for t in timers]
    fwd_s = sum(fwd_ms) / len(fwd_ms) / 1e3
    # Average duration of one decode launch: the replayed block of Sd launches
    # on the launch stream, divided by Sd (includes the small gaps between
    # back-to-back kernels, so it is an upper bound on the kernel time).
    dec_s = sum(dec_ms) / len(dec_ms) / 1e3 / Sd

    tokens_step = B * T + Bd * Sd
    ms_step = wall / args.steps * 1e3
    value = tokens_step * args.steps / wall

    head_tokens = B * T * H
    fl = forward_flops_per_head_token(dk, dv) * head_tokens
    fb = forward_bytes(B, T, H, dk, dv)
    db = decode_bytes(Bd, H, dk, dv)
    dec_bw = db / dec_s
    med = lambda xs: sorted(xs)[len(xs) // 2]
    prefill = dict(tokens_per_s=B * T / fwd_s, ms=fwd_s * 1e3, ms_median=med(fwd_ms),
                   tflops=fl / fwd_s / 1e12, mfma_frac=fl / fwd_s / PEAK_BF16,
                   hbm_GBps=fb / fwd_s / 1e9, hbm_frac=fb / fwd_s / PEAK_HBM,
                   algorithmic_flop=fl, algorithmic_bytes=fb)
    cold_state = None
    if n_cold:
        cold_med = cold_us[n_cold // 2] * 1e-6
        cold_state = dict(
            note=f"{n_cold} single launches, each after a 1 GiB read sweep that evicts the "
                 "state to HBM; median launch",
            us_per_step=cold_med * 1e6, min_us=cold_us[0], max_us=cold_us[-1],
            GBps=db / cold_med / 1e9, hbm_frac=db / cold_med / PEAK_HBM,
            box_copy_GBps=copy_Bps / 1e9, frac_of_box_copy=db / cold_med / copy_Bps,
            box_copy_note="torch device copy of 2 GiB, bytes read plus written",
            state_rmw_reference=rmw,
            frac_of_state_rmw=(db / cold_med) / (rmw["cold_GBps"] * 1e9))
    decode = dict(tokens_per_s=Bd / dec_s, us_per_step=dec_s * 1e6,
                  us_per_step_median=med(dec_ms) * 1e3 / Sd,
                  GBps=dec_bw / 1e9, hbm_frac=dec_bw / PEAK_HBM, algorithmic_bytes=db,
                  steps_per_bench_step=Sd, batch=Bd,
                  state_residency="last-level cache (MALL): the 64 MiB state stays in the "
                                  "256 MiB MALL between back-to-back steps",
                  frac_of_state_rmw_warm=(dec_bw / (rmw["warm_GBps"] * 1e9)) if n_cold else None,
                  cold_state=cold_state)
    t_dec_total = dec_s * Sd
    dominant = "decode" if t_dec_total >= fwd_s else "prefill"
    if dominant == "decode":
        roofline = dict(kernel="decode_wave_kernel<KLA,bf16,128,32,4>", bound="hbm",
                        achieved=dec_bw / 1e9, peak=PEAK_HBM / 1e9, unit="GB/s",
                        frac=dec_bw / PEAK_HBM,
                        state_residency="MALL (warm, as timed); with the state in HBM see "
                                        "decode.cold_state",
                        frac_state_in_hbm=cold_state["hbm_frac"] if cold_state else None,
                        traffic=measured_traffic("decode_wave_kernel",
                                                 "gated_delta_rule_85_amd/csrc/decode.hip"),
                        traffic_unit="bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                     "copy-calibrated)",
                        per_launch_bytes=db, avg_launch_us=dec_s * 1e6)
    else:
        roofline = dict(kernel="chunked forward", bound="hbm", achieved=fb / fwd_s / 1e9,
                        peak=PEAK_HBM / 1e9, unit="GB/s", frac=fb / fwd_s / PEAK_HBM,
                        traffic=None)

    cpu = None
    if not args.no_cpu:
        log("timing the CPU oracle on a bounded sample")
        try:
            threads = min(16, len(os.sched_getaffinity(0)))
        except AttributeError:
            threads = 16
        cpu = cpu_baseline(wl, args.cpu_tokens, args.cpu_decode_steps, threads)

    out = {
        "metric": "chunked-forward tokens/s + %MFMA peak; decode tokens/s + HBM GB/s",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"Kaczmarz LA layer: prefill B={B} H={H} T={T} d_k=d_v={dk} bf16 "
                         f"(fp32 gates/state) + {Sd} decode steps at batch {Bd}"),
            "variant": wl.variant, "B": B, "H": H, "T": T, "dk": dk, "dv": dv, "chunk": C,
            "decode_batch": Bd, "decode_steps": Sd,
            "tokens_per_step": tokens_step,
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "prefill": prefill,
        "decode": decode,
        "forward_other_workloads": others,
        "forward_few_heads": few,
        "git": git_sha(),
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
