"""Benchmark of the causal SATA hot path on one MI355X.

One step = the decode workload end to end: 256 resident states (batch 8 x 32
heads), d_k = d_v = 64, P = 4, bf16 q/k/v with fp32 state: a 4096-token causal
prefill from empty states, then 1024 single-token decode steps.  Inputs are
seeded synthetic data (workloads.py), resident in HBM before timing starts.

Prints one JSON line.  `value` is head-tokens/s over the whole step (every
prefill and decode token of every state).  The prefill and decode legs are
also reported on their own, each against its roofline; `roofline` describes
the dominant kernel (the decode update/readout, bound by HBM).  After the
timed steps, `configs` reports the other workloads, each against its own
roofline (a few repetitions each): the same decode on the mixed-precision
state (orders >= 2 of S in float16), the d8 / d16 fp32 and d64 bf16 prefills,
the long-context d32 prefill at 2^16, 2^18 and 2^20 tokens with its per-token
cost ratio, the orders 0..4 (P = 5) prefill and decode legs, few-head long
prefills with and without sequence segments, and exact causal
softmax attention beside the SATA prefill over n = 2^12..2^16 (the crossover);
`ceilings` gives the box's own stream and matrix-core rates from the ceiling
kernels, with the decode and prefill legs as fractions of them.  The CPU
baseline is the float64 oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6    # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3     # MI355X dense fp32 MFMA
METRIC = "causal SATA tokens/sec/head (prefill, decode) + % of HBM/MFMA roofline"
# HBM bytes moved by one decode_update_readout launch of this workload, from the
# FETCH_SIZE / WRITE_SIZE counters scaled by a 1 GiB copy
# (profiles/decode_update_readout_256x4096_d64_hbm_traffic.txt).  Re-measure after any
# change to the decode kernel.
DECODE_TRAFFIC_BYTES = 6.5784e9
# The same for one decode_mixed launch (mixed-precision state, same workload).
MIXED_DECODE_TRAFFIC_BYTES = 3.4166e9


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (timed after the headline step: the d8/d16/d64 prefills, "
                         "the long-context sweep at 2^16..2^20 and the orders 0..4 legs)")
    ap.add_argument("--no-mixed", action="store_true", help="skip the mixed-precision decode-state leg")
    ap.add_argument("--mixed-steps", type=int, default=256,
                    help="timed decode steps on the mixed-precision state")
    ap.add_argument("--config-steps", type=int, default=5,
                    help="timed repetitions of each of the other workloads (one warmup each)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--flatness", action="store_true",
                    help="instead of the step: prefill cost per token of the long-context workload "
                         "(16 heads, d_k=d_v=32, P=4, bf16) at n = 2^16, 2^18, 2^20")
    ap.add_argument("--configs", action="store_true",
                    help="instead of the step: prefill throughput of the other workloads at their full "
                         "sizes (d8 n256 fp32, d16 n4096 fp32, d64 n16384 bf16), each against the MFMA "
                         "peak of its arithmetic")
    ap.add_argument("--order5", action="store_true",
                    help="instead of the step: orders 0..4 (P=5) at d_k=d_v=64, 32 states, bf16 -- a "
                         "4096-token prefill against the MFMA peak, then --order5-steps decode steps "
                         "against the HBM peak")
    ap.add_argument("--order5-steps", type=int, default=64)
    ap.add_argument("--ceilings", action="store_true",
                    help="instead of the step: what this box sustains with plain library kernels -- a "
                         "1 GiB device copy, an in-place read-modify-write and a read of 3 GiB, and a "
                         "bf16 GEMM -- next to the published peaks")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 1 GiB device copy (read 1 GiB, write 1 GiB), the "
                         "reference for scaling hardware byte counters")
    return ap.parse_args()


def cpu_baseline(w, q, k, v, qs, ks, vs, budget_s):
    """The float64 oracle, as it stands, on a bounded sample: whole states'
    prefill rows plus their decode rows, until the time budget is used."""
    from oracle import sata_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    S = w.B * w.H
    qf = q.reshape(S, w.n, w.d_k).astype(np.float64)
    kf = k.reshape(S, w.n, w.d_k).astype(np.float64)
    vf = v.reshape(S, w.n, w.d_v).astype(np.float64)
    dsteps = qs.shape[0]
    rows = 0
    states = 0
    t0 = time.perf_counter()
    while states < S and (time.perf_counter() - t0) < budget_s:
        s = states
        O.direct_taylor(qf[s], kf[s], vf[s], w.P, w.c)
        qq = np.concatenate([qf[s], qs[:, s].astype(np.float64)])
        kk = np.concatenate([kf[s], ks[:, s].astype(np.float64)])
        vv = np.concatenate([vf[s], vs[:, s].astype(np.float64)])
        O.direct_taylor(qq, kk, vv, w.P, w.c, rows=np.arange(w.n, w.n + dsteps))
        rows += w.n + dsteps
        states += 1
    el = time.perf_counter() - t0
    return {"value": rows / el, "unit": "head-tokens/s", "cores": int(blas_threads),
            "host_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{states} of {S} states: all {w.n} prefill rows and {dsteps} decode rows each "
                      f"({rows} head-tokens, float64 numpy, {el:.1f} s)"}


def _time_prefill(sa, basis, Q, K, V, state, out, ws, stream, reps, warmup):
    """Median HIP-event time (ms) of a prefill from empty states."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ms = []
    for it in range(warmup + reps):
        state.zero_()
        ev[0].record(stream)
        sa.prefill(basis, Q, K, V, state=state, out=out, ws=ws)
        ev[1].record(stream)
        torch.cuda.synchronize()
        if it >= warmup:
            ms.append(ev[0].elapsed_time(ev[1]))
    return float(np.median(ms))


def flatness_points(reps, warmup, lgs=(16, 18, 20)):
    """Prefill time per token of the long-context workload (16 heads, d = 32,
    P = 4, bf16) at growing context: the state is fixed-size, so the per-token
    cost should not grow with n.  Inputs: seeded unit-norm Gaussian q, k and
    Gaussian v generated on the device (same distribution as the seeded host
    generators, which would take minutes at 2^20 tokens)."""
    import torch
    import constant_cost_taylor_amd as sa
    import workloads as W
    from oracle import sata_oracle as O
    w = W.WORKLOADS["long_d32_n1m"]
    dev = torch.device("cuda:0")
    basis = sa.build_basis(w.d_k, w.P, w.c)
    g = torch.Generator(device=dev)
    g.manual_seed(1000 * w.seed)
    stream = torch.cuda.current_stream(dev)
    _, page_flops = O.cost_model(w.d_k, w.d_v, w.P)
    rows = []
    for lg in lgs:
        n = 1 << lg
        shape = (w.B, w.H, n, w.d_k)
        q = torch.randn(shape, generator=g, device=dev)
        q = (q / q.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
        k = torch.randn(shape, generator=g, device=dev)
        k = (k / k.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
        v = torch.randn(shape, generator=g, device=dev).to(torch.bfloat16)
        out = torch.empty(shape, dtype=torch.float32, device=dev)
        state = sa.new_state(basis, w.B * w.H, dev)
        ws = sa.workspace(sa.prefill_workspace_bytes(basis, w.B, w.H, n, w.d_v, sa.SATA_BF16), dev)
        t = _time_prefill(sa, basis, q, k, v, state, out, ws, stream, reps, warmup)
        tok = w.B * w.H * n
        tf = tok * page_flops / (t * 1e-3) / 1e12
        rows.append({"n": n, "ms": t, "ns_per_head_token": 1e6 * t / tok, "head_tokens_per_s": tok / (t * 1e-3),
                     "page_tflops": tf, "mfma_bf16_frac": tf / BF16_PEAK_TFLOPS,
                     "finite": bool(torch.isfinite(out).all())})
        print(f"long-context prefill n=2^{lg}: {t:.2f} ms", file=sys.stderr, flush=True)
        del q, k, v, out, state, ws
        torch.cuda.empty_cache()
    costs = np.array([r["ns_per_head_token"] for r in rows])
    return {"workload": f"long-context prefill: batch {w.B} x {w.H} heads, d_k=d_v={w.d_k}, P={w.P}, bf16 inputs, "
                        f"f32 state, n = 2^16, 2^18, 2^20 (device-generated inputs)",
            "steps": reps, "warmup": warmup, "points": rows,
            "per_token_cost_ratio_last_over_first": float(costs[-1] / costs[0]),
            # largest departure of a point's per-token cost from the mean over the points
            "per_token_cost_max_dev_from_mean": float(np.max(np.abs(costs / costs.mean() - 1.0)))}


def flatness(args):
    torch = __import__("torch")
    torch.cuda.set_device(0)
    res = flatness_points(args.steps, args.warmup)
    print(json.dumps({"metric": "prefill per-token cost vs context length", "unit": "ns/head-token", **res}),
          flush=True)


def segment_points(reps, warmup, cases=((1, 20, 32), (4, 18, 32), (1, 16, 64))):
    """Prefill of few heads over long sequences, with the sequence segments
    the library takes for such batches and with them turned off
    (SATA_PREFILL_SEGMENTS=0): (heads, log2 n, d) each, P = 4, bf16 inputs
    generated on the device (seeded unit-norm Gaussian q, k; Gaussian v)."""
    import torch
    import constant_cost_taylor_amd as sa
    from oracle import sata_oracle as O
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    rows = []
    for H, lg, d in cases:
        n = 1 << lg
        basis = sa.build_basis(d, 4, 1.0)
        _, page_flops = O.cost_model(d, d, 4)
        g = torch.Generator(device=dev)
        g.manual_seed(7000 + lg + d)
        shape = (1, H, n, d)
        q = torch.randn(shape, generator=g, device=dev)
        q = (q / q.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
        k = torch.randn(shape, generator=g, device=dev)
        k = (k / k.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
        v = torch.randn(shape, generator=g, device=dev).to(torch.bfloat16)
        out = torch.empty(shape, dtype=torch.float32, device=dev)
        state = sa.new_state(basis, H, dev)
        row = {"heads": H, "n": n, "d": d}
        for mode in ("segments", "no_segments"):
            if mode == "no_segments":
                os.environ["SATA_PREFILL_SEGMENTS"] = "0"
            ws = sa.workspace(sa.prefill_workspace_bytes(basis, 1, H, n, d, sa.SATA_BF16), dev)
            t = _time_prefill(sa, basis, q, k, v, state, out, ws, stream, reps, warmup)
            os.environ.pop("SATA_PREFILL_SEGMENTS", None)
            tf = H * n * page_flops / (t * 1e-3) / 1e12
            row[mode] = {"ms": t, "head_tokens_per_s": H * n / (t * 1e-3), "page_tflops": tf,
                         "mfma_bf16_frac": tf / BF16_PEAK_TFLOPS, "finite": bool(torch.isfinite(out).all())}
            del ws
            torch.cuda.empty_cache()
        row["speedup"] = row["no_segments"]["ms"] / row["segments"]["ms"]
        rows.append(row)
        del q, k, v, out, state
        torch.cuda.empty_cache()
    return {"workload": "prefill of few heads over long sequences, P=4, bf16 inputs, f32 state, from empty "
                        "states, with and without sequence segments (device-generated inputs)",
            "steps": reps, "warmup": warmup, "points": rows}


def config_points(reps, warmup, names=("tiny_d8_n256", "d16_n4096", "d64_n16384")):
    """Prefill of the other workloads at their full sizes, from empty states,
    inputs from the seeded generators (workloads.py), each against the MFMA
    peak of its arithmetic (page FLOPs / time)."""
    import torch
    import constant_cost_taylor_amd as sa
    import workloads as W
    from oracle import sata_oracle as O
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    res = {}
    for name in names:
        w = W.WORKLOADS[name]
        basis = sa.build_basis(w.d_k, w.P, w.c)
        q, k, v = W.workload_inputs(w)
        bf16 = w.dtype == W.BF16
        tdt = torch.bfloat16 if bf16 else torch.float32
        Q, K, V = (torch.from_numpy(np.ascontiguousarray(x)).to(tdt).to(dev) for x in (q, k, v))
        out = torch.empty((w.B, w.H, w.n, w.d_v), dtype=torch.float32, device=dev)
        state = sa.new_state(basis, w.B * w.H, dev)
        ws = sa.workspace(sa.prefill_workspace_bytes(basis, w.B, w.H, w.n, w.d_v,
                                                     sa.SATA_BF16 if bf16 else sa.SATA_F32), dev)
        t = _time_prefill(sa, basis, Q, K, V, state, out, ws, stream, reps, warmup)
        tok = w.B * w.H * w.n
        _, page_flops = O.cost_model(w.d_k, w.d_v, w.P)
        tflops = tok * page_flops / (t * 1e-3) / 1e12
        peak = BF16_PEAK_TFLOPS if bf16 else FP32_PEAK_TFLOPS
        res[name] = {"workload": f"batch {w.B} x {w.H} heads, n={w.n}, d_k=d_v={w.d_k}, P={w.P}, "
                                 f"{'bf16' if bf16 else 'fp32'} inputs, f32 state, prefill from empty states",
                     "ms": t, "head_tokens_per_s": tok / (t * 1e-3), "page_tflops": tflops,
                     "mfma_peak_tflops": peak, "mfma_frac": tflops / peak,
                     "finite": bool(torch.isfinite(out).all())}
        print(f"prefill {name}: {t:.3f} ms", file=sys.stderr, flush=True)
        del Q, K, V, out, state, ws
        torch.cuda.empty_cache()
    return res


def configs(args):
    torch = __import__("torch")
    torch.cuda.set_device(0)
    res = config_points(args.steps, args.warmup)
    print(json.dumps({"metric": "prefill throughput per workload", "unit": "head-tokens/s", "steps": args.steps,
                      "warmup": args.warmup, "points": res}), flush=True)


def order5_point(reps, warmup, dsteps):
    """Orders 0..4 at d = 64: the prefill leg and the decode leg of a 32-state
    step, each against its roofline, with a sampled check of the last decode
    outputs against the oracle."""
    import torch
    import constant_cost_taylor_amd as sa
    import workloads as W
    from oracle import sata_oracle as O
    w = W.WORKLOADS["order5_32x4096_d64"]
    S = w.B * w.H
    q, k, v = W.workload_inputs(w)
    qs, ks, vs = W.decode_inputs(w, dsteps)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    basis = sa.build_basis(w.d_k, w.P, w.c)
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).to(dev)
    Q, K, V = bf(q), bf(k), bf(v)
    DQ, DK, DV = bf(qs), bf(ks), bf(vs)
    state = sa.new_state(basis, S, dev)
    out = torch.empty((w.B, w.H, w.n, w.d_v), dtype=torch.float32, device=dev)
    dout = torch.empty((dsteps, S, w.d_v), dtype=torch.float32, device=dev)
    pws = sa.workspace(sa.prefill_workspace_bytes(basis, w.B, w.H, w.n, w.d_v, sa.SATA_BF16), dev)
    dws = sa.workspace(sa.decode_workspace_bytes(basis, S, w.d_v, sa.SATA_BF16), dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(dsteps + 2)]
    pre_ms, dec_ms = [], []
    for it in range(warmup + reps):
        state.zero_()
        ev[0].record(stream)
        sa.prefill(basis, Q, K, V, state=state, out=out, ws=pws)
        ev[1].record(stream)
        for t in range(dsteps):
            sa.decode_step(basis, DQ[t], DK[t], DV[t], state, out=dout[t], ws=dws)
            ev[t + 2].record(stream)
        torch.cuda.synchronize()
        if it >= warmup:
            pre_ms.append(ev[0].elapsed_time(ev[1]))
            dec_ms.extend(ev[t + 1].elapsed_time(ev[t + 2]) for t in range(dsteps))
        print(f"order5 step {it}: prefill {ev[0].elapsed_time(ev[1]):.2f} ms", file=sys.stderr, flush=True)
    got = dout[:, [0, S - 1]].cpu().numpy()
    qf, kf, vf = (x.reshape(S, w.n, -1) for x in (q, k, v))
    errs = []
    for j, s in enumerate([0, S - 1]):
        rr = np.arange(w.n, w.n + dsteps, max(1, dsteps // 8))
        ref = O.direct_taylor(np.concatenate([qf[s], qs[:, s]]).astype(np.float64),
                              np.concatenate([kf[s], ks[:, s]]).astype(np.float64),
                              np.concatenate([vf[s], vs[:, s]]).astype(np.float64), w.P, w.c, rows=rr)
        errs.append(O.row_normwise_error(got[rr - w.n, j], ref))
    pre = float(np.median(pre_ms))
    dec = float(np.mean(dec_ms))
    D = basis.total_rows
    dec_bytes = S * (2 * 4 * (w.d_v + 1) * D + 3 * w.d_k * 2 + w.d_v * 4)
    _, page_flops = O.cost_model(w.d_k, w.d_v, w.P)
    pre_tflops = S * w.n * page_flops / (pre * 1e-3) / 1e12
    dec_gbs = dec_bytes / (dec * 1e-3) / 1e9
    del Q, K, V, DQ, DK, DV, state, out, dout, pws, dws
    torch.cuda.empty_cache()
    return {"workload": f"order5: {S} states (batch {w.B} x {w.H} heads), d_k=d_v={w.d_k}, P={w.P}, D={D}, bf16 "
                        f"inputs, f32 state, {w.n}-token prefill + {dsteps} decode steps",
            "steps": reps, "warmup": warmup,
            "prefill": {"ms": pre, "head_tokens_per_s": S * w.n / (pre * 1e-3), "page_tflops": pre_tflops,
                        "mfma_bf16_frac": pre_tflops / BF16_PEAK_TFLOPS},
            "decode": {"ms_per_step": dec, "head_tokens_per_s": S / (dec * 1e-3), "hbm_gbs": dec_gbs,
                       "hbm_frac": dec_gbs / HBM_PEAK_GBS, "algorithmic_bytes": dec_bytes},
            "check": {"decode_row_normwise_err": max(errs)}}


def order5(args):
    torch = __import__("torch")
    torch.cuda.set_device(0)
    res = order5_point(args.steps, args.warmup, args.order5_steps)
    print(json.dumps({"metric": "orders 0..4 (P=5) prefill and decode vs roofline", "unit": "head-tokens/s",
                      **res}), flush=True)


def mixed_leg(sa, basis, w, Q, K, V, DQ, DK, DV, state, out, pws, q, k, v, qs, ks, vs, stream, dsteps, f32_ms):
    """The same workload's decode on the mixed-precision state (orders >= 2 of
    S in float16, per-tile scales): prefill on the float32 state, hand-off,
    then dsteps timed decode steps, against HBM on the mixed state's own
    bytes."""
    import torch
    from oracle import sata_oracle as O
    S = w.B * w.H
    D = basis.total_rows
    state.zero_()
    sa.prefill(basis, Q, K, V, state=state, out=out, ws=pws)
    mixed = sa.to_mixed(basis, state)
    dws = sa.workspace(sa.decode_mixed_workspace_bytes(basis, S, w.d_v, sa.SATA_BF16), Q.device)
    dout = torch.empty((dsteps, S, w.d_v), dtype=torch.float32, device=Q.device)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(dsteps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for t in range(dsteps):
        sa.decode_step_mixed(basis, DQ[t], DK[t], DV[t], mixed, out=dout[t], ws=dws)
        ev[t + 1].record(stream)
    torch.cuda.synchronize()
    ms = [ev[t].elapsed_time(ev[t + 1]) for t in range(dsteps)]
    dec = float(np.mean(ms[1:])) if dsteps > 1 else ms[0]
    lo, r16 = 1 + w.d_k, 2 * (128 // (w.d_v // 8))
    nt16 = -(-(D - lo) // r16)
    state_bytes = 2 * (lo * w.d_v * 4 + (D - lo) * w.d_v * 2 + D * 4 + nt16 * 4)
    io_bytes = 3 * w.d_k * 2 + w.d_v * 4
    dec_bytes = S * (state_bytes + io_bytes)
    gbs = dec_bytes / (dec * 1e-3) / 1e9
    got = dout[:, [0, S - 1]].cpu().numpy()
    qf, kf, vf = (x.reshape(S, w.n, -1) for x in (q, k, v))
    errs = []
    for j, s_ in enumerate([0, S - 1]):
        rr = np.arange(w.n, w.n + dsteps, max(1, dsteps // 8))
        ref = O.direct_taylor(np.concatenate([qf[s_], qs[:dsteps, s_]]).astype(np.float64),
                              np.concatenate([kf[s_], ks[:dsteps, s_]]).astype(np.float64),
                              np.concatenate([vf[s_], vs[:dsteps, s_]]).astype(np.float64), w.P, w.c, rows=rr)
        errs.append(O.row_normwise_error(got[rr - w.n, j], ref))
    del mixed, dws, dout
    return {"workload": f"same states, orders 0-1 of S and z fp32, orders >= 2 of S float16 with per-tile "
                        f"power-of-two scales; {dsteps} decode steps after the {w.n}-token prefill",
            "ms_per_step": dec, "head_tokens_per_s": S / (dec * 1e-3), "algorithmic_bytes": dec_bytes,
            "hbm_gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS, "speedup_vs_f32_state": f32_ms / dec,
            "traffic": MIXED_DECODE_TRAFFIC_BYTES, "traffic_unit": "bytes per launch (HBM, counter-measured)",
            "check": {"decode_row_normwise_err": max(errs)}}


def crossover_points(reps, warmup, heads=(4, 32), lgs=(12, 13, 14, 15, 16)):
    """Exact causal softmax attention (sata_softmax_attention, bf16 MFMA)
    beside the SATA prefill on the same inputs (d = 64, P = 4, bf16,
    device-generated unit-norm q, k and Gaussian v) over growing n: SATA's
    cost per token is flat, exact attention's grows with n.  The crossover n
    is interpolated on log-log axes between the sweep points around it."""
    import torch
    import constant_cost_taylor_amd as sa
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    basis = sa.build_basis(64, 4, 1.0)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(fn):
        ms = []
        for it in range(warmup + reps):
            ev[0].record(stream)
            fn()
            ev[1].record(stream)
            torch.cuda.synchronize()
            if it >= warmup:
                ms.append(ev[0].elapsed_time(ev[1]))
        return float(np.median(ms))

    res = {}
    for H in heads:
        pts = []
        for lg in lgs:
            n = 1 << lg
            g = torch.Generator(device=dev)
            g.manual_seed(7000 + lg)
            shape = (1, H, n, 64)
            q = torch.randn(shape, generator=g, device=dev)
            q = (q / q.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
            k = torch.randn(shape, generator=g, device=dev)
            k = (k / k.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
            v = torch.randn(shape, generator=g, device=dev).to(torch.bfloat16)
            out = torch.empty(shape, dtype=torch.float32, device=dev)
            t_exact = timed(lambda: sa.softmax_attention(q, k, v, 1.0, out=out))
            state = sa.new_state(basis, H, dev)
            ws = sa.workspace(sa.prefill_workspace_bytes(basis, 1, H, n, 64, sa.SATA_BF16), dev)
            t_sata = timed(lambda: sa.prefill(basis, q, k, v, state=state.zero_(), out=out, ws=ws))
            pts.append({"n": n, "exact_ms": t_exact, "sata_ms": t_sata,
                        "exact_ns_per_head_token": 1e6 * t_exact / (H * n),
                        "sata_ns_per_head_token": 1e6 * t_sata / (H * n)})
            print(f"crossover H={H} n=2^{lg}: exact {t_exact:.2f} ms, SATA {t_sata:.2f} ms", file=sys.stderr,
                  flush=True)
            del q, k, v, out, state, ws
            torch.cuda.empty_cache()
        cross = None
        for a_, b_ in zip(pts, pts[1:]):
            ra, rb = a_["exact_ms"] / a_["sata_ms"], b_["exact_ms"] / b_["sata_ms"]
            if ra < 1.0 <= rb:
                f = np.log(1.0 / ra) / np.log(rb / ra)
                cross = float(np.exp(np.log(a_["n"]) + f * (np.log(b_["n"]) - np.log(a_["n"]))))
                break
        res[f"heads_{H}"] = {"points": pts, "crossover_n": cross}
    return {"workload": "exact causal softmax (bf16 MFMA) vs SATA prefill, d_k=d_v=64, P=4, bf16 inputs, "
                        "device-generated inputs", "steps": reps, "warmup": warmup, **res}


def box_ceilings(reps=10):
    """Ceilings of this box from the ceiling kernels (libsata_ceilings.so, HIP
    events): a 1 GiB read+write copy, a 3 GiB in-place read-modify-write in the
    decode step's access shape, a 3 GiB read, and the bf16 and fp32 matrix-core
    loops (eight independent MFMA chains a wave, 1024 workgroups of 8 waves)."""
    import torch
    from constant_cost_taylor_amd import ceilings as CL
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    def timed(fn):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            ev[0].record(stream)
            fn()
            ev[1].record(stream)
            torch.cuda.synchronize()
            ms.append(ev[0].elapsed_time(ev[1]))
        return float(np.median(ms))

    res = {}
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    res["copy_1GiB_read_write_gbs"] = 2 * (1 << 30) / (timed(lambda: CL.copy(src, dst, sp)) * 1e-3) / 1e9
    del src, dst
    big = torch.ones(3 << 28, dtype=torch.float32, device=dev)
    res["rmw_3GiB_gbs"] = 2 * (3 << 30) / (timed(lambda: CL.rmw(big, sp)) * 1e-3) / 1e9
    part = torch.empty(CL.read_partials(3 << 30), dtype=torch.float32, device=dev)
    res["read_3GiB_gbs"] = (3 << 30) / (timed(lambda: CL.read(big, part, sp)) * 1e-3) / 1e9
    del big, part
    torch.cuda.empty_cache()
    blocks = 1024
    out = torch.empty(blocks * 512, dtype=torch.float32, device=dev)
    for code, name, iters in ((1, "mfma_bf16_tflops", 4000), (0, "mfma_f32_tflops", 2000)):
        t = timed(lambda: CL.mfma(code, blocks, iters, out, sp))
        res[name] = CL.mfma_flops(code, blocks, iters) / (t * 1e-3) / 1e12
    del out
    torch.cuda.empty_cache()
    return res


def ceilings(args):
    """Measured ceilings of this machine (torch / hipBLASLt kernels, HIP events):
    the bandwidth a read+write stream, an in-place read-modify-write stream
    and a read stream reach, and the bf16 matrix rate of a large GEMM."""
    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    def timed(fn, reps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            ev[0].record(stream)
            fn()
            ev[1].record(stream)
            torch.cuda.synchronize()
            ms.append(ev[0].elapsed_time(ev[1]))
        return float(np.median(ms))

    res = {}
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    t = timed(lambda: dst.copy_(src), 20)
    res["copy_1GiB_read_write_gbs"] = 2 * src.numel() * 4 / (t * 1e-3) / 1e9
    del src, dst
    big = torch.ones(3 << 28, dtype=torch.float32, device=dev)
    t = timed(lambda: big.add_(1.0), 10)
    res["inplace_rmw_3GiB_gbs"] = 2 * big.numel() * 4 / (t * 1e-3) / 1e9
    acc = torch.empty((), dtype=torch.float32, device=dev)
    t = timed(lambda: torch.sum(big, dim=0, out=acc), 10)
    res["read_3GiB_sum_gbs"] = big.numel() * 4 / (t * 1e-3) / 1e9
    del big, acc
    torch.cuda.empty_cache()
    n = 8192
    a = torch.randn((n, n), device=dev).to(torch.bfloat16)
    b = torch.randn((n, n), device=dev).to(torch.bfloat16)
    c = torch.empty((n, n), dtype=torch.bfloat16, device=dev)
    t = timed(lambda: torch.matmul(a, b, out=c), 20)
    res["gemm_bf16_8192_tflops"] = 2 * n ** 3 / (t * 1e-3) / 1e12
    del a, b, c
    torch.cuda.empty_cache()
    print(json.dumps({"metric": "measured ceilings of this box", "peaks": {"hbm_gbs": HBM_PEAK_GBS,
                      "bf16_tflops": BF16_PEAK_TFLOPS, "fp32_tflops": FP32_PEAK_TFLOPS},
                      "ceiling_kernels": box_ceilings(), "library_kernels": res}),
          flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on exactly one GPU (heads are independent; the multi-GPU "
              "sharding is a design note only). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.flatness:
        flatness(args)
        return
    if args.configs:
        configs(args)
        return
    if args.ceilings:
        ceilings(args)
        return
    if args.order5:
        order5(args)
        return
    import torch
    import constant_cost_taylor_amd as sa
    import workloads as W
    from oracle import sata_oracle as O

    w = W.WORKLOADS["decode_256x4096_d64"]
    S = w.B * w.H
    dsteps = args.decode_steps
    q, k, v = W.workload_inputs(w)
    qs, ks, vs = W.decode_inputs(w, dsteps)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    basis = sa.build_basis(w.d_k, w.P, w.c)
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).to(dev)
    Q, K, V = bf(q), bf(k), bf(v)
    DQ, DK, DV = bf(qs), bf(ks), bf(vs)
    state = sa.new_state(basis, S, dev)
    out = torch.empty((w.B, w.H, w.n, w.d_v), dtype=torch.float32, device=dev)
    dout = torch.empty((dsteps, S, w.d_v), dtype=torch.float32, device=dev)
    pws = sa.workspace(sa.prefill_workspace_bytes(basis, w.B, w.H, w.n, w.d_v, sa.SATA_BF16), dev)
    dws = sa.workspace(sa.decode_workspace_bytes(basis, S, w.d_v, sa.SATA_BF16), dev)
    stream = torch.cuda.current_stream(dev)
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ev_p = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev_d = [torch.cuda.Event(enable_timing=True) for _ in range(dsteps + 1)]
    pre_ms, dec_ms = [], []

    def step(record):
        state.zero_()
        if record:
            ev_p[0].record(stream)
        sa.prefill(basis, Q, K, V, state=state, out=out, ws=pws)
        if record:
            ev_p[1].record(stream)
            ev_d[0].record(stream)
        for t in range(dsteps):
            sa.decode_step(basis, DQ[t], DK[t], DV[t], state, out=dout[t], ws=dws)
            if record:
                ev_d[t + 1].record(stream)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
        torch.cuda.synchronize()
        pre_ms.append(ev_p[0].elapsed_time(ev_p[1]))
        dec_ms.extend(ev_d[t].elapsed_time(ev_d[t + 1]) for t in range(dsteps))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # sanity check of the last step against the oracle on a few decode rows
    s_chk = [0, S - 1]
    got = dout[:, s_chk].cpu().numpy()
    qf = q.reshape(S, w.n, w.d_k)
    kf = k.reshape(S, w.n, w.d_k)
    vf = v.reshape(S, w.n, w.d_v)
    errs = []
    for j, s in enumerate(s_chk):
        rr = np.arange(w.n, w.n + dsteps, max(1, dsteps // 16))
        ref = O.direct_taylor(np.concatenate([qf[s], qs[:, s]]).astype(np.float64),
                              np.concatenate([kf[s], ks[:, s]]).astype(np.float64),
                              np.concatenate([vf[s], vs[:, s]]).astype(np.float64), w.P, w.c, rows=rr)
        errs.append(O.row_normwise_error(got[rr - w.n, j], ref))

    ms_step = 1000.0 * wall / args.steps
    pre = float(np.median(pre_ms))
    dec = float(np.mean(dec_ms))
    D = basis.total_rows
    state_bytes = 2 * 4 * (w.d_v + 1) * D                  # read + write of one state
    io_bytes = 3 * w.d_k * 2 + w.d_v * 4                   # q, k, v bf16 in, fp32 out
    dec_bytes = S * (state_bytes + io_bytes)
    dec_gbs = dec_bytes / (dec * 1e-3) / 1e9
    _, page_flops = O.cost_model(w.d_k, w.d_v, w.P)
    pre_tokens = S * w.n
    pre_tflops = pre_tokens * page_flops / (pre * 1e-3) / 1e12
    tokens = S * (w.n + dsteps)
    value = tokens / (ms_step * 1e-3)

    res = {
        "metric": METRIC,
        "value": value,
        "unit": "head-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 inputs, f32 state",
        "data": "synthetic (seeded unit-norm Gaussian q,k; Gaussian v)",
        "config": {"workload": f"decode workload: {S} states (batch {w.B} x {w.H} heads), d_k=d_v={w.d_k}, "
                               f"P={w.P}, {w.n}-token prefill + {dsteps} decode steps",
                   "global_batch": w.B, "heads": w.H, "seq_len": w.n, "decode_steps": dsteps,
                   "parallelism": "single GPU"},
        "prefill": {"head_tokens_per_s": pre_tokens / (pre * 1e-3), "ms": pre,
                    "page_tflops": pre_tflops, "mfma_bf16_frac": pre_tflops / BF16_PEAK_TFLOPS},
        "decode": {"head_tokens_per_s": S / (dec * 1e-3), "ms_per_step": dec,
                   "first_last_ratio": float(np.mean(dec_ms[:8]) / np.mean(dec_ms[-8:])),
                   "hbm_gbs": dec_gbs, "hbm_frac": dec_gbs / HBM_PEAK_GBS},
        "roofline": {"bound": "hbm", "kernel": "decode step: decode_update_readout + decode_reduce",
                     "achieved": dec_gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": dec_gbs / HBM_PEAK_GBS,
                     "traffic": DECODE_TRAFFIC_BYTES if dsteps else None,
                     "traffic_unit": "bytes per launch (HBM, counter-measured)",
                     "algorithmic_bytes": dec_bytes},
        "check": {"decode_row_normwise_err": max(errs)},
    }
    if not args.no_mixed:
        res["decode_mixed_state"] = mixed_leg(sa, basis, w, Q, K, V, DQ, DK, DV, state, out, pws, q, k, v,
                                              qs, ks, vs, stream, min(dsteps, args.mixed_steps), dec)
    if not args.no_configs:
        # the other workloads, timed after the headline step with its buffers freed
        del Q, K, V, DQ, DK, DV, state, out, dout, pws, dws
        torch.cuda.empty_cache()
        res["configs"] = {"prefill": config_points(args.config_steps, 1),
                          "long_context": flatness_points(args.config_steps, 1),
                          "order5": order5_point(args.config_steps, 1, 64),
                          "segments": segment_points(args.config_steps, 1),
                          "softmax_crossover": crossover_points(3, 1)}
    if not args.no_configs:
        # the box's own ceilings (ceiling kernels), and the two legs against them
        ceil = box_ceilings()
        ceil["decode_frac_of_rmw"] = dec_gbs / ceil["rmw_3GiB_gbs"]
        ceil["prefill_frac_of_mfma_bf16"] = pre_tflops / ceil["mfma_bf16_tflops"]
        res["ceilings"] = ceil
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, q, k, v, qs, ks, vs, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
