#!/usr/bin/env python3
"""Benchmark of exact shared-prefix attention, forward + backward, on one MI355X.

One step is the whole hot path over one replay tree, as eleven single C-ABI steps
(identical kernels to the four composite calls): prompt prefill forward; replay against
the stationary prompt K/V; response-local replay; LSE merge; row dots; prompt K/V gradient
summed over all branches; branch K/V gradient; branch dQ; prefill K/V gradient (adding
the branch sum); prefill dQ. Inputs are seeded, synthetic and resident in HBM before the
timed region.

Prints one JSON line: algorithmic TFLOP/s of the step (reuse work only: 4*D flops per
visible (query, key) pair forward, 10*D backward, summed over query heads), the roofline
of the dominant kernel (HIP events around its launch inside the timed steps), and the
fp64 CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "shared-prefix attn fwd+bwd TFLOP/s and % bf16 MFMA peak, 1 MI355X"
BF16_PEAK_TFLOPS = 2516.6   # 256 CU x 4096 flop/clk x 2.4 GHz, dense
F32_PEAK_TFLOPS = 157.3

STAGES = ["prefill_fwd", "replay_prompt_fwd", "replay_local_fwd", "merge", "row_dot_r",
          "replay_prompt_bwd", "replay_local_bwd", "replay_dq", "row_dot_p", "prefill_kv_bwd",
          "prefill_dq"]


def stage_flops(shape):
    """Algorithmic flops of each MFMA stage (per launch), by the pair counts it covers.
    Forward stages: 4*D per pair (QK^T, PV). Key-stationary gradient stages: 8*D per
    pair (QK^T, dO V^T, P^T dO, dS^T Q). dQ stages: 2*D per pair (dS K), the remaining
    algorithmic backward share; their recomputation of QK^T and dO V^T is not counted."""
    P, T, D, Hq = shape.P, shape.T, shape.D, shape.Hq
    tri_p = P * (P + 1) // 2
    cross = T * P
    tri_r = sum(r * (r + 1) // 2 for r in shape.lens)
    return {
        "prefill_fwd": 4 * D * tri_p * Hq,
        "replay_prompt_fwd": 4 * D * cross * Hq,
        "replay_local_fwd": 4 * D * tri_r * Hq,
        "replay_prompt_bwd": 8 * D * cross * Hq,
        "replay_local_bwd": 8 * D * tri_r * Hq,
        "replay_dq": 2 * D * (cross + tri_r) * Hq,
        "prefill_kv_bwd": 8 * D * tri_p * Hq,
        "prefill_dq": 2 * D * tri_p * Hq,
    }


def stage_bytes(shape, parts: int = 2):
    """Algorithmic HBM bytes of the HBM-bound stages (per launch); ``parts`` partial states
    per branch row are merged (2: the whole prompt and the branch)."""
    T, P, D, Hq = shape.T, shape.P, shape.D, shape.Hq
    esz = 2 if shape.dtype == "bf16" else 4
    return {
        # the fp32 partial outputs and LSEs read, output + LSE written
        "merge": T * Hq * (parts * (4 * D + 4) + esz * D + 4),
        # O and dO read, one float written
        "row_dot_r": T * Hq * (2 * esz * D + 4),
        "row_dot_p": P * Hq * (2 * esz * D + 4),
    }


def cpu_baseline(w, budget_s: float = 12.0):
    """The fp64 oracle, unmodified, on branch 0's flattened sequence (P + R_0 tokens), one
    query head at a time (head h with its key/value head), forward + backward, until about
    ``budget_s`` seconds of CPU work are done; extrapolated to the whole workload by
    flattened pair count x Hq / heads done and converted to algorithmic TFLOP/s."""
    import torch
    from oracle import flattened_tree_attention
    from workloads import algorithmic_flops, pairs_flattened, make_shape

    s = w.shape
    R0 = s.lens[0]
    group = s.Hq // s.Hkv
    sub = make_shape(s.P, [R0], 1, 1, s.D, dtype=s.dtype, std=s.std)
    heads = 0
    t0 = time.perf_counter()
    while heads < s.Hq and (heads == 0 or time.perf_counter() - t0 < budget_s):
        h, g = heads, heads // group
        flattened_tree_attention(w.q_p[:, h:h + 1], w.k_p[:, g:g + 1], w.v_p[:, g:g + 1],
                                 w.q_r[:R0, h:h + 1], w.k_r[:R0, g:g + 1], w.v_r[:R0, g:g + 1], [0, R0],
                                 do_p=w.do_p[:, h:h + 1], do_r=w.do_r[:R0, h:h + 1])
        heads += 1
    dt = time.perf_counter() - t0
    factor = pairs_flattened(s) * s.Hq / (pairs_flattened(sub) * heads)
    full_time = dt * factor
    value = algorithmic_flops(s) / full_time / 1e12
    return {"value": value, "unit": "TFLOP/s", "cores": torch.get_num_threads(), "kind": "oracle",
            "sample": f"branch 0 flattened ({s.P}+{R0} tokens), query heads 0..{heads - 1}, fwd+bwd in "
                      f"fp64: {dt:.2f} s; extrapolated x{factor:.1f} (flattened pairs x Hq / heads) to "
                      f"{full_time:.0f} s for the whole workload",
            "sample_seconds": dt, "extrapolated_seconds": full_time}


def gemm_reference(dev, n=8192, reps=10):
    """The vendor library's dense bf16 GEMM (torch.matmul of two contiguous n x n matrices)
    timed right after the step: the matrix-core rate reachable at the clocks the chip runs at
    under this load, as a yardstick beside the spec peak. Not part of the path."""
    import torch
    g = torch.Generator(device="cpu").manual_seed(1)
    a = torch.randn(n, n, generator=g).to(device=dev, dtype=torch.bfloat16).contiguous()
    b = torch.randn(n, n, generator=g).to(device=dev, dtype=torch.bfloat16).contiguous()
    c = torch.matmul(a, b)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b, c
    return {"kind": f"torch.matmul bf16 {n}x{n}x{n}", "TFLOP/s": round(2 * n ** 3 / (ms / 1e3) / 1e12, 1)}


def small_grid(shape):
    """Whether the replay kernels' grids are too small to fill 256 compute units for long
    (fewer than 8 rounds of the branch-row workgroups): then independent steps run on
    separate streams, so one kernel's tail and idle units take another's workgroups."""
    group = shape.Hq // shape.Hkv
    hg = 4 if group % 4 == 0 else (2 if group % 2 == 0 else 1)
    rows = 32 * 8 // hg
    wgs = -(-shape.T // rows) * (shape.Hq // hg)
    return wgs < 8 * 256


def schedule(stages, nstreams):
    """Issue plan: (kind, stream, name) with kind "run", "mark" (record an event) or "wait".
    Three streams: the prompt prefill, its row dot and the prefill dQ on one stream, beside the
    replay; the branch-local forward beside the replay against the prompt; after the merge, the
    prompt K/V gradient (then the prefill K/V gradient, which adds it) beside the branch K/V
    gradient and branch dQ. Every dependency of the path is an event; results are identical to the
    one-stream order (no step's arithmetic depends on the schedule)."""
    if nstreams == 1:
        return [("run", 0, n) for n in stages]
    p = [("run", 0, "prefill_fwd"), ("run", 2, "replay_local_fwd"), ("mark", 2, "f3"),
         ("run", 1, "replay_prompt_fwd"), ("wait", 1, "f3"), ("run", 1, "merge")]
    if "row_dot_r" not in stages:
        return p
    p += [("run", 0, "row_dot_p"), ("mark", 0, "rdp"),
          ("run", 1, "row_dot_r"), ("mark", 1, "rdr"), ("run", 1, "replay_prompt_bwd"),
          ("wait", 2, "rdr"), ("run", 2, "replay_local_bwd"), ("run", 2, "replay_dq"),
          ("wait", 1, "rdp"), ("run", 1, "prefill_kv_bwd"),
          ("run", 0, "prefill_dq")]
    return p


class Runner:
    """One pass of the whole hot path over a tree (eleven single C-ABI steps, the identical
    kernels of the four composite calls) on 1 or 3 streams, with every buffer allocated once.
    ``step(ev)`` issues a pass; ``buf`` holds the outputs."""

    def __init__(self, w, t, dev, nstreams: int = 1, nsh: int = 1):
        import torch
        from shared_prefix_attention_prompt_amd import _lib, ops
        s = w.shape
        self.shape = s
        tr = ops.Tree(s.P, s.offsets, s.Hq, s.Hkv, s.D, s.torch_dtype, dev)
        f32 = torch.float32
        b = self.buf = {
            "o_p": tr.empty(s.P, s.Hq, s.D), "lse_p": tr.empty(s.Hq, s.P, dtype=f32),
            "oa": tr.empty(s.T, s.Hq, s.D, dtype=f32), "la": tr.empty(s.Hq, s.T, dtype=f32),
            "ob": tr.empty(s.T, s.Hq, s.D, dtype=f32), "lb": tr.empty(s.Hq, s.T, dtype=f32),
            "o_r": tr.empty(s.T, s.Hq, s.D), "lse_r": tr.empty(s.Hq, s.T, dtype=f32),
            "rd_r": tr.empty(s.Hq, s.T, dtype=f32), "rd_p": tr.empty(s.Hq, s.P, dtype=f32),
            "dk_acc": tr.empty(s.P, s.Hkv, s.D, dtype=f32), "dv_acc": tr.empty(s.P, s.Hkv, s.D, dtype=f32),
            "dk_r": torch.empty_like(t["k_r"]), "dv_r": torch.empty_like(t["v_r"]),
            "dq_r": torch.empty_like(t["q_r"]), "dk_p": torch.empty_like(t["k_p"]),
            "dv_p": torch.empty_like(t["v_p"]), "dq_p": torch.empty_like(t["q_p"]),
        }
        cuts = [min(s.P, round(s.P * i / nsh / 256) * 256) for i in range(nsh)] + [s.P]
        if any(q <= p for p, q in zip(cuts, cuts[1:])):
            raise ValueError(f"--kv-shards {nsh}: the prompt of {s.P} keys cannot be cut into {nsh} non-empty "
                             "ranges of whole 256-key blocks")
        self.cuts = cuts
        shard_bufs = [(tr.empty(s.T, s.Hq, s.D, dtype=f32), tr.empty(s.Hq, s.T, dtype=f32)) for _ in range(nsh - 1)]
        nws = max(_lib.workspace_bytes(tr.dims, op) for op in range(13))
        # shard layout: each shard's float32 dQ partial over its key range, plus the own-branch one
        dq_parts = [tr.empty(s.T, s.Hq, s.D, dtype=f32) for _ in range(nsh + 1)] if nsh > 1 else []
        main = torch.cuda.current_stream(dev)
        self.nstreams = nstreams
        streams = [main] if nstreams == 1 else [torch.cuda.Stream(dev) for _ in range(3)]
        wss = [torch.empty(max(nws, 256), dtype=torch.uint8, device=dev) for _ in streams]
        run = {
            "prefill_fwd": lambda ws: _lib._check(_lib.augtree_prefill_fwd(
                tr.dims, t["q_p"].data_ptr(), t["k_p"].data_ptr(), t["v_p"].data_ptr(), b["o_p"].data_ptr(),
                b["lse_p"].data_ptr(), ws.data_ptr(), ws.numel(), tr.stream()), "augtree_prefill_fwd"),
            "replay_prompt_fwd": lambda ws: [ops.replay_prompt_fwd(
                tr, t["k_p"], t["v_p"], t["q_r"], cuts[i], cuts[i + 1],
                out=(b["oa"], b["la"]) if i == 0 else shard_bufs[i - 1], ws=ws) for i in range(nsh)],
            "replay_local_fwd": lambda ws: ops.replay_local_fwd(tr, t["q_r"], t["k_r"], t["v_r"],
                                                                out=(b["ob"], b["lb"]), ws=ws),
            "merge": lambda ws: ops.merge_partials(tr, [(b["oa"], b["la"])] + shard_bufs + [(b["ob"], b["lb"])],
                                                   out=(b["o_r"], b["lse_r"])),
            "row_dot_r": lambda ws: ops.row_dot(tr, b["o_r"], t["do_r"], out=b["rd_r"]),
            "replay_prompt_bwd": lambda ws: [ops.replay_prompt_bwd(
                tr, t["k_p"], t["v_p"], t["q_r"], b["lse_r"], b["rd_r"], t["do_r"], cuts[i], cuts[i + 1],
                dk_acc=b["dk_acc"], dv_acc=b["dv_acc"], ws=ws) for i in range(nsh)],
            "replay_local_bwd": lambda ws: ops.replay_local_bwd(
                tr, t["q_r"], t["k_r"], t["v_r"], b["lse_r"], b["rd_r"], t["do_r"], out=(b["dk_r"], b["dv_r"]),
                ws=ws),
            "replay_dq": (lambda ws: ops.replay_dq(tr, t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"], b["lse_r"],
                                                   b["rd_r"], t["do_r"], out=b["dq_r"], ws=ws)) if nsh == 1 else
                         (lambda ws: ([ops.replay_prompt_dq(tr, t["k_p"], t["v_p"], t["q_r"], b["lse_r"], b["rd_r"],
                                                            t["do_r"], cuts[i], cuts[i + 1], out=dq_parts[i], ws=ws)
                                       for i in range(nsh)],
                                      ops.replay_local_dq(tr, t["q_r"], t["k_r"], t["v_r"], b["lse_r"], b["rd_r"],
                                                          t["do_r"], out=dq_parts[nsh], ws=ws),
                                      ops.sum_parts(tr, dq_parts, out=b["dq_r"]))),
            "row_dot_p": lambda ws: ops.row_dot(tr, b["o_p"], t["do_p"], out=b["rd_p"]),
            "prefill_kv_bwd": lambda ws: ops.prefill_kv_bwd(
                tr, t["q_p"], t["k_p"], t["v_p"], b["lse_p"], b["rd_p"], t["do_p"], b["dk_acc"], b["dv_acc"],
                out=(b["dk_p"], b["dv_p"]), ws=ws),
            "prefill_dq": lambda ws: ops.prefill_dq(tr, t["q_p"], t["k_p"], t["v_p"], b["lse_p"], b["rd_p"],
                                                    t["do_p"], out=b["dq_p"], ws=ws),
        }
        self.stages = STAGES if s.backward else STAGES[:4]
        plan = schedule(self.stages, nstreams)
        self._torch, self._main, self._streams, self._wss, self._run, self._plan = torch, main, streams, wss, run, plan

    def step(self, ev=None):
        """One pass of the whole path. ev: per-stage (start, end) timing events, recorded on
        the stream each stage runs on."""
        torch, main, streams = self._torch, self._main, self._streams
        if self.nstreams > 1:
            fork = torch.cuda.Event()
            fork.record(main)
            for x in streams:
                x.wait_event(fork)
        marks = {}
        for kind, si, name in self._plan:
            st = streams[si]
            if kind == "wait":
                st.wait_event(marks[name])
                continue
            if kind == "mark":
                marks[name] = torch.cuda.Event()
                marks[name].record(st)
                continue
            with torch.cuda.stream(st):
                if ev is not None:
                    ev[name][0].record(st)
                self._run[name](self._wss[si])
                if ev is not None:
                    ev[name][1].record(st)
        if self.nstreams > 1:
            for x in streams:
                j = torch.cuda.Event()
                j.record(x)
                main.wait_event(j)


def kernel_source_digest():
    """sha256 over the HIP sources, so stored counter readings are only reported for the
    kernels they were taken on."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "shared_prefix_attention_prompt_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp", ".h")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def _stored(name, stage, workload):
    """Record of ``stage`` in the committed counter summary profiles/<name>, or None when it was
    taken on other kernel sources or another workload."""
    path = os.path.join(ROOT, "profiles", name)
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sources_sha256") != kernel_source_digest():
        return None
    if "workloads" in rec:   # several workloads in one record
        return rec["workloads"].get(workload, {}).get("stages", {}).get(stage)
    return rec.get("stages", {}).get(stage) if rec.get("workload") == workload else None


def stored_traffic(stage, workload):
    """HBM bytes per launch of ``stage`` (FETCH_SIZE + WRITE_SIZE counter runs, calibrated)."""
    return _stored("traffic.json", stage, workload)


def stored_mfma(stage, workload):
    """Matrix-core counters of ``stage``'s kernels per launch: issued flops
    (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512) and the busy fraction of the matrix cores."""
    return _stored("mfma.json", stage, workload)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=4, help="workload number (1..5)")
    ap.add_argument("--workload", default=None,
                    help="a group-size / prompt:response-ratio sweep tree by name (group_g8, "
                         "group_g16, group_g32, group_g64, response_heavy); overrides --config")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--streams", type=int, default=0, choices=[0, 1, 3],
                    help="1: every step on one stream; 3: independent steps on three streams; "
                         "0 (default): three when the kernels' grids are too small to fill the GPU")
    ap.add_argument("--no-gemm-reference", action="store_true",
                    help="skip timing the vendor bf16 GEMM reported beside the roofline peak")
    ap.add_argument("--kv-shards", type=int, default=1, choices=range(1, 8), metavar="{1..7}",
                    help="split the prompt K/V into this many stationary shards (the paper's MoveQ "
                         "layout): the replay forward, the prompt K/V gradient and the branch dQ run "
                         "once per shard's key range; the merge combines shards + 1 partial states and "
                         "the dQ partials (shards + own branch) are summed in a fixed order")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the timed steps, run a plain elementwise copy of this many MiB "
                         "three times (a known-size kernel to scale HBM byte counters by)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the shared-prefix "
              "path is measured on one MI355X's share; no multi-GPU figure is produced.", file=sys.stderr)
        return 2

    import torch
    from shared_prefix_attention_prompt_amd import _lib, ops
    from workloads import SWEEPS, algorithmic_flops, config_seed, make_inputs, workload_name

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    _lib.load()
    dev = torch.device("cuda:0")
    if args.workload is not None and args.workload not in SWEEPS:
        print(f"unknown sweep tree {args.workload!r}; one of {sorted(SWEEPS)}", file=sys.stderr)
        return 2
    cfg = args.workload if args.workload is not None else args.config
    t_gen = time.perf_counter()
    w = make_inputs(cfg)
    s = w.shape
    t = {k: getattr(w, k).to(dev) for k in ["q_p", "k_p", "v_p", "q_r", "k_r", "v_r", "do_p", "do_r"]
         if getattr(w, k) is not None}
    torch.cuda.synchronize()
    print(f"# inputs for config {cfg} ready in {time.perf_counter() - t_gen:.1f} s "
          f"(P={s.P}, T_R={s.T}, G={s.G}, Hq={s.Hq}, Hkv={s.Hkv}, D={s.D})", file=sys.stderr, flush=True)

    nsh = args.kv_shards
    nstreams = args.streams if args.streams > 0 else (3 if small_grid(s) else 1)
    try:
        runner = Runner(w, t, dev, nstreams, nsh)
    except ValueError as e:
        print(str(e), file=sys.stderr)
        return 2
    stages, step = runner.stages, runner.step
    main = torch.cuda.current_stream(dev)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [{n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for n in stages}
              for _ in range(args.steps)]
    # one event per step boundary on the main stream (every stream joins it at each step's
    # end): the K steps' total time, and the median step
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    marks[0].record(main)
    for i in range(args.steps):
        step(events[i])
        marks[i + 1].record(main)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    ms_per_step = marks[0].elapsed_time(marks[-1]) / args.steps
    ms_median = step_ms[len(step_ms) // 2] if len(step_ms) % 2 else 0.5 * (
        step_ms[len(step_ms) // 2 - 1] + step_ms[len(step_ms) // 2])

    stage_ms = {}
    for name in stages:
        stage_ms[name] = sum(e[name][0].elapsed_time(e[name][1]) for e in events) / args.steps
    flops = algorithmic_flops(s)
    tflops = flops / (ms_per_step / 1e3) / 1e12
    peak = BF16_PEAK_TFLOPS if s.dtype == "bf16" else F32_PEAK_TFLOPS
    sf = {k: v for k, v in stage_flops(s).items() if k in stages}
    sb = {k: v for k, v in stage_bytes(s, parts=nsh + 1).items() if k in stages}
    kernels = {}
    for name in stages:
        ms = stage_ms[name]
        entry = {"ms": round(ms, 4)}
        if name in sf:
            entry["TFLOP/s"] = round(sf[name] / (ms / 1e3) / 1e12, 1)
        if name in sb:
            entry["GB/s"] = round(sb[name] / (ms / 1e3) / 1e9, 1)
        kernels[name] = entry
    wl = workload_name(cfg)
    for name in sf:
        mf = stored_mfma(name, wl) if nsh == 1 else None
        if mf is not None:
            # issued matrix work from the committed counter run of the same kernels and workload,
            # over this run's time: makes the dQ passes' recompute visible
            kernels[name]["issued_TFLOP/s"] = round(mf["issued_flops"] / (stage_ms[name] / 1e3) / 1e12, 1)
            kernels[name]["mfma_busy"] = mf["busy"]
    dom = max(sf, key=lambda n: stage_ms[n])
    achieved = sf[dom] / (stage_ms[dom] / 1e3) / 1e12
    tr_rec = stored_traffic(dom, wl) if nsh == 1 else None
    mf_rec = stored_mfma(dom, wl) if nsh == 1 else None
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": tr_rec["bytes_per_launch"] if tr_rec else None,
                "alg_flops_per_launch": sf[dom], "avg_launch_ms": round(stage_ms[dom], 4),
                "issued": (None if mf_rec is None else
                           {"TFLOP/s": round(mf_rec["issued_flops"] / (stage_ms[dom] / 1e3) / 1e12, 1),
                            "flops_per_launch": mf_rec["issued_flops"], "mfma_busy": mf_rec["busy"],
                            "clock_GHz": mf_rec.get("clock_GHz"), "source": "profiles/mfma.json"})}
    if s.dtype == "bf16" and not args.no_gemm_reference:
        roofline["gemm_reference"] = gemm_reference(dev)

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline and s.backward:
        cpu = cpu_baseline(w)
        cpu["value"] = round(cpu["value"], 6)

    line = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_median": round(ms_median, 4), "ms_per_step_min": round(step_ms[0], 4),
        "ms_per_step_max": round(step_ms[-1], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": s.dtype,
        "data": "synthetic", "pct_bf16_peak": round(100 * tflops / peak, 2),
        "config": {"workload": workload_name(cfg), "P": s.P, "G": s.G, "branch_lens": list(s.lens),
                   "T_R": s.T, "Hq": s.Hq, "Hkv": s.Hkv, "D": s.D,
                   "passes": "fwd+bwd" if s.backward else "fwd",
                   "alg_flops": flops, "seed": config_seed(cfg), "streams": nstreams,
                   "kv_shards": nsh},
        "roofline": roofline, "cpu_baseline": cpu, "kernels": kernels,
        "wall_s": round(wall, 3),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
