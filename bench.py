"""Benchmark: CSA2 decode tokens/s/layer and fraction of the HBM roofline.

Default workload: a decoder group of 4 layers (Full + 3 Reuse), decode batch 8,
context 131072 per sequence -- the 128K-context decode configuration.  One
step = every layer of the group once (indexer scan, Top-512, FP4 gather +
dequantisation + attention with the 128-token window) for one batch.

Prints ONE JSON line.  See --help for the options; with no flags it runs on
one GPU and finishes within a few minutes.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense


def parse():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="decode_128k",
                   choices=["decode_128k", "decode_1m", "prefill", "serving", "model38", "causal_prefill"],
                   help="decode_128k: Full + 3 Reuse, batch 8 at 131072; decode_1m: hierarchical group at 1048576; "
                        "prefill: 4096-row chunk over 131072 entries; serving: 20 decoder layers, batch 32, paged; "
                        "model38: the 38 CSA2 layers of one decode step, encoder at ratio 2 + decoder, batch 8 at "
                        "128K; causal_prefill: the prefill chunk with its own compressed entries under the "
                        "completion mask")
    p.add_argument("--replicas", type=int, default=3,
                   help="input replicas cycled per step so the 256 MB last-level cache cannot serve them")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-1m", action="store_true", help="skip the 1M-context group (reported beside the default)")
    p.add_argument("--no-model", action="store_true",
                   help="skip the 38-layer decode step (reported beside the default)")
    p.add_argument("--no-fp8", action="store_true",
                   help="skip the 128K group on FP8 indexer keys (reported beside the default)")
    p.add_argument("--no-others", action="store_true",
                   help="skip the full_4k, prefill and serving sub-objects (the default line keeps the rest)")
    p.add_argument("--no-extras", action="store_true",
                   help="report the default workload alone (no 1M, 4K, prefill, serving, FP8-key or 38-layer "
                        "sub-objects)")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum CPU time of the oracle baseline")
    p.add_argument("--copy-probe", action="store_true",
                   help="only run a plain 1 GiB device copy (for counter scaling)")
    return p.parse_args()


def algorithmic_bytes(w, key_bytes=128):
    """Per step: indexer keys key_bytes/position (128 bf16, 68 FP8) + q_idx
    512 B + Top-512 out 2048 B per Full row; per attention row-layer 460 800 B
    (512 FP4 entries of 288 B, window K+V 2*128*1024 B, query 16 KiB, output
    32 KiB fp32, indices 2 KiB)."""
    per_attn = 512 * 288 + 2 * 128 * 1024 + 16 * 512 * 2 + 16 * 512 * 4 + 512 * 4
    scan = 0
    attn_layers = 0
    for m in w.schedule:
        if m == "F":
            scan += sum(key_bytes * L + 512 + 2048 for L in w.seq_lens)
            if w.hier:
                scan += 8192 * w.B
        elif m == "I":
            scan += w.B * (2048 * 8 * key_bytes + 8192 + 512 + 2048)
    for li, m in enumerate(w.schedule):
        if not (m == "F" and w.hier and w.full_blocks_only):
            attn_layers += 1
    return scan + attn_layers * w.R * per_attn, scan, attn_layers


def src_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profiles(kernel_src):
    """HBM bytes per launch of the scan kernel from the committed counter
    summary (rocprofv3 FETCH_SIZE and WRITE_SIZE, scaled by the same counters
    on a 1 GiB device copy), if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "index_scan_decode_F3R_b8_L131072_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
        if d.get("src_sha") != src_sha(kernel_src):
            return None
        return float(d["bytes_per_launch"])
    except Exception:
        return None


def _oracle_inputs(w):
    """The workload's inputs as the oracle takes them (numpy, host): the FP4
    main KV and indexer keys at their slots, and every layer's own inputs.
    Set-up, not timed."""
    import numpy as np
    from fp4_kv_cache_02_amd import synth
    from oracle import csa2_oracle as O

    n_slots, pt, _ = synth.slots_layout(w)
    K = np.zeros((n_slots, 64), np.uint16)
    q_full = synth.gen_q_idx(w, 0) if w.planted > 0 else None
    P = np.zeros((n_slots, 256), np.uint8)
    S = np.zeros((n_slots, 32), np.uint8)
    if w.raw_fp4:
        P, S = synth.gen_fp4_raw(w, n_slots)
    elif w.kv_pool:
        pool_p, pool_s = O.quantize_fp4(synth.gen_kv_pool(w))
    if w.shared_slots:
        K[:w.n_max] = synth.gen_k_idx_seq(w, 0, q_full, L=w.n_max)
    for b in range(0 if w.shared_slots else w.B):
        L = w.seq_lens[b]
        sl = synth.slot_index(w, pt, b, np.arange(L))
        K[sl] = synth.gen_k_idx_seq(w, b, q_full)
        if w.raw_fp4:
            continue
        if w.kv_pool:
            m = synth.gen_kv_pool_map(w, b)
            P[sl], S[sl] = pool_p[m], pool_s[m]
        else:
            P[sl], S[sl] = O.quantize_fp4(synth.gen_kv_values(w, b, 0, L))
    arrays = {"P": P, "S": S, "K": K}
    if pt is not None:
        arrays["pt"] = pt
    for li, m in enumerate(w.schedule):
        k, v, _, st, ln = synth.gen_swa(w, li)
        arrays.update({f"q{li}": synth.gen_q(w, li), f"k{li}": k, f"v{li}": v, f"st{li}": st, f"ln{li}": ln})
        if m in "FI":
            arrays[f"qi{li}"] = synth.gen_q_idx(w, li)
    return arrays


class _OracleGroup:
    """Runs the oracle's layer steps of workload w for chosen rows."""

    def __init__(self, w, arrays):
        from oracle import csa2_oracle as O
        self.w = w
        self.a = arrays
        self.cache = O.Cache(arrays["P"], arrays["S"], arrays["K"], w.seq_lens, arrays.get("pt"), 64,
                             w.slot_stride)
        self.row_seq = list(w.row_seq())

    def run_rows(self, rs):
        """The group's layers over rows rs (their own Top-k state); returns
        the number of row-layers attended."""
        from fp4_kv_cache_02_amd import synth
        from oracle import csa2_oracle as O
        w, a = self.w, self.a
        state = O.GroupState(w.R)
        n = 0
        for li, m in enumerate(w.schedule):
            blocks_only = m == "F" and w.hier and w.full_blocks_only
            O.layer_step(synth.MODES[m], self.cache, state, self.row_seq, a.get(f"qi{li}"), a[f"q{li}"],
                         a[f"k{li}"], a[f"v{li}"], a[f"st{li}"], a[f"ln{li}"], 1.0 / math.sqrt(512), hier=w.hier,
                         blocks_only=blocks_only, rows=rs, swa_shared=w.shared_slots)
            n += 0 if blocks_only else len(rs)
        return n


_WORKER = {}


def _oracle_worker_init(kind, folder, names):
    """Process-pool worker set-up: one numpy thread, the inputs memory-mapped
    from the files the parent wrote."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_limits
        _WORKER["limits"] = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        pass
    from fp4_kv_cache_02_amd import synth
    w = synth.workload(kind)
    arrays = {n: np.load(os.path.join(folder, n + ".npy"), mmap_mode="r") for n in names}
    _WORKER["group"] = _OracleGroup(w, arrays)


def _oracle_worker_rows(rs):
    return _WORKER["group"].run_rows(rs)


def cpu_baseline(w, kind, min_seconds, procs=1, arrays=None):
    """The oracle, untuned, on the same workload: rows through every layer of
    the group (scan + Top-512 + attention per layer, each row with its own
    Top-k state), repeated until at least `min_seconds` have passed.  procs =
    1: in this process, one numpy thread.  procs > 1: a pool of that many
    processes (spawned, one numpy thread each, the inputs memory-mapped from
    files the parent writes), one row per task, kept busy until the time is
    up.  Input generation (and the oracle's quantisation of the main KV) is
    set-up and not timed."""
    import numpy as np
    rows = list(range(w.R if not w.prefill_rows else 4))   # prefill: a sample of 4 chunk rows
    if arrays is None:
        arrays = _oracle_inputs(w)
    if procs <= 1:
        try:
            from threadpoolctl import threadpool_limits
            ctx = threadpool_limits(limits=1)
        except Exception:  # pragma: no cover
            ctx = None
        grp = _OracleGroup(w, arrays)
        t0 = time.perf_counter()
        attended = reps = 0
        while True:
            attended += grp.run_rows(rows)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds:
                break
        if ctx is not None:
            ctx.restore_original_limits()
        how = "in one process, one numpy thread"
    else:
        import multiprocessing as mp
        import shutil
        import tempfile
        from concurrent.futures import FIRST_COMPLETED, ProcessPoolExecutor, wait
        base = "/dev/shm" if os.path.isdir("/dev/shm") else None
        folder = tempfile.mkdtemp(prefix="csa2_oracle_", dir=base)
        try:
            for n, arr in arrays.items():
                np.save(os.path.join(folder, n + ".npy"), np.ascontiguousarray(arr))
            with ProcessPoolExecutor(max_workers=procs, mp_context=mp.get_context("spawn"),
                                     initializer=_oracle_worker_init,
                                     initargs=(kind, folder, sorted(_oracle_names(w)))) as pool:
                # warm every worker (start-up and memory-mapping are not timed)
                list(pool.map(_oracle_worker_rows, [[]] * procs))
                t0 = time.perf_counter()
                attended = reps = 0
                nxt = 0
                pending = set()
                while len(pending) < procs:
                    pending.add(pool.submit(_oracle_worker_rows, [rows[nxt % len(rows)]]))
                    nxt += 1
                while pending:
                    done, pending = wait(pending, return_when=FIRST_COMPLETED)
                    for f in done:
                        attended += f.result()
                    if time.perf_counter() - t0 < min_seconds:
                        for _ in done:
                            pending.add(pool.submit(_oracle_worker_rows, [rows[nxt % len(rows)]]))
                            nxt += 1
                dt = time.perf_counter() - t0
                reps = nxt / len(rows)
        finally:
            shutil.rmtree(folder, ignore_errors=True)
        how = f"in a pool of {procs} spawned processes (one numpy thread each), one row per task"
    sample = ("the whole workload" if len(rows) == w.R else f"{len(rows)} of the {w.R} rows of the workload")
    return {"value": attended / dt, "unit": "tokens/s/layer", "cores": procs, "kind": "oracle",
            "sample": f"{sample} ({len(rows)} rows x {len(w.schedule)} layers) run {reps:g} times, "
                      f"{attended} row-layers in {dt:.1f} s {how} (numpy elementwise float32 scores, "
                      f"float64 attention); input generation not timed",
            "host_cores_available": len(os.sched_getaffinity(0))}


def _oracle_names(w):
    names = {"P", "S", "K"}
    if w.paged:
        names.add("pt")
    for li, m in enumerate(w.schedule):
        names.update({f"q{li}", f"k{li}", f"v{li}", f"st{li}", f"ln{li}"})
        if m in "FI":
            names.add(f"qi{li}")
    return names


def data_desc(w):
    if w.raw_fp4:
        kv = "main KV drawn as raw FP4 nibbles and E4M3 scale codes 0x20-0x37"
    elif w.kv_pool:
        kv = f"N(0,1) main KV quantised on the GPU from a pool of {w.kv_pool} vectors"
    else:
        kv = "N(0,1) main KV quantised on the GPU"
    extra = f", {w.planted:.0%} planted indexer keys" if w.planted else ""
    return f"synthetic (seeded; {kv}; bf16 N(0,1) queries, indexer keys and windows{extra})"


def fp8_keys(inp):
    """The workload's bf16 indexer keys as FP8 keys, quantised on the GPU by
    the library's FP8 key quantiser (input preparation, not timed): per slot
    scale = max |k| / 448 and codes = E4M3(k / scale)."""
    import dataclasses
    import torch
    from fp4_kv_cache_02_amd import csa2
    n = inp.k_idx.shape[0]
    codes = torch.zeros((n, 64), dtype=torch.uint8, device=inp.k_idx.device)
    scale = torch.zeros((n,), dtype=torch.float32, device=inp.k_idx.device)
    csa2.csa2_fp8_key_quantize(inp.k_idx, codes, scale)
    return dataclasses.replace(inp, k_idx=codes, k_scale=scale)


def replica(base):
    """A copy of a workload's device inputs in separate memory, so that
    cycling replicas step by step leaves no input in the 256 MB last-level
    cache from the step before."""
    import dataclasses
    from fp4_kv_cache_02_amd import group

    def cl(t):
        return None if t is None else t.clone()
    layers = [group.LayerInputs(q=cl(L.q), swa_k=cl(L.swa_k), swa_v=cl(L.swa_v), swa_start=cl(L.swa_start),
                                swa_len=cl(L.swa_len), q_idx=cl(L.q_idx)) for L in base.layers]
    return dataclasses.replace(base, kv_fp4=cl(base.kv_fp4), kv_scale=cl(base.kv_scale), k_idx=cl(base.k_idx),
                               k_scale=cl(base.k_scale), seq_len=cl(base.seq_len), page_table=cl(base.page_table),
                               row_seq=cl(base.row_seq), layers=layers)


def measure(w, steps, warmup, n_replicas, fp8=False):
    """Times `steps` whole steps of workload w (every group once) and, apart,
    back-to-back launches of its dominant kernel (the Full layer's scan, with
    the arguments, grid and outputs of the step).  fp8: the indexer keys in
    the FP8 form.  Returns a dict."""
    import torch
    from fp4_kv_cache_02_amd import csa2, group

    t_setup = time.perf_counter()
    base = group.build_inputs(w)
    if fp8:
        base = fp8_keys(base)
    reps = [base]
    # extra replicas: every input the step reads (caches, queries, windows)
    # in memory of its own
    for _ in range(max(0, n_replicas - 1)):
        reps.append(replica(base))
    runners = [group.GroupRunner(w, inp) for inp in reps]
    torch.cuda.synchronize()
    t_setup = time.perf_counter() - t_setup

    stream = torch.cuda.current_stream()
    for i in range(warmup):
        runners[i % len(runners)].step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        runners[i % len(runners)].step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps

    key_bytes = 68 if fp8 else 128
    algo, scan_bytes, attn_layers = algorithmic_bytes(w, key_bytes)
    res = {"ms": ms, "value": w.R * attn_layers / (ms * 1e-3), "attn_layers": attn_layers, "algo": algo,
           "replicas": len(runners), "setup_s": t_setup}
    if w.prefill_rows:
        return res              # prefill: the step as a whole is priced against the MFMA peak
    li_full = w.schedule.index("F")
    n_scan = max(10, steps)
    scores = torch.empty((w.R, w.n_max), dtype=torch.float32, device="cuda")
    bmax = torch.empty((w.R, (w.n_max + 7) // 8), dtype=torch.float32, device="cuda")

    def scan(i):
        r = runners[i % len(runners)]
        csa2.csa2_index_score(r.inp.layers[li_full].q_idx, r.kidx, r.inp.seq_len, scores, row_seq=r.inp.row_seq,
                              n_max=w.n_max, block_max=bmax)
    for i in range(3):
        scan(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(n_scan):
        scan(i)
    b.record(stream)
    torch.cuda.synchronize()
    kern_ms = a.elapsed_time(b) / n_scan
    scan_algo = sum(key_bytes * L + 512 for L in w.seq_lens)   # indexer keys + query, per launch
    res.update({"kern_ms": kern_ms, "scan_algo": scan_algo})
    return res


def measure_model(ws, steps, warmup, n_replicas):
    """Times `steps` decode steps of the 38 CSA2 layers: every layer of the
    encoder workload, then every layer of the decoder workload, each over its
    own caches (cycled over replicas like measure())."""
    import torch
    from fp4_kv_cache_02_amd import group

    t_setup = time.perf_counter()
    runners = []            # runners[replica] = [encoder runner, decoder runner]
    bases = [group.build_inputs(w) for w in ws]
    for i in range(max(1, n_replicas)):
        row = []
        for w, base in zip(ws, bases):
            inp = base if i == 0 else replica(base)
            row.append(group.GroupRunner(w, inp))
        runners.append(row)
    torch.cuda.synchronize()
    t_setup = time.perf_counter() - t_setup

    def step(i):
        for r in runners[i % len(runners)]:
            r.step()
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    algo = sum(algorithmic_bytes(w)[0] for w in ws)
    layers = sum(algorithmic_bytes(w)[2] for w in ws)
    rows = ws[0].R
    return {"ms": ms, "value": rows * layers / (ms * 1e-3), "attn_layers": layers, "algo": algo,
            "replicas": len(runners), "setup_s": t_setup}


def decode_summary(w, m):
    """A decode workload's figures for the JSON line: step time, tokens/s/layer,
    algorithmic bytes and their rate against the HBM peak, and the Full
    layer's scan timed on its own."""
    a = m["scan_algo"] / (m["kern_ms"] * 1e-3) / 1e9
    gbps = m["algo"] / (m["ms"] * 1e-3) / 1e9
    return {"workload": w.name, "value": m["value"], "unit": "tokens/s/layer", "ms_per_step": m["ms"],
            "step_algorithmic_bytes": m["algo"], "step_gbps": gbps, "step_frac_of_hbm_peak": gbps / HBM_PEAK_GBPS,
            "scan_avg_launch_ms": m["kern_ms"], "scan_achieved_gbps": a, "scan_frac": a / HBM_PEAK_GBPS,
            "replicas": m["replicas"], "batch": w.B, "context_max": w.n_max, "layers": w.schedule}


def prefill_summary(w, m):
    """A prefill workload's figures: the step's algorithmic flops (indexer
    512 flop per visible (row, entry), counted once for the group; attention
    2 x 2 x 16 x 512 x (512 + 128) flop per row-layer) against the dense bf16
    MFMA peak."""
    visible = sum(w.seq_lens) if w.shared_slots else w.R * w.n_max
    flops = visible * 512 + m["attn_layers"] * w.R * 2 * 2 * 16 * 512 * (512 + 128)
    tflops = flops / (m["ms"] * 1e-3) / 1e12
    return {"workload": w.name, "value": m["value"], "unit": "tokens/s/layer", "ms_per_step": m["ms"],
            "flops_per_step": flops, "achieved_tflops": tflops, "mfma_peak_tflops": MFMA_BF16_PEAK_TFLOPS,
            "mfma_frac": tflops / MFMA_BF16_PEAK_TFLOPS, "rows": w.R, "entries": w.n_max, "layers": w.schedule}


def copy_bandwidth_gbps(nbytes=1 << 30, reps=5):
    """Device-to-device copy of nbytes (read + write = 2 x nbytes moved) timed
    with events on the current stream: the HBM rate a plain streaming kernel
    reaches on this GPU, beside the vendor peak."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(reps):
        b.copy_(a)
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    torch.cuda.empty_cache()
    return 2 * nbytes / (ms * 1e-3) / 1e9


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the multi-GPU design "
                                   "(sequence- or context-parallel) is not built", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    if args.copy_probe:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": 1 << 30, "launches": 3}))
        return

    from fp4_kv_cache_02_amd import synth

    if args.workload == "model38":
        ws = synth.model_step()
        m5 = measure_model(ws, args.steps, args.warmup, args.replicas)
        out = {
            "metric": "CSA2 decode tokens/s/layer over the 38 CSA2 layers of one decode step",
            "value": m5["value"], "unit": "tokens/s/layer", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": m5["ms"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None,
            "dtype": "fp4(e2m1)+e4m3 main KV, bf16 indexer/query/window, f32 accumulate",
            "data": data_desc(ws[1]),
            "config": {"workload": "+".join(w.name for w in ws), "batch": ws[0].B, "layers": m5["attn_layers"],
                       "topk": 512, "window": 128, "replicas": m5["replicas"]},
            "step_algorithmic_bytes": m5["algo"], "step_gbps": m5["algo"] / (m5["ms"] * 1e-3) / 1e9,
            "setup_s": m5["setup_s"],
        }
        print(json.dumps(out), flush=True)
        return

    w = synth.workload(args.workload)
    m = measure(w, args.steps, args.warmup, args.replicas if not w.prefill_rows else 1)
    if w.prefill_rows:
        pf = prefill_summary(w, m)
        roof = {"kernel": "whole prefill group step (MFMA indexer pass, candidate filter, selection, attention)", "bound": "mfma",
                "achieved": pf["achieved_tflops"], "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": pf["mfma_frac"], "traffic": None, "flops_per_step": pf["flops_per_step"]}
    else:
        achieved = m["scan_algo"] / (m["kern_ms"] * 1e-3) / 1e9
        traffic = traffic_from_profiles(os.path.join(ROOT, "fp4_kv_cache_02_amd", "csrc", "index_score.hip"))
        if args.workload != "decode_128k":
            traffic = None          # the committed counter summary covers the 128K decode scan only
        copy_gbps = copy_bandwidth_gbps()
        roof = {"kernel": "index_scan_kernel (Full-layer indexer scan)", "bound": "hbm",
                "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                "algorithmic_bytes_per_launch": m["scan_algo"], "avg_launch_ms": m["kern_ms"],
                "copy_gbps_measured": copy_gbps, "frac_of_copy": achieved / copy_gbps}

    out = {
        "metric": "CSA2 decode tokens/s/layer + % of HBM roofline at 128K and 1M ctx",
        "value": m["value"],
        "unit": "tokens/s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4(e2m1)+e4m3 main KV, bf16 indexer/query/window, f32 accumulate",
        "data": data_desc(w),
        "config": {"workload": w.name, "batch": w.B, "context": w.n_max, "layers": w.schedule,
                   "topk": 512, "window": 128, "replicas": m["replicas"]},
        "step_algorithmic_bytes": m["algo"],
        "step_gbps": m["algo"] / (m["ms"] * 1e-3) / 1e9,
        "step_frac_of_hbm_peak": m["algo"] / (m["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "roofline": roof,
        "setup_s": m["setup_s"],
    }
    default = args.workload == "decode_128k" and not args.no_extras
    if default and not args.no_1m:
        # the metric's second context: the 1M decode group (hierarchical Full
        # layer building 2048 candidate blocks, then Reindex + 3 Reuse)
        w2 = synth.workload("decode_1m")
        out["context_1m"] = decode_summary(w2, measure(w2, args.steps, args.warmup, args.replicas))
    if default and not args.no_others:
        # the other workloads, each timed the same way: one Full layer at 4096
        # positions, the 4096-row prefill chunk (priced against the MFMA
        # peak) and the mixed 20-layer serving batch
        w0 = synth.workload("full_4k")
        out["full_4k"] = decode_summary(w0, measure(w0, args.steps, args.warmup, args.replicas))
        w3 = synth.workload("prefill")
        out["prefill"] = prefill_summary(w3, measure(w3, args.steps, args.warmup, 1))
        w4 = synth.workload("serving")
        out["serving"] = decode_summary(w4, measure(w4, args.steps, args.warmup, args.replicas))
    if default and not args.no_fp8:
        # the same 128K group with the indexer keys in the FP8 form (68 B per
        # position: 64 E4M3 codes and a float32 scale)
        m8 = measure(w, args.steps, args.warmup, args.replicas, fp8=True)
        a8 = m8["scan_algo"] / (m8["kern_ms"] * 1e-3) / 1e9
        out["fp8_indexer_keys"] = {"workload": w.name + "_fp8keys", "value": m8["value"], "unit": "tokens/s/layer",
                                   "ms_per_step": m8["ms"], "scan_avg_launch_ms": m8["kern_ms"],
                                   "scan_algorithmic_bytes_per_launch": m8["scan_algo"],
                                   "scan_achieved_gbps": a8, "scan_frac": a8 / HBM_PEAK_GBPS,
                                   "step_frac_of_hbm_peak": m8["algo"] / (m8["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                                   "replicas": m8["replicas"]}
    if default and not args.no_model:
        # the whole decode step's CSA2 layers: encoder (18, ratio 2) + decoder (20)
        ws = synth.model_step()
        m5 = measure_model(ws, args.steps, args.warmup, args.replicas)
        out["model_38_layers"] = {"workload": "+".join(w.name for w in ws), "layers": m5["attn_layers"],
                                  "value": m5["value"], "unit": "tokens/s/layer", "ms_per_step": m5["ms"],
                                  "step_gbps": m5["algo"] / (m5["ms"] * 1e-3) / 1e9,
                                  "step_frac_of_hbm_peak": m5["algo"] / (m5["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                                  "replicas": m5["replicas"]}
    if not args.no_cpu:
        arrays = _oracle_inputs(w)
        out["cpu_baseline"] = cpu_baseline(w, args.workload, args.cpu_seconds, arrays=arrays)
        # the same oracle over every host core this process may use, one
        # process per core
        n_cores = len(os.sched_getaffinity(0))
        if n_cores > 1:
            out["cpu_baseline_all_cores"] = cpu_baseline(w, args.workload, args.cpu_seconds, procs=n_cores,
                                                         arrays=arrays)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
