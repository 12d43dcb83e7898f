"""Benchmark: MLA speculative-decoding verify attention on one MI355X.

One step = one mla_verify_run call (split partials + merge) over one batch of
synthetic, seeded inputs already resident in HBM.  The timed region replays a
captured HIP graph of 10 back-to-back calls (as inside a captured decode step),
so `value` is the steady-state time per call; single-call graph replays, whose
time includes the launch gap in front of each replay, are reported beside it.
Prints one JSON line.  Default workload: B=1, H=64, 16 draft tokens,
65,536-token context, 2M-slot pool, nsplit=32.

    python bench.py [--steps K] [--warmup W] [--workload ctx64k] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0       # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
METRIC = "µs/call, KV GB/s and MFMA TFLOP/s (% of MI355X roofline) at 64k-ctx verify"


def algorithmic_counts(x):
    """FLOPs (QK + PV over visible pairs) and bytes (each kv row once, slot ids, q, out, lse)."""
    H = x.heads
    pairs = sum(Q * L - Q * (Q - 1) // 2 for L, Q in zip(x.seq_lens.tolist(), x.q_lens.tolist()))
    flops = 2.0 * H * (576 + 512) * pairs
    keys = int(x.seq_lens.sum())
    t_q = int(x.q_lens.sum())
    kv_bytes = keys * 1152
    alg_bytes = kv_bytes + keys * 4 + t_q * H * (1152 + 1024 + 4) + 8 * len(x.seq_lens)
    return flops, kv_bytes, alg_bytes


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per kernel-1 launch from the committed rocprofv3 counter summary, or None.

    The summary (profiles/<kernel>_<workload>_traffic.md) records the sha256 of the kernel
    source it was taken on; once the source differs, the counters no longer describe the kernel
    and None is returned.
    """
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    src = os.path.join(ROOT, "speculative_decode_mla_amd", "csrc", "mla_verify_kernels.hip")
    if not (os.path.exists(path) and os.path.exists(src)):
        return None
    fields = {}
    for line in open(path):
        key, sep, val = line.partition(":")
        if sep and key.strip() in ("kernel_source_sha256", "traffic_bytes_per_launch"):
            fields[key.strip()] = val.strip()
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if fields.get("kernel_source_sha256") != digest or "traffic_bytes_per_launch" not in fields:
        return None
    return int(fields["traffic_bytes_per_launch"])


def cpu_baseline(x, budget_s: float):
    """Time the oracle on the first k draft tokens of request 0 (their exact key ranges); extrapolate."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = cores
    pool = x.sparse_pool()
    L, Q = int(x.seq_lens[0]), int(x.q_lens[0])
    k, elapsed, spent = 0, 0.0, 0.0

    def run(k):
        Lk = L - Q + k
        t0 = time.perf_counter()
        oracle.verify_attention(x.q[:k], pool, x.slot_idx[:Lk], np.array([Lk], np.int32), np.array([k], np.int32),
                                x.scale)
        return time.perf_counter() - t0

    while k < Q and spent < budget_s:
        k = min(Q, max(1, k * 2))
        elapsed = run(k)
        spent += elapsed
    runs = [elapsed]
    if k == Q:  # the whole of request 0 fits the budget: repeat it and take the median
        while spent < budget_s and len(runs) < 50:
            runs.append(run(k))
            spent += runs[-1]
        elapsed = statistics.median(runs)
    total_q = int(x.q_lens.sum())
    # the sample is request 0's first k tokens; scale by visible pairs
    pairs_sample = sum(L - Q + t + 1 for t in range(k))
    pairs_all = sum(Lb * Qb - Qb * (Qb - 1) // 2 for Lb, Qb in zip(x.seq_lens.tolist(), x.q_lens.tolist()))
    us = elapsed * 1e6 * pairs_all / pairs_sample
    return {"value": us, "unit": "us/call", "cores": threads, "kind": "oracle",
            "sample": f"fp64 numpy oracle on draft tokens 0..{k - 1} of request 0 (all {x.heads} heads, "
                      f"their exact visible keys), median {elapsed * 1e3:.1f} ms of {len(runs)} runs ({spent:.1f} s in all), "
                      f"scaled by visible (row, key) pairs to the whole call ({total_q} tokens); "
                      f"{cores} host cores visible"}


def _graph_us(torch, fn, reps=10, rounds=20):
    """Median time per call of `fn`, from `rounds` replays of a graph of `reps` back-to-back calls."""
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        fn()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(rounds)]
    for a, b in ev:
        a.record(stream)
        g.replay()
        b.record(stream)
    torch.cuda.synchronize()
    return statistics.median(a.elapsed_time(b) * 1e3 / reps for a, b in ev)


def kernel1_name(w, x, nsplit, form, cus):
    """The kernel-1 form a call takes (include/mla_verify.h, MLA_VERIFY_FORM_*): a fixed `form`, or
    the library's choice for FORM_AUTO (0)."""
    names = {1: "mla_verify_partial", 2: "mla_verify_partial_2s", 3: "mla_verify_partial_4s"}
    if form:
        return names[form]
    req_rows = x.heads * int(x.q_lens.max())
    range_plan = req_rows > 64 and 2 <= w.batch <= 64
    two_stream = req_rows <= 64 or (not range_plan and 2 * w.batch * nsplit * -(-req_rows // 128) <= cus)
    if two_stream and 2 * w.batch * nsplit * -(-req_rows // 64) <= cus:
        return names[3]
    return names[2] if two_stream else names[1]


def bench_compact(args, w, x, h, q, pool, slot_idx, seq_lens, q_lens, out, lse, nsplit):
    """KV compaction of every row the workload references into a fresh contiguous buffer (one
    launch, HBM-bound: each 1152-B row read once and written once), then kernel 1 and the whole
    call over the compacted rows against the scattered ones.  Prints one JSON line."""
    import torch

    from speculative_decode_mla_amd import api
    from speculative_decode_mla_amd import inputs as I

    n = len(x.slot_idx)
    dst = torch.empty((n, I.D_QK), dtype=torch.bfloat16, device="cuda")
    new = torch.empty((n,), dtype=torch.int32, device="cuda")
    api.compact(pool, slot_idx, dst, 0, new)
    torch.cuda.synchronize()
    # parity: the compacted rows are the generator's kv_rows bit for bit (closed form), and the
    # verify call over them equals the scattered call bit for bit
    exact = bool(np.array_equal(dst.view(torch.int16).cpu().numpy().view(np.uint16), x.kv_rows)
                 and np.array_equal(new.cpu().numpy(), np.arange(n, dtype=np.int32)))
    h.run(q, pool, slot_idx, seq_lens, q_lens, out, lse, nsplit)
    o1, l1 = out.clone(), lse.clone()
    h.run(q, dst, new, seq_lens, q_lens, out, lse, nsplit)
    torch.cuda.synchronize()
    same = bool(torch.equal(o1.view(torch.int16), out.view(torch.int16)) and torch.equal(l1, lse))
    print(f"# compaction of {n} rows: bit-exact {exact}; verify over compacted rows bitwise equal {same}",
          file=sys.stderr, flush=True)
    t_c = _graph_us(torch, lambda: api.compact(pool, slot_idx, dst, 0, new))
    moved = 2 * n * I.D_QK * 2 + 2 * n * 4  # rows read and written, slot ids read and written
    k1_s = _graph_us(torch, lambda: h.partials(q, pool, slot_idx, seq_lens, q_lens, nsplit))
    k1_c = _graph_us(torch, lambda: h.partials(q, dst, new, seq_lens, q_lens, nsplit))
    run_s = _graph_us(torch, lambda: h.run(q, pool, slot_idx, seq_lens, q_lens, out, lse, nsplit))
    run_c = _graph_us(torch, lambda: h.run(q, dst, new, seq_lens, q_lens, out, lse, nsplit))
    gbps = moved / (t_c * 1e-6) / 1e9
    res = {
        "metric": "KV compaction GB/s (rows moved per launch) and kernel-1 time over compacted vs scattered rows",
        "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "higher_is_better": True,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "rows": n, "row_bytes": I.D_QK * 2, "pool_slots": w.num_slots,
                   "replay": "hipGraph, 10 launches per graph"},
        "compact_us": round(t_c, 3),
        "parity": {"rows_bit_exact": exact, "verify_bitwise_equal": same},
        "partial_kernel_us": {"scattered": round(k1_s, 3), "compacted": round(k1_c, 3)},
        "call_us": {"scattered": round(run_s, 3), "compacted": round(run_c, 3)},
        "roofline": {"bound": "hbm", "kernel": "mla_kv_compact_kernel", "achieved": round(gbps, 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4),
                     "traffic": None, "bytes_per_launch": moved},
    }
    print(json.dumps(res), flush=True)


def bench_metadata(args, w, x, h, q, pool, slot_idx, seq_lens, q_lens, out, lse, nsplit):
    """Device-side step metadata for the workload's requests, from a request-to-token table
    (request b in table row 2b+1, rows as wide as the longest request): one launch against the
    host path it replaces (numpy gather of the table rows + copy to the device), and inside a
    captured step together with the verify call.  Prints one JSON line."""
    import torch

    import oracle
    from speculative_decode_mla_amd import api

    B = len(x.seq_lens)
    width = int(x.seq_lens.max())
    table = np.zeros((2 * B + 1, width), dtype=np.int32)
    ids = np.array([2 * b + 1 for b in range(B)], dtype=np.int32)
    ko = np.concatenate([[0], np.cumsum(x.seq_lens)])
    for b in range(B):
        table[ids[b], :x.seq_lens[b]] = x.slot_idx[ko[b]:ko[b + 1]]
    pre = (x.seq_lens - x.q_lens).astype(np.int32)
    dr = x.q_lens.astype(np.int32)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    t_table, t_ids, t_pre, t_dr = d(table), d(ids), d(pre), d(dr)
    cap = int(w.num_slots)
    m_slots = torch.zeros((cap,), dtype=torch.int32, device="cuda")
    m_seq = torch.zeros((B,), dtype=torch.int32, device="cuda")
    m_q = torch.zeros((B,), dtype=torch.int32, device="cuda")
    m_st = torch.zeros((1,), dtype=torch.int32, device="cuda")
    build = lambda: api.build_metadata(t_table, t_ids, t_pre, t_dr, m_slots, m_seq, m_q, m_st)  # noqa: E731
    build()
    torch.cuda.synchronize()
    hs, hseq, hql, hst = oracle.build_step_metadata(table, ids, pre, dr, cap)
    total = len(hs)
    exact = bool(int(m_st.item()) == hst == 0 and np.array_equal(m_slots[:total].cpu().numpy(), hs)
                 and np.array_equal(m_seq.cpu().numpy(), hseq) and np.array_equal(m_q.cpu().numpy(), hql))
    h.run(q, pool, slot_idx, seq_lens, q_lens, out, lse, nsplit)
    o1 = out.clone()
    h.run(q, pool, m_slots, m_seq, m_q, out, lse, nsplit)
    torch.cuda.synchronize()
    same = bool(torch.equal(o1.view(torch.int16), out.view(torch.int16)))
    print(f"# metadata for {B} requests, {total} slots: bit-exact {exact}; verify on it bitwise equal {same}",
          file=sys.stderr, flush=True)
    t_dev = _graph_us(torch, build)
    t_step = _graph_us(torch, lambda: (build(), h.run(q, pool, m_slots, m_seq, m_q, out, lse, nsplit)))
    t_run = _graph_us(torch, lambda: h.run(q, pool, slot_idx, seq_lens, q_lens, out, lse, nsplit))
    # the host path it replaces: gather the rows on the host, copy the three arrays to the device
    host_slots = torch.empty((cap,), dtype=torch.int32, device="cuda")
    ht = []
    for _ in range(20):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        flat = np.concatenate([table[ids[b], :pre[b] + dr[b]] for b in range(B)])
        host_slots[:len(flat)].copy_(torch.from_numpy(flat))
        seq_lens.copy_(torch.from_numpy(pre + dr))
        q_lens.copy_(torch.from_numpy(dr))
        torch.cuda.synchronize()
        ht.append((time.perf_counter() - t0) * 1e6)
    moved = 2 * total * 4 + 4 * B * 4 + 4
    gbps = moved / (t_dev * 1e-6) / 1e9
    res = {
        "metric": "device-side step metadata: us per build, beside the host gather + copy it replaces",
        "value": round(t_dev, 3), "unit": "us/build", "n_gpus": 1, "higher_is_better": False,
        "dtype": "int32", "data": "synthetic",
        "config": {"workload": w.name, "requests": B, "slots": total, "table": list(table.shape),
                   "replay": "hipGraph, 10 launches per graph"},
        "parity": {"bit_exact": exact, "verify_bitwise_equal": same},
        "host_gather_and_copy_us_p50": round(statistics.median(ht), 1),
        "captured_step_us": {"metadata_and_verify": round(t_step, 3), "verify_only": round(t_run, 3)},
        "roofline": {"bound": "hbm", "kernel": "mla_step_metadata_kernel", "achieved": round(gbps, 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 5),
                     "traffic": None, "bytes_per_launch": moved},
    }
    print(json.dumps(res), flush=True)


def _smi_sample(delay_s: float):
    """Start a read-only `amd-smi metric` sample of socket power and the XCD clocks, taken delay_s
    from now; returns a function that collects it ({} when the tool is absent or fails)."""
    import subprocess
    try:
        proc = subprocess.Popen(["bash", "-c", f"sleep {delay_s}; timeout -k 5 20 amd-smi metric -g 0 -p -c"],
                                stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)
    except OSError:
        return lambda: {}

    def collect():
        text = proc.communicate()[0]
        power = [l.split(":", 1)[1].strip() for l in text.splitlines() if "SOCKET_POWER" in l]
        clk, in_gfx = [], False  # the CLK line of each GFX_<n> block (one per XCD), not the other clocks
        for l in text.splitlines():
            t = l.strip()
            if t.startswith("GFX_") and t.endswith(":"):
                in_gfx = True
            elif in_gfx and t.startswith("CLK:"):
                clk.append(t.split()[1])
                in_gfx = False
        out = {}
        if power and power[0].endswith("W") and power[0][:-1].strip().isdigit():
            out["socket_power_w"] = int(power[0][:-1])
        clk = [int(c) for c in clk if c.isdigit()]
        if clk:
            out["xcd_clock_mhz"] = clk
        return out
    return collect


def bench_mfma_ceiling(torch):
    """What dense bf16 MFMA work sustains on this GPU with random data: the vendor GEMM
    (torch.matmul, i.e. hipBLASLt) on N(0,1) operands for a few large shapes, each after 1 s of
    untimed GEMMs and timed over 2.5 s, with one power and clock sample in the middle.  MFMA power
    depends on the operand bits, so with random data the chip runs at its power limit below its
    top clock; this is the practical ceiling against which kernel 1's fraction of the published
    2.5 PFLOP/s can be read."""
    gen = torch.Generator(device="cuda").manual_seed(0)
    rows = []
    for m, n, k in [(8192, 8192, 8192), (16384, 16384, 8192), (4096, 4096, 16384)]:
        a = torch.randn(m, k, device="cuda", dtype=torch.bfloat16, generator=gen)
        b = torch.randn(k, n, device="cuda", dtype=torch.bfloat16, generator=gen)
        c = torch.empty(m, n, device="cuda", dtype=torch.bfloat16)
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 1.0:
            for _ in range(10):
                torch.matmul(a, b, out=c)
            torch.cuda.synchronize()
        sample = _smi_sample(1.0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 0
        e0.record()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 2.5:
            for _ in range(20):
                torch.matmul(a, b, out=c)
            reps += 20
            torch.cuda.synchronize()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        tflops = 2.0 * m * n * k / us / 1e6
        rows.append({"shape_mnk": [m, n, k], "us": round(us, 1), "tflops": round(tflops, 1),
                     "frac_of_2500": round(tflops / 2500.0, 4), **sample()})
        print(f"# {m}x{n}x{k}: {us:.1f} us, {tflops:.0f} TFLOP/s", file=sys.stderr, flush=True)
        del a, b, c
    print(json.dumps({"mfma_ceiling": rows, "what": "torch.matmul bf16 (hipBLASLt), N(0,1) operands",
                      "peak_tflops": 2500.0}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # The GPU takes about 0.1 s of sustained work to settle: at ctx64k the first timed graphs of a
    # fresh process ran ~5 % slower than the same graphs 0.1 s later.  1,000 untimed calls (0.13 s at
    # ctx64k) cover that.
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--settle", type=float, default=0.5,
                    help="seconds of untimed back-to-back calls before the timed region (besides --warmup)")
    ap.add_argument("--workload", default="ctx64k")
    ap.add_argument("--nsplit", type=int, default=None)
    ap.add_argument("--form", type=int, default=0, choices=[0, 1, 2, 3],
                    help="kernel-1 layout: 0 the library's choice, 1 128-row, 2 two-stream, 3 four-stream")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold", type=int, default=50, help="single-call replays, each after reading 1 GiB to flush the caches")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time for the CPU baseline")
    ap.add_argument("--eager", action="store_true", help="plain launches, no graph (for profilers)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a plain 256 MiB device copy (reference size for HBM traffic counters)")
    ap.add_argument("--power-window", type=float, default=2.0,
                    help="seconds of back-to-back calls after the timed region with one amd-smi power and clock "
                         "sample in the middle (0: none)")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only time the vendor bf16 GEMM on random data (the MFMA rate this GPU sustains)")
    ap.add_argument("--metadata", action="store_true",
                    help="measure the device-side step-metadata build for the workload instead")
    ap.add_argument("--compact", action="store_true",
                    help="measure KV compaction of the workload's rows instead (and kernel 1 over the compacted rows)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU sharding is described, not built", file=sys.stderr)
        sys.exit(2)

    import torch

    import oracle
    from speculative_decode_mla_amd import api
    from speculative_decode_mla_amd import inputs as I

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calib:
        n = 256 << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 3}))
        return
    if args.mfma_ceiling:
        bench_mfma_ceiling(torch)
        return
    w = I.WORKLOADS[args.workload]
    nsplit = args.nsplit or w.nsplit
    print(f"# workload {w.name}: B={w.batch} H={w.heads} Q={w.q_len} L={w.ctx or 'log-uniform'} "
          f"pool={w.num_slots} nsplit={nsplit}", file=sys.stderr, flush=True)
    x = I.make_inputs(w)
    dev = torch.device("cuda:0")
    q = torch.from_numpy(x.q.view(np.int16)).to(dev).view(torch.bfloat16)
    pool = torch.full((x.num_slots, I.D_QK), I.BF16_QNAN, dtype=torch.int16, device=dev)
    pool[torch.from_numpy(x.slot_idx.astype(np.int64)).to(dev)] = torch.from_numpy(x.kv_rows.view(np.int16)).to(dev)
    pool = pool.view(torch.bfloat16)
    slot_idx = torch.from_numpy(x.slot_idx).to(dev)
    seq_lens = torch.from_numpy(x.seq_lens).to(dev)
    q_lens = torch.from_numpy(x.q_lens).to(dev)
    t_q = x.q.shape[0]
    out = torch.empty((t_q, x.heads, I.D_V), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((t_q, x.heads), dtype=torch.float32, device=dev)
    h = api.MlaVerify(x.heads, w.batch, int(x.q_lens.max()), nsplit, x.num_slots, x.scale, form=args.form)
    step = lambda: h.run(q, pool, slot_idx, seq_lens, q_lens, out, lse, nsplit)  # noqa: E731
    part = lambda: h.partials(q, pool, slot_idx, seq_lens, q_lens, nsplit)  # noqa: E731
    if args.compact:
        bench_compact(args, w, x, h, q, pool, slot_idx, seq_lens, q_lens, out, lse, nsplit)
        h.close()
        return
    if args.metadata:
        bench_metadata(args, w, x, h, q, pool, slot_idx, seq_lens, q_lens, out, lse, nsplit)
        h.close()
        return

    # parity on sampled rows (the oracle evaluates them one by one)
    step()
    torch.cuda.synchronize()
    rng = np.random.default_rng(123)
    rows = [(int(t), int(hh)) for t, hh in zip(rng.integers(0, t_q, 12), rng.integers(0, x.heads, 12))]
    rows += [(t_q - 1, 0), (0, x.heads - 1)]
    ro, rl = oracle.verify_attention_rows(x.q, x.sparse_pool(), x.slot_idx, x.seq_lens, x.q_lens, x.scale, rows)
    o_np = out.float().cpu().numpy()
    l_np = lse.cpu().numpy()
    err_o = max(float(np.max(np.abs(o_np[t, hh] - ro[i]))) for i, (t, hh) in enumerate(rows))
    err_l = max(abs(float(l_np[t, hh]) - rl[i]) for i, (t, hh) in enumerate(rows))
    print(f"# parity on {len(rows)} sampled rows: max|out err| {err_o:.3e}, max|lse err| {err_l:.3e}",
          file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    settle_s, settle_calls = 0.0, 0
    power = {}
    if args.eager:
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        us = wall / args.steps * 1e6
        times_us = [us]
        steady_us = [us]
        cold_us = []
        k1_us = float("nan")
    else:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
            part()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        # steady state: `reps` calls back to back inside one graph, as in a captured decode step
        reps = 10 if args.steps % 10 == 0 else 1
        gs = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gs):
            for _ in range(reps):
                step()
        gk = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gk):
            for _ in range(10):
                part()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        # Untimed settle, whatever --warmup is: the GPU needs about 0.1 s of sustained work before
        # its clocks (and so the timings) are steady, and a handful of warm-up calls is far less.
        # Replays of the 10-call graph until args.settle seconds have passed.
        t_settle = time.perf_counter()
        settle_calls = 0
        while time.perf_counter() - t_settle < args.settle:
            for _ in range(10):
                gs.replay()
            settle_calls += 10 * reps
            torch.cuda.synchronize()
        settle_s = time.perf_counter() - t_settle
        # the timed region: exactly `steps` calls
        n_rep = args.steps // reps
        sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_rep)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for a, b in sev:
            a.record(stream)
            gs.replay()
            b.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        steady_us = sorted(a.elapsed_time(b) * 1e3 / reps for a, b in sev)
        # single calls, one graph replay each (includes the launch gap before each replay)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for a, b in ev:
            a.record(stream)
            g.replay()
            b.record(stream)
        torch.cuda.synchronize()
        times_us = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
        # kernel 1 alone: `reps` back-to-back launches per replay, timed with events on the same stream
        # (interleaved with replays of the call graph, so that the GPU stays as busy as in the timed
        # region); then the merge's share of a call as the difference
        gk.replay()
        torch.cuda.synchronize()
        kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(40)]
        for a, b in kev:
            gs.replay()
            a.record(stream)
            gk.replay()
            b.record(stream)
        torch.cuda.synchronize()
        k1_us = statistics.median(a.elapsed_time(b) * 1e3 / 10 for a, b in kev)
        # Socket power and XCD clocks while the call runs back to back (read-only amd-smi query, after
        # the timed region so that it cannot disturb it): MFMA power grows with the operand bits, and
        # with random data the GPU reaches its power limit below its top clock.
        if args.power_window > 0:
            sample = _smi_sample(args.power_window / 2)
            t_pw = time.perf_counter()
            while time.perf_counter() - t_pw < args.power_window:
                for _ in range(10):
                    gs.replay()
                torch.cuda.synchronize()
            power = sample()
            if power:
                power["during"] = f"{args.power_window:g} s of back-to-back calls after the timed region"
        # (last: the flushes disturb the timings that follow them)
        # cold single calls: 1 GiB read before each replay (outside the events) evicts the KV rows from
        # the L2s and the 256 MB MALL, so the call reads them from HBM.  A read, not a write: written
        # lines would still be dirty in the caches and their write-back would land inside the call.
        flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        flush.sum()
        torch.cuda.synchronize()
        cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.cold)]
        for a, b in cev:
            flush.sum()
            a.record(stream)
            g.replay()
            b.record(stream)
        torch.cuda.synchronize()
        cold_us = sorted(a.elapsed_time(b) * 1e3 for a, b in cev)
        del flush
        us = sum(steady_us) / len(steady_us)

    flops, kv_bytes, alg_bytes = algorithmic_counts(x)
    p95 = times_us[min(len(times_us) - 1, int(0.95 * len(times_us)))]
    k1_tflops = flops / (k1_us * 1e-6) / 1e12 if k1_us == k1_us else None
    # kernel 1's roof: bf16 MFMA above the ridge (flop per byte of the call's algorithmic bytes),
    # HBM below it (q_len = 1 decode: H flop/B ~ 121 against a ridge of 312)
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9)
    k1_kernel = kernel1_name(w, x, nsplit, args.form, torch.cuda.get_device_properties(0).multi_processor_count)
    # `achieved`/`frac` are the dominant kernel's (kernel 1: all of the call's FLOPs, and its KV
    # stream); `call_achieved`/`call_frac` hold the whole captured call (kernel 1, the merge and the
    # gap between them) against the same roof.
    if flops / alg_bytes >= ridge:
        call_tflops = flops / (us * 1e-6) / 1e12
        roofline = {"bound": "mfma", "kernel": k1_kernel,
                    "achieved": round(k1_tflops, 1) if k1_tflops else None, "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(k1_tflops / PEAK_BF16_TFLOPS, 4) if k1_tflops else None,
                    "traffic": measured_traffic(k1_kernel, w.name), "traffic_unit": "bytes/launch",
                    "flops_per_launch": flops,
                    "call_achieved": round(call_tflops, 1), "call_frac": round(call_tflops / PEAK_BF16_TFLOPS, 4)}
    else:
        k1_gbps = alg_bytes / (k1_us * 1e-6) / 1e9 if k1_us == k1_us else None
        call_gbps = alg_bytes / (us * 1e-6) / 1e9
        roofline = {"bound": "hbm", "kernel": k1_kernel,
                    "achieved": round(k1_gbps, 1) if k1_gbps else None, "peak": PEAK_HBM_GBPS,
                    "unit": "GB/s", "frac": round(k1_gbps / PEAK_HBM_GBPS, 4) if k1_gbps else None,
                    "traffic": measured_traffic(k1_kernel, w.name), "traffic_unit": "bytes/launch",
                    "bytes_per_launch": alg_bytes,
                    "call_achieved": round(call_gbps, 1), "call_frac": round(call_gbps / PEAK_HBM_GBPS, 4)}
    res = {
        "metric": METRIC,
        "value": round(us, 3),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "draft_tokens": w.q_len,
                   "context": w.ctx if w.ctx else "log-uniform[1024,65536] (seed 5)",
                   "pool_slots": w.num_slots, "nsplit": nsplit, "replay": "eager" if args.eager else "hipGraph, 10 calls per graph",
                   "seed": w.seed},
        "settle_s": round(settle_s, 3),
        "settle_calls": settle_calls,
        "steady_p50_us": round(statistics.median(steady_us), 3),
        "single_call_p50_us": round(statistics.median(times_us), 3),
        "single_call_p95_us": round(p95, 3),
        "cold_single_call_p50_us": round(statistics.median(cold_us), 3) if cold_us else None,
        "cold_kv_gbps": round(kv_bytes / (statistics.median(cold_us) * 1e-6) / 1e9, 1) if cold_us else None,
        "wall_us_per_step": round(wall / args.steps * 1e6, 3),
        "kv_gbps": round(kv_bytes / (us * 1e-6) / 1e9, 1),
        "kv_frac_of_hbm": round(kv_bytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
        "tflops": round(flops / (us * 1e-6) / 1e12, 1),
        "tflops_frac_of_mfma": round(flops / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "partial_kernel_us": round(k1_us, 3) if k1_us == k1_us else None,
        "parity_sampled": {"rows": len(rows), "max_abs_err_out": err_o, "max_abs_err_lse": err_l},
        "roofline": roofline,
        "power_sample": power,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(x, args.cpu_budget)
    h.close()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
