"""Benchmark of the MTP draft sweep on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config large]

A step is one whole draft sweep (gather, both norms, concat, eh_proj, head norm,
lm_head over the full vocabulary, argmax) for one batch of synthetic input
already resident in HBM.  The default workload is the Large draft sweep
(H = 6144, vocab = 154880, B = 1); `value` is BF16-head draft sweeps per second,
and the FP8-head sweep is timed the same way and reported beside it.

The roofline object covers the dominant kernel, the lm_head sweep: algorithmic
bytes per launch (the weight matrix once, plus the per-row scales for FP8, the
normed activation and the logits written) divided by the head call's average
duration, timed with HIP events on the stream the kernels run on.  The
cpu_baseline object times the FP64 oracle on a bounded sample of the same
workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "draft sweeps/sec and lm_head achieved HBM GB/s (% of peak), BF16 vs FP8"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense BF16 matrix-core peak (no sparsity)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", default="large", choices=["tiny", "mid", "large", "batched", "neartie"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="approximate budget for the oracle baseline sample")
    p.add_argument("--no-batched", action="store_true",
                   help="skip the batched (B = 16 FP8, B = 8) timings")
    p.add_argument("--no-chain", action="store_true",
                   help="skip the chained-draft (K = 4 drafts per call) timings")
    p.add_argument("--no-context", action="store_true",
                   help="skip the context-row (prompt / catch-up rows) timings")
    p.add_argument("--no-shards", action="store_true",
                   help="skip the head timings at vocabulary-shard shapes (V/2, V/4, V/8 rows)")
    p.add_argument("--no-ceiling", action="store_true",
                   help="skip the plain streaming-read probe (the practical HBM ceiling)")
    p.add_argument("--no-agreement", action="store_true",
                   help="skip the BF16-vs-FP8 draft agreement study")
    p.add_argument("--calib-copy", action="store_true",
                   help="also run a plain 1 GiB device-to-device copy three times "
                        "(the known-size kernel that HBM counters are scaled by)")
    return p.parse_args()


def kernel_source_hash() -> str:
    """SHA-256 of the sources of the single-sequence head kernel."""
    import hashlib
    h = hashlib.sha256()
    for f in ("row_gemv.hip", "common.hpp", "kernels.hpp"):
        with open(os.path.join(ROOT, "mtp_draft_head_embed_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def committed_traffic(name: str):
    """HBM bytes per launch of the BF16 head kernel from the committed counter
    summary, or None when the summary is missing or the kernel changed since."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and line.strip().startswith("- "):
            k, v = line.strip()[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return int(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def head_bytes(H: int, V: int, B: int, fp8: bool) -> int:
    """Algorithmic bytes of one lm_head launch: every weight byte once (plus
    one f32 scale per row for FP8), the x vectors and head-norm weight read,
    and BF16 logits written."""
    w = V * H * (1 if fp8 else 2) + (V * 4 if fp8 else 0)
    return w + B * H * 2 + H * 2 + B * V * 2


def sweep_bytes(H: int, V: int, B: int, fp8: bool) -> int:
    """Algorithmic bytes of one whole sweep: eh_proj [H][2H] BF16, the head,
    and per sequence the embedding row, the hidden row and the two norm weights."""
    return 2 * H * H * 2 + head_bytes(H, V, B, fp8) + B * 2 * H * 2 + 2 * H * 2


def cpu_info() -> dict:
    """The host CPU as /proc/cpuinfo names it, and how many processors it lists."""
    info = {"model_name": "unknown", "vendor_id": None, "cpu_family": None, "model": None,
            "processors_listed": 0}
    keys = {"model name": "model_name", "vendor_id": "vendor_id", "cpu family": "cpu_family",
            "model": "model"}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" not in line:
                continue
            k, v = (t.strip() for t in line.split(":", 1))
            if k == "processor":
                info["processors_listed"] += 1
            elif k in keys and info["processors_listed"] <= 1:
                info[keys[k]] = v
    except OSError:
        pass
    return info


def _time_calls(fn, seconds: float):
    """Run fn until `seconds` have passed (at least once): (calls, elapsed s)."""
    n, t0 = 0, time.perf_counter()
    while True:
        fn()
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            return n, el


def cpu_baseline_leg(args, cfg, wts, tokens, hidden) -> dict:
    """The FP64 oracle timed on the host: the bench configuration's BF16 sweep
    (the reported value), then every configuration and head path for a bounded
    time each, the quantiser, and one-thread figures from row samples."""
    import numpy as np

    import oracle
    import synth

    nthreads = oracle.default_threads()
    H, V, B = cfg.hidden, cfg.vocab, cfg.batch

    def sweeps(w, tk, hd, fp8=None, nt=nthreads):
        for b in range(tk.size):
            oracle.draft(w, int(tk[b]), hd[b], fp8=fp8, nthreads=nt)

    n, el = _time_calls(lambda: sweeps(wts, tokens, hidden), args.cpu_seconds * 0.5)
    cpu = {"value": round(n / el, 4), "unit": "draft sweeps/s" if B == 1 else "calls/s",
           "cores": nthreads, "kind": "oracle",
           "sample": f"{n} full {cfg.name} BF16 draft sweep call(s) (B={B}) through the FP64 "
                     f"oracle in {el:.1f}s on {nthreads} threads splitting vocab rows"}
    hc = oracle.host_cores()
    detail = {"cpu": cpu_info(), "host_cores": hc, "threads": nthreads,
              "thread_rule": f"min(os.cpu_count(), affinity, cgroup quota, {oracle.THREAD_CAP}): "
                             f"a one-GPU host grants a process about {oracle.THREAD_CAP} host cores"}
    # the FP8 copy of the bench weights (timed: the quantiser on the host)
    tq = time.perf_counter()
    ref8 = oracle.quantize_fp8(wts["lm_head"], nthreads=nthreads)
    detail["quantiser_s"] = round(time.perf_counter() - tq, 3)

    # every configuration and path, each for about a second (one call at least);
    # batched and near-tie share the large shape, so they run on the bench's
    # weights with their own tokens and hidden rows (values do not change the
    # oracle's cost)
    per_s = max(0.5, args.cpu_seconds / 12)
    per = {}
    own = {(H, V): (wts, ref8)}
    for name, paths in (("tiny", ("bf16", "fp8")), ("mid", ("bf16",)),
                        ("large", ("bf16", "fp8")), ("batched", ("fp8",)),
                        ("neartie", ("bf16", "fp8"))):
        c = synth.CONFIGS[name]
        if (c.hidden, c.vocab) not in own:
            w2 = synth.make_weights(c)
            own[(c.hidden, c.vocab)] = (w2, oracle.quantize_fp8(w2["lm_head"], nthreads=nthreads)
                                        if "fp8" in paths else None)
        w2, r8 = own[(c.hidden, c.vocab)]
        tk, hd = synth.make_inputs(c)
        ent = {"hidden": c.hidden, "vocab": c.vocab, "batch": c.batch}
        for path in paths:
            n2, el2 = _time_calls(lambda: sweeps(w2, tk, hd, r8 if path == "fp8" else None), per_s)
            ent[path] = {"calls_per_s": round(n2 / el2, 4),
                         "sequences_per_s": round(n2 * c.batch / el2, 4),
                         "ms_per_call": round(el2 / n2 * 1e3, 2), "calls": n2}
        per[name] = ent
        if name == "mid":
            del own[(c.hidden, c.vocab)]  # 2.5 GB of weights no longer needed
    detail["per_config"] = per

    # one thread: eh_proj whole, row samples of lm_head and of the quantiser,
    # scaled to the whole matrix (every row costs the same)
    rows = min(V, 16384)
    xs = synth.to_bf16(np.ones(H, np.float32))
    cs = synth.to_bf16(np.ones(2 * H, np.float32))
    t1 = time.perf_counter()
    oracle.gemv_bf16(wts["eh_proj"], cs, nthreads=1)
    t_front = time.perf_counter() - t1
    t1 = time.perf_counter()
    oracle.gemv_bf16(wts["lm_head"][:rows], xs, nthreads=1)
    t_head = (time.perf_counter() - t1) * V / rows
    detail["bf16_sweeps_per_s_1thread"] = round(1.0 / (t_front + t_head), 4)
    t1 = time.perf_counter()
    oracle.quantize_fp8(wts["lm_head"][:rows // 4], nthreads=1)
    detail["quantiser_s_1thread"] = round((time.perf_counter() - t1) * V / (rows // 4), 3)
    detail["one_thread_sample"] = (f"eh_proj GEMV whole, lm_head GEMV over {rows} rows and "
                                   f"the quantiser over {rows // 4} rows, scaled to {V} rows")
    cpu["detail"] = detail
    print(f"[bench] cpu baseline: {cpu}", file=sys.stderr, flush=True)
    return cpu


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the sweep has no "
              "multi-GPU path (it runs the whole vocabulary on one GPU).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mtp_draft_head_embed_amd as mtp
    import synth
    from tests import harness

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = synth.CONFIGS[args.config]
    H, V, B = cfg.hidden, cfg.vocab, cfg.batch
    t0 = time.time()
    wts = synth.make_weights(cfg)
    tokens, hidden = synth.make_inputs(cfg)
    print(f"[bench] {cfg.name}: weights generated in {time.time() - t0:.1f}s", file=sys.stderr,
          flush=True)
    dw = harness.upload(wts)
    q, s = harness.quantize_dev(dw)
    torch.cuda.synchronize()

    # the load-time FP8 copy of lm_head (timed apart from the sweep): reads the
    # BF16 matrix, writes the codes and the per-row scales
    qws = torch.empty(256, dtype=torch.uint8, device=dev)
    qt = []
    for _ in range(6):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(torch.cuda.current_stream())
        mtp.mtp_quantize_head_fp8(dw.tensors["lm_head"], V, H, q, s, qws)
        e1.record(torch.cuda.current_stream())
        torch.cuda.synchronize()
        qt.append(e0.elapsed_time(e1) * 1e3)
    q_us = float(np.median(qt[1:]))
    q_bytes = V * H * 3 + 4 * V
    quant = {"call_us": round(q_us, 1), "call_GBps": round(q_bytes / q_us / 1e3, 1),
             "call_frac_of_peak": round(q_bytes / q_us / 1e3 / HBM_PEAK_GBPS, 4),
             "bytes": q_bytes, "note": "median of 5 calls after one warm-up, HIP events around "
             "the whole call: the flag clear, the quantise kernel, and the synchronising read "
             "of the non-finite flag (the kernel alone is in the rocprofv3 trace)"}
    print(f"[bench] quantiser: {quant}", file=sys.stderr, flush=True)

    tk = torch.from_numpy(tokens.astype(np.uint32).view(np.int32)).to(dev)
    hd = harness.to_dev_bf16(hidden)
    draft = torch.empty(B, dtype=torch.int32, device=dev)
    logits = torch.empty((B, V), dtype=torch.bfloat16, device=dev)
    ws = mtp.new_workspace(H, V, B)
    x = torch.empty((B, H), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    def sweep(fp8):
        if fp8:
            mtp.mtp_draft_fp8w(dw.w, q, s, B, tk, hd, draft, logits, ws, stream)
        else:
            mtp.mtp_draft_bf16(dw.w, B, tk, hd, draft, logits, ws, stream)

    def head(fp8):
        if fp8:
            mtp.mtp_head_fp8w(dw.w, q, s, B, x, draft, logits, ws, stream)
        else:
            mtp.mtp_head_bf16(dw.w, B, x, draft, logits, ws, stream)

    def timed(fn, steps, warmup):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t_wall = time.perf_counter()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_wall
        return e0.elapsed_time(e1) / 1e3, wall

    mtp.mtp_front(dw.w, B, tk, hd, x, ws, stream)
    torch.cuda.synchronize()

    # three copies of eh_proj (3 x 151 MB at the Large shape, more than the
    # 256 MB last-level cache), used in turn by the cold-front sweeps and the
    # context rows, so those calls stream eh_proj from HBM
    t = dw.tensors
    ehc = [t["eh_proj"]] + [t["eh_proj"].clone() for _ in range(2)]
    cw = [dw.w] + [mtp.mtp_weights(t["embed"], t["enorm_w"], t["hnorm_w"], t["head_norm_w"],
                                   e, t["lm_head"], float(wts["rms_eps"])) for e in ehc[1:]]

    def spread(fn, blocks=20, per=10):
        """Per-call µs from HIP events around blocks of back-to-back calls:
        p10, median, p90 over the blocks."""
        for _ in range(per):
            fn()
        vals = []
        for _ in range(blocks):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(per):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            vals.append(e0.elapsed_time(e1) * 1e3 / per)
        p10, med, p90 = np.percentile(vals, [10, 50, 90])
        return {"p10_us": round(float(p10), 2), "median_us": round(float(med), 2),
                "p90_us": round(float(p90), 2), "blocks": blocks, "calls_per_block": per}

    def synced(fn, n=100):
        """Host latency of one call that is waited for and whose draft is read
        back (4 bytes), as a caller that needs the token at once sees it."""
        for _ in range(5):
            fn()
            draft.cpu()
        vals = []
        for _ in range(n):
            t1 = time.perf_counter()
            fn()
            draft.cpu()
            vals.append((time.perf_counter() - t1) * 1e6)
        return round(float(np.median(vals)), 2)

    res = {}
    for name, fp8 in (("bf16", False), ("fp8", True)):
        gpu_s, wall_s = timed(lambda: sweep(fp8), args.steps, args.warmup)
        head_s, _ = timed(lambda: head(fp8), args.steps, args.warmup)
        hb = head_bytes(H, V, B, fp8)
        head_us = head_s / args.steps * 1e6
        gbps = hb / (head_s / args.steps) / 1e9
        res[name] = {
            "sweeps_per_s": args.steps / wall_s,
            "ms_per_step": wall_s / args.steps * 1e3,
            "event_ms_per_step": gpu_s / args.steps * 1e3,
            "head_us": head_us,
            "lm_head_GBps": gbps,
            "lm_head_frac_of_peak": gbps / HBM_PEAK_GBPS,
            "sweep_GBps": sweep_bytes(H, V, B, fp8) / (gpu_s / args.steps) / 1e9,
        }
        turn = [0]

        def cold(fp8=fp8):
            turn[0] = (turn[0] + 1) % len(cw)
            if fp8:
                mtp.mtp_draft_fp8w(cw[turn[0]], q, s, B, tk, hd, draft, logits, ws, stream)
            else:
                mtp.mtp_draft_bf16(cw[turn[0]], B, tk, hd, draft, logits, ws, stream)
        cold_s, cold_wall = timed(cold, args.steps, args.warmup)
        res[name]["detail"] = {
            "sweep_per_call": spread(lambda: sweep(fp8)),
            "head_per_call": spread(lambda: head(fp8)),
            "sync_each_call_us": synced(lambda: sweep(fp8)),
            "cold_eh_proj_sweeps_per_s": round(args.steps / cold_wall, 2),
            "cold_eh_proj_ms_per_step": round(cold_wall / args.steps * 1e3, 5),
        }
        print(f"[bench] {name}: {res[name]}", file=sys.stderr, flush=True)

    # The per-GPU kernel of a vocabulary-sharded head (the pages' TP sweep):
    # the head over V/G rows, what one of G GPUs would sweep before the
    # cross-GPU pick.  Only the kernel is timed here; the exchange of the
    # per-shard (max, index) is not built.
    shards = None
    if not args.no_shards:
        shards = {}
        t = dw.tensors

        def shard_tables(G):
            # Consecutive calls read different row ranges of the tables (up to
            # three shards of V/G rows): one shard read over and over would
            # partly stay in the 256 MB last-level cache, which a sharded
            # sweep, reading its rows once per draft, does not get.
            Vs = V // G
            tabs = []
            for i in range(min(G, 3)):
                r = slice(i * Vs, (i + 1) * Vs)
                tabs.append((mtp.mtp_weights(t["embed"][r], t["enorm_w"], t["hnorm_w"],
                                             t["head_norm_w"], t["eh_proj"], t["lm_head"][r],
                                             float(wts["rms_eps"])), q[r], s[r]))
            return [a for a, _, _ in tabs], [b for _, b, _ in tabs], [c for _, _, c in tabs]

        # A plain streaming read of the same bytes, rotated the same way (best
        # of one and two workgroups per CU): the practical floor at this size,
        # launch and drain included, against which the head's fixed costs show.
        probe_out = torch.zeros(1, dtype=torch.int32, device=dev)
        probe_cache = {}

        def read_floor_us(G, fp8):
            if (G, fp8) not in probe_cache:
                Vs = V // G
                bufs = [(q if fp8 else t["lm_head"])[i * Vs:(i + 1) * Vs] for i in range(min(G, 3))]
                best = None
                for per_cu in (1, 2):
                    def rd(c=[0]):
                        mtp.mtp_probe_stream_read(bufs[c[0] % len(bufs)], probe_out, per_cu, stream)
                        c[0] += 1
                    g_s, _ = timed(rd, args.steps, args.warmup)
                    us = g_s / args.steps * 1e6
                    best = us if best is None else min(best, us)
                probe_cache[(G, fp8)] = round(best, 2)
            return probe_cache[(G, fp8)]
        for G in (2, 4, 8):
            Vs = V // G
            sws_, qs_, ss_ = shard_tables(G)
            slg = torch.empty((B, Vs), dtype=torch.bfloat16, device=dev)
            sws = mtp.new_workspace(H, Vs, B)
            ent = {"rows": Vs, "row_ranges": len(sws_)}
            for name, fp8 in (("bf16", False), ("fp8", True)):
                def shead(c=[0]):
                    i = c[0] % len(sws_)
                    c[0] += 1
                    if fp8:
                        mtp.mtp_head_fp8w(sws_[i], qs_[i], ss_[i], B, x, draft, slg, sws, stream)
                    else:
                        mtp.mtp_head_bf16(sws_[i], B, x, draft, slg, sws, stream)
                g_s, _ = timed(shead, args.steps, args.warmup)
                per = g_s / args.steps
                ent[name] = {"head_us": round(per * 1e6, 2),
                             "GBps": round(head_bytes(H, Vs, B, fp8) / per / 1e9, 1),
                             "frac_of_peak": round(head_bytes(H, Vs, B, fp8) / per / 1e9
                                                   / HBM_PEAK_GBPS, 4),
                             "weight_read_floor_us": read_floor_us(G, fp8)}
            shards[f"G{G}"] = ent
        if args.config == "large":
            # the same shard shapes for the batched configuration's 16 sequences
            # (the batched head on matrix cores)
            btok16, bhid16 = synth.make_inputs(synth.CONFIGS["batched"])
            xb = harness.to_dev_bf16(bhid16)
            db = torch.empty(16, dtype=torch.int32, device=dev)
            for G in (1, 2, 4, 8):
                Vs = V // G
                sws_, qs_, ss_ = shard_tables(G)
                slg = torch.empty((16, Vs), dtype=torch.bfloat16, device=dev)
                sws = mtp.new_workspace(H, Vs, 16)
                ent = {"rows": Vs, "batch": 16, "row_ranges": len(sws_)}
                for name, fp8 in (("bf16", False), ("fp8", True)):
                    def shead(c=[0]):
                        i = c[0] % len(sws_)
                        c[0] += 1
                        if fp8:
                            mtp.mtp_head_fp8w(sws_[i], qs_[i], ss_[i], 16, xb, db, slg, sws, stream)
                        else:
                            mtp.mtp_head_bf16(sws_[i], 16, xb, db, slg, sws, stream)
                    g_s, _ = timed(shead, args.steps, args.warmup)
                    per = g_s / args.steps
                    ent[name] = {"head_us": round(per * 1e6, 2),
                                 "GBps": round(head_bytes(H, Vs, 16, fp8) / per / 1e9, 1),
                                 "frac_of_peak": round(head_bytes(H, Vs, 16, fp8) / per / 1e9
                                                       / HBM_PEAK_GBPS, 4),
                                 "weight_read_floor_us": read_floor_us(G, fp8)}
                shards[f"B16_G{G}"] = ent
        print(f"[bench] vocab shards: {shards}", file=sys.stderr, flush=True)

    batched = None
    if not args.no_batched and args.config == "large":
        batched = {}
        for bname, bcfg, paths, nb in (("B16", synth.CONFIGS["batched"], ("fp8",), 16),
                                       ("B8", synth.CONFIGS["neartie"], ("bf16", "fp8"), 8),
                                       ("B4", synth.CONFIGS["batched"], ("bf16", "fp8"), 4)):
            btok, bhid = synth.make_inputs(bcfg)
            btok, bhid = btok[:nb], np.ascontiguousarray(bhid[:nb])
            Bb = nb
            btk = torch.from_numpy(btok.astype(np.uint32).view(np.int32)).to(dev)
            bhd = harness.to_dev_bf16(bhid)
            bdr = torch.empty(Bb, dtype=torch.int32, device=dev)
            blg = torch.empty((Bb, V), dtype=torch.bfloat16, device=dev)
            bws = mtp.new_workspace(H, V, Bb)
            for path in paths:
                def bsweep():
                    if path == "fp8":
                        mtp.mtp_draft_fp8w(dw.w, q, s, Bb, btk, bhd, bdr, blg, bws, stream)
                    else:
                        mtp.mtp_draft_bf16(dw.w, Bb, btk, bhd, bdr, blg, bws, stream)
                g_s, w_s = timed(bsweep, args.steps, args.warmup)
                per = g_s / args.steps
                batched[f"{bname}_{path}"] = {
                    "batch": Bb, "calls_per_s": round(args.steps / w_s, 2),
                    "sequences_per_s": round(Bb * args.steps / w_s, 1),
                    "ms_per_call": round(per * 1e3, 5),
                    "sweep_GBps": round(sweep_bytes(H, V, Bb, path == "fp8") / per / 1e9, 1),
                    # dense multiply-adds of the call (eh_proj + lm_head), as MFMA work
                    "sweep_TFLOPs": round(2.0 * Bb * (V * H + 2 * H * H) / per / 1e12, 1),
                }
        print(f"[bench] batched: {batched}", file=sys.stderr, flush=True)

    chain = None
    if not args.no_chain:
        # K chained drafts per call (each step takes the previous draft and
        # block output), one sequence: the propose loop without host round trips.
        K = 4
        cdr = torch.empty((K, B), dtype=torch.int32, device=dev)
        cws = torch.empty(mtp.mtp_chain_workspace_bytes(H, V, B), dtype=torch.uint8, device=dev)
        chain = {"steps": K}
        for name, fp8 in (("bf16", False), ("fp8", True)):
            def ccall():
                if fp8:
                    mtp.mtp_draft_chain_fp8w(dw.w, q, s, K, B, tk, hd, cdr, None, cws, stream)
                else:
                    mtp.mtp_draft_chain_bf16(dw.w, K, B, tk, hd, cdr, None, cws, stream)
            n = max(10, args.steps // K)
            g_s, w_s = timed(ccall, n, max(2, args.warmup // K))
            chain[name] = {"ms_per_call": round(g_s / n * 1e3, 4),
                           "drafts_per_s": round(K * B * n / w_s, 1)}
        print(f"[bench] chain: {chain}", file=sys.stderr, flush=True)

    context = None
    if not args.no_context and args.config == "large":
        # Context rows through the front half (embed gather, dual norm, eh_proj
        # as a GEMM over T rows), at the drafter's Large shape.
        Tmax = 4096
        ccfg = synth.custom(H, V, Tmax + 1, 2002)
        ctok, chid = synth.make_inputs(ccfg)
        ctk = torch.from_numpy(ctok.astype(np.uint32).view(np.int32)).to(dev)
        chd = harness.to_dev_bf16(chid[:Tmax])
        cx = torch.empty((Tmax, H), dtype=torch.bfloat16, device=dev)
        cws = torch.empty(mtp.mtp_context_workspace_bytes(H, Tmax), dtype=torch.uint8,
                          device=dev)
        turn = [0]

        def ctx_call(T):
            turn[0] = (turn[0] + 1) % len(cw)
            mtp.mtp_context_rows(cw[turn[0]], T, ctk, chd, cx, cws, stream)

        context = {"eh_proj_copies": len(cw)}
        for T in (4, 16, 128, 1024, 4096):
            n = max(10, min(args.steps, 100 if T <= 128 else 20))
            g_s, _ = timed(lambda: ctx_call(T), n, max(2, min(args.warmup, 5)))
            per = g_s / n
            flops = 2.0 * T * H * 2 * H
            # eh_proj once, per row an embedding row, a hidden row, an x row and a
            # token, plus the two norm weights
            nbytes = H * (2 * H) * 2 + T * (H * 2 + H * 2 + H * 2 + 4) + 2 * H * 2
            t_roof = max(flops / (MFMA_BF16_PEAK_TFLOPS * 1e12), nbytes / (HBM_PEAK_GBPS * 1e9))
            context[f"T{T}"] = {
                "us_per_call": round(per * 1e6, 2), "rows_per_s": round(T / per, 1),
                "TFLOPs": round(flops / per / 1e12, 1), "GBps": round(nbytes / per / 1e9, 1),
                "bound": "mfma" if flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) > nbytes / (
                    HBM_PEAK_GBPS * 1e9) else "hbm",
                "roofline_frac": round(t_roof / per, 3),
            }
        # The vendor library on the same product (torch's BF16 matmul, which
        # runs hipBLASLt): the GEMM alone, with the weight pre-transposed so no
        # transposed view reaches it.  A reference point for ctx_gemm_kernel,
        # not part of the path.
        wt = dw.tensors["eh_proj"].t().contiguous()
        lib_gemm = {}
        for T in (1024, 4096):
            a = torch.randn(T, 2 * H, device=dev).to(torch.bfloat16)
            n = max(10, min(args.steps, 20))
            g_s, _ = timed(lambda: torch.matmul(a, wt), n, max(2, min(args.warmup, 5)))
            per = g_s / n
            lib_gemm[f"T{T}"] = {"us_per_call": round(per * 1e6, 2),
                                 "TFLOPs": round(2.0 * T * H * 2 * H / per / 1e12, 1)}
            del a
        del wt
        context["library_gemm"] = lib_gemm
        print(f"[bench] context rows: {context}", file=sys.stderr, flush=True)

    agreement = None
    if not args.no_agreement:
        # How often the FP8 drafting copy proposes the same token as the BF16
        # head (the page's reason for the copy: it may change acceptance, never
        # an emitted token).  Random-init weights: a synthetic proxy only.  The
        # oracle's own rate on the same sequences comes from the agreement
        # tests, which need minutes of FP64 work.
        def agree_on(w, qq, ss, Hh, Vv, atok, ahid):
            n = atok.size
            d16 = np.empty(n, np.int64)
            d8 = np.empty(n, np.int64)
            gaps = np.empty(n)
            for b0 in range(0, n, 64):
                bb = min(64, n - b0)
                atk = torch.from_numpy(atok[b0:b0 + bb].astype(np.uint32).view(np.int32)).to(dev)
                ahd = harness.to_dev_bf16(np.ascontiguousarray(ahid[b0:b0 + bb]))
                a16 = torch.empty(bb, dtype=torch.int32, device=dev)
                a8 = torch.empty(bb, dtype=torch.int32, device=dev)
                alg = torch.empty((bb, Vv), dtype=torch.bfloat16, device=dev)
                aws = mtp.new_workspace(Hh, Vv, bb)
                mtp.mtp_draft_bf16(w, bb, atk, ahd, a16, alg, aws, stream)
                mtp.mtp_draft_fp8w(w, qq, ss, bb, atk, ahd, a8, None, aws, stream)
                torch.cuda.synchronize()
                d16[b0:b0 + bb] = a16.cpu().numpy()
                d8[b0:b0 + bb] = a8.cpu().numpy()
                top2 = torch.topk(alg.float(), 2, dim=1).values.cpu().numpy()
                gaps[b0:b0 + bb] = top2[:, 0] - top2[:, 1]
            agree = int((d16 == d8).sum())
            return {"sequences": n, "agree": agree, "rate": round(agree / n, 4),
                    "median_bf16_top2_gap": round(float(np.median(gaps)), 4)}

        agreement = {"data": "synthetic random-init weights (a proxy, not an acceptance rate)"}
        if args.config == "large":
            tw = synth.make_weights(synth.CONFIGS["tiny"])
            tdw = harness.upload(tw)
            tq, ts = harness.quantize_dev(tdw)
            ttok, thid = synth.make_inputs(synth.custom(256, 4096, 256, 3001))
            agreement["tiny"] = agree_on(tdw.w, tq, ts, 256, 4096, ttok, thid)
            atok, ahid = synth.make_inputs(synth.custom(H, V, 64, 2001))
            agreement["large"] = agree_on(dw.w, q, s, H, V, atok, ahid)
            btok, bhid = synth.make_inputs(synth.CONFIGS["batched"])
            agreement["batched_inputs_on_large_weights"] = agree_on(dw.w, q, s, H, V, btok, bhid)
            del tdw, tq, ts
        else:
            atok, ahid = synth.make_inputs(synth.custom(H, V, 64, 2001))
            agreement[cfg.name] = agree_on(dw.w, q, s, H, V, atok, ahid)
        print(f"[bench] agreement: {agreement}", file=sys.stderr, flush=True)

    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # The practical ceiling: a plain streaming read of the same lm_head bytes
    # (16-byte non-temporal loads, nothing computed), best over grid sizes.
    ceiling = None
    if not args.no_ceiling:
        pout = torch.zeros(1, dtype=torch.int32, device=dev)
        lmh = dw.tensors["lm_head"]
        nb = lmh.numel() * lmh.element_size()
        best = None
        per = {}
        for per_cu in (1, 2, 4, 8):
            g_s, _ = timed(lambda: mtp.mtp_probe_stream_read(lmh, pout, per_cu, stream),
                           max(20, args.steps // 4), 5)
            gbps = nb / (g_s / max(20, args.steps // 4)) / 1e9
            per[f"wg_per_cu_{per_cu}"] = round(gbps, 1)
            if best is None or gbps > best[0]:
                best = (gbps, per_cu)
        ceiling = {"GBps": round(best[0], 1), "frac_of_peak": round(best[0] / HBM_PEAK_GBPS, 4),
                   "wg_per_cu": best[1], "by_grid": per,
                   "buffer": f"the BF16 lm_head, {nb} bytes",
                   "lm_head_bf16_frac_of_ceiling": round(res["bf16"]["lm_head_GBps"] / best[0], 4),
                   "lm_head_fp8_frac_of_ceiling": round(res["fp8"]["lm_head_GBps"] / best[0], 4)}
        if B == 1:
            # The sweep against plain reads of its two weight matrices: the same
            # probe over eh_proj (the three copies in turn, as the cold-front
            # sweeps read them) plus the lm_head read above.
            eh_us = None
            for per_cu in (1, 2):
                def rd(c=[0]):
                    mtp.mtp_probe_stream_read(ehc[c[0] % len(ehc)], pout, per_cu, stream)
                    c[0] += 1
                g_s, _ = timed(rd, max(20, args.steps // 4), 5)
                us = g_s / max(20, args.steps // 4) * 1e6
                eh_us = us if eh_us is None else min(eh_us, us)
            lm_us = nb / best[0] / 1e3
            sweep_us = res["bf16"]["ms_per_step"] * 1e3
            ceiling["bf16_sweep_vs_plain_reads"] = {
                "eh_proj_read_us": round(eh_us, 2), "lm_head_read_us": round(lm_us, 2),
                "sum_us": round(eh_us + lm_us, 2), "sweep_us": round(sweep_us, 2),
                "sweep_over_sum": round(sweep_us / (eh_us + lm_us), 4)}
        print(f"[bench] streaming-read ceiling: {ceiling}", file=sys.stderr, flush=True)

    main_path = "bf16"
    r = res[main_path]
    hb = head_bytes(H, V, B, False)
    roof = {
        "bound": "hbm",
        "achieved": round(r["lm_head_GBps"], 1),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(r["lm_head_GBps"] / HBM_PEAK_GBPS, 4),
        "traffic": committed_traffic(f"lm_head_bf16_{cfg.name}_traffic.md"),
        "kernel": "row_gemv_kernel<BF16, head-norm prologue, argmax-partials epilogue>; the "
                  "timed mtp_head_bf16 call also runs the one-workgroup-per-sequence "
                  "argmax_final_kernel after it",
        "traffic_source": f"profiles/lm_head_bf16_{cfg.name}_traffic.md (null when there is "
                          "none for this configuration or the kernel sources changed since the "
                          "counters were taken)",
        "algorithmic_bytes_per_launch": hb,
        "avg_launch_us": round(r["head_us"], 2),
    }

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_leg(args, cfg, wts, tokens, hidden)
    line = {
        "metric": METRIC,
        "value": round(r["sweeps_per_s"], 2),
        "unit": "draft sweeps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name} draft sweep", "hidden": H, "vocab": V, "batch": B,
                   "head": "bf16", "parallelism": "single GPU"},
        "lm_head": {k: {"GBps": round(v["lm_head_GBps"], 1),
                        "frac_of_peak": round(v["lm_head_frac_of_peak"], 4),
                        "head_us": round(v["head_us"], 2),
                        "sweeps_per_s": round(v["sweeps_per_s"], 2),
                        "ms_per_step": round(v["ms_per_step"], 5),
                        **v["detail"]} for k, v in res.items()},
        "fp8_quantiser": quant,
        "vocab_shard_heads": shards,
        "batched": batched,
        "chained_drafts": chain,
        "context_rows": context,
        "draft_agreement_fp8_vs_bf16": agreement,
        "streaming_read_ceiling": ceiling,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
