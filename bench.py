#!/usr/bin/env python3
"""Decode-step benchmark of the EntmaxKV HIP path on one MI355X.

One step = one decode step for every (sequence, KV head) of the workload:
refresh of each sequence's tail-page metadata and Gaussian page scoring (one
launch), Gaussian-aware selection, gathered entmax attention (scores,
threshold, apply).  The headline value is decode tokens/s = batch / median step time,
with the inputs resident in HBM and the caches flushed between steps
(a 1 GiB read, so that no dirty lines are left to write back), outside the
timed events.  Beside it the top-k path and the
full-cache entmax and split-K softmax baselines are timed the same way.

Each kernel of a step is bracketed by HIP events on the stream the library
launches on (torch's current stream), which gives the per-kernel durations
and picks the dominant kernel.  Since an event between two kernels delays
the second one's dispatch, the dominant kernel's duration for the roofline
is taken without one: the step cut just after that kernel minus the step cut
just before it, both timed like the headline pass.  The events are created with
a device-scope release (hipEventReleaseToDevice): the default system-scope
release flushes the caches at every record and would add several
microseconds between the kernels of a step.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

REPO = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, REPO)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, 8 TB/s

# hipEventReleaseToDevice: the event is recorded with a device-scope
# release.  The default (system-scope) release writes back and invalidates
# the caches at every record, which adds several microseconds between
# kernels and would be charged to the decode step.
HIP_EVENT_RELEASE_TO_DEVICE = 0x40000000


class DeviceEvents:
    """Timing events on the HIP runtime that torch already loaded."""

    def __init__(self):
        import ctypes
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("HIP runtime not loaded")
        self.ct = ctypes
        self.lib = ctypes.CDLL(path)
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.pool = []

    def new(self):
        e = self.ct.c_void_p()
        rc = self.lib.hipEventCreateWithFlags(self.ct.byref(e), HIP_EVENT_RELEASE_TO_DEVICE)
        if rc != 0:
            raise RuntimeError("hipEventCreateWithFlags failed (%d)" % rc)
        self.pool.append(e)
        return e

    def record(self, e, stream):
        rc = self.lib.hipEventRecord(e, self.ct.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError("hipEventRecord failed (%d)" % rc)

    def ms(self, a, b):
        out = self.ct.c_float()
        rc = self.lib.hipEventElapsedTime(self.ct.byref(out), a, b)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed (%d)" % rc)
        return out.value

    def close(self):
        for e in self.pool:
            self.lib.hipEventDestroy(e)
        self.pool = []


TRAFFIC_FILE = os.path.join(REPO, "profiles", "hbm_traffic_cluster_1m.txt")
KERNEL_SOURCES = ("kpass.hip", "decode_common.h", "ekv_device.h", "ekv_kernels.h")


def kernel_source_hash():
    """sha256 over the sources the key-pass kernel is built from."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(REPO, "sparse_entmax_attention_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (L2-to-memory read and write requests counted by size), or None when
    there is none or the kernel's sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith("#"))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("kernel") != kernel or kv.get("source_sha256") != kernel_source_hash():
        return None
    try:
        return int(kv["fetch_bytes_per_launch"]) + int(kv["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="cluster_1m")
    ap.add_argument("--seed", type=int, default=3000)
    ap.add_argument("--flush", choices=["read", "write", "none"], default="read",
                    help="cache flush between timed steps (outside the events): "
                         "read a 1 GiB buffer (default), write 512 MiB, or none")
    ap.add_argument("--cpu-units", type=int, default=-1,
                    help="(sequence, KV head) units the oracle is timed on; "
                         "-1 (default) all units of one step, 0 skips")
    ap.add_argument("--legs", default="gauss,topk,topk_split,softmax_topk,entmax_full,softmax_full")
    ap.add_argument("--extra", default="cluster_128k_b4,ragged_pool_b16",
                    help="other workloads timed after the main legs (comma "
                         "separated; empty for none): the Gaussian step on "
                         "cluster_128k_b4, and on ragged_pool_b16 with one "
                         "token appended per sequence per step")
    ap.add_argument("--extra-steps", type=int, default=64)
    ap.add_argument("--extra-warmup", type=int, default=8)
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the headline line: time the top-k and "
                         "Gaussian steps on prefixes of the workload's "
                         "sequences (16k tokens up to their full length) and "
                         "print one JSON line with the selection and step "
                         "times per length")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the decode step on one GPU only; units are "
              "independent, and the multi-GPU split is not implemented "
              "(got --gpus %d, WORLD_SIZE %d)" % (args.gpus, world),
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_entmax_attention_amd as ekv
    import workloads
    from sparse_entmax_attention_amd.quality import matched_budget_quality

    dev = torch.device("cuda:0")
    spec = workloads.workload(args.workload)
    log = lambda *a: print(*a, file=sys.stderr, flush=True)
    log("[bench] generating %s seed %d" % (spec.name, args.seed))
    t0 = time.time()
    inp = workloads.generate(spec, args.seed, dev)
    torch.cuda.synchronize()
    log("[bench] inputs ready in %.1fs" % (time.time() - t0))
    kv = ekv.PagedKV(inp.k, inp.v, inp.page_table, inp.seq_lens, spec.group)
    buf = ekv.DecodeBuffers(kv, softmax=True)
    stream = torch.cuda.current_stream()
    B, H, G, D, P = spec.batch, spec.num_kv_heads, spec.group, spec.head_dim, spec.page_size
    e = 2 if spec.kv_dtype == "bf16" else 4
    alpha = spec.alphas[0]
    k_top = spec.topk or 16
    delta = spec.delta
    q = inp.q
    if args.flush == "read":
        flush_buf = torch.ones(256 << 20, dtype=torch.float32, device=dev)  # 1 GiB
        flush = lambda s: torch.amax(flush_buf)
    elif args.flush == "write":
        flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        flush = lambda s: flush_buf.fill_(s & 0xFF)
    else:
        flush = None

    # Measured HBM read ceiling: the library's streaming-read probe over
    # 2 GiB (well beyond the 256 MB last-level cache), median of 5.
    probe = torch.ones(512 << 20, dtype=torch.float32, device=dev)
    sink = torch.empty(ekv.EKV_READ_PROBE_SINK, dtype=torch.int32, device=dev)
    dev_ev = DeviceEvents()
    pe = [dev_ev.new() for _ in range(12)]
    for i in range(6):
        dev_ev.record(pe[2 * i], stream)
        ekv.ekv_read_probe(probe, sink)
        dev_ev.record(pe[2 * i + 1], stream)
    torch.cuda.synchronize()
    probe_ms = statistics.median(dev_ev.ms(pe[2 * i], pe[2 * i + 1]) for i in range(1, 6))
    dev_ev.close()
    read_probe_gbps = probe.numel() * 4 / (probe_ms * 1e-3) / 1e9
    del probe, sink
    # A write of known size (256 MiB), the reference for hardware write counters.
    calib = torch.empty(64 << 20, dtype=torch.float32, device=dev)
    calib.fill_(1.0)
    torch.cuda.synchronize()
    del calib

    # Full metadata build (once; timed on its own).
    ev0, ev1 = dev_ev.new(), dev_ev.new()
    dev_ev.record(ev0, stream)
    buf.build_meta()
    dev_ev.record(ev1, stream)
    torch.cuda.synchronize()
    meta_build_ms = dev_ev.ms(ev0, ev1)
    dev_ev.close()

    # Each leg is a list of (phase name, callable).
    n_keep = min(k_top, inp.max_pages)
    topk_front = [
        # the tail page's box refresh runs inside the scoring launch
        ("score_bbox", lambda: buf.refresh_score(q, ekv.EKV_SCORE_BBOX)),
        ("select_topk", lambda: buf.select_topk(k_top)),
    ]
    split_decode = [
        ("entmax_scores", lambda: ekv.ekv_entmax_scores(
            kv, q, buf.scale, alpha, buf.sel, buf.count, buf.ws_decode)),
        ("entmax_threshold", lambda: ekv.ekv_entmax_threshold(
            kv, alpha, buf.sel, buf.count, buf.tau, buf.out, buf.ws_decode)),
        ("entmax_apply", lambda: ekv.ekv_entmax_apply(
            kv, alpha, buf.sel, buf.count, buf.out, None, buf.ws_decode)),
    ]
    legs = {
        "gauss": [
            # the tail page's metadata refresh runs inside the scoring launch
            ("score_gauss", lambda: buf.refresh_score(q, ekv.EKV_SCORE_GAUSS)),
            ("select_gauss", lambda: buf.select_gauss(alpha, delta)),
            # the selector's threshold estimates are the decode's hint
            ("entmax_scores", lambda: ekv.ekv_entmax_scores(
                kv, q, buf.scale, alpha, buf.sel, buf.count, buf.ws_decode,
                tau_hint=buf.tau_hat)),
            ("entmax_threshold", lambda: ekv.ekv_entmax_threshold(
                kv, alpha, buf.sel, buf.count, buf.tau, buf.out, buf.ws_decode)),
            ("entmax_apply", lambda: ekv.ekv_entmax_apply(
                kv, alpha, buf.sel, buf.count, buf.out, None, buf.ws_decode)),
        ],
        # top-k: the k pages' decode in one launch when they fit on chip
        # (the split decode otherwise); "topk_split" always takes the split
        # decode (key pass, threshold step), for comparison
        "topk": topk_front + ([
            ("entmax_small", lambda: buf.entmax_small(q, alpha, n_keep)),
        ] if buf.small_fits(n_keep) else split_decode),
        "topk_split": topk_front + split_decode,
        "entmax_full": [
            ("entmax_scores", lambda: ekv.ekv_entmax_scores(
                kv, q, buf.scale, alpha, None, None, buf.ws_decode)),
            ("entmax_threshold", lambda: ekv.ekv_entmax_threshold(
                kv, alpha, None, None, buf.tau, buf.out, buf.ws_decode)),
            ("entmax_apply", lambda: ekv.ekv_entmax_apply(
                kv, alpha, None, None, buf.out, None, buf.ws_decode)),
        ],
        "softmax_full": [
            ("softmax", lambda: buf.softmax(q)),
        ],
        # split-K softmax over the same top-k pages (the pages' softmax
        # top-k comparison)
        "softmax_topk": topk_front + [
            ("softmax", lambda: buf.softmax(q, selected=True)),
        ],
    }

    def step_median(phases, steps, warmup):
        """Median time of the given phases run as one step, one event pair
        per step and the cache flush between steps (as the headline pass)."""
        for _ in range(warmup):
            for _, fn in phases:
                fn()
        torch.cuda.synchronize()
        evs = [(dev_ev.new(), dev_ev.new()) for _ in range(steps)]
        for s in range(steps):
            if flush is not None:
                flush(s)
            dev_ev.record(evs[s][0], stream)
            for _, fn in phases:
                fn()
            dev_ev.record(evs[s][1], stream)
        torch.cuda.synchronize()
        med = statistics.median(dev_ev.ms(a, b) for a, b in evs)
        dev_ev.close()
        return med

    def run_leg(name, steps, warmup):
        """Headline pass: one event pair per step (start, end).  Breakdown
        pass: the same steps with an event after every kernel, for the
        per-kernel durations (each event between kernels adds a few
        microseconds of dispatch delay, so it is kept out of the headline)."""
        phases = legs[name]
        for _ in range(warmup):
            for _, fn in phases:
                fn()
        torch.cuda.synchronize()

        evs = [(dev_ev.new(), dev_ev.new()) for _ in range(steps)]
        t_start = time.perf_counter()
        for s in range(steps):
            if flush is not None:
                flush(s)
            dev_ev.record(evs[s][0], stream)
            for _, fn in phases:
                fn()
            dev_ev.record(evs[s][1], stream)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t_start) / steps
        step_ms = [dev_ev.ms(a, b) for a, b in evs]
        dev_ev.close()

        pev = [[dev_ev.new() for _ in range(len(phases) + 1)] for _ in range(steps)]
        for s in range(steps):
            if flush is not None:
                flush(s)
            dev_ev.record(pev[s][0], stream)
            for i, (_, fn) in enumerate(phases):
                fn()
                dev_ev.record(pev[s][i + 1], stream)
        torch.cuda.synchronize()
        phase_ms = {pname: statistics.mean(dev_ev.ms(pev[s][i], pev[s][i + 1])
                                           for s in range(steps))
                    for i, (pname, _) in enumerate(phases)}
        phased_step_ms = statistics.median(dev_ev.ms(pev[s][0], pev[s][-1])
                                           for s in range(steps))
        dev_ev.close()
        return {"median_ms": statistics.median(step_ms),
                "p10_ms": float(np.percentile(step_ms, 10)),
                "p90_ms": float(np.percentile(step_ms, 90)),
                "wall_ms_incl_flush": wall * 1e3, "phase_ms": phase_ms,
                "median_ms_with_phase_events": phased_step_ms}

    def selection_stats():
        cnt = buf.count.cpu().numpy()
        sel = buf.sel.cpu().numpy()
        tok = 0
        for b in range(B):
            L = inp.lens[b]
            for h in range(H):
                pages = sel[b, h, :cnt[b, h]]
                tok += int(sum(min(P, L - p * P) for p in pages))
        return int(cnt.sum()), tok

    def support_rows(selected):
        probs = torch.zeros(B, H * G, inp.max_pages * P, device=dev)
        buf.entmax(q, alpha, selected=selected, probs=probs)
        torch.cuda.synchronize()
        rows = (probs.view(B, H, G, -1) > 0).any(dim=2).sum().item()
        del probs
        return int(rows)

    n_pages_total = sum((L + P - 1) // P for L in inp.lens)
    tokens_total = sum(inp.lens)
    meta_gauss_bytes = n_pages_total * H * 2 * D * 4
    meta_bbox_bytes = n_pages_total * H * 2 * D * e
    tail_bytes = B * H * (P * D * e)

    if args.sweep:
        # Prefixes of every sequence, multiples of the page size, so that the
        # metadata built for the whole cache is that of each prefix.
        full_lens = list(inp.lens)
        lengths = [L for L in (1 << 14, 1 << 15, 1 << 16, 1 << 17, 1 << 18,
                               1 << 19, 1 << 20) if L <= max(full_lens)]
        rows = []
        for L in lengths:
            lens = [min(L, n) for n in full_lens]
            inp.lens[:] = lens
            inp.seq_lens.copy_(torch.tensor(lens, dtype=torch.int32))
            n_pages = sum((n + P - 1) // P for n in lens)
            row = {"seq_len": L}
            for name, sel_phases in (("topk", ("score_bbox", "select_topk")),
                                     ("gauss", ("score_gauss", "select_gauss"))):
                r = run_leg(name, args.steps, args.warmup)
                pages, toks = selection_stats()
                meta = n_pages * H * 2 * D * (4 if name == "gauss" else e)
                row[name] = {
                    "step_us": round(r["median_ms"] * 1e3, 2),
                    "select_us": round(sum(r["phase_ms"][k] for k in sel_phases) * 1e3, 2),
                    "selected_pages": pages,
                    "phase_us": {k: round(v * 1e3, 2) for k, v in r["phase_ms"].items()},
                    "metadata_bytes": meta,
                    "selected_k_bytes": toks * D * e,
                }
            log("[sweep] %7d tokens: top-k select %.1f us, step %.1f us | "
                "gauss select %.1f us, step %.1f us (%d pages kept)" % (
                    L, row["topk"]["select_us"], row["topk"]["step_us"],
                    row["gauss"]["select_us"], row["gauss"]["step_us"],
                    row["gauss"]["selected_pages"]))
            rows.append(row)
        print(json.dumps({"sweep": rows, "workload": spec.name, "batch": B,
                          "kv_heads": H, "group": G, "head_dim": D, "page_size": P,
                          "alpha": alpha, "delta": delta, "topk": k_top,
                          "steps": args.steps, "warmup": args.warmup,
                          "note": "select_us sums the per-phase event times "
                                  "(scoring with the tail refresh, selection); "
                                  "step_us is the headline pass of the whole step"}),
              flush=True)
        return

    results = {}
    wanted = [x for x in args.legs.split(",") if x]
    for name in wanted:
        steps = args.steps
        warm = args.warmup
        log("[bench] leg %s: %d warmup + %d timed steps" % (name, warm, steps))
        r = run_leg(name, steps, warm)
        if name in ("gauss", "topk", "topk_split", "softmax_topk"):
            pages, toks = selection_stats()
            # what the selection costs each attention (same pages for both),
            # measured after the timed steps from the selection they left
            qm = matched_budget_quality(buf, q, alpha)
            r["quality"] = {k: {"mean": round(v.mean().item(), 6),
                                "min": round(v.min().item(), 6),
                                "max": round(v.max().item(), 6)}
                            for k, v in qm.items()}
            rows = support_rows(True)
            kbytes = toks * D * e
            # softmax weights every selected token: all their value rows
            vbytes = (toks if name == "softmax_topk" else rows) * D * e
            mbytes = meta_gauss_bytes if name == "gauss" else meta_bbox_bytes
            r.update(selected_pages=pages, selected_tokens=toks, support_v_rows=rows,
                     bytes={"metadata": mbytes, "tail_refresh": tail_bytes,
                            "selected_k": kbytes, "support_v": vbytes})
            step_bytes = mbytes + tail_bytes + kbytes + vbytes
            sel_positions = pages * P
            # scoring: metadata read and per-page values written; the launch
            # also refreshes the tail pages (keys of each sequence's last
            # page read)
            r["kernel_bytes"] = {
                "score_gauss" if name == "gauss" else "score_bbox":
                    mbytes + n_pages_total * H * G * (8 if name == "gauss" else 4) +
                    tail_bytes,
                # the key pass reads the selected keys; unhinted it writes
                # every score, hinted only those near the support (a few
                # hundred per head: left out)
                "entmax_scores": kbytes + (0 if name == "gauss" else sel_positions * G * 4),
            }
            if "softmax" in r["phase_ms"]:
                r["kernel_bytes"]["softmax"] = kbytes + vbytes
            if "entmax_small" in r["phase_ms"]:
                # keys of the selection and value rows of the support read,
                # the output rows written
                rbytes = B * H * G * D * 4
                r["kernel_bytes"]["entmax_small"] = kbytes + vbytes + rbytes
        elif name == "entmax_full":
            rows = support_rows(False)
            kbytes = tokens_total * H * D * e
            r.update(support_v_rows=rows,
                     bytes={"k": kbytes, "support_v": rows * D * e})
            step_bytes = kbytes + rows * D * e
            r["kernel_bytes"] = {"entmax_scores": kbytes + n_pages_total * P * H * G * 4}
        else:
            step_bytes = 2 * tokens_total * H * D * e
            r.update(bytes={"kv": step_bytes})
            r["kernel_bytes"] = {"softmax": step_bytes}
        r["step_bytes"] = step_bytes
        r["hbm_gbps"] = step_bytes / (r["median_ms"] * 1e-3) / 1e9
        r["tokens_per_s"] = B / (r["median_ms"] * 1e-3)
        results[name] = r
        log("[bench] %s: median %.1f us, %.0f tokens/s, %.0f GB/s" % (
            name, r["median_ms"] * 1e3, r["tokens_per_s"], r["hbm_gbps"]))

    head = results.get("gauss") or next(iter(results.values()))
    head_name = "gauss" if "gauss" in results else next(iter(results))
    # Dominant kernel of the headline step and its roofline.
    kb = {k: v for k, v in head["kernel_bytes"].items() if k in head["phase_ms"]}
    dom = max(kb, key=lambda kname: head["phase_ms"][kname])
    # Its duration without an event around it: the step cut just after the
    # kernel minus the step cut just before it, each timed like the headline
    # pass (one event pair per step), so that no event delays the kernel's
    # dispatch; the difference includes its launch after the previous kernel.
    # The per-kernel event time is kept beside it.
    names = [n for n, _ in legs[head_name]]
    k_dom = names.index(dom)
    with_ms = step_median(legs[head_name][:k_dom + 1], args.steps, 2)
    without_ms = (step_median(legs[head_name][:k_dom], args.steps, 2)
                  if k_dom > 0 else 0.0)
    dom_ms = with_ms - without_ms
    if not dom_ms > 0.0:  # noise on a short kernel: fall back to the events
        dom_ms = head["phase_ms"][dom]
    achieved = kb[dom] / (dom_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBPS, 4),
                "traffic": (measured_traffic("k_entmax_scores_mfma")
                            if dom == "entmax_scores" and head_name == "gauss" else None),
                "bytes_per_launch": kb[dom], "avg_launch_ms": dom_ms,
                "avg_launch_ms_event_pair": head["phase_ms"][dom],
                "duration_method": "step through the kernel minus step before it"}

    speedups = {}
    for base in ("softmax_full", "entmax_full"):
        if base in results and head_name in results:
            speedups["%s_over_%s" % (head_name, base)] = round(
                results[base]["median_ms"] / head["median_ms"], 3)
        for tk in ("topk", "topk_split", "softmax_topk"):
            if base in results and tk in results:
                speedups["%s_over_%s" % (tk, base)] = round(
                    results[base]["median_ms"] / results[tk]["median_ms"], 3)

    if "topk" in results and "softmax_topk" in results:
        speedups["topk_over_softmax_topk"] = round(
            results["softmax_topk"]["median_ms"] / results["topk"]["median_ms"], 3)
    # The same speedups against full-cache baselines priced at the measured
    # 2 GiB read probe's rate: the bytes each baseline must read, divided by
    # that rate.  A reference point for how much of a speedup comes from
    # bytes not read; not a strict floor (a streaming kernel can exceed the
    # probe, as the split-K softmax does).
    floor_ms = {}
    for base in ("softmax_full", "entmax_full"):
        if base in results:
            floor_ms[base] = results[base]["step_bytes"] / (read_probe_gbps * 1e9) * 1e3
    for base, fms in floor_ms.items():
        for leg in (head_name, "topk"):
            if leg in results:
                speedups["%s_over_%s_at_read_probe_rate" % (leg, base)] = round(
                    fms / results[leg]["median_ms"], 3)

    extra = {}
    names = [x for x in args.extra.split(",") if x]
    if names:
        del buf, kv
        for name in names:
            extra[name] = other_workload(name, args, flush, dev_ev, log)

    cpu, cpu_more = None, None
    n_cpu = B * H if args.cpu_units < 0 else args.cpu_units
    if n_cpu > 0:
        cpu, cpu_more = cpu_baseline(inp, spec, min(n_cpu, B * H), alpha, delta, log)

    line = {
        "metric": "decode tokens/s at 1M ctx (1 GPU); achieved HBM GB/s vs peak",
        "value": round(head["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["median_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": spec.name, "batch": B, "seq_len": inp.lens[0] if B == 1 else list(inp.lens),
                   "kv_heads": H, "group": G, "head_dim": D, "page_size": P,
                   "kv_dtype": spec.kv_dtype, "alpha": alpha, "selector": head_name,
                   "delta": delta, "topk": k_top, "parallelism": "single GPU",
                   "cache_flush_between_steps": args.flush},
        "hbm_gbps": round(head["hbm_gbps"], 1),
        "hbm_frac_of_peak": round(head["hbm_gbps"] / PEAK_HBM_GBPS, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "cpu_baseline_more": cpu_more,
        "speedups": speedups,
        "meta_build_ms": round(meta_build_ms, 4),
        "hbm_read_probe_gbps": round(read_probe_gbps, 1),
        "baseline_floor_ms_at_read_probe_rate": {k: round(v, 4) for k, v in floor_ms.items()},
        "legs": {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv)
                     for kk, vv in v.items()} for k, v in results.items()},
        "workloads": extra,
    }
    print(json.dumps(line), flush=True)


def fresh_queries(inp, gen):
    """A new query set of the workload's recipe, drawn on the device in one
    pass: for clustered keys each query head is the sum of 1-3 distinct
    cluster means of its KV head over sqrt(count); else N(0, I)."""
    import torch
    spec = inp.spec
    B, H, G, D = spec.batch, spec.num_kv_heads, spec.group, spec.head_dim
    dev = inp.q.device
    if inp.cluster_means is None:
        return torch.randn(B, H * G, D, generator=gen, device=dev)
    C = spec.n_clusters
    cnt = torch.randint(1, 4, (B, H, G), generator=gen, device=dev)
    order = torch.rand(B, H, G, C, generator=gen, device=dev).argsort(dim=-1)
    pick = torch.zeros(B, H, G, C, device=dev)
    pick.scatter_(-1, order[..., :3], (torch.arange(3, device=dev) < cnt[..., None]).float())
    q = torch.matmul(pick, inp.cluster_means.contiguous()) / cnt[..., None].float().sqrt()
    return q.reshape(B, H * G, D).contiguous()


def other_workload(name, args, flush, dev_ev, log):
    """The Gaussian decode step on another workload, timed per step with a
    HIP event pair (the cache flush outside).  On a workload with spare
    pages (ragged_pool_b16) every step first appends one token to every
    sequence (key from the sequence's last cluster, value N(0, I), written
    into the pool through the page table), and draws a fresh query set; the
    tail-page metadata refresh runs inside the scoring launch.  The step
    time includes the append; decode_ms is the part after it."""
    import numpy as np
    import torch

    import sparse_entmax_attention_amd as ekv
    import workloads

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    spec = workloads.workload(name)
    log("[bench] generating %s seed %d" % (name, args.seed))
    inp = workloads.generate(spec, args.seed, dev)
    kv = ekv.PagedKV(inp.k, inp.v, inp.page_table, inp.seq_lens, spec.group)
    buf = ekv.DecodeBuffers(kv, bbox=False)
    buf.build_meta()
    B, H, G, D, P = spec.batch, spec.num_kv_heads, spec.group, spec.head_dim, spec.page_size
    alpha, delta = spec.alphas[0], spec.delta
    n_steps = args.extra_warmup + args.extra_steps
    appending = spec.spare_pages > 0
    if appending and n_steps > spec.spare_pages * P:
        raise SystemExit("%s: %d steps do not fit %d spare pages" % (name, n_steps, spec.spare_pages))
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed + 1)
    if appending:
        dt = spec.torch_dtype
        newk = (inp.cluster_means[None, :, :, -1, :] +
                0.3 * torch.randn(n_steps, B, H, D, generator=gen, device=dev)).to(dt)
        newv = torch.randn(n_steps, B, H, D, generator=gen, device=dev).to(dt)
        qs = [fresh_queries(inp, gen) for _ in range(n_steps)]
        bidx = torch.arange(B, device=dev)
    else:
        qs = [inp.q] * n_steps
    torch.cuda.synchronize()

    def append(s):
        pos = inp.seq_lens.long()
        slot = inp.page_table[bidx, pos // P].long()
        off = pos % P
        inp.k[slot, :, off, :] = newk[s]
        inp.v[slot, :, off, :] = newv[s]
        inp.seq_lens += 1

    def decode(s):
        buf.refresh_score(qs[s], ekv.EKV_SCORE_GAUSS)
        buf.select_gauss(alpha, delta)
        buf.entmax(qs[s], alpha, tau_hint=buf.tau_hat)

    evs = [(dev_ev.new(), dev_ev.new(), dev_ev.new()) for _ in range(n_steps)]
    for s in range(n_steps):
        if flush is not None:
            flush(s)
        dev_ev.record(evs[s][0], stream)
        if appending:
            append(s)
        dev_ev.record(evs[s][1], stream)
        decode(s)
        dev_ev.record(evs[s][2], stream)
    torch.cuda.synchronize()
    timed = evs[args.extra_warmup:]
    step = [dev_ev.ms(a, c) for a, _, c in timed]
    dec = [dev_ev.ms(b2, c) for _, b2, c in timed]
    dev_ev.close()
    med = statistics.median(step)
    lens = inp.seq_lens.cpu().tolist()
    n_pages = sum((L + P - 1) // P for L in lens)
    cnt = buf.count.cpu().numpy()
    meta = n_pages * H * 2 * D * 4
    res = {"steps": args.extra_steps, "warmup": args.extra_warmup,
           "median_ms": med, "p10_ms": float(np.percentile(step, 10)),
           "p90_ms": float(np.percentile(step, 90)),
           "decode_median_ms": statistics.median(dec),
           "tokens_per_s": B / (med * 1e-3),
           "config": {"batch": B, "kv_heads": H, "group": G, "head_dim": D,
                      "page_size": P, "kv_dtype": spec.kv_dtype, "alpha": alpha,
                      "delta": delta, "selector": "gauss",
                      "seq_lens_after": lens,
                      "append_per_step": appending},
           "selected_pages_last_step": int(cnt.sum()),
           "metadata_bytes": meta}
    log("[bench] %s: median %.1f us per step (%s), %.0f tokens/s" % (
        name, med * 1e3, "with the append" if appending else "Gaussian step",
        res["tokens_per_s"]))
    return {k: (round(v, 5) if isinstance(v, float) else v) for k, v in res.items()}


def _oracle_unit_worker(task):
    """One unit of the Gaussian step by the oracle on one thread, in a
    process of its own: the unit's keys and values come from shared memory
    (float32, exact for bf16 inputs); the time is that of decode_unit."""
    import numpy as np
    from multiprocessing import shared_memory

    from threadpoolctl import threadpool_limits

    import oracle as O
    shm_name, n, D, qs, P, scale, alpha, delta = task
    shm = shared_memory.SharedMemory(name=shm_name)
    try:
        kv = np.ndarray((2, n, D), dtype=np.float32, buffer=shm.buf)
        keys = kv[0].astype(np.float64)
        vals = kv[1].astype(np.float64)
        del kv
    finally:
        shm.close()
    with threadpool_limits(1):
        t0 = time.perf_counter()
        O.decode_unit(qs, keys, vals, P, scale, alpha, "gauss", delta=delta)
        return time.perf_counter() - t0


def cpu_parallel_units(inp, spec, alpha, delta, log):
    """The oracle's Gaussian step with every unit in a process of its own
    (one thread each), all at once: the step takes as long as its slowest
    unit."""
    import multiprocessing as mp
    from multiprocessing import shared_memory

    import numpy as np
    P, G, D = spec.page_size, spec.group, spec.head_dim
    scale = 1.0 / math.sqrt(D)
    units = spec.batch * spec.num_kv_heads
    workers = min(units, len(os.sched_getaffinity(0)))
    shms, tasks = [], []
    try:
        for u in range(units):
            b, h = divmod(u, spec.num_kv_heads)
            n = inp.lens[b]
            rows = inp.page_table[b, :(n + P - 1) // P].long()
            shm = shared_memory.SharedMemory(create=True, size=2 * n * D * 4)
            shms.append(shm)
            kv = np.ndarray((2, n, D), dtype=np.float32, buffer=shm.buf)
            kv[0] = inp.k[rows, h].reshape(-1, D)[:n].float().cpu().numpy()
            kv[1] = inp.v[rows, h].reshape(-1, D)[:n].float().cpu().numpy()
            del kv
            qs = inp.q[b, h * G:(h + 1) * G].double().cpu().numpy()
            tasks.append((shm.name, n, D, qs, P, scale, alpha, delta))
        log("[bench] oracle: %d units in %d processes" % (units, workers))
        t0 = time.perf_counter()
        with mp.get_context("spawn").Pool(workers) as pool:
            dts = pool.map(_oracle_unit_worker, tasks, chunksize=1)
        wall = time.perf_counter() - t0
    except Exception as e:  # no shared memory or no processes on this host
        return {"value": None, "reason": "%s: %s" % (type(e).__name__, e)}
    finally:
        for shm in shms:
            shm.close()
            shm.unlink()
    rounds = (units + workers - 1) // workers
    step = max(dts) * rounds if rounds > 1 else max(dts)
    return {"value": round(spec.batch / step, 6), "unit": "tokens/s",
            "cores": workers,
            "sample": "all %d units of one Gaussian step, one process and one "
                      "thread per unit, fp64 numpy; step time = the slowest "
                      "unit's %.2f s%s (%.1f s from the processes' start to "
                      "the last result)" % (units, max(dts),
                                            " x %d rounds" % rounds if rounds > 1 else "",
                                            wall)}


def cpu_baseline(inp, spec, n_units, alpha, delta, log):
    """Time the fp64 oracle on a bounded sample of the same step."""
    import numpy as np
    import torch

    import oracle as O

    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(1)
    except Exception:  # pragma: no cover - threadpoolctl is installed here
        limiter = None
    P, G, D = spec.page_size, spec.group, spec.head_dim
    scale = 1.0 / math.sqrt(D)
    times = []
    for u in range(n_units):
        b, h = divmod(u, spec.num_kv_heads)
        n = inp.lens[b]
        rows = inp.page_table[b, :(n + P - 1) // P].long()
        keys = inp.k[rows, h].reshape(-1, D)[:n].double().cpu().numpy()
        vals = inp.v[rows, h].reshape(-1, D)[:n].double().cpu().numpy()
        qs = inp.q[b, h * G:(h + 1) * G].double().cpu().numpy()
        log("[bench] oracle unit %d (%d tokens)" % (u, n))
        t0 = time.perf_counter()
        O.decode_unit(qs, keys, vals, P, scale, alpha, "gauss", delta=delta)
        times.append(time.perf_counter() - t0)
        if u == 0:
            qs0, keys0, vals0 = qs, keys, vals
    units_per_step = spec.batch * spec.num_kv_heads

    def rate(per_unit_s):
        return round(spec.batch / (per_unit_s * units_per_step), 6)

    # The same oracle on unit 0 for the full-cache baselines (every token,
    # every query head of the group), still on one thread.
    more = {}
    for kind, fn in (("entmax_full", lambda q: O.entmax_attend(q, keys0, vals0, scale, alpha)),
                     ("softmax_full", lambda q: O.softmax_attend(q, keys0, vals0, scale))):
        log("[bench] oracle %s, unit 0" % kind)
        t0 = time.perf_counter()
        for g in range(G):
            fn(qs0[g])
        dt = time.perf_counter() - t0
        more[kind] = {"value": rate(dt), "unit": "tokens/s", "cores": 1,
                      "sample": "every token of unit 0 for its %d query heads, "
                                "fp64 numpy, %.2f s; step time = that x %d units"
                                % (G, dt, units_per_step)}
    if limiter is not None:
        limiter.restore_original_limits()
    # Unit 0 of the Gaussian step again with numpy free to use every core
    # of this process (the oracle is not parallelised beyond that).
    cores = len(os.sched_getaffinity(0))
    log("[bench] oracle unit 0 on %d cores" % cores)
    t0 = time.perf_counter()
    O.decode_unit(qs0, keys0, vals0, P, scale, alpha, "gauss", delta=delta)
    dt = time.perf_counter() - t0
    more["gauss_all_cores"] = {"value": rate(dt), "unit": "tokens/s",
                               "cores": cores,
                               "sample": "unit 0 of the Gaussian step, numpy "
                                         "free to use every core, %.2f s; step "
                                         "time = that x %d units" % (dt, units_per_step)}
    par = cpu_parallel_units(inp, spec, alpha, delta, log)
    per_unit = statistics.mean(times)
    one_core = {"value": rate(per_unit), "unit": "tokens/s",
                "cores": 1, "kind": "oracle",
                "sample": "%d of %d (sequence, KV head) units of one decode step "
                          "(metadata build, Gaussian scoring, threshold estimate, "
                          "selection, entmax over the kept pages), fp64 numpy, "
                          "%.2f s per unit; step time = per-unit time x %d units"
                          % (n_units, units_per_step, per_unit, units_per_step)}
    # The headline CPU figure: every unit in a process of its own, all at
    # once (the oracle itself unchanged); the one-core figure otherwise.
    if par.get("value") is not None:
        more["gauss_one_core"] = one_core
        par["kind"] = "oracle"
        return par, more
    more["gauss_parallel_units"] = par
    return one_core, more


if __name__ == "__main__":
    main()
