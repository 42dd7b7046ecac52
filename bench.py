"""Throughput of the corrector pass on one GPU.

One step = one corrector_run (top-K, projections, transition scores, walk)
over one batch of synthetic draft blocks already resident in HBM.  The batch
rotates over several independently generated input sets (more logits than
the 256 MB Infinity Cache holds) so the logits stream from HBM.

Prints ONE JSON line: blocks/s, the roofline of the dominant kernel (HIP-event
timed on the launch stream inside this run), and the CPU oracle timed on the
host cores on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "corrected draft blocks/s at batch 32 (V=151936,B=16,K=16); % HBM/MFMA peak"
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
# vector-ALU ceiling for GELU evaluations: the published float32 vector rate
# (157.3 TFLOP/s = 78.6 T lane multiply-adds/s: 256 CUs x 128 lanes x 2.4 GHz),
# at 17 issue slots per evaluation in the MLP's inner loop: 9 single-rate
# instructions (the add of P and Q, 7 for the GELU itself, the w2
# multiply-add) and the two transcendentals v_rcp_f32 and v_exp_f32 at a
# quarter of that rate (4 slots each)
PEAK_GELU_T = 256 * 128 * 2.4e9 / 17 / 1e12   # 4.63 T evaluations/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "draft_correction_amd", "csrc")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """C++ source without its comments and with whitespace runs collapsed:
    what the compiler sees of the code (string and character literals kept)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code (comments and layout ignored): the
    recorded HBM traffic stands while it matches."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(CSRC, name), encoding="utf-8") as f:
                h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


def algorithmic_work(cfg: dict, n: int) -> dict:
    """Bytes a kernel must move and flops it must do, per launch, by definition
    of its step (not counting re-reads): the unit figures times the units one
    launch processes."""
    B, K, V, d, de, r, h = cfg["B"], cfg["K"], cfg["V"], cfg["d"], cfg["de"], cfg["r"], cfg["h"]
    esz = 2 if cfg["logits_dtype"] == "bf16" else 4
    rows, pairs = n * B, n * (B - 1)
    w = {}
    # top-K: every logit of every drafted slot row read once
    w["topk_partial"] = dict(bound="hbm", bytes=rows * V * esz, unit="drafted slot row of V logits",
                             per_unit=V * esz, units=rows)
    w["topk_merge"] = dict(bound="hbm", bytes=rows * K * 8, per_unit=K * 8, units=rows,
                           unit="slot row (K ids + values out)")
    # the fused top-K + normalisation reads the same logits once; its merge
    # also writes log Z and five confidence scalars per candidate
    w["topk_partial_lse"] = dict(w["topk_partial"])
    w["topk_merge_lse"] = dict(bound="hbm", bytes=rows * (K * 8 + 4 + K * 20), per_unit=K * 28 + 4, units=rows,
                               unit="slot row (K ids, values, 5 scalars and log Z out)")
    hn = 3 * r if cfg["variant"] == "mlp" else r
    w["hproj"] = dict(bound="hbm", bytes=rows * d * 2 + hn * d * 2, flops=2 * rows * d * hn,
                      per_unit=d * 2, units=rows, unit="hidden row")
    w["cand_gemm"] = dict(bound="hbm", bytes=rows * K * de * 2 + r * de * 2, flops=2 * rows * K * de * r,
                          per_unit=de * 2, units=rows * K, unit="gathered embedding row")
    # one launch: the gathered candidate projection and the hidden-state
    # projection side by side
    w["proj_gemm"] = dict(bound="hbm", bytes=w["cand_gemm"]["bytes"] + w["hproj"]["bytes"],
                          flops=w["cand_gemm"]["flops"] + w["hproj"]["flops"],
                          per_unit=de * 2, units=rows * K + rows,
                          unit="gathered embedding row or hidden row (d_e = d)")
    # one launch: the top-K merge and the hidden-state projection side by side
    w["topk_merge_hproj"] = dict(bound="hbm", bytes=w["topk_merge"]["bytes"] + w["hproj"]["bytes"],
                                 flops=w["hproj"]["flops"], per_unit=d * 2, units=rows,
                                 unit="slot row (K winners out; hidden row projected)")
    # the candidate kernel reads the split partials of u and writes z (hi | lo)
    w["cand"] = dict(bound="hbm", bytes=rows * K * (r * 4 * 2), flops=2 * rows * K * 2 * r * r,
                     per_unit=r * 8, units=rows * K, unit="candidate (u in; z out)")
    w["finish"] = w["finish_walk"] = w["finish_viterbi"] = w["finish_beam"] = dict(bound="hbm", bytes=n * (B - 1) * K * K * 4 * 2,
                                          per_unit=(B - 1) * K * K * 8, units=n, unit="block")
    # the transition MLP epilogue is bound by the vector ALU: K m h GELU
    # evaluations per pair (m = K unless sparsified; 17 VALU issue slots each)
    # against 256 CUs x 64 lanes x 2.4 GHz
    ms = cfg.get("succ_top_m", 0)
    ms = ms if 0 < ms < K else K   # successors scored per predecessor
    # (its prologue also forms U = W1_za z and V = W1_zb z of the pair's
    # candidates on MFMA: 2 K h r multiply-adds per pair, small next to these)
    w["mlp"] = dict(bound="alu", gelu=pairs * K * ms * h, flops=2 * pairs * K * ms * h,
                    per_unit=h, units=pairs * K * ms, unit="transition (h GELU evaluations)")
    # few pairs: the finishing step and the walk run in the MLP's launch
    w["mlp_walk"] = dict(w["mlp"])
    w["cosine"] = w["cosine_walk"] = w["cosine_viterbi"] = w["cosine_beam"] = dict(
        bound="hbm", bytes=pairs * 2 * K * cfg["dvec"] * 4, per_unit=2 * K * cfg["dvec"] * 4, units=pairs, unit="pair")
    w["walk"] = dict(bound="hbm", bytes=n * (B - 1) * K * 4, per_unit=(B - 1) * K * 4, units=n,
                     unit="block (scores rows read)")
    # the Global-Sum path reads every score of the block once
    w["viterbi"] = w["beam"] = dict(bound="hbm", bytes=n * (B - 1) * K * K * 4, per_unit=(B - 1) * K * K * 4, units=n,
                        unit="block (all scores read)")
    return w


def measure_topk_softmax(corr, cfg, dev_sets, host_logits, st, stream, steps, warmup, cpu=True) -> dict:
    """corrector_topk_softmax (with the confidence scalars) over the same
    rotated logits, beside plain corrector_topk; the partial kernel's HBM rate
    against the peak; the oracle (top-K, log Z and scalars) on one batch."""
    import torch
    n, B, K = cfg["n"], cfg["B"], cfg["K"]
    ids = torch.empty((n, B, K), dtype=torch.int32, device="cuda")
    vals = torch.empty((n, B, K), dtype=torch.float32, device="cuda")
    logz = torch.empty((n, B), dtype=torch.float32, device="cuda")
    conf = torch.empty((n, B, K, 5), dtype=torch.float32, device="cuda")
    ws = corr.new_workspace(n)

    def fused(i):
        corr.topk_softmax(n, dev_sets[i % len(dev_sets)]["logits"], st["l_req"], st["l_slot"], ids, vals, logz, ws,
                          conf=conf, offset=st["l_off"], stream=stream)

    def plain(i):
        corr.topk(n, dev_sets[i % len(dev_sets)]["logits"], st["l_req"], st["l_slot"], ids, vals, ws,
                  offset=st["l_off"], stream=stream)

    out = {}
    for name, fn in (("fused", fused), ("topk_only", plain)):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(steps):
            fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        corr.set_timing(True)
        per = {}
        for i in range(steps):
            fn(i)
            for k, t in corr.kernel_times():
                per.setdefault(k, []).append(t)
        corr.set_timing(False)
        torch.cuda.synchronize()
        out[name] = dict(us=round(ms * 1e3, 3), kernels_us={k: round(float(np.mean(v)) * 1e3, 3)
                                                            for k, v in per.items()})
    work = algorithmic_work(cfg, n)["topk_partial_lse"]
    t = out["fused"]["kernels_us"]["topk_partial_lse"] / 1e6
    gbs = work["bytes"] / t / 1e9
    res = {"value": round(n * B / (out["fused"]["us"] / 1e6), 1), "unit": "slot rows/s",
           "call": "corrector_topk_softmax (ids, values, log Z, 5 scalars per candidate)",
           "us": out["fused"]["us"], "kernels_us": out["fused"]["kernels_us"],
           "topk_only_us": out["topk_only"]["us"],
           "roofline": {"bound": "hbm", "kernel": "topk_partial_lse", "achieved": round(gbs, 1),
                        "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)}}
    if cpu:
        import oracle
        oracle.build(force=False)
        d = oracle.OracleDesc.from_config(cfg)
        V = cfg["V"]
        t0, reps = time.perf_counter(), 0
        while True:
            _, ov = oracle.topk(d, host_logits, n, (B + 1) * V, V, offset=V)
            oz = oracle.log_normaliser(d, host_logits, n, (B + 1) * V, V, offset=V)
            oracle.confidence(ov, oz)
            reps += 1
            el = time.perf_counter() - t0
            if el >= 5.0 or reps >= 64:
                break
        res["cpu_baseline"] = {"value": round(reps * n * B / el, 1), "unit": "slot rows/s",
                               "cores": oracle.get_threads(), "kind": "oracle",
                               "sample": "%d pass(es) over one %d-row batch: full-sort top-K, log Z and scalars "
                                         "(%.1f s)" % (reps, n * B, el)}
    return res


def measure_ceilings(steps: int = 20) -> dict:
    """The box's own reference ceilings: a large device-to-device copy (HBM
    read + write) and a large bf16 matrix product through PyTorch's library
    GEMM (MFMA).  Context for the roofline fractions, not part of the path."""
    import torch
    out = {}
    nb = 2 << 30
    src = torch.empty(nb, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    t = a.elapsed_time(b) / steps / 1e3
    out["copy"] = {"bytes": 2 * nb, "us": round(t * 1e6, 1), "GB/s": round(2 * nb / t / 1e9, 1),
                   "what": "torch copy_ of 2 GiB (read + write)"}
    del src, dst
    n = 8192
    x = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    y = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    for _ in range(3):
        torch.matmul(x, y)
    torch.cuda.synchronize()
    a.record()
    for _ in range(steps):
        torch.matmul(x, y)
    b.record()
    torch.cuda.synchronize()
    t = a.elapsed_time(b) / steps / 1e3
    out["gemm_bf16"] = {"flops": 2 * n ** 3, "us": round(t * 1e6, 1), "TFLOP/s": round(2 * n ** 3 / t / 1e12, 1),
                        "what": "torch.matmul bf16 8192 x 8192 x 8192"}
    return out


def _median_pass_seconds(cfg, inputs, n: int, reps: int = 3) -> float:
    import oracle
    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        oracle.run(cfg, inputs, n=n)
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts))


def cpu_baseline(cfg, inputs, single_blocks: int = 4) -> dict:
    """The CPU oracle on the host cores: the median of 3 full passes over the
    batch with every OpenMP thread, and the median of 3 passes over its first
    `single_blocks` blocks with one thread (the oracle's cost is linear in the
    blocks of a pass)."""
    import oracle
    oracle.build(force=False)
    threads = oracle.get_threads()
    n = cfg["n"]
    t_all = _median_pass_seconds(cfg, inputs, n)
    oracle.set_threads(1)
    try:
        ns = min(single_blocks, n)
        t_one = _median_pass_seconds(cfg, inputs, ns)
    finally:
        oracle.set_threads(threads)
    cpu = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": n / t_all, "unit": "blocks/s", "cores": threads, "kind": "oracle",
            "sample": "median of 3 full passes of the CPU oracle over one %d-block batch of the same workload "
                      "(%.2f s each, %d OpenMP threads)" % (n, t_all, threads),
            "single_thread": {"value": round(ns / t_one, 3), "unit": "blocks/s", "cores": 1,
                              "sample": "median of 3 passes over the first %d blocks of the batch, one thread "
                                        "(%.2f s each)" % (ns, t_one)},
            "cpu_model": cpu}


def measure_pass(corr, cfg, dev_sets, st, stream, steps: int, warmup: int) -> dict:
    """Back-to-back corrector_run passes over the rotated input sets: the
    pass time over exactly `steps` passes (HIP events around the whole
    region), then per-kernel durations from the library's kernel-stamped
    events over the same number of passes."""
    import torch
    n, B = cfg["n"], cfg["B"]
    tokens = torch.empty((n, B), dtype=torch.int32, device="cuda")
    ws = corr.new_workspace(n)

    def step(i):
        s = dev_sets[i % len(dev_sets)]
        corr.run(n, s["logits"], st["l_req"], st["l_slot"], s["hidden"], st["h_req"], st["h_slot"],
                 tokens, ws, l_offset=st["l_off"], h_offset=st["h_off"], stream=stream)

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
    corr.set_timing(True)
    per = {}
    for i in range(steps):
        step(i)
        for name, t in corr.kernel_times():
            per.setdefault(name, []).append(t)
    corr.set_timing(False)
    torch.cuda.synchronize()
    return {"ms": ms, "kernels_ms": {k: float(np.mean(v)) for k, v in per.items()}}


def measure_graph(corr, cfg, dev_sets, st, stream, steps: int, warmup: int) -> dict:
    """The same pass captured into graphs (one per rotated input set, each
    capturing one corrector_run on that set's buffers) and replayed `steps`
    times back to back: the pass time without per-launch host work."""
    import torch
    n, B = cfg["n"], cfg["B"]
    tokens = torch.empty((n, B), dtype=torch.int32, device="cuda")
    ws = corr.new_workspace(n)
    s0 = dev_sets[0]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        corr.run(n, s0["logits"], st["l_req"], st["l_slot"], s0["hidden"], st["h_req"], st["h_slot"], tokens, ws,
                 l_offset=st["l_off"], h_offset=st["h_off"], stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for s in dev_sets:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            corr.run(n, s["logits"], st["l_req"], st["l_slot"], s["hidden"], st["h_req"], st["h_slot"], tokens, ws,
                     l_offset=st["l_off"], h_offset=st["h_off"])
        graphs.append(g)
    torch.cuda.synchronize()
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(cur)
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    e1.record(cur)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del graphs
    return {"us": round(ms * 1e3, 3), "value": round(n / (ms / 1e3), 1),
            "note": "one graph per rotated input set, each capturing one corrector_run; replays back to back"}


def roofline_of(work: dict, name: str, ms: float, traffic=None) -> dict:
    wk = work[name]
    t_s = ms / 1e3
    if wk["bound"] == "mfma":
        achieved, peak, unit = wk["flops"] / t_s / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    elif wk["bound"] == "alu":
        achieved, peak, unit = wk["gelu"] / t_s / 1e12, PEAK_GELU_T, "T GELU/s"
    else:
        achieved, peak, unit = wk["bytes"] / t_s / 1e9, PEAK_HBM_GBS, "GB/s"
    return {"bound": wk["bound"], "achieved": round(achieved, 2), "peak": round(peak, 3), "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": name, "kernel_us": round(ms * 1e3, 3)}


def kernel_table(work: dict, kms: dict) -> dict:
    kernels = {}
    for k, v in kms.items():
        wkk = work.get(k, {})
        ent = {"us": round(v * 1e3, 3)}
        if "bytes" in wkk:
            ent["GB/s"] = round(wkk["bytes"] / (v / 1e3) / 1e9, 1)
        if "flops" in wkk:
            ent["TFLOP/s"] = round(wkk["flops"] / (v / 1e3) / 1e12, 2)
        if "gelu" in wkk:
            ent["T GELU/s"] = round(wkk["gelu"] / (v / 1e3) / 1e12, 3)
        kernels[k] = ent
    return kernels


def load_workload(name: str, copies: int, args, head: str):
    """Synthetic inputs of a named workload (several independent input sets),
    weights and the embedding table, on the device."""
    from draft_correction_amd import device
    from workload import config
    from workload.gen import gen_embed, gen_hidden, gen_logits, gen_weights
    cfg = config(name, path_rule=args.path_rule, path_lambda=args.path_lambda, beam_width=args.beam_width,
                 succ_top_m=args.top_m)
    t0 = time.perf_counter()
    embed = gen_embed(cfg)
    weights = gen_weights(cfg, head=head)
    sets = []
    for c in range(copies):
        cc = dict(cfg, seed=c)
        sets.append(dict(logits=gen_logits(cc), hidden=gen_hidden(cc)))
    log("generated %s inputs (%d copies) in %.1f s" % (name, copies, time.perf_counter() - t0))
    dev_w = device.weights_to_device(weights, embed)
    dev_sets = [dict(logits=device.tensor(s["logits"]), hidden=device.tensor(s["hidden"])) for s in sets]
    corr = device.make_corrector(cfg, dict(weights=dev_w), max_requests=cfg["n"])
    return cfg, corr, dev_sets, sets, weights, embed, dev_w


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="b32")
    ap.add_argument("--copies", type=int, default=4, help="independent input sets rotated per step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--head", default="normal")
    ap.add_argument("--path-rule", default="greedy", choices=["greedy", "global_sum", "geometric", "beam"],
                    help="how the path through the candidate lattice is chosen")
    ap.add_argument("--path-lambda", type=float, default=0.75, help="lambda of the Geometric path rule")
    ap.add_argument("--beam-width", type=int, default=4, help="width of the beam path rule (1..4)")
    ap.add_argument("--top-m", type=int, default=0,
                    help="score only the first m successors of each predecessor (0: all K)")
    ap.add_argument("--no-fold", action="store_true", help="skip the folded-table measurement")
    ap.add_argument("--no-b1", action="store_true", help="skip the batch-1 measurement")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-replay measurements")
    ap.add_argument("--ceilings", action="store_true",
                    help="also measure the box's copy and large-GEMM ceilings (reference figures)")
    ap.add_argument("--no-softmax", action="store_true",
                    help="skip the fused top-K + normalisation measurement")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="first run a plain device copy of this many MiB (a known-size reference "
                         "for hardware traffic counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(requests shard across GPUs with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    from draft_correction_amd import device

    torch.cuda.set_device(0)
    cfg, corr, dev_sets, sets, weights, embed, dev_w = load_workload(args.workload, args.copies, args, args.head)
    n, B, K = cfg["n"], cfg["B"], cfg["K"]
    st = device.strides(cfg)
    stream = torch.cuda.current_stream()

    if args.calibrate_copy:
        nb = args.calibrate_copy << 20
        src = torch.empty(nb, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: %d bytes read, %d bytes written" % (nb, nb))
        del src, dst

    # ---- timed region: exactly `steps` passes, then per-kernel durations
    # (HIP events stamped by the library around each of its launches, on the
    # same stream, over the same number of passes)
    main_pass = measure_pass(corr, cfg, dev_sets, st, stream, args.steps, args.warmup)
    ms, avg = main_pass["ms"], main_pass["kernels_ms"]
    log("pass: %.2f us (%d steps)" % (ms * 1e3, args.steps))
    for k, v in avg.items():
        log("  %-16s %8.2f us" % (k, v * 1e3))

    graph = None
    if not args.no_graph:
        graph = measure_graph(corr, cfg, dev_sets, st, stream, args.steps, args.warmup)
        log("graph-replayed pass: %.2f us" % graph["us"])

    # ---- the same pass with the folded candidate projection (E W_cand^T
    # tabulated once; the table is computed outside the timed region)
    folded = None
    if not args.no_fold:
        table = torch.empty(corr.table_bytes() // 4, dtype=torch.float32, device="cuda")
        corr.fold_table(table, stream=stream)
        corr.use_table(table)
        fp = measure_pass(corr, cfg, dev_sets, st, stream, args.steps, args.warmup)
        corr.use_table(None)
        torch.cuda.synchronize()
        folded = {"value": round(n / (fp["ms"] / 1e3), 1), "ms_per_step": round(fp["ms"], 5),
                  "kernels_us": {k: round(v * 1e3, 3) for k, v in fp["kernels_ms"].items()},
                  "note": "candidate projection gathers rows of the folded table E W_cand^T "
                          "(computed once, outside the timed region)"}
        log("folded pass: %.2f us" % (fp["ms"] * 1e3))
        del table

    fused_softmax = None
    if not args.no_softmax:
        fused_softmax = measure_topk_softmax(corr, cfg, dev_sets, sets[0]["logits"], st, stream, args.steps,
                                             args.warmup, cpu=not args.no_cpu_baseline)
        log("fused top-K + normalisation: %.2f us (top-K alone %.2f us)"
            % (fused_softmax["us"], fused_softmax["topk_only_us"]))

    work = algorithmic_work(cfg, n)
    dom = max(avg, key=avg.get)
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        ent = tr.get("kernels", {}).get(dom)
        if ent and tr.get("source_hash") == kernel_source_hash() and tr.get("workload") == args.workload:
            traffic = ent.get("bytes_per_launch")
    roof = roofline_of(work, dom, avg[dom], traffic)
    mk = "mlp" if "mlp" in avg else ("mlp_walk" if "mlp_walk" in avg else None)
    roof_mlp = roofline_of(work, mk, avg[mk]) if mk else None
    kernels = kernel_table(work, avg)

    # ---- batch 1 (the pages' concurrency-1 serving point), same run
    b1 = None
    if not args.no_b1 and args.workload != "b1":
        del dev_sets
        torch.cuda.empty_cache()
        cfg1, corr1, dev1, _, _, _, _ = load_workload("b1", args.copies, args, args.head)
        st1 = device.strides(cfg1)
        p1 = measure_pass(corr1, cfg1, dev1, st1, stream, args.steps, args.warmup)
        work1 = algorithmic_work(cfg1, 1)
        b1 = {"value": round(1 / (p1["ms"] / 1e3), 1), "unit": "blocks/s", "ms_per_step": round(p1["ms"], 5),
              "us": round(p1["ms"] * 1e3, 3), "kernels": kernel_table(work1, p1["kernels_ms"]),
              "config": {"workload": "b1: 1 request x %d drafted slots (+anchor), V=%d, K=%d, d=%d, r=%d"
                                     % (cfg1["B"], cfg1["V"], cfg1["K"], cfg1["d"], cfg1["r"])}}
        log("b1 pass: %.2f us" % b1["us"])
        if not args.no_graph:
            b1["graph"] = measure_graph(corr1, cfg1, dev1, st1, stream, args.steps, args.warmup)
            log("b1 graph-replayed pass: %.2f us" % b1["graph"]["us"])
        corr1.close()
        del dev1

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        inputs = dict(cfg=cfg, logits=sets[0]["logits"], hidden=sets[0]["hidden"], weights=weights,
                      embed=embed)
        cpu = cpu_baseline(cfg, inputs)

    out = {
        "metric": METRIC,
        "value": round(n / (ms / 1e3), 1),
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%s: %d requests x %d drafted slots (+anchor), V=%d, K=%d, d=%d, r=%d, "
                               "MLP %d->%d->1, %s" % (args.workload, n, B, cfg["V"], K, cfg["d"],
                                                      cfg["r"], 3 * cfg["r"] + 2, cfg["h"], cfg["variant"])
                               + {"greedy": "", "global_sum": ", Global-Sum path",
                                  "geometric": ", Geometric path (lambda %g)" % args.path_lambda,
                                  "beam": ", beam path (width %d)" % args.beam_width}[args.path_rule]
                               + (", top-%d successors scored" % args.top_m if 0 < args.top_m < cfg["K"] else ""),
                   "global_batch": n, "rotating_input_sets": args.copies},
        "roofline": roof,
        "roofline_mlp": roof_mlp,
        "kernels": kernels,
        "cpu_baseline": cpu,
        "b1": b1,
        "graph": graph,
        "folded_table": folded,
        "fused_softmax": fused_softmax,
    }
    if args.ceilings:
        out["ceilings"] = measure_ceilings()
        log("ceilings: %s" % json.dumps(out["ceilings"]))
    print(json.dumps(out), flush=True)
    corr.close()


if __name__ == "__main__":
    main()
