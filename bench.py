#!/usr/bin/env python3
"""Throughput of the causal token-block MXFP8 attention training call on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic packed input already
resident in HBM: quantise Q, K, V -> forward -> quantise dO (+ D) -> backward.  The work lists
are built once per micro-batch (jaehun.me review §3.4) and are timed separately.

value = algorithmic FLOP per step / step time, with the causal FLOP count
14 * d * Hq * sum_docs L (L + 1) / 2 (forward 4d, backward 10d per visible query-key pair);
--non-causal times the non-causal variant instead (14 * d * Hq * sum_docs L^2).

Prints one JSON line.  Extra objects: `roofline` (dominant kernel vs the MI355X dense FP8
peak, timed with HIP events on the launch stream), `quantize` (HBM roofline of the quantiser
passes), `stages_ms`, `worklist_ms`, and `cpu_baseline` (the CPU oracle on a bounded sample
of the same workload).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal MXFP8 attn fwd+bwd TFLOPS incl. quantize; % of MI355X MXFP8 peak"
METRIC_NC = "non-causal MXFP8 attn fwd+bwd TFLOPS incl. quantize; % of MI355X MXFP8 peak"
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense FP8 / MXFP8 matrix peak
PEAK_HBM_GBPS = 8000.0       # MI355X HBM3E

# HBM bytes per flamia_bwd call (prologue, small-document pass, key-tile + dQ kernels) on the
# `long` workload, from the FETCH_SIZE / WRITE_SIZE passes summarised in
# profiles/flamia_long_hbm_traffic.md (FETCH scaled by 2.000 and WRITE by 1.000, the factors a
# 1 GiB copy gives).  Valid only for the backward sources it was measured on (sha256 prefix over
# attn_bwd.hip, attn_small.hip, device_common.h, kernels.h); any other build reports null.
BWD_TRAFFIC = {"workload": "long", "src": "9cafb9f6f4e63e8a", "read_bytes": 18.116e9, "write_bytes": 13.033e9}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long")
    ap.add_argument("--causal-dq", action="store_true", help="causal dQ prescale option")
    ap.add_argument("--non-causal", action="store_true",
                    help="time the non-causal variant (every key of a row's document visible)")
    ap.add_argument("--hadamard", action="store_true",
                    help="rotate Q and K by H / sqrt(d) in the quantiser, dQ and dK back in the backward")
    ap.add_argument("--qk4", action="store_true",
                    help="time the 4-bit score path (MXFP4 copy of Q and K, log-domain probability operand)")
    ap.add_argument("--precise", action="store_true",
                    help="time the precision options (per-token scales, folded exponents, row-wise dS exponents)")
    ap.add_argument("--store-gb", type=float, default=None,
                    help="cap the backward's dShat store at this many GiB (chunked backward); default: one chunk")
    ap.add_argument("--cpu-pairs", type=float, default=1.5e8,
                    help="query-key pairs (summed over heads) in the CPU-oracle sample")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one step captured in a HIP graph (stage times from eager steps after "
                         "the timed region)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibration-copy-mb", type=int, default=0,
                    help="before warmup, run one plain device-to-device copy of this many MiB (reference "
                         "kernel of known traffic for hardware byte counters)")
    return ap.parse_args()


def bwd_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in ("attn_bwd.hip", "attn_small.hip", "device_common.h", "kernels.h"):
        with open(os.path.join(ROOT, "precision_causal_attention_token_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or the platform's processor string."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(workload_name, pairs_budget):
    """Time the oracle (test infrastructure, untuned) on a bounded sample: documents of the
    workload in order, each truncated to 4096 tokens, until pairs_budget query-key pairs per
    head are covered; then the query heads of the first KV heads, whole groups, until
    pairs_budget pairs in all (or every head)."""
    import numpy as np
    import torch

    import oracle
    from precision_causal_attention_token_amd import workloads

    cu, shp, (q, k, v, do) = workloads.workload(workload_name)
    lens, spans, pairs = [], [], 0
    for a, b in zip(cu[:-1], cu[1:]):
        L = min(int(b - a), 4096)
        if L <= 0:
            continue
        lens.append(L)
        spans.append((int(a), int(a) + L))
        pairs += L * (L + 1) // 2
        if pairs >= pairs_budget:
            break
    idx = np.concatenate([np.arange(a, b) for a, b in spans])
    cs = workloads.cu_seqlens(lens)
    grp = shp.Hq // shp.Hkv
    n_kv = min(shp.Hkv, max(1, -(-int(pairs_budget) // (pairs * grp))))
    n_q = n_kv * grp

    def bits(x, nh):
        return x[idx][:, :nh].contiguous().view(torch.int16).numpy().view(np.uint16)

    oracle.lib()
    t0 = time.perf_counter()
    qc = [oracle.quantize(bits(x, nh), cs) for x, nh in ((q, n_q), (k, n_kv), (v, n_kv))]
    o, lse, _ = oracle.fwd(*qc[0], *qc[1], *qc[2], cs)
    dc, dsc, D = oracle.quantize_do(bits(do, n_q), o, cs)
    oracle.bwd(*qc[0], *qc[1], *qc[2], dc, dsc, lse, D, cs)
    dt = time.perf_counter() - t0
    flop = 14.0 * shp.d * n_q * pairs
    return {"value": flop / dt / 1e12, "unit": "TFLOPS", "cores": oracle.num_threads(), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": "%s workload: first %d documents (each truncated to 4096 tokens, %d tokens), query heads "
                      "0..%d (KV heads 0..%d), %d query-key pairs per head; quantise + forward + dO pass + "
                      "backward in %.2f s" % (workload_name, len(lens), len(idx), n_q - 1, n_kv - 1, pairs, dt),
            "seconds": dt}


def main():
    args = parse()
    if args.non_causal and args.causal_dq:
        print("bench.py: the causal dQ prescale applies to causal attention only", file=sys.stderr)
        sys.exit(2)
    if args.precise and (args.non_causal or args.hadamard or args.qk4):
        print("bench.py: the precision options are timed alone on causal attention", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1:
        print("bench.py measures one GPU: the path has no multi-GPU component (--gpus %d refused)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import precision_causal_attention_token_amd as fl
    from precision_causal_attention_token_amd import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cu, shp, (q, k, v, do) = workloads.workload(args.workload)
    T, Hq, Hkv, d = shp.T, shp.Hq, shp.Hkv, shp.d
    causal = not args.non_causal
    pairs = workloads.visible_pairs(cu, causal)
    flop = 14.0 * d * Hq * pairs
    q, k, v, do = (x.to(dev) for x in (q, k, v, do))
    cu_d = torch.as_tensor(cu).to(dev)
    print("bench: workload %s T=%d Hq=%d Hkv=%d d=%d docs=%d pairs=%d" % (args.workload, T, Hq, Hkv, d,
                                                                          len(cu) - 1, pairs), file=sys.stderr,
          flush=True)

    # work lists: built once per micro-batch, timed on their own
    ev = lambda: torch.cuda.Event(enable_timing=True)
    wl_ms = []
    for _ in range(5):
        e0, e1 = ev(), ev()
        e0.record()
        lists = fl.Lists(cu_d, T, causal)
        e1.record()
        torch.cuda.synchronize()
        wl_ms.append(e0.elapsed_time(e1))
    # backward workspace: one key-tile chunk for this micro-batch's documents (sized from the
    # lengths the data loader holds on the host; --store-gb caps the store instead)
    if args.precise:  # nothing is stored: the smallest workspace
        ws_bytes = fl.bwd_workspace_bytes(len(cu) - 1, T, Hq, d, 0)
    elif args.store_gb is None:
        ws_bytes = fl.bwd_workspace_bytes_for(cu, T, Hq, d, causal)
    else:
        ws_bytes = fl.bwd_workspace_bytes(len(cu) - 1, T, Hq, d, int(args.store_gb * (1 << 30)))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    # the longest document, from the same host lengths: the backward launches its key-tile chunks
    # for documents no longer than this
    max_doc_len = int(np.max(np.diff(cu))) if len(cu) > 1 else 0

    stage_names = ("quantize_qkv", "fwd", "quantize_do", "bwd")

    def step(evs=None):
        if evs: evs[0].record()
        qz, kz, vz = fl.quantize([q, k, v], cu_d, hadamard=(args.hadamard, args.hadamard, False),
                                 per_token=args.precise, mx4=(args.qk4, args.qk4, False))
        if evs: evs[1].record()
        o, lse = fl.fwd(qz, kz, vz, cu_d, lists.fwd, causal=causal, precise=args.precise, qk4=args.qk4)
        if evs: evs[2].record()
        dc, dsc, D = fl.quantize_do(do, o, cu_d, per_token=args.precise)
        if evs: evs[3].record()
        out = fl.bwd(qz, kz, vz, (dc, dsc), lse, D, cu_d, lists, None, args.causal_dq, workspace=ws, causal=causal,
                     hadamard=args.hadamard, precise=args.precise, qk4=args.qk4, max_doc_len=max_doc_len)
        if evs: evs[4].record()
        return out

    if args.calibration_copy_mb > 0:
        n = args.calibration_copy_mb << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print("bench: calibration copy of %d bytes done" % n, file=sys.stderr, flush=True)
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    status, chunks = fl.bwd_status(ws)
    assert status == 0
    graph = None
    if args.graph:  # one step captured on a side stream's graph, after one call there
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()

    # timed region: exactly K steps, bracketed by device synchronisation
    all_evs = [[ev() for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            step(all_evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    if graph is not None:  # stage times: the same number of eager steps, after the timed region
        for i in range(args.steps):
            step(all_evs[i])
        torch.cuda.synchronize()
    stages = {nm: float(np.median([e[j].elapsed_time(e[j + 1]) for e in all_evs])) for j, nm in enumerate(stage_names)}
    assert fl.bwd_status(ws)[0] == 0

    value = flop / (ms_per_step * 1e-3) / 1e12
    fwd_flop, bwd_flop = 4.0 * d * Hq * pairs, 10.0 * d * Hq * pairs
    dom = "bwd" if stages["bwd"] >= stages["fwd"] else "fwd"
    dom_flop = bwd_flop if dom == "bwd" else fwd_flop
    achieved = dom_flop / (stages[dom] * 1e-3) / 1e12
    traffic = None
    if (dom == "bwd" and causal and not args.hadamard and not args.precise and not args.qk4
            and args.workload == BWD_TRAFFIC["workload"]
            and bwd_source_hash() == BWD_TRAFFIC["src"]):
        traffic = BWD_TRAFFIC["read_bytes"] + BWD_TRAFFIC["write_bytes"]
    roofline = {"bound": "mfma",
                "kernel": ("flamia_bwd (bwd_prologue + bwd_kernel + %s)" % ("dqp_kernel" if args.precise else "dq_kernel")
                           if dom == "bwd" else "flamia_fwd"),
                "achieved": achieved, "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_FP8_TFLOPS,
                "traffic": traffic, "traffic_unit": "bytes per launch"}
    n_qkv = T * (Hq + 2 * Hkv) * d
    qkv_bytes = 3 * n_qkv + T * (Hq + 2 * Hkv)
    if args.qk4:  # the 4-bit copies of Q and K: d/2 code bytes and d/32 exponent bytes per row
        qkv_bytes += T * (Hq + Hkv) * (d // 2 + d // 32)
    do_bytes = 5 * T * Hq * d + 5 * T * Hq
    quant = {"qkv_GBps": qkv_bytes / (stages["quantize_qkv"] * 1e-3) / 1e9,
             "do_GBps": do_bytes / (stages["quantize_do"] * 1e-3) / 1e9, "peak_GBps": PEAK_HBM_GBPS}
    quant["qkv_frac"] = quant["qkv_GBps"] / PEAK_HBM_GBPS
    quant["do_frac"] = quant["do_GBps"] / PEAK_HBM_GBPS

    res = {
        "metric": METRIC if causal else METRIC_NC, "value": value, "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "mxfp8_e4m3", "data": "synthetic",
        "config": {"workload": args.workload, "T": T, "Hq": Hq, "Hkv": Hkv, "d": d, "docs": len(cu) - 1,
                   "visible_pairs": pairs, "flop_per_step": flop, "causal_dq_scale": bool(args.causal_dq),
                   "causal": causal, "hadamard": bool(args.hadamard), "precise": bool(args.precise),
                   "qk4": bool(args.qk4), "graph": bool(args.graph)},
        "frac_of_peak": value / PEAK_FP8_TFLOPS,
        "roofline": roofline,
        "quantize": quant,
        "stages_ms": stages,
        "worklist_ms": float(np.median(wl_ms)),
        "peak_mem_GB": torch.cuda.max_memory_allocated() / 1e9,
        "bwd_workspace_GB": ws_bytes / 1e9, "bwd_chunks": chunks,
    }
    if not args.no_cpu_baseline and causal and not args.hadamard and not args.precise and not args.qk4:
        res["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_pairs)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
