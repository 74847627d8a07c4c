"""Benchmark of the k8v4 decode step on one MI355X.

One step = one decode step of one layer at 64K context: quantize-and-append
the new token's key/value (32 query / 8 kv heads, D 128, bf16) and attend the
65536 cached tokens with the single bf16 query token.  Steps rotate over
distinct layer caches whose total size exceeds 4 x 256 MiB (the MI355X
last-level cache), so every step streams its cache from HBM.  After W eager
warm-up steps, exactly K steps are captured in one HIP graph; one untimed
replay is checked against the eager result, and one replay is timed with
HIP events on the stream it runs on.

Prints one JSON line.  ``value`` is the achieved algorithmic HBM bandwidth of
the whole step (GB/s); ``tok_s_per_layer`` is query tokens per second per
layer; ``roofline`` reports the attention launch alone (a K-launch graph of
it, timed the same way); ``probe`` streams the same page-head blocks with no
compute (q8k4v_hbm_probe) and a contiguous buffer (q8k4v_stream_probe):
what the memory system gives this access pattern, the attention launch's
practical ceiling; ``cpu_baseline`` times the CPU oracle on the same
workload (a bounded number of steps).

    python bench.py [--steps K] [--warmup W] [--workload NAME|all] [--no-cpu-baseline]
    python bench.py --cpu-report       # the oracle on every workload, default BLAS pool and one thread
    python bench.py --tune             # tune_select first, gated by the stored oracle references
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

HBM_PEAK_GBS = 8000.0
LLC_BYTES = 256 << 20
WORKLOADS = ["tiny_decode_256", "gqa_decode_4096", "gqa_decode_65536", "verify_65536_w8", "multi_session_16x32768"]
LONG_WORKLOADS = ["gqa_decode_131072", "gqa_decode_200000", "verify_131072_w8", "verify_200000_w8",
                  "multi_session_16x32768_prefix", "multi_session_16_suffixes", "batch_decode_16x4096"]
TUNE_REFS = os.path.join(ROOT, "tests", "golden", "tune_refs_32q8kv_d128_w8.npz")
TUNE_SESSION_REFS = os.path.join(ROOT, "tests", "golden", "tune_refs_32q4kv_d128_s16.npz")
MAX_LAYERS = 512


def cache_bytes_per_token_head(D: int, affine: bool = False) -> int:
    # key codes D + key scale 2 + value codes D/2 + value scales 2*D/32
    # (+ key zero point 1 + value zero points D/32 with the affine codec)
    return D + 2 + D // 2 + 2 * (D // 32) + ((1 + D // 32) if affine else 0)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="gqa_decode_65536", choices=WORKLOADS + LONG_WORKLOADS + ["all"],
                    help="all: one JSON line per workload (attention launches, no CPU baseline)")
    ap.add_argument("--layers", type=int, default=0, help="rotating layer caches (0: enough for 4x LLC)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--cpu-steps", type=int, default=20)
    ap.add_argument("--tune", action="store_true",
                    help="run tune_select first (oracle gate from the stored references) and use its choice")
    ap.add_argument("--tune-budget-ms", type=int, default=60000)
    ap.add_argument("--tune-report", default="", help="write tune_select's JSON report to this file")
    ap.add_argument("--config", default="", help="JSON dict of launch config fields")
    ap.add_argument("--kernel-only", action="store_true", help="time only the attention launches (profiling)")
    ap.add_argument("--contiguous-pages", action="store_true", help="identity page table (profiling)")
    ap.add_argument("--codec", default="symmetric", choices=["symmetric", "affine"],
                    help="cache codec (affine: unsigned codes with zero points)")
    ap.add_argument("--separate-append", action="store_true",
                    help="decode steps: the append kernel, then the attention launch")
    ap.add_argument("--no-cascade", action="store_true",
                    help="shared-prefix workload: plain decode instead of the prefix cascade")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run device-to-device copies of MIB MiB (counter calibration) and exit")
    ap.add_argument("--cpu-report", action="store_true",
                    help="only time the CPU oracle on every workload (no GPU) and exit")
    return ap.parse_args()


def main() -> int:
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU (--gpus must be 1): across GPUs the path "
                                   "would shard by kv head or by session, with no communication, and no "
                                   "multi-GPU figure is measured"}))
        return 2
    if args.cpu_report:
        return cpu_report()
    import torch

    import decode_attention_quantized_kv_amd as q8
    import workloads

    if args.copy_calibration:
        return copy_calibration(torch, args.copy_calibration)
    q8.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    cfg = q8.make_config(**json.loads(args.config)) if args.config else None
    tuned = None
    if args.tune:
        # the multi-session workload (32 q / 4 kv heads) tunes with its
        # session unit; the others at 32 q / 8 kv heads
        sessions = args.workload == "multi_session_16x32768"
        dcfg, vcfg, mcfg, rep = run_tuner(torch, q8, workloads, args.tune_budget_ms, sessions)
        if args.tune_report:
            with open(args.tune_report, "w") as f:
                json.dump(rep, f)
        w0 = workloads.NAMED[args.workload if args.workload != "all" else "gqa_decode_65536"]()
        cfg = mcfg if sessions else vcfg if w0.n_draft else dcfg
        tuned = {"decode": dcfg.as_dict(), "verify": vcfg.as_dict(),
                 "status": rep.get("status"), "units": [{k: u.get(k) for k in
                                                          ("unit", "qualified", "chosen_cost", "oracle_gate",
                                                           "admitted", "rejected", "rejected_by", "invalid")}
                                                         for u in rep.get("units", [])]}
        if sessions:
            tuned["multi_session"] = mcfg.as_dict()

    names = WORKLOADS if args.workload == "all" else [args.workload]
    for name in names:
        w = workloads.NAMED[name]()
        res = run_workload(args, torch, q8, w, cfg, tuned, full_line=args.workload != "all")
        if args.workload != "all" and not args.no_cpu_baseline:
            res["cpu_baseline"] = cpu_baseline(w, args.cpu_steps, res["step_bytes"], res["tokens_per_step"])
        print(json.dumps(res), flush=True)
    return 0


def run_tuner(torch, q8, workloads, budget_ms, sessions=False):
    """tune_select over decode / verify at 4096 and 65536 tokens (32 q / 8 kv
    heads, D 128, 8 drafts), each term gated by the oracle outputs stored in
    tests/golden (written by tests/golden/make_tune_refs.py) at 2e-3 sigma.
    With ``sessions``: at 32 q / 4 kv heads with the 16-session unit, whose
    two terms are gated the same way (the decode / verify units there by the
    alpha gate alone)."""
    refs = {}
    keep = []
    if not sessions:
        z = np.load(TUNE_REFS)
        for size, ctx, seed in (("small", 4096, 11), ("large", 65536, 12)):
            w = workloads.tune_reference(ctx, 8, seed)
            cache = _upload(torch, q8, w)
            pt = _dev(torch, np.ascontiguousarray(w.page_table[0]))
            keep.append(cache)
            sigma = z["sigma_" + size]
            refs["decode_" + size] = {"cache": cache, "q": _dev(torch, np.ascontiguousarray(w.q[0, 0]), True),
                                      "page_table": pt, "length": ctx, "out": z["decode_" + size], "sigma": sigma}
            refs["verify_" + size] = {"cache": cache, "q": _dev(torch, np.ascontiguousarray(w.q[0]), True),
                                      "page_table": pt, "length": ctx + 8, "out": z["verify_" + size],
                                      "sigma": sigma}
    else:
        z = np.load(TUNE_SESSION_REFS)
        for size, ctx, seed in (("small", 4096, 13), ("large", 65536, 14)):
            w = workloads.tune_sessions_reference(ctx, 16, seed)
            cache = _upload(torch, q8, w)
            keep.append(cache)
            refs["multi_session_" + size] = {
                "cache": cache, "q": _dev(torch, w.q, True), "page_table": _dev(torch, w.page_table),
                "length": int(w.seq_lens.max()), "seq_lens": _dev(torch, w.seq_lens),
                "n_prefix_pages": w.shared_prefix // 16, "out": z["multi_session_" + size],
                "sigma": z["sigma_" + size]}
    torch.cuda.synchronize()
    return q8.tune_select(32, 4 if sessions else 8, 128, n_draft=8, ctx_small=4096, ctx_large=65536,
                          budget_ms=budget_ms, install=True, refs=refs, ref_tol=2e-3,
                          n_sessions=16 if sessions else 0)


def _upload(torch, q8, w):
    cache = q8.PagedKVCache(w.num_pages, w.num_kv_heads, w.head_dim)
    for a in w.appends:
        q8.kv_quant_append(cache, _dev(torch, a.k, True), _dev(torch, a.v, True), _dev(torch, a.cu_new),
                           _dev(torch, a.start_pos), _dev(torch, a.page_table))
    return cache


def _dev(torch, a, bf=False):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if bf:
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.to("cuda:0")


def run_workload(args, torch, q8, w, cfg, tuned, full_line: bool) -> dict:
    """Times exactly args.steps steps of workload w (and as many attention
    launches, and the probes) and returns the JSON record."""
    dev = torch.device("cuda:0")
    if args.contiguous_pages:
        # relabel physical pages so that sequence 0's pages are in logical order
        perm = np.argsort(w.page_table[0][: (int(w.seq_lens[0]) + 15) // 16])
        full = np.arange(w.num_pages)
        full[: len(perm)] = perm
        relabel = lambda t: full[t].astype(np.int32)
        w.page_table = relabel(w.page_table)
        for a in w.appends:
            a.page_table = relabel(a.page_table)
    Hq, H, D = w.num_q_heads, w.num_kv_heads, w.head_dim
    per_th = cache_bytes_per_token_head(D, args.codec == "affine")
    unique = w.unique_tokens()
    layer_bytes = w.num_pages * H * 16 * per_th
    # enough distinct layer caches that the rotation streams 4x the LLC, at
    # most MAX_LAYERS: a cache of a few pages (the 256-token workload) stays
    # LLC-resident whatever the rotation, and tens of thousands of caches
    # would only slow the setup
    layers = args.layers or min(MAX_LAYERS, max(2, -(-4 * LLC_BYTES // layer_bytes) + 1))
    K = args.steps

    bf = w.dtype == "bf16"
    to_dev = lambda a, b=False: _dev(torch, a, b)
    caches = [q8.PagedKVCache(w.num_pages, H, D, codec=args.codec) for _ in range(layers)]
    batches = [(to_dev(a.k, bf), to_dev(a.v, bf), to_dev(a.cu_new), to_dev(a.start_pos), to_dev(a.page_table))
               for a in w.appends]
    for c in caches:
        for (k, v, cu, sp, pt) in batches:
            q8.kv_quant_append(c, k, v, cu, sp, pt)
    torch.cuda.synchronize()
    del batches
    # the step's new token: the last cached token of every sequence, re-appended
    last = w.appends[-1]
    B = w.n_seqs
    rows = (last.cu_new[1:] - 1).astype(np.int64)
    step_k = to_dev(last.k[rows], bf)
    step_v = to_dev(last.v[rows], bf)
    step_cu = to_dev(np.arange(B + 1, dtype=np.int32))
    step_pos = to_dev((w.seq_lens - 1).astype(np.int32))
    page_table = to_dev(w.page_table)
    seq_lens = to_dev(w.seq_lens)
    q = to_dev(w.q, bf)
    msl = int(w.seq_lens.max())
    nd = w.n_draft
    # sessions over one shared prefix run the prefix cascade
    n_pref = 0 if (nd or args.no_cascade) else w.shared_prefix // 16
    if n_pref:
        nws = q8.prefix_workspace_bytes(B, Hq, H, D, msl, n_pref, cfg)
    else:
        nws = q8.workspace_bytes(B, Hq, H, D, msl, nd, cfg)
    ws = torch.zeros(max(16, nws), dtype=torch.uint8, device=dev)
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def attend(c):
        if nd:
            q8.attn_verify_q8k4v(c, q, seq_lens, msl, page_table, w.softmax_scale, out=out, cfg=cfg, workspace=ws)
        elif n_pref:
            q8.attn_decode_prefix_q8k4v(c, q, seq_lens, msl, page_table, n_pref, w.softmax_scale, out=out, cfg=cfg,
                                        workspace=ws)
        else:
            q8.attn_decode_q8k4v(c, q, seq_lens, msl, page_table, w.softmax_scale, out=out, cfg=cfg, workspace=ws)

    # decode steps append their token inside the attention launch where the
    # plan allows (attn_decode_append_q8k4v); other steps append, then attend
    fused_step = not nd and not n_pref and not args.separate_append

    def step(i):
        c = caches[i % layers]
        if fused_step:
            q8.attn_decode_append_q8k4v(c, step_k, step_v, q, seq_lens, msl, page_table, w.softmax_scale, out=out,
                                        cfg=cfg, workspace=ws)
            return
        q8.kv_quant_append(c, step_k, step_v, step_cu, step_pos, page_table, total_new=B)
        attend(c)

    # a graph of exactly n calls of fn(i), i = 0 .. n-1 (rotating layers)
    def capture(fn, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(i)
        return g

    def timed(g, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # eager reference of the last step's layer; the graphs' untimed replay must match it
    last_layer = (K - 1) % layers
    attend(caches[last_layer])
    torch.cuda.synchronize()
    ref_out = out.clone()
    step_graph = capture(step, K)
    attn_graph = capture(lambda i: attend(caches[i % layers]), K)
    for g in (step_graph, attn_graph):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        if not torch.equal(out, ref_out):
            raise RuntimeError("graph replay differs from the eager result")
    t0 = time.perf_counter()
    ms_step = timed(attn_graph if args.kernel_only else step_graph, K)
    wall = time.perf_counter() - t0
    ms_attn = timed(attn_graph, K)
    del step_graph, attn_graph

    q_bytes = q.numel() * q.element_size()
    o_bytes = out.numel() * 4
    cache_read = unique * H * per_th
    attn_bytes = cache_read + q_bytes + o_bytes
    elem = 2 if bf else 4
    append_bytes = B * H * D * 2 * elem + B * H * per_th
    step_bytes = attn_bytes + (0 if args.kernel_only else append_bytes)
    tokens = B * max(1, nd)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    achieved = attn_bytes / (ms_attn * 1e-3) / 1e9

    probe = None
    if not args.no_probe and args.codec == "symmetric":
        probe = run_probes(torch, q8, caches, seq_lens, msl, page_table, K, layers, cache_read, w, n_pref)

    res = {
        "metric": "achieved HBM GB/s (% of peak) + decode tok/s/layer, q8K/q4V attn at 64K ctx",
        "value": round(value, 1),
        "unit": "GB/s",
        "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "tok_s_per_layer": round(tokens / (ms_step * 1e-3), 1),
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in, int8 K / int4 V codes, int8 and fp16 MFMA, fp32 accumulate",
        "data": "synthetic (seeded N(0,1), 1% outlier channels x8, bf16), random page permutation",
        "config": {"workload": w.name, "codec": args.codec, "num_q_heads": Hq, "num_kv_heads": H, "head_dim": D,
                   "context": int(w.seq_lens.max()), "n_seqs": B, "n_draft": nd, "page_size": 16,
                   "rotating_layer_caches": layers, "layer_cache_bytes": layer_bytes,
                   "launch_config": tuned or (cfg.as_dict() if cfg else "default"),
                   "shared_prefix_pages": n_pref},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_bytes(w.name if args.codec == "symmetric" else w.name + "_affine", nd),
                     "kernel": attention_launch_name(nd, n_pref, w, cfg, q8),
                     "algorithmic_bytes": attn_bytes, "avg_launch_us": round(ms_attn * 1e3, 3)},
        "tokens_per_step": tokens,
        "step_bytes": step_bytes,
        "wall_s": round(wall, 3),
    }
    if probe:
        res["probe"] = probe
        res["pct_of_probe"] = round(100 * achieved / probe["paged_GBs"], 1)
    if full_line:
        res["device"] = device_info(torch)
    return res


def attention_launch_name(nd, n_pref, w, cfg, q8) -> str:
    if n_pref:
        return "attn_decode_prefix_q8k4v launch (prefix and suffix passes + cascade combine kernel)"
    entry = "attn_verify_q8k4v" if nd else "attn_decode_q8k4v"
    msl = int(w.seq_lens.max())
    if q8.workspace_bytes(w.n_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, msl, max(1, nd), cfg) == 0:
        return entry + " launch (one split per sequence and kv head: the attention kernel alone)"
    fused = bool(cfg and cfg.fused_combine)
    return entry + (" launch (split-K attention kernel with the in-launch split merge)" if fused else
                    " launch (split-K attention kernel + LSE combine kernel)")


def run_probes(torch, q8, caches, seq_lens, msl, page_table, K, layers, cache_read, w, n_pref):
    """The streaming references: q8k4v_hbm_probe over the same caches
    (rotating as the steps do; the best of its launch shapes) and
    q8k4v_stream_probe over contiguous 256 MiB slices of a 2 GiB buffer."""
    stream = torch.cuda.current_stream()

    def time_graph(fn, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(i)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    res = {"paged_bytes": cache_read}
    if not n_pref:   # the probe streams each sequence's own pages (a shared prefix would be re-read)
        best, best_grouped = None, None
        H = caches[0].num_kv_heads
        shapes = [(4, 2, 1), (4, 3, 1), (4, 4, 1), (8, 2, 1), (8, 3, 1),
                  (4, 3, 2), (4, 3, 4), (8, 3, 2), (8, 3, 4), (8, 2, 8), (8, 3, 8)]
        for waves, stages, hpw in shapes:
            if H % hpw:
                continue
            ms = time_graph(lambda i: q8.hbm_probe(caches[i % layers], seq_lens, msl, page_table, waves, stages, hpw),
                            min(K, 4 * layers))
            gbs = cache_read / (ms * 1e-3) / 1e9
            res[f"paged_GBs_w{waves}s{stages}h{hpw}"] = round(gbs, 1)
            if hpw == 1 and (best is None or gbs > best[0]):
                best = (gbs, ms, waves, stages)
            if hpw > 1 and (best_grouped is None or gbs > best_grouped[0]):
                best_grouped = (gbs, ms, waves, stages, hpw)
        # the decode kernel's own mapping (one kv head per workgroup)
        res["paged_GBs"] = round(best[0], 1)
        res["paged_us"] = round(best[1] * 1e3, 3)
        res["paged_shape"] = {"waves_per_wg": best[2], "stages": best[3]}
        if best_grouped:
            res["paged_grouped_GBs"] = round(best_grouped[0], 1)
            res["paged_grouped_shape"] = {"waves_per_wg": best_grouped[2], "stages": best_grouped[3],
                                          "heads_per_wg": best_grouped[4]}
    seg = 256 << 20
    buf = torch.empty(8 * seg, dtype=torch.uint8, device="cuda:0")
    ms = time_graph(lambda i: q8.stream_probe(buf[(i % 8) * seg:(i % 8 + 1) * seg], 8, 3), 16)
    res["stream_GBs"] = round(seg / (ms * 1e-3) / 1e9, 1)
    del buf
    if "paged_GBs" not in res:
        res["paged_GBs"] = res["stream_GBs"]
    return res


# Kernel sources whose HBM traffic the committed counter summary describes;
# the summary is used only while these files are unchanged.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    False: ["attn_paged.hip", "attn_common.h", "q8k4v_device.h", "q8k4v_internal.h", "abi.cpp", "combine.hip"],
    True: ["attn_paged.hip", "attn_common.h", "q8k4v_device.h", "q8k4v_internal.h", "abi.cpp", "combine.hip"],
}


def kernel_sources_sha(verify: bool) -> str:
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "decode_attention_quantized_kv_amd", "csrc")
    for name in KERNEL_SOURCES[verify]:
        h.update(name.encode())
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()[:16]


def traffic_bytes(workload: str, n_draft: int):
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE
    counters, each scaled by what the same counter reads for a plain copy of
    known size; None when absent or taken on other kernel sources."""
    try:
        t = json.load(open(TRAFFIC_FILE))
        e = t["workloads"][workload]
    except (OSError, KeyError, ValueError):
        return None
    if e.get("kernel_sources_sha") != kernel_sources_sha(bool(n_draft)):
        return None
    kib = e["fetch_kib"] * t["copy_factor"]["fetch"] + e["write_kib"] * t["copy_factor"]["write"]
    return int(round(kib * 1024))


def copy_calibration(torch, mib: int) -> int:
    """Device-to-device copies of a known size: the reference that scales the
    FETCH_SIZE / WRITE_SIZE counters to bytes."""
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "copies": 5}), flush=True)
    return 0


def device_info(torch) -> dict:
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", ""), "cus": p.multi_processor_count,
            "mem_gib": round(p.total_memory / 2**30, 1)}


def cpu_baseline(w, steps: int, step_bytes: int, tokens: int) -> dict:
    """The CPU oracle as it stands, on this host: one step = quantize-append
    the new token + fp64 attention over the dequantized cache."""
    from oracle import attention, codec
    cache = codec.PagedCache(w.num_pages, w.num_kv_heads, w.head_dim)
    for a in w.appends:
        codec.append(cache, a.k, a.v, w.dtype, a.cu_new, a.start_pos, a.page_table)
    last = w.appends[-1]
    B = w.n_seqs
    rows = (last.cu_new[1:] - 1).astype(np.int64)
    times = []
    for _ in range(steps):
        t0 = time.perf_counter()
        codec.append(cache, last.k[rows], last.v[rows], w.dtype, np.arange(B + 1, dtype=np.int32),
                     (w.seq_lens - 1).astype(np.int32), w.page_table)
        if w.n_draft:
            attention.verify(cache, w.q, w.dtype, w.page_table, w.seq_lens, w.softmax_scale)
        else:
            attention.decode(cache, w.q, w.dtype, w.page_table, w.seq_lens, w.softmax_scale)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        pass
    return {"value": round(step_bytes / t / 1e9, 4), "unit": "GB/s", "cores": threads or 1,
            "kind": "oracle", "s_per_step": round(t, 3), "tok_s_per_layer": round(tokens / t, 4),
            "host_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{steps} full steps of {w.name} (median); numpy elementwise work is single-threaded, "
                      f"matmuls use the BLAS pool"}


def cpu_report(reps: int = 3) -> int:
    """The CPU oracle as it stands, timed on this host for every workload:
    the quantizer filling each workload's cache, and one fp64 attention call
    (decode, verify or the multi-session decode) over the filled cache, each
    with the BLAS pool at its default size and limited to one thread (numpy's
    elementwise work is single-threaded either way).  Medians of `reps` runs
    (one run where the first takes over 60 s).  Prints one JSON line per
    measurement."""
    import contextlib

    from threadpoolctl import threadpool_info, threadpool_limits

    import workloads
    from oracle import attention, codec

    pool = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    print(json.dumps({"host": {"sched_getaffinity": len(os.sched_getaffinity(0)), "os_cpu_count": os.cpu_count(),
                               "blas_threads_default": pool, "reps": reps}}), flush=True)

    def median_time(fn):
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
            if ts[0] > 60.0:
                break
        return float(np.median(ts)), len(ts)

    for name in ["tiny_decode_256", "gqa_decode_4096", "gqa_decode_65536", "verify_65536_w8",
                 "multi_session_16x32768"]:
        w = workloads.NAMED[name]()
        H, D = w.num_kv_heads, w.head_dim
        nbytes = w.unique_tokens() * H * cache_bytes_per_token_head(D)
        tokens = w.n_seqs * max(1, w.n_draft)

        def fill():
            cache = codec.PagedCache(w.num_pages, H, D)
            for a in w.appends:
                codec.append(cache, a.k, a.v, w.dtype, a.cu_new, a.start_pos, a.page_table)
            return cache

        cache = fill()
        fn = attention.verify if w.n_draft else attention.decode

        def attend():
            fn(cache, w.q, w.dtype, w.page_table, w.seq_lens, w.softmax_scale)

        for threads in (None, 1):
            limit = threadpool_limits(threads) if threads else contextlib.nullcontext()
            with limit:
                for what, run in (("attention", attend), ("quantize_fill", fill)):
                    t, n = median_time(run)
                    rec = {"workload": name, "step": what, "blas_threads": threads or pool, "runs": n,
                           "s": round(t, 4)}
                    if what == "attention":
                        rec.update({"GB_s_algorithmic": round(nbytes / t / 1e9, 4),
                                    "tok_s_per_layer": round(tokens / t, 4)})
                    else:
                        rec["tokens_quantized"] = int(sum(len(a.k) for a in w.appends)) * H
                    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
