"""Throughput of the MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--pass train]

A step is one moe_forward call (route, dispatch, expert FFN, combine) over one
batch of synthetic, seeded inputs already resident in HBM.  W untimed steps,
then exactly K steps back to back between two device synchronisations; value
is tokens/s over those K steps.  A second, equally long region runs the same
kernels through the stage entry points (route, dispatch indices, the expert
FFN gathering its rows from x, combine: the launches moe_forward makes) with
HIP events between the stages on the stream the kernels run on, after a
512 MiB write that evicts the L2 and MALL caches before each step, to get
each stage's duration and its achieved HBM bandwidth; the expert FFN stage
is two launches of the grouped-GEMM kernel with equal flops, which gives the
per-launch roofline of the dominant kernel.  The fp64 oracle is timed on the
host cores on a bounded sample of the same workload, and its result gives
the sample's near-tie count and the GPU output's error.  One JSON line is
printed.

--pass train times a training step of the layer instead: moe_forward_train
then moe_backward (same inputs, a seeded output gradient), with the backward's
expert GEMMs timed through moe_expert_ffn_backward for their roofline.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import moe_inputs as mi  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 (vector and matrix)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "MoE layer fwd tokens/s (T=2048,H=4096,E=8,k=2) + % MFMA/HBM roofline"


def workload(a) -> "mi.MoEConfig":
    """--shape's layer, else the named workload."""
    if not a.shape:
        return mi.CONFIGS[a.config]
    f = a.shape.split(",")
    if len(f) not in (5, 6) or (len(f) == 6 and f[5] not in ("bf16", "f32")):
        raise SystemExit(f"--shape wants T,H,E,K,F[,bf16|f32], got {a.shape!r}")
    T, H, E, k, F = (int(v) for v in f[:5])
    dt = f[5] if len(f) == 6 else "bf16"
    return mi.MoEConfig(f"shape_T{T}_H{H}_E{E}_k{k}_F{F}_{dt}", T=T, H=H, E=E, k=k, F=F, dtype=dt)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--config", default="mixtral_bf16", choices=list(mi.CONFIGS))
    ap.add_argument("--shape", default=None, metavar="T,H,E,K,F[,DTYPE]",
                    help="a layer of this shape (DTYPE bf16, the default, or f32; seed 0, "
                         "the workloads' input recipe) instead of --config")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true",
                    help="stage timing without the cache-evicting write before each step")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0,
                    help="tokens in the oracle's timed sample (0: per-workload default)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--summarize-traffic", nargs="+", metavar="CSV",
                    help="READ_CSV WRITE_CSV COPY_READ_CSV COPY_WRITE_CSV [MFMA_CSV]: turn "
                         "rocprofv3 request-counter files into the traffic record under "
                         "profiles/ and exit")
    ap.add_argument("--copy-mib", type=int, default=1024, help="size of the calibration copy")
    ap.add_argument("--pass", dest="pass_", default="forward", choices=["forward", "train"],
                    help="forward (default): moe_forward steps; train: moe_forward_train + "
                         "moe_backward steps (a training step of the layer)")
    return ap.parse_args()


GEMM_SOURCES = ["mixture_experts_layer_21_amd/csrc/gemm_bf16.hip",
                "mixture_experts_layer_21_amd/csrc/common.h"]
PROFILES = os.path.join(ROOT, "profiles")


def gemm_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_record_path(workload: str) -> str:
    return os.path.join(PROFILES, f"traffic_gemm_bf16_grouped_{workload}.md")


def calibrate_copy(mib: int):
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": n}))


def attainable_hbm(mib: int = 1024, reps: int = 5) -> dict:
    """A diagnostic beside the published peak: a plain device copy of `mib`
    MiB (read + write) timed with HIP events, best of `reps`."""
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = float("inf")
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        b.synchronize()
        best = min(best, a.elapsed_time(b) * 1e-3)
    del src, dst
    return {"hbm_copy_gbs": 2 * n / best / 1e9, "copy_bytes": 2 * n}


def attainable_gemm(reps: int = 5) -> dict:
    """Diagnostics beside the published bf16 peak: torch.matmul (hipBLASLt)
    in bf16 on an 8192^3 product and on one expert's first GEMM at the
    Mixtral shape (512 x 4096 by 4096 x 14336), best of `reps` with HIP
    events.  Not part of the hot path."""
    out = {}
    g = torch.Generator(device="cuda").manual_seed(0)
    for name, (m, k, n) in {"matmul_8192_tflops": (8192, 8192, 8192),
                            "matmul_expert_tflops": (512, 4096, 14336)}.items():
        a = torch.randn(m, k, device="cuda", generator=g).bfloat16()
        b = torch.randn(k, n, device="cuda", generator=g).bfloat16()
        c = a @ b
        best = float("inf")
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            torch.matmul(a, b, out=c)
            e1.record()
            e1.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e-3)
        out[name] = 2 * m * k * n / best / 1e12
        del a, b, c
    return out


def _counter_totals(csv_path: str, counter: str, kernel_substr: str, required: bool = True):
    """(sum over dispatches, number of dispatches) of a counter for the kernels
    whose name contains kernel_substr."""
    import csv
    vals = {}
    for r in csv.DictReader(open(csv_path)):
        if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter:
            vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not vals and required:
        raise SystemExit(f"no {counter} rows for kernels matching {kernel_substr!r} in {csv_path}")
    return sum(vals.values()), len(vals)


READ_COUNTERS = ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum",
                 "TCC_EA0_RDREQ_128B_sum")
WRITE_COUNTERS = ("TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum")
MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "GRBM_GUI_ACTIVE")


def _bytes(rd_csv: str, wr_csv: str, kernel: str, required: bool = True):
    """(read bytes, written bytes, dispatches) of the L2 <-> memory traffic of
    the matching kernels, from the request counts by size: reads 32 n32 +
    64 n64 + 128 n128, writes 64 n64 + 32 (n - n64)."""
    n, nd = _counter_totals(rd_csv, READ_COUNTERS[0], kernel, required)
    n32, _ = _counter_totals(rd_csv, READ_COUNTERS[1], kernel, required)
    n64, _ = _counter_totals(rd_csv, READ_COUNTERS[2], kernel, required)
    n128, _ = _counter_totals(rd_csv, READ_COUNTERS[3], kernel, required)
    w, _ = _counter_totals(wr_csv, WRITE_COUNTERS[0], kernel, required)
    w64, _ = _counter_totals(wr_csv, WRITE_COUNTERS[1], kernel, required)
    return (32 * n32 + 64 * n64 + 128 * n128, 64 * w64 + 32 * (w - w64), nd,
            {"rdreq": n, "rdreq_32b": n32, "rdreq_64b": n64, "rdreq_128b": n128,
             "wrreq": w, "wrreq_64b": w64})


def summarize_traffic(a):
    """HBM-side traffic of one launch of the grouped GEMM (the main kernel
    plus the split-tile reduce that follows it) from rocprofv3 request
    counters, checked against a plain device copy of known size under the
    same counters, plus the matrix-pipe busy fraction of the main kernel."""
    rd, wr, cr, cw = a.summarize_traffic[:4]
    mf = a.summarize_traffic[4] if len(a.summarize_traffic) > 4 else None
    rg, wg, nd, raw = _bytes(rd, wr, "gemm_bf16_grouped")
    rr, wrr, nr, _ = _bytes(rd, wr, "gemm_split_reduce", False)
    crd, cwr, ncopy, craw = _bytes(cr, cw, "copy")
    crd, cwr = crd / ncopy, cwr / ncopy
    nbytes = a.copy_mib << 20
    per = {"read": (rg + rr) / nd, "write": (wg + wrr) / nd}
    rec = {"kernel": "gemm_bf16_grouped", "workload": a.config, "source_hash": gemm_source_hash(),
           "dispatches": nd, "reduce_dispatches": nr,
           "read_bytes_per_launch": per["read"], "write_bytes_per_launch": per["write"],
           "reduce_read_bytes_per_launch": rr / nd, "reduce_write_bytes_per_launch": wrr / nd,
           "copy_bytes": nbytes, "copy_read_counted": crd / 1, "copy_write_counted": cwr,
           "copy_read_ratio": crd / nbytes, "copy_write_ratio": cwr / nbytes,
           "traffic_bytes_per_launch": per["read"] + per["write"], "counts": raw,
           "copy_counts": craw}
    if mf:
        busy, n1 = _counter_totals(mf, MFMA_COUNTERS[0], "gemm_bf16_grouped")
        mops, _ = _counter_totals(mf, MFMA_COUNTERS[1], "gemm_bf16_grouped")
        gui, _ = _counter_totals(mf, MFMA_COUNTERS[2], "gemm_bf16_grouped")
        # GRBM_GUI_ACTIVE is summed over the 8 XCDs (one count each);
        # SQ_VALU_MFMA_BUSY_CYCLES over all 1024 SIMDs
        xcds, simds = 8, 4 * 256
        rec["mfma_busy_frac"] = busy / (gui / xcds * simds)
        rec["mfma_flops_per_launch"] = mops * 512 / n1
        rec["gui_active_cycles_per_launch"] = gui / xcds / n1
    path = traffic_record_path(a.config)
    cmd = ("rocprofv3 --pmc {c} --output-format csv -d <dir> -o {o} -- python3 bench.py "
           "--config {w} --steps 3 --warmup 1 --no-cpu-baseline")
    with open(path, "w") as fh:
        fh.write(f"# HBM traffic of gemm_bf16_grouped on {a.config}\n\n")
        fh.write("L2-to-memory traffic of one launch of the grouped GEMM (the main kernel plus "
                 "the gemm_split_reduce kernel that follows it), from rocprofv3 request counters "
                 "by size: read bytes = 32 RDREQ_32B + 64 RDREQ_64B + 128 RDREQ_128B, written "
                 "bytes = 64 WRREQ_64B + 32 (WRREQ - WRREQ_64B), summed over the 16 channels of "
                 "the 8 XCDs and averaged over the launches.  A plain device copy of "
                 f"{a.copy_mib} MiB (torch copy kernel) under the same counters checks the "
                 "formula: its counted bytes over its true bytes are the ratios below (no "
                 "scale factor is applied).\n\n")
        fh.write("Commands (run from the repository root on the GPU host):\n\n```\n")
        fh.write(cmd.format(c=" ".join(READ_COUNTERS), o="r", w=a.config) + "\n")
        fh.write(cmd.format(c=" ".join(WRITE_COUNTERS), o="w", w=a.config) + "\n")
        if mf:
            fh.write(cmd.format(c=" ".join(MFMA_COUNTERS), o="m", w=a.config) + "\n")
        fh.write(f"rocprofv3 --pmc {' '.join(READ_COUNTERS)} --output-format csv -d <dir> -o cr "
                 f"-- python3 bench.py --calibrate-copy-mib {a.copy_mib}\n")
        fh.write(f"rocprofv3 --pmc {' '.join(WRITE_COUNTERS)} --output-format csv -d <dir> -o cw "
                 f"-- python3 bench.py --calibrate-copy-mib {a.copy_mib}\n")
        fh.write(f"python3 bench.py --config {a.config} --summarize-traffic <r csv> <w csv> "
                 f"<cr csv> <cw csv>{' <m csv>' if mf else ''}\n```\n\n")
        fh.write("| quantity | value |\n|---|---|\n")
        fh.write(f"| GEMM launches averaged (reduce dispatches) | {nd} ({nr}) |\n")
        fh.write(f"| read per launch (of it, reduce) | {per['read'] / 1e9:.4f} GB "
                 f"({rr / nd / 1e9:.4f} GB) |\n")
        fh.write(f"| written per launch (of it, reduce) | {per['write'] / 1e9:.4f} GB "
                 f"({wrr / nd / 1e9:.4f} GB) |\n")
        fh.write(f"| copy of {nbytes} B: counted read / written | {crd / nbytes:.4f} / "
                 f"{cwr / nbytes:.4f} of the true bytes |\n")
        fh.write(f"| HBM-side bytes per launch | {rec['traffic_bytes_per_launch'] / 1e9:.4f} GB |\n")
        if mf:
            fh.write(f"| matrix pipe busy (SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 "
                     f"XCDs x 1024 SIMDs)) | {rec['mfma_busy_frac']:.3f} |\n")
            fh.write(f"| GPU active cycles per launch (one XCD) | "
                     f"{rec['gui_active_cycles_per_launch']:.0f} |\n")
            fh.write(f"| bf16 MFMA flops per launch (MOPS x 512) | "
                     f"{rec['mfma_flops_per_launch'] / 1e9:.1f} G |\n")
        fh.write("\nThe record below is read by bench.py; it is ignored once the GEMM sources "
                 "change (source_hash).\n\n```json\n" + json.dumps(rec, indent=1) + "\n```\n")
    print(f"wrote {path}")


def read_traffic(workload: str):
    path = traffic_record_path(workload)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    try:
        rec = json.loads(text.split("```json")[1].split("```")[0])
    except (IndexError, ValueError):
        return None
    if rec.get("source_hash") != gemm_source_hash():
        return None
    return rec["traffic_bytes_per_launch"]


def alg_counts(cfg, ids: np.ndarray):
    """Algorithmic flops and HBM bytes of one forward (padding excluded)."""
    es = 4 if cfg.dtype == "f32" else 2
    touched = len(np.unique(ids))
    flops = 2 * cfg.T * cfg.H * cfg.E + 4 * cfg.T * cfg.k * cfg.H * cfg.F
    bytes_ = es * (cfg.T * cfg.H + cfg.H * cfg.E + 2 * touched * cfg.H * cfg.F + cfg.T * cfg.H) \
        + 8 * cfg.T * cfg.k
    return flops, bytes_, touched


def gemm_launch_counts(cfg, touched):
    """Per launch of the grouped expert GEMM (both FFN GEMMs are equal; a
    launch is the main kernel plus its split-tile reduce): flops 2*R*H*F;
    bytes = the touched experts' weight matrix + the A operand rows read + the
    C rows written."""
    es = 4 if cfg.dtype == "f32" else 2
    R = cfg.R
    flops = 2 * R * cfg.H * cfg.F
    bytes_ = es * (touched * cfg.H * cfg.F + R * cfg.H + R * cfg.F)
    return flops, bytes_


def time_forward(moe, L, cfg, steps, warmup, ws, y):
    args = (L["x"], L["w_r"], L["router_bias"], L["w1"], L["w2"], cfg.k)
    for _ in range(warmup):
        moe.moe_forward(*args, y=y, ws=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        moe.moe_forward(*args, y=y, ws=ws)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


FLUSH_BYTES = 512 << 20     # twice the MALL (256 MB); the L2s are 4 MB per XCD


def time_stages(moe, L, cfg, steps, bufs, flush=True):
    """Per-stage durations (ms) from HIP events on the launch stream.  The
    stages are the launches moe_forward makes: routing, the dispatch indices
    (bf16: no row copy), the expert FFN (bf16: its first GEMM gathers the rows
    from x), the combine.  With flush, a 512 MiB write before each step (not
    timed) leaves nothing of the previous step in the L2 or MALL caches."""
    names = ["route", "permute", "expert_ffn", "combine"]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    ids, w, off, st, inv, xp, yp, y, ws = bufs
    junk = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda") if flush else None
    bf16 = cfg.dtype == "bf16"
    torch.cuda.synchronize()
    for i in range(steps):
        if flush:
            junk.fill_(i & 0xFF)
        e = ev[i]
        e[0].record()
        moe.moe_route(L["x"], L["w_r"], L["router_bias"], cfg.k, topk_ids=ids, topk_w=w, ws=ws)
        e[1].record()
        moe.moe_permute(L["x"], ids, cfg.E, expert_offsets=off, sorted_token=st, inv_pos=inv,
                        xp=xp, ws=ws, with_rows=not bf16)
        e[2].record()
        if bf16:
            moe.moe_expert_ffn_gather(L["x"], st, off, L["w1"], L["w2"], yp=yp, ws=ws)
        else:
            moe.moe_expert_ffn(xp, off, L["w1"], L["w2"], yp=yp, ws=ws)
        e[3].record()
        moe.moe_combine(yp, inv, w, y=y)
        e[4].record()
    torch.cuda.synchronize()
    out = {}
    for j, n in enumerate(names):
        out[n] = float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(steps)]))
    return out


def pass_bytes(cfg, touched):
    """Algorithmic HBM bytes of the passes around the expert GEMMs (what each
    must read and write at least):
      route    x, W_r, router bias; ids and gate weights written
      permute  ids read; offsets, sorted_token, inv_pos written
      combine  yp, gate weights and inv_pos read; y written"""
    es = 4 if cfg.dtype == "f32" else 2
    T, H, E, k, R = cfg.T, cfg.H, cfg.E, cfg.k, cfg.R
    route = es * (T * H + H * E) + (4 * E if cfg.bias0 else 0) + 8 * T * k
    permute = 4 * R + 4 * (E + 1) + 8 * R + (es * R * H * 2 if cfg.dtype == "f32" else 0)
    combine = es * R * H + 8 * R + es * T * H
    return {"route": route, "permute": permute, "combine": combine}


def blas_threads() -> int:
    """Threads of the BLAS library numpy's matmul runs on (what the oracle
    uses); the CPU count this process may run on if it cannot be read."""
    try:
        import threadpoolctl
        n = [d["num_threads"] for d in threadpoolctl.threadpool_info()
             if d.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_baseline(cfg, L, n_tokens, y_gpu, ids_gpu):
    """The fp64 oracle on the first n_tokens tokens of the workload (all the
    experts they route to), timed on the host cores.  Its result also gives
    the sample's routing agreement and the GPU output's error (returned
    separately: they are not part of the timing)."""
    import oracle
    sel = torch.arange(n_tokens, device="cuda")
    x = L["x"][sel].cpu()
    w_r = L["w_r"].cpu()
    b = None if L["router_bias"] is None else L["router_bias"].cpu()
    w1 = L["w1"].cpu()
    w2 = L["w2"].cpu()
    cores = blas_threads()
    t0 = time.perf_counter()
    up = lambda t: t.to(torch.float64).numpy()  # noqa: E731  (the oracle's own upcast)
    ref = oracle.forward(up(x), up(w_r), None if b is None else up(b),
                         lambda e: up(w1[e]), lambda e: up(w2[e]), cfg.k)
    dt = time.perf_counter() - t0
    base = {"value": n_tokens / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {n_tokens} of {cfg.T} tokens of {cfg.name}, fp64 numpy "
                      f"({cores} BLAS threads), {dt:.2f} s"}
    # routing and output against the oracle on the same tokens: y is compared
    # on the tokens whose ids agree (a near-tie token may pick another expert)
    ids_g = ids_gpu[:n_tokens].astype(np.int64)
    same = (ids_g == ref["ids"]).all(axis=1)
    yg = y_gpu[:n_tokens].to(torch.float64).cpu().numpy()
    err = np.abs(yg[same] - ref["y"][same]).max() / np.abs(ref["y"][same]).max()
    near = oracle.boundary_near_tie(ref["logits"], cfg.k)
    kinds = classify_ids(ids_g, ref["ids"], ref["logits"], near)
    check = {"tokens": n_tokens,
             "boundary_near_ties": int(near.sum()),
             "ids_differ": int((~same).sum()),
             "near_ties": kinds,
             "max_err_rel": float(err)}
    return base, check


def classify_ids(ids_g, ids_ref, logits, near, rel=1e-3) -> dict:
    """Tokens whose ids differ from the oracle's, by the routing acceptance
    rule: "within" (the same set, slots swapped only between logits closer
    than `rel` relative), "boundary" (another set, on a token whose k-th and
    (k+1)-th oracle logits are that close), "other" (neither: a failure)."""
    out = {"boundary": 0, "within": 0, "other": 0}
    for t in np.nonzero((ids_g != ids_ref).any(axis=1))[0]:
        g, l = ids_g[t], logits[t]
        if set(g.tolist()) == set(ids_ref[t].tolist()):
            s = l[g]
            ok = all(s[j] >= s[j + 1] - rel * max(abs(s[j]), abs(s[j + 1]))
                     for j in range(len(s) - 1))
            out["within" if ok else "other"] += 1
        else:
            out["boundary" if near[t] else "other"] += 1
    return out


METRIC_TRAIN = "MoE layer fwd+bwd (training step) tokens/s + % MFMA/HBM roofline"


def time_train(moe, L, cfg, steps, warmup, bufs):
    y, ids, w, saved, ws_f, ws_b, out, dy = bufs
    args = (L["x"], L["w_r"], L["router_bias"], L["w1"], L["w2"], cfg.k)

    def step():
        moe.moe_forward_train(*args, y=y, topk_ids=ids, topk_w=w, saved=saved, ws=ws_f)
        moe.moe_backward(dy, L["x"], L["w_r"], L["w1"], L["w2"], cfg.k, ids, w, saved, out=out,
                         ws=ws_b)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def time_train_stages(moe, L, cfg, steps, bufs):
    """HIP events on the launch stream: the training forward, the backward, and
    the backward's expert stage alone (moe_expert_ffn_backward: four GEMM
    launches of equal flops, 2 R H F each)."""
    y, ids, w, saved, ws_f, ws_b, out, dy = bufs
    args = (L["x"], L["w_r"], L["router_bias"], L["w1"], L["w2"], cfg.k)
    dev = "cuda"
    R = cfg.R
    off = torch.empty(cfg.E + 1, dtype=torch.int32, device=dev)
    st = torch.empty(R, dtype=torch.int32, device=dev)
    inv = torch.empty(R, dtype=torch.int32, device=dev)
    xp = torch.empty((R, cfg.H), dtype=cfg.torch_dtype, device=dev)
    moe.moe_permute(L["x"], ids, cfg.E, expert_offsets=off, sorted_token=st, inv_pos=inv, xp=xp,
                    ws=ws_f)
    rows = mi.MoEConfig("rows", T=R, H=cfg.F, E=1, k=1, F=8, dtype=cfg.dtype, seed=cfg.seed + 2)
    z = mi.make_x(rows, dev)                 # [R, F] seeded values for z and h
    dyp = torch.empty((R, cfg.H), dtype=cfg.torch_dtype, device=dev)
    dyp.copy_(xp)
    dw1, dw2 = out["dw1"], out["dw2"]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        e = ev[i]
        e[0].record()
        moe.moe_forward_train(*args, y=y, topk_ids=ids, topk_w=w, saved=saved, ws=ws_f)
        e[1].record()
        moe.moe_backward(dy, L["x"], L["w_r"], L["w1"], L["w2"], cfg.k, ids, w, saved, out=out,
                         ws=ws_b)
        e[2].record()
        moe.moe_expert_ffn_backward(dyp, xp, off, z, z, L["w1"], L["w2"], dxp=dyp, dw1=dw1,
                                    dw2=dw2, ws=ws_b)
        e[3].record()
    torch.cuda.synchronize()
    names = ["forward_train", "backward", "expert_ffn_backward"]
    return {n: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(steps)]))
            for j, n in enumerate(names)}


def cpu_baseline_train(cfg, L, dy, n_tokens):
    """The fp64 oracle's forward and backward on the first n_tokens tokens
    (every expert they route to), timed on the host cores."""
    import oracle
    up = lambda t: t.cpu().to(torch.float64).numpy()  # noqa: E731
    x = up(L["x"][:n_tokens])
    g = up(dy[:n_tokens])
    w_r = up(L["w_r"])
    b = None if L["router_bias"] is None else up(L["router_bias"])
    w1c, w2c = L["w1"].cpu(), L["w2"].cpu()
    ids = oracle.topk_ids(oracle.router_logits(x, w_r, b), cfg.k)
    used = sorted(set(ids.ravel().tolist()))
    w1 = np.zeros((cfg.E, cfg.H, cfg.F))
    w2 = np.zeros((cfg.E, cfg.F, cfg.H))
    for e in used:
        w1[e] = w1c[e].to(torch.float64).numpy()
        w2[e] = w2c[e].to(torch.float64).numpy()
    cores = blas_threads()
    t0 = time.perf_counter()
    oracle.forward(x, w_r, b, w1, w2, cfg.k)
    oracle.backward(x, w_r, b, w1, w2, cfg.k, g)
    dt = time.perf_counter() - t0
    return {"value": n_tokens / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {n_tokens} of {cfg.T} tokens of {cfg.name}: fp64 forward + "
                      f"backward (weight gradients of the {len(used)} experts they use), "
                      f"{dt:.2f} s"}


def main_train(a, moe, cfg):
    dev = "cuda"
    L = mi.make_inputs(cfg, dev)
    dy = mi.make_dy(cfg, dev)
    T, H, E, k, F, td = cfg.T, cfg.H, cfg.E, cfg.k, cfg.F, cfg.torch_dtype
    bufs = (torch.empty((T, H), dtype=td, device=dev),
            torch.empty((T, k), dtype=torch.int32, device=dev),
            torch.empty((T, k), dtype=torch.float32, device=dev),
            torch.empty(moe.moe_saved_bytes(T, H, E, k, F, td), dtype=torch.uint8, device=dev),
            torch.empty(moe.moe_workspace_bytes(T, H, E, k, F, td), dtype=torch.uint8,
                        device=dev),
            torch.empty(moe.moe_backward_workspace_bytes(T, H, E, k, F, td), dtype=torch.uint8,
                        device=dev),
            {"dx": torch.empty((T, H), dtype=td, device=dev),
             "dw_r": torch.empty((H, E), dtype=td, device=dev),
             "dw1": torch.empty((E, H, F), dtype=td, device=dev),
             "dw2": torch.empty((E, F, H), dtype=td, device=dev),
             "dw": torch.empty((T, k), dtype=torch.float32, device=dev)},
            dy)
    torch.cuda.synchronize()
    print(f"[bench] {cfg.name} train: inputs ready", file=sys.stderr, flush=True)
    sec = time_train(moe, L, cfg, a.steps, a.warmup, bufs)
    print(f"[bench] timed region done: {sec * 1e3:.3f} ms/step", file=sys.stderr, flush=True)
    stages = time_train_stages(moe, L, cfg, a.steps, bufs)
    R = cfg.R
    es = 2 if cfg.dtype == "bf16" else 4
    # per GEMM launch of the expert backward (four of them, equal flops):
    # 2 R H F flops; bytes: the touched experts' weight (NT) or gradient (TN)
    # matrix plus the two R-row operands read
    ids = bufs[1].cpu().numpy()
    touched = len(np.unique(ids))
    g_flops = 2 * R * H * F
    g_bytes = es * (touched * H * F + R * H + R * F)
    g_sec = stages["expert_ffn_backward"] / 4 * 1e-3
    peak_mm = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    ridge = peak_mm * 1e12 / (PEAK_HBM_GBS * 1e9)
    if g_flops / g_bytes >= ridge:
        roof = {"bound": "mfma" if cfg.dtype == "bf16" else "alu",
                "achieved": g_flops / g_sec / 1e12, "peak": peak_mm, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": g_bytes / g_sec / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    roof["kernel"] = ("expert backward GEMMs: gemm_bf16_grouped NT (dz, dxp) and "
                      "gemm_bf16_wgrad (dW2, dW1), average of the four launches"
                      if cfg.dtype == "bf16" else "gemm_f32_bwd, average of four launches")
    roof["per_launch"] = {"flops": g_flops, "bytes": g_bytes, "ms": g_sec * 1e3}
    cpu = None
    if not a.no_cpu_baseline:
        # (about 10 s of host work each)
        n = a.cpu_sample_tokens or {"tiny_fp32": 64, "mixtral_bf16": 1024, "skewed_bf16": 1024,
                                    "many_experts_bf16": 2048,
                                    "weight_bound_bf16": 16}.get(cfg.name, min(T, 64))
        cpu = cpu_baseline_train(cfg, L, dy, min(n, T))
    # training-step flops: forward (router + 2 GEMMs) and backward (router
    # weight and input gradients + 4 GEMMs)
    flops = 2 * T * H * E * 3 + 6 * 2 * R * H * F
    out = {
        "metric": METRIC_TRAIN, "value": T / sec, "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": sec * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded counter-based generator; random-init weights)",
        "config": {"workload": cfg.name + " (training step)", "T": T, "H": H, "E": E,
                   "top_k": k, "F": F, "router_bias0": cfg.bias0, "seed": cfg.seed},
        "step_tflops": flops / sec / 1e12,
        "stages_ms": stages,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def main():
    a = parse()
    if a.summarize_traffic:
        summarize_traffic(a)
        return
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {a.gpus} requested): the MoE forward "
              "here is a single-GPU hot path with no collectives.", file=sys.stderr)
        sys.exit(2)
    import mixture_experts_layer_21_amd as moe
    cfg = workload(a)
    torch.cuda.set_device(0)
    if a.calibrate_copy_mib:
        calibrate_copy(a.calibrate_copy_mib)
        return
    if a.pass_ == "train":
        main_train(a, moe, cfg)
        return
    L = mi.make_inputs(cfg, "cuda")
    dev = "cuda"
    nbytes = moe.moe_workspace_bytes(cfg.T, cfg.H, cfg.E, cfg.k, cfg.F, cfg.torch_dtype)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    y = torch.empty((cfg.T, cfg.H), dtype=cfg.torch_dtype, device=dev)
    torch.cuda.synchronize()
    print(f"[bench] {cfg.name}: inputs ready, workspace {nbytes / 2**20:.0f} MiB", file=sys.stderr,
          flush=True)

    sec = time_forward(moe, L, cfg, a.steps, a.warmup, ws, y)
    print(f"[bench] timed region done: {sec * 1e3:.3f} ms/step", file=sys.stderr, flush=True)

    R = cfg.R
    bufs = (torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=dev),
            torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=dev),
            torch.empty(cfg.E + 1, dtype=torch.int32, device=dev),
            torch.empty(R, dtype=torch.int32, device=dev),
            torch.empty(R, dtype=torch.int32, device=dev),
            torch.empty((R, cfg.H), dtype=cfg.torch_dtype, device=dev),
            torch.empty((R, cfg.H), dtype=cfg.torch_dtype, device=dev),
            torch.empty((cfg.T, cfg.H), dtype=cfg.torch_dtype, device=dev), ws)
    stages = time_stages(moe, L, cfg, a.steps, bufs, flush=not a.no_flush)
    ids = bufs[0].cpu().numpy()
    flops, bytes_, touched = alg_counts(cfg, ids)
    counts = np.bincount(ids.ravel(), minlength=cfg.E)
    pb = pass_bytes(cfg, touched)
    hbm = {}
    for n, b in pb.items():
        gbs = b / (stages[n] * 1e-3) / 1e9
        hbm[n] = {"bytes": b, "gb_s": gbs, "frac": gbs / PEAK_HBM_GBS}

    g_flops, g_bytes = gemm_launch_counts(cfg, touched)
    g_sec = stages["expert_ffn"] / 2 * 1e-3         # two launches per FFN stage
    peak_mm = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    ridge = peak_mm * 1e12 / (PEAK_HBM_GBS * 1e9)
    if g_flops / g_bytes >= ridge:
        roof = {"bound": "mfma" if cfg.dtype == "bf16" else "alu",
                "achieved": g_flops / g_sec / 1e12, "peak": peak_mm, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": g_bytes / g_sec / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = read_traffic(cfg.name) if cfg.dtype == "bf16" else None
    roof["kernel"] = ("gemm_bf16_grouped + gemm_split_reduce" if cfg.dtype == "bf16"
                      else "gemm_f32_grouped")
    roof["per_launch"] = {"flops": g_flops, "bytes": g_bytes, "ms": g_sec * 1e3}

    cpu = check = None
    if not a.no_cpu_baseline:
        # (about 10 s of host work at most: the whole batch)
        n = a.cpu_sample_tokens or {"tiny_fp32": 64, "mixtral_bf16": 2048, "skewed_bf16": 2048,
                                    "many_experts_bf16": 4096,
                                    "weight_bound_bf16": 64}.get(cfg.name, min(cfg.T, 256))
        moe.moe_forward(L["x"], L["w_r"], L["router_bias"], L["w1"], L["w2"], cfg.k, y=y,
                        topk_ids_out=bufs[0], ws=ws)
        torch.cuda.synchronize()
        cpu, check = cpu_baseline(cfg, L, min(n, cfg.T), y, bufs[0].cpu().numpy())

    layer_tflops = flops / sec / 1e12
    out = {
        "metric": METRIC,
        "value": cfg.T / sec,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": sec * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded counter-based generator; random-init weights)",
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "E": cfg.E, "top_k": cfg.k,
                   "F": cfg.F, "router_bias0": cfg.bias0, "seed": cfg.seed},
        "layer_tflops": layer_tflops,
        "layer_alg_gflop": flops / 1e9,
        "layer_alg_gbytes": bytes_ / 1e9,
        "layer_roofline_frac": max(layer_tflops / peak_mm,
                                   bytes_ / sec / 1e9 / PEAK_HBM_GBS),
        "experts_touched": int(touched),
        "expert_rows": {"min": int(counts.min()), "max": int(counts.max())},
        "stages_ms": stages,
        "stages_flushed": not a.no_flush,
        "pass_hbm": hbm,
        "oracle_check": check,
        "attainable": {**attainable_hbm(), **attainable_gemm()},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
