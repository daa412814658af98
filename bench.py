"""Throughput of the NVFP4 hot path on one MI355X.

One step = one pass over every kernel of the path on its full-size synthetic
workload: dynamic quantize and dequantize of a 65536 x 6144 heavy-tailed bf16
tensor, and its columnwise quantization and transposed dequantization; the W4A16 GEMV at batch 1, 2, 4, 8 on o_proj (6144 x 16384) and
q_b_proj (16384 x 2048); the W4A4 GEMM (from bf16 and from a pre-packed
activation) and the W4A16 GEMM at M in {1, 8, ..., 4096} on both shapes; the routed-expert MoE layer (4096 tokens, 256 experts, top-8, hidden
6144, intermediate 2048) in W4A16 and W4A4 mode, with and without a rank-64
bf16 LoRA on its experts.  Inputs are resident in HBM
before timing starts.  GEMV and GEMM rows cycle through enough weight copies
(10 of o_proj, 30 of q_b_proj: about 565 MB each) that every launch reads its
weights from HBM, not from the 256 MB last-level cache.

The headline value is the batch-1 o_proj GEMV's effective HBM bandwidth
(packed codes + scale bytes per launch / mean launch time).  Per-kernel times
come from HIP events on the stream the kernels run on, around back-to-back
launches that the host enqueued ahead of the GPU.

Prints one JSON line.  --gpus N with N > 1 exits: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2516.6  # dense fp16 / bf16 MFMA
FP4_PEAK_TFLOPS = 10066.0      # dense MXFP4 (context only)
METRIC = "NVFP4 bs1 GEMV HBM TB/s; W4A4 GEMM/MoE TFLOPS; % of roofline"
TRAFFIC_FILE = "profiles/gemv_w4a16_o_proj_M1_hbm_traffic.md"
COPY_BYTES = 512 << 20
# sources of the kernel the traffic figure belongs to: a change to any of
# them voids the recorded figure
TRAFFIC_SOURCES = ("nvfp4_bit_block_amd/csrc/gemv.hip", "nvfp4_bit_block_amd/csrc/nvfp4_device.hpp")


def _sources_digest():
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_probe():
    import torch
    import nvfp4_bit_block_amd as nv
    import workloads as wl
    dev = torch.device("cuda", 0)
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    w, x = wl.gemv_inputs("o_proj")
    c, s, g = nv.quantize(torch.from_numpy(w.view(np.int16)).to(dev))
    x1 = torch.from_numpy(np.ascontiguousarray(x[:1]).view(np.int16)).to(dev)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    for _ in range(3):
        nv.gemv_w4a16(x1, c, s, g)
    torch.cuda.synchronize()
    print("traffic probe done", flush=True)


def _counter_per_dispatch(db, counter):
    import sqlite3
    con = sqlite3.connect(db)
    q = ("select dispatch_id, kernel_name, sum(value) from counters_collection "
         "where counter_name = ? group by dispatch_id order by dispatch_id")
    return [(k, v) for _, k, v in con.execute(q, (counter,))]


def traffic_parse(fetch_db, write_db):
    """Scale each counter by its reading for the copy of COPY_BYTES (read
    once, written once) and record the GEMV's HBM bytes per launch."""
    out = {}
    for counter, db in (("FETCH_SIZE", fetch_db), ("WRITE_SIZE", write_db)):
        rows = _counter_per_dispatch(db, counter)
        copy = [v for k, v in rows if "copy" in k.lower() or "elementwise" in k.lower()]
        gemv = [v for k, v in rows if "k_gemv" in k]
        if not copy or not gemv:
            raise SystemExit(f"{db}: no copy or GEMV dispatch with {counter}")
        factor = COPY_BYTES / (float(np.median(copy)) * 1024.0)
        out[counter] = {"copy_kib": float(np.median(copy)), "factor": factor,
                        "gemv_kib": float(np.median(gemv)), "gemv_bytes": float(np.median(gemv)) * 1024.0 * factor}
    algo = 6144 * 16384 // 2 + 6144 * 16384 // 16
    total = out["FETCH_SIZE"]["gemv_bytes"] + out["WRITE_SIZE"]["gemv_bytes"]
    rec = {"kernel": "k_gemv<1> batch-1 o_proj 6144x16384", "sources_sha256_16": _sources_digest(),
           "fetch_bytes": round(out["FETCH_SIZE"]["gemv_bytes"]), "write_bytes": round(out["WRITE_SIZE"]["gemv_bytes"]),
           "traffic_bytes": round(total), "algorithmic_bytes": algo}
    lines = [
        "# HBM traffic: batch-1 W4A16 GEMV, o_proj 6144 x 16384", "",
        "Commands (repository root on an MI355X; $OUT is an output directory; two counter passes, then this file):", "",
        "```",
        "cd /tmp && export TMPDIR=/tmp",
        "timeout -s KILL 60 rocprofv3 --pmc FETCH_SIZE -d $OUT/pmc_fetch -o run -- "
        "python3 $REPO/bench.py --traffic-probe",
        "timeout -s KILL 60 rocprofv3 --pmc WRITE_SIZE -d $OUT/pmc_write -o run -- "
        "python3 $REPO/bench.py --traffic-probe",
        "python3 bench.py --traffic-parse $OUT/pmc_fetch/run_results.db $OUT/pmc_write/run_results.db",
        "```", "",
        f"Each counter is scaled by bytes / counter for a plain {COPY_BYTES >> 20} MiB device copy "
        "(torch copy_: the same bytes read and written), medians over three dispatches.", "",
        "| counter | copy (KiB) | scale | GEMV (KiB) | GEMV bytes |", "|---|---|---|---|---|",
    ]
    for ctr, d in out.items():
        lines.append(f"| {ctr} | {d['copy_kib']:.0f} | {d['factor']:.4f} | {d['gemv_kib']:.0f} | {d['gemv_bytes']:.0f} |")
    lines += ["", f"Algorithmic bytes per launch (codes + scales): {algo}; measured HBM traffic per launch: "
              f"{total:.0f} ({total / algo:.3f} x).", "",
              "traffic-json: " + json.dumps(rec)]
    with open(os.path.join(ROOT, TRAFFIC_FILE), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(json.dumps(rec))


def counter_probe(kind):
    """Launch a plain 512 MiB copy three times, then the kernels of one row
    three times, for a rocprofv3 --pmc pass (kind: quantize, gemm, gemm_small
    or moe)."""
    import torch
    import nvfp4_bit_block_amd as nv
    import workloads as wl
    dev = torch.device("cuda", 0)
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    if kind == "quantize":
        x = to_dev(wl.heavy_tailed(65536, 6144, seed=1))
        ws = nv.workspace(nv.quantize_workspace_size(65536, 6144), dev)
        run = lambda: nv.quantize(x, ws=ws)
    elif kind == "gemm":
        w, _ = wl.gemv_inputs("q_b_proj")
        wq = nv.quantize(to_dev(w))
        wo, _ = wl.gemv_inputs("o_proj")
        woq = nv.quantize(to_dev(wo))
        xs = {}
        for name, K in (("q_b_proj", 2048), ("o_proj", 16384)):
            x = to_dev(wl.activations(4096, K, seed=4))
            isc = torch.empty(1, dtype=torch.float32, device=dev)
            nv.quantize(x, global_scale=isc)
            xs[name] = (x, isc)

        def run():
            nv.gemm_w4a4(xs["q_b_proj"][0], xs["q_b_proj"][1], *wq)
            nv.gemm_w4a4(xs["o_proj"][0], xs["o_proj"][1], *woq)
    elif kind == "gemm_small":
        # the weight-streaming regime: W4A4 at M = 32 on both layers
        w, _ = wl.gemv_inputs("q_b_proj")
        wq = nv.quantize(to_dev(w))
        wo, _ = wl.gemv_inputs("o_proj")
        woq = nv.quantize(to_dev(wo))
        xs = {}
        for name, K in (("q_b_proj", 2048), ("o_proj", 16384)):
            x = to_dev(wl.activations(32, K, seed=4))
            isc = torch.empty(1, dtype=torch.float32, device=dev)
            nv.quantize(x, global_scale=isc)
            xs[name] = (x, isc)

        def run():
            nv.gemm_w4a4(xs["q_b_proj"][0], xs["q_b_proj"][1], *wq)
            nv.gemm_w4a4(xs["o_proj"][0], xs["o_proj"][1], *woq)
    elif kind == "moe":
        # the bench's MoE layer (T 4096, 256 experts, top-8, H 6144, I 2048)
        T, E, k, H, I = wl.MOE_T, wl.MOE_E, wl.MOE_TOPK, wl.MOE_H, wl.MOE_I
        ids, wts = wl.moe_routing(T, E, k, seed=5)
        xm = to_dev(wl.moe_tokens(T, H, seed=55))
        w13 = [torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device=dev),
               torch.empty((E, 2 * I, H // 16), dtype=torch.uint8, device=dev),
               torch.empty(E, dtype=torch.float32, device=dev)]
        w2 = [torch.empty((E, H, I // 2), dtype=torch.uint8, device=dev),
              torch.empty((E, H, I // 16), dtype=torch.uint8, device=dev),
              torch.empty(E, dtype=torch.float32, device=dev)]
        for e, a, b in wl.moe_expert_weights_iter(E, H, I, seed=50, threads=16):
            nv.quantize(to_dev(a), codes=w13[0][e], scales=w13[1][e], global_scale=w13[2][e:e + 1])
            nv.quantize(to_dev(b), codes=w2[0][e], scales=w2[1][e], global_scale=w2[2][e:e + 1])
        ids_d, wts_d = torch.from_numpy(ids).to(dev), torch.from_numpy(wts).to(dev)
        tmp = torch.empty(1, dtype=torch.float32, device=dev)
        nv.quantize(xm, global_scale=tmp)
        a13 = tmp.expand(E).contiguous()
        a2 = torch.full((E,), 2.0 * H * 0.02 ** 2 * float(np.log(T * k * I)) / 2688.0, dtype=torch.float32,
                        device=dev)

        def run():
            nv.moe_grouped_gemm(xm, ids_d, wts_d, *w13, *w2, mode=nv.MODE_W4A16)
            nv.moe_grouped_gemm(xm, ids_d, wts_d, *w13, *w2, mode=nv.MODE_W4A4, a13_scale=a13, a2_scale=a2)
    else:
        raise SystemExit(f"unknown counter probe {kind!r}")
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    print(f"counter probe {kind} done", flush=True)


def counter_report(dbs):
    """Median per-dispatch value of every counter in rocprofv3 --pmc databases,
    per kernel and launch shape (markdown)."""
    import sqlite3
    print("| kernel | grid | counter | dispatches | median per dispatch |")
    print("|---|---|---|---|---|")
    for db in dbs:
        con = sqlite3.connect(db)
        cols = {r[1] for r in con.execute("pragma table_info(counters_collection)")}
        grid = next((c for c in ("grid_size", "grid_x", "grid_size_x") if c in cols), "0")
        q = (f"select dispatch_id, kernel_name, {grid}, counter_name, sum(value) from counters_collection "
             "group by dispatch_id, counter_name order by dispatch_id")
        vals = {}
        for _, k, grid, ctr, v in con.execute(q):
            short = k.replace("(anonymous namespace)::", "").replace("nvfp4::", "")
            short = short[5:].split(">(")[0] + ">" if short.startswith("void ") else short.split("(")[0]
            vals.setdefault((short[:90], grid, ctr), []).append(v)
        for (k, grid, ctr), v in vals.items():
            print(f"| `{k}` | {grid} | {ctr} | {len(v)} | {float(np.median(v)):.6g} |")


def trace_summary(db, filt):
    """Per-kernel durations from a rocprofv3 kernel-trace database, one row per
    kernel and launch shape, sorted by total time."""
    import sqlite3
    con = sqlite3.connect(db)
    q = ("select name, grid_x, workgroup_x, count(*), avg(duration) / 1000.0, min(duration) / 1000.0, "
         "max(duration) / 1000.0, sum(duration) / 1000.0, vgpr_count, accum_vgpr_count, lds_size, scratch_size "
         "from kernels group by name, grid_x, grid_y, grid_z order by sum(duration) desc")
    print("| kernel | grid (work-items) | wg | launches | avg us | min us | max us | total us | VGPR | AGPR | LDS B | scratch B |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|")
    for r in con.execute(q):
        name = r[0]
        if "nvfp4::" not in name or (filt and filt not in name):
            continue
        short = name.replace("(anonymous namespace)::", "").replace("nvfp4::", "")
        if short.startswith("void "):        # a template instantiation: keep its arguments
            short = short[5:].split(">(")[0] + ">"
        else:
            short = short.split("(")[0]
        print(f"| `{short[:100]}` | {r[1]} | {r[2]} | {r[3]} | {r[4]:.2f} | {r[5]:.2f} | {r[6]:.2f} | {r[7]:.0f} | "
              f"{r[8]} | {r[9]} | {r[10]} | {r[11]} |")


def recorded_traffic():
    """HBM bytes per launch of the batch-1 o_proj GEMV from the committed
    counter summary, or None when it is missing or the kernel changed."""
    try:
        with open(os.path.join(ROOT, TRAFFIC_FILE)) as fh:
            for line in fh:
                if line.startswith("traffic-json: "):
                    rec = json.loads(line[len("traffic-json: "):])
                    if rec.get("sources_sha256_16") == _sources_digest():
                        return rec
    except OSError:
        pass
    return None


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--rows", default="all", help="comma list of row groups: quant,gemv,gemm,moe or all")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target oracle time for the CPU baseline")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="only launch a plain 512 MiB copy and the batch-1 o_proj GEMV, three times each "
                         "(run this under rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE)")
    ap.add_argument("--counter-probe", choices=("quantize", "gemm", "gemm_small", "moe"),
                    help="only launch a plain 512 MiB copy, then the quantize of 65536 x 6144, the W4A4 GEMM at "
                         "M = 4096 on q_b_proj and o_proj, or the MoE layer in both modes, three times each "
                         "(run under rocprofv3 --pmc)")
    ap.add_argument("--counter-report", nargs="+", metavar="DB",
                    help="median per-dispatch counter values of rocprofv3 --pmc databases (markdown)")
    ap.add_argument("--trace-summary", nargs=2, metavar=("DB", "FILTER"),
                    help="print a markdown table of a rocprofv3 --kernel-trace database (kernels whose name "
                         "contains FILTER; '' for all library kernels)")
    ap.add_argument("--traffic-parse", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="turn the two rocprofv3 databases of --traffic-probe into " + TRAFFIC_FILE)
    return ap.parse_args()


class Row:
    """One kernel configuration: `calls` are zero-argument launchers that
    enqueue one launch each; `reps` launches per step cycle through them."""

    def __init__(self, name, calls, reps, nbytes=0.0, flops=0.0, info=None, keep=()):
        self.name, self.calls, self.reps = name, calls, reps
        self.keep = list(keep)      # device tensors the raw-pointer launches use
        self.nbytes, self.flops, self.info = nbytes, flops, dict(info or {})
        self.total_ms = 0.0
        self.launches = 0
        self.k = 0

    def enqueue(self):
        for _ in range(self.reps):
            self.calls[self.k % len(self.calls)]()
            self.k += 1


def main():
    args = parse()
    if args.traffic_parse:
        traffic_parse(*args.traffic_parse)
        return
    if args.trace_summary:
        trace_summary(*args.trace_summary)
        return
    if args.traffic_probe:
        traffic_probe()
        return
    if args.counter_probe:
        counter_probe(args.counter_probe)
        return
    if args.counter_report:
        counter_report(args.counter_report)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs the NVFP4 path on exactly one GPU; --gpus {args.gpus} "
              f"(WORLD_SIZE={world}) is not supported: the library has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import nvfp4_bit_block_amd as nv
    import workloads as wl

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    L = nv.lib()
    stream = torch.cuda.current_stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)
    groups = set(args.rows.split(",")) if args.rows != "all" else {"quant", "gemv", "gemm", "moe"}
    P = lambda t: ctypes.c_void_p(t.data_ptr())

    def check(st, what):
        if st != 0:
            raise RuntimeError(f"{what}: {L.nvfp4_last_error().decode()}")

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    t_setup = time.time()
    rows: list[Row] = []

    def progress(msg):
        print(f"[bench {time.time() - t_setup:6.1f}s] {msg}", file=sys.stderr, flush=True)

    # ------------------------------------------------------------ quantize --
    if "quant" in groups:
        R, C = 65536, 6144
        xq = to_dev(wl.heavy_tailed(R, C, seed=1))
        qc = torch.empty((R, C // 2), dtype=torch.uint8, device=dev)
        qs = torch.empty((R, C // 16), dtype=torch.uint8, device=dev)
        qg = torch.empty(4, dtype=torch.float32, device=dev)
        qws = nv.workspace(nv.quantize_workspace_size(R, C), dev)
        yq = torch.empty((R, C), dtype=torch.int16, device=dev)
        qargs = (P(xq), R, C, None, P(qc), P(qs), P(qg), P(qws), qws.numel(), sptr)
        dargs = (P(qc), P(qs), P(qg), R, C, P(yq), sptr)
        n = R * C
        qkeep = (xq, qc, qs, qg, qws, yq)
        rows.append(Row("quantize_65536x6144", [lambda: check(L.nvfp4_quantize(*qargs), "quantize")], 3, keep=qkeep,
                        nbytes=n * (2 + 2 + 0.5 + 0.0625),
                        info={"unique_bytes": n * 2.5625, "bound": "hbm",
                              "bytes_model": "two-pass: 2 B read (amax) + 2 B read + 0.5625 B written per element"}))
        progress("quantize workload ready")
        rows.append(Row("dequantize_65536x6144", [lambda: check(L.nvfp4_dequantize(*dargs), "dequantize")], 3, keep=qkeep,
                        nbytes=n * (0.5625 + 2), info={"bound": "hbm"}))
        # the Dgrad layouts: the columnwise copy (NVFP4 of x^T) and the rowwise
        # copy dequantized to bf16 and transposed
        ct = torch.empty((C, R // 2), dtype=torch.uint8, device=dev)
        st_ = torch.empty((C, R // 16), dtype=torch.uint8, device=dev)
        gt = torch.empty(4, dtype=torch.float32, device=dev)
        yt = torch.empty((C, R), dtype=torch.int16, device=dev)
        cargs = (P(xq), R, C, None, P(ct), P(st_), P(gt), P(qws), qws.numel(), sptr)
        targs = (P(qc), P(qs), P(qg), R, C, P(yt), sptr)
        tkeep = (ct, st_, gt, yt) + qkeep
        rows.append(Row("quantize_columnwise_65536x6144",
                        [lambda: check(L.nvfp4_quantize_columnwise(*cargs), "quantize_columnwise")], 3, keep=tkeep,
                        nbytes=n * (2 + 2 + 0.5 + 0.0625), info={"bound": "hbm", "bytes_model": "as quantize"}))
        rows.append(Row("dequantize_transpose_65536x6144",
                        [lambda: check(L.nvfp4_dequantize_transpose(*targs), "dequantize_transpose")], 3,
                        keep=tkeep, nbytes=n * (0.5625 + 2), info={"bound": "hbm"}))

    # ---------------------------------------------------------------- GEMV --
    layers = {}
    if "gemv" in groups or "gemm" in groups:
        for name, copies in (("o_proj", 10), ("q_b_proj", 30)):
            w, x = wl.gemv_inputs(name)
            N, K = w.shape
            c, s, g = nv.quantize(to_dev(w))
            torch.cuda.synchronize()
            cs = [(c.clone(), s.clone(), g.clone()) for _ in range(copies)]
            layers[name] = (N, K, cs, to_dev(x))
            del w
            progress(f"{name} weights ready ({copies} copies)")
    if "gemv" in groups:
        for name, (N, K, cs, x8) in layers.items():
            for M in wl.GEMV_M:
                y = torch.empty((M, N), dtype=torch.int16, device=dev)
                xm = x8[:M].contiguous()
                calls = []
                for c, s, g in cs:
                    a = (P(xm), M, N, K, P(c), P(s), P(g), P(y), sptr)
                    calls.append(lambda a=a: check(L.nvfp4_gemv_w4a16(*a), "gemv"))
                wbytes = N * K // 2 + N * K // 16
                # about 100 back-to-back launches per step, so the mean is the
                # steady state of a decode loop rather than the first launches
                # after the prefill spin
                reps = len(calls) * max(2, -(-100 // len(calls)))
                rows.append(Row(f"gemv_w4a16_{name}_M{M}", calls, reps, nbytes=wbytes, keep=(y, xm, cs),
                                flops=2.0 * M * N * K,
                                info={"bound": "hbm", "bytes_with_x_y": wbytes + 2 * M * K + 2 * M * N,
                                      "weight_copies": len(cs)}))

    # ---------------------------------------------------------------- GEMM --
    if "gemm" in groups:
        for name, (N, K, cs, _) in layers.items():
            for M in wl.GEMM_M_SWEEP:
                x = to_dev(wl.activations(M, K, seed=4))
                isc = torch.empty(4, dtype=torch.float32, device=dev)
                # static input_scale = amax(X)/(6*448), taken from the library's dynamic quantize
                nv.quantize(x, global_scale=isc[:1])
                y = torch.empty((M, N), dtype=torch.int16, device=dev)
                ws = nv.workspace(nv.gemm_w4a4_workspace_size(M, N, K), dev)
                use = cs   # launches cycle through all copies across steps (more than the 256 MB cache)
                calls = []
                for c, s, g in use:
                    a = (P(x), P(isc), M, N, K, P(c), P(s), P(g), P(y), P(ws), ws.numel(), sptr)
                    calls.append(lambda a=a: check(L.nvfp4_gemm_w4a4(*a), "gemm"))
                reps = max(2, min(2 * len(calls), (4 * 4096) // max(M, 1)))
                wbytes = N * K // 2 + N * K // 16
                rows.append(Row(f"gemm_w4a4_{name}_M{M}", calls, reps, nbytes=wbytes + 2 * M * K + 2 * M * N,
                                keep=(x, isc, y, ws, use),
                                flops=2.0 * M * N * K, info={"M": M, "N": N, "K": K}))
                # the same product on the activation pre-packed by a static quantize (serving split)
                ac = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
                asc = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
                ag = torch.empty(4, dtype=torch.float32, device=dev)
                check(L.nvfp4_quantize(P(x), M, K, P(isc), P(ac), P(asc), P(ag), None, 0, sptr), "static quantize")
                wsp = nv.workspace(L.nvfp4_gemm_w4a4_packed_workspace_size(M, N, K), dev)
                callsp = []
                for c, s, g in use:
                    a = (P(ac), P(asc), P(ag), M, N, K, P(c), P(s), P(g), P(y), P(wsp), wsp.numel(), sptr)
                    callsp.append(lambda a=a: check(L.nvfp4_gemm_w4a4_packed(*a), "gemm_packed"))
                rows.append(Row(f"gemm_w4a4_packed_{name}_M{M}", callsp, reps,
                                nbytes=wbytes + M * K * (0.5 + 1 / 16) + 2 * M * N, keep=(ac, asc, ag, y, wsp, use),
                                flops=2.0 * M * N * K, info={"M": M, "N": N, "K": K}))
                # the weight-only path on the same activation (bf16 operand, no quantize)
                ws16 = nv.workspace(nv.gemm_w4a16_workspace_size(M, N, K), dev)
                calls16 = []
                for c, s, g in use:
                    a = (P(x), M, N, K, P(c), P(s), P(g), P(y), P(ws16), ws16.numel(), sptr)
                    calls16.append(lambda a=a: check(L.nvfp4_gemm_w4a16(*a), "gemm_w4a16"))
                rows.append(Row(f"gemm_w4a16_{name}_M{M}", calls16, reps, nbytes=wbytes + 2 * M * K + 2 * M * N,
                                keep=(x, y, ws16, use),
                                flops=2.0 * M * N * K, info={"M": M, "N": N, "K": K}))

    # ----------------------------------------------------------------- MoE --
    moe_host = None
    if "moe" in groups:
        T, E, k, H, I = wl.MOE_T, wl.MOE_E, wl.MOE_TOPK, wl.MOE_H, wl.MOE_I
        ids, wts = wl.moe_routing(T, E, k, seed=5)
        xm = to_dev(wl.moe_tokens(T, H, seed=55))
        w13c = torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device=dev)
        w13s = torch.empty((E, 2 * I, H // 16), dtype=torch.uint8, device=dev)
        w13g = torch.empty(E, dtype=torch.float32, device=dev)
        w2c = torch.empty((E, H, I // 2), dtype=torch.uint8, device=dev)
        w2s = torch.empty((E, H, I // 16), dtype=torch.uint8, device=dev)
        w2g = torch.empty(E, dtype=torch.float32, device=dev)
        for e, w13, w2 in wl.moe_expert_weights_iter(E, H, I, seed=50, threads=16):
            nv.quantize(to_dev(w13), codes=w13c[e], scales=w13s[e], global_scale=w13g[e:e + 1])
            nv.quantize(to_dev(w2), codes=w2c[e], scales=w2s[e], global_scale=w2g[e:e + 1])
            if e % 32 == 31:
                progress(f"moe experts {e + 1}/{E} quantized")
        ids_d = torch.from_numpy(ids).to(dev)
        wts_d = torch.from_numpy(wts).to(dev)
        out = torch.empty((T, H), dtype=torch.int16, device=dev)
        # static input scales, one per expert: a13 = amax(X)/(6*448) from the
        # library's dynamic quantize of X, the same value for every expert (the
        # serving form, with the activation quantized once before routing: the
        # layer then quantizes each token once); a2 is a generous analytic estimate
        # for h = silu(g)*u with g, u ~ N(0, s2), s2 = H * 0.02^2 * E[x^2]:
        # |h| stays below s2 * ln(#h) with margin, doubled (the pages' static
        # input_scale is likewise a generous per-tensor heuristic).
        a13 = torch.empty(E, dtype=torch.float32, device=dev)
        tmp = torch.empty(4, dtype=torch.float32, device=dev)
        nv.quantize(xm, global_scale=tmp[:1])
        a13[:] = tmp[0]
        s2 = H * 0.02 ** 2
        a2 = torch.full((E,), 2.0 * s2 * float(np.log(T * k * I)) / 2688.0, dtype=torch.float32, device=dev)
        def moe_host(ts=4):
            # the first ts tokens and the experts they use (renumbered), for
            # the CPU baseline
            used = sorted(set(int(e) for e in ids[:ts].ravel()))
            remap = {e: i for i, e in enumerate(used)}
            idx = torch.tensor(used, device=dev)
            pick = lambda t: t.index_select(0, idx).cpu().numpy()
            return {"x": xm[:ts].view(torch.int16).cpu().numpy().view(np.uint16),
                    "ids": np.vectorize(remap.get)(ids[:ts]).astype(np.int32), "wts": wts[:ts],
                    "w": [pick(t) for t in (w13c, w13s, w13g, w2c, w2s, w2g)], "a13": pick(a13), "a2": pick(a2),
                    "tokens": T, "experts": len(used)}

        moe_bytes = E * (2 * I * H + H * I) * (0.5 + 1 / 16) + 2 * T * H * 2
        moe_flops = 2.0 * T * k * (2 * I * H + H * I)
        for mode in (0, 1):
            p = nv.MoeProblem(T, E, k, H, I, mode)
            ws = nv.workspace(L.nvfp4_moe_workspace_size(ctypes.byref(p)), dev)
            tens = nv.MoeTensors(xm.data_ptr(), ids_d.data_ptr(), wts_d.data_ptr(), w13c.data_ptr(),
                                 w13s.data_ptr(), w13g.data_ptr(), w2c.data_ptr(), w2s.data_ptr(),
                                 w2g.data_ptr(), a13.data_ptr() if mode else None,
                                 a2.data_ptr() if mode else None, out.data_ptr())
            a = (ctypes.byref(p), ctypes.byref(tens), P(ws), ws.numel(), sptr)
            call = (lambda a=a, p=p, tens=tens, ws=ws: check(L.nvfp4_moe_grouped_gemm(*a), "moe"))
            rows.append(Row(f"moe_{'w4a16' if mode == 0 else 'w4a4'}", [call], 1, nbytes=moe_bytes,
                            keep=(xm, ids_d, wts_d, w13c, w13s, w13g, w2c, w2s, w2g, a13, a2, out, ws),
                            flops=moe_flops, info={"T": T, "E": E, "top_k": k, "H": H, "I": I,
                                                   "bytes_model": "NVFP4 expert weights + x + out"}))
        # the same layer with a rank-64 bf16 LoRA on every expert projection
        # (one A shared by the experts, one B per expert)
        R = wl.MOE_LORA_RANK
        lo = {n: to_dev(v) for n, v in wl.moe_lora(E, H, I, rank=R, seed=56).items()}
        lcs = nv.MoeLora(R, 1.0, lo["a13"].data_ptr(), lo["b13"].data_ptr(), lo["a2"].data_ptr(),
                         lo["b2"].data_ptr())
        lora_bytes = 2 * R * (H + I) + 2 * E * R * (2 * I + H)
        lora_flops = 2.0 * R * (T * H + T * k * (2 * I + I + H))
        for mode in (0, 1):
            p = nv.MoeProblem(T, E, k, H, I, mode)
            ws = nv.workspace(L.nvfp4_moe_lora_workspace_size(ctypes.byref(p), ctypes.byref(lcs)), dev)
            tens = nv.MoeTensors(xm.data_ptr(), ids_d.data_ptr(), wts_d.data_ptr(), w13c.data_ptr(),
                                 w13s.data_ptr(), w13g.data_ptr(), w2c.data_ptr(), w2s.data_ptr(),
                                 w2g.data_ptr(), a13.data_ptr() if mode else None,
                                 a2.data_ptr() if mode else None, out.data_ptr())
            a = (ctypes.byref(p), ctypes.byref(tens), ctypes.byref(lcs), P(ws), ws.numel(), sptr)
            call = (lambda a=a, p=p, tens=tens, ws=ws: check(L.nvfp4_moe_grouped_gemm_lora(*a), "moe lora"))
            rows.append(Row(f"moe_{'w4a16' if mode == 0 else 'w4a4'}_lora_r{R}", [call], 1,
                            nbytes=moe_bytes + lora_bytes,
                            keep=(xm, ids_d, wts_d, w13c, w13s, w13g, w2c, w2s, w2g, a13, a2, out, ws, lo, lcs),
                            flops=moe_flops + lora_flops,
                            info={"T": T, "E": E, "top_k": k, "H": H, "I": I, "lora_rank": R,
                                  "bytes_model": "NVFP4 expert weights + bf16 adapter + x + out"}))

    torch.cuda.synchronize()
    setup_s = time.time() - t_setup

    # ------------------------------------------------------------- timing --
    sleeper = _Sleeper(torch)

    def step(record):
        for r in rows:
            sleeper.prefill(r)
            if record:
                ev0 = torch.cuda.Event(enable_timing=True)
                ev1 = torch.cuda.Event(enable_timing=True)
                ev0.record(stream)
            r.enqueue()
            if record:
                ev1.record(stream)
                r._ev = (ev0, ev1)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    progress(f"warmup done; timing {args.steps} steps")
    events = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
        events.append([(r, r._ev) for r in rows])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for per_step in events:
        for r, (e0, e1) in per_step:
            r.total_ms += e0.elapsed_time(e1)
            r.launches += r.reps

    # Per-launch spread of the batch-1 GEMVs: one more pass with an event
    # between consecutive launches (the event markers add a little time of
    # their own, so the mean above stays the reported figure).
    spread = {}
    for r in rows:
        if r.name not in ("gemv_w4a16_o_proj_M1", "gemv_w4a16_q_b_proj_M1"):
            continue
        sleeper.prefill(r)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(r.reps + 1)]
        evs[0].record(stream)
        for i in range(r.reps):
            r.calls[r.k % len(r.calls)]()
            r.k += 1
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        per = np.array([1e3 * evs[i].elapsed_time(evs[i + 1]) for i in range(r.reps)])
        spread[r.name] = {"marked_us_median": round(float(np.median(per)), 3),
                          "marked_us_p10": round(float(np.percentile(per, 10)), 3),
                          "marked_us_p90": round(float(np.percentile(per, 90)), 3),
                          "marked_launches": int(r.reps),
                          "marked_note": "per-launch times with an event marker between launches "
                                         "(each marker adds a few us); for the spread, not the rate"}

    report = {}
    for r in rows:
        us = 1e3 * r.total_ms / max(r.launches, 1)
        d = {"us_per_launch": round(us, 3)}
        if r.nbytes:
            gbs = r.nbytes / (us * 1e-6) / 1e9
            d["GB_s"] = round(gbs, 1)
            d["frac_hbm_peak"] = round(gbs / HBM_PEAK_GBS, 4)
        if r.flops:
            tf = r.flops / (us * 1e-6) / 1e12
            d["TFLOPS"] = round(tf, 2)
            d["frac_mfma_f16_peak"] = round(tf / MFMA_F16_PEAK_TFLOPS, 4)
        d.update({k: v for k, v in r.info.items() if k not in ("M", "N", "K")})
        d.update(spread.get(r.name, {}))
        report[r.name] = d

    head = report.get("gemv_w4a16_o_proj_M1")
    value = head["GB_s"] / 1e3 if head else None
    roofline = None
    if head:
        tr = recorded_traffic()
        roofline = {"kernel": "k_gemv<1> (nvfp4_gemv_w4a16, o_proj 6144x16384, M=1)", "bound": "hbm",
                    "achieved": head["GB_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(head["GB_s"] / HBM_PEAK_GBS, 4),
                    "traffic": None if tr is None else tr["traffic_bytes"],
                    "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-scaled; " + TRAFFIC_FILE + ")",
                    "bytes_per_launch": 6144 * 16384 // 2 + 6144 * 16384 // 16,
                    "us_per_launch": head["us_per_launch"]}
    progress("timed steps done")
    ceil = measure_ceilings(torch, dev, stream, sleeper)
    if roofline is not None:
        roofline["ceiling"] = ceil
        roofline["frac_of_copy_ceiling"] = round(roofline["achieved"] / ceil["copy_1GiB_GB_s"], 4)
        roofline["frac_of_same_size_read_ceiling"] = round(roofline["achieved"] / ceil["read_56.6MB_GB_s"], 4)
    progress("ceilings measured")
    cpu = None
    if not args.no_cpu_baseline:
        host = {}
        if layers:
            host["layers"] = {name: (cs[0][0].cpu().numpy(), cs[0][1].cpu().numpy(), np.float32(cs[0][2].item()),
                                     x8.view(torch.int16).cpu().numpy().view(np.uint16))
                              for name, (N, K, cs, x8) in layers.items()}
        if moe_host is not None:
            host["moe"] = moe_host()
        cpu = cpu_baseline(args.cpu_seconds, host)
        progress("cpu baseline done")
    line = {
        "metric": METRIC, "value": None if value is None else round(value, 4), "unit": "TB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(1e3 * (t1 - t0) / args.steps, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded numpy draws, bf16; NVFP4 weights quantized on the GPU)",
        "config": {"workload": "W4A16 batch-1 decode GEMV on NVFP4 o_proj [6144 x 16384]; step also runs "
                               "quantize/dequantize (rowwise, columnwise, transposed) 65536x6144, GEMV M=1..8 on o_proj and q_b_proj, "
                               "W4A4 (bf16 and pre-packed activation) and W4A16 GEMM M=1..4096 on both, MoE T=4096 E=256 top-8 H=6144 I=2048",
                   "gpu": torch.cuda.get_device_name(0), "setup_s": round(setup_s, 1),
                   "timing": "HIP events around back-to-back launches enqueued behind a prefill kernel"},
        "roofline": roofline, "cpu_baseline": cpu, "hbm_ceiling": ceil, "rows": report,
    }
    print(json.dumps(line))


def measure_ceilings(torch, dev, stream, sleeper):
    """HBM ceilings measured in the same run: a plain device copy of 1 GiB
    (bytes read + written per second), and the read ceiling of one launch
    of the headline GEMV's size: the probe kernel of libnvfp4_probe.so,
    which only streams 56,623,104 bytes with 16-byte non-temporal loads
    (each wave instruction 1 KB contiguous), over ten buffers in turn so that
    each launch reads HBM, back to back like the GEMV rows; the best of
    several grid sizes and load depths is the ceiling."""
    out = {}

    def timed(fn, reps):
        fn(0)
        torch.cuda.synchronize()
        if sleeper.ok:
            torch.cuda._sleep(sleeper.cycles)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    t = timed(lambda i: dst.copy_(src), 10)
    out["copy_1GiB_GB_s"] = round(2 * n / t / 1e9, 1)
    del src, dst
    from nvfp4_bit_block_amd import build as nvbuild
    probe = ctypes.CDLL(nvbuild.PROBE_PATH)
    probe.nvfp4probe_stream_read.restype = ctypes.c_int32
    probe.nvfp4probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_void_p, ctypes.c_void_p]
    nb = 6144 * 16384 // 2 + 6144 * 16384 // 16
    bufs = [torch.ones(nb, dtype=torch.uint8, device=dev) for _ in range(10)]
    sink = torch.empty(4096, dtype=torch.int32, device=dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    best = None
    for wgs in (256, 512, 768, 1024):
        for unroll in (4, 8):
            def run(i, wgs=wgs, unroll=unroll):
                st = probe.nvfp4probe_stream_read(ctypes.c_void_p(bufs[i % 10].data_ptr()), nb, wgs, unroll,
                                                  ctypes.c_void_p(sink.data_ptr()), sp)
                if st != 0:
                    raise RuntimeError(f"read probe status {st}")
            t = timed(run, 100)
            if best is None or t < best[0]:
                best = (t, wgs, unroll)
    out["read_56.6MB_us"] = round(best[0] * 1e6, 3)
    out["read_56.6MB_GB_s"] = round(nb / best[0] / 1e9, 1)
    out["read_probe_config"] = f"{best[1]} workgroups x 512 threads, {best[2]} loads in flight per thread"
    out["note"] = ("same-run ceilings: a device copy_ of 1 GiB (read + write bytes); the read-only probe over the "
                   "headline GEMV's 56,623,104 bytes, one launch per buffer, ten buffers rotated, best of 8 launch shapes")
    del bufs
    return out


class _Sleeper:
    """Enqueues a short GPU spin before each row so the host can queue that
    row's launches ahead of the GPU (the events then time GPU work only)."""

    def __init__(self, torch):
        self.torch = torch
        self.ok = hasattr(torch.cuda, "_sleep")
        self.cycles = 2_000_000
        if self.ok:
            try:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                torch.cuda._sleep(self.cycles)
                e1.record()
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1)
                self.cycles = int(self.cycles * min(4.0, max(0.05, 1.0 / max(ms, 1e-3))))  # ~1 ms
            except Exception:
                self.ok = False

    def prefill(self, row):
        if self.ok:
            self.torch.cuda._sleep(self.cycles)


def _cpu_model():
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except Exception:
        pass
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(target_s: float, host=None):
    """The oracle (as it stands) on the host cores, on bounded samples of the
    step's workloads.  The headline value is the W4A16 GEMV over the full
    o_proj weight at batch 1, repeated for about `target_s` seconds; the rows
    time the other workloads once each: the GEMV at batch 1-8 on both layers
    (full size), the quantize on the first 4096 rows of the 65536 x 6144
    tensor, the W4A4 GEMM sweep on sampled weight rows (all M, both layers)
    and the MoE layer in both modes on 4 sampled tokens with the experts they
    use.  `host` carries the weights the GPU part set up (NVFP4 bytes copied
    back), when those row groups ran."""
    import oracle
    import workloads as wl
    threads = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(threads))
    host = host or {}
    rows = {}

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    layers = host.get("layers")
    if layers is None:
        layers = {}
        for name in ("o_proj", "q_b_proj"):
            w, x = wl.gemv_inputs(name)
            layers[name] = (*oracle.quantize(w), x)
    c, s, g, x8 = layers["o_proj"]
    n, t0 = 0, time.perf_counter()
    while True:
        oracle.gemv_w4a16(x8[:1], c, s, g)
        n += 1
        if time.perf_counter() - t0 >= target_s:
            break
    dt = (time.perf_counter() - t0) / n
    head = (c.nbytes + s.nbytes) / dt / 1e12
    for name, (c, s, g, x8) in layers.items():
        N, K = c.shape[0], c.shape[1] * 2
        wbytes = c.nbytes + s.nbytes
        for M in wl.GEMV_M:
            t = timed(lambda: oracle.gemv_w4a16(x8[:M], c, s, g))
            rows[f"gemv_w4a16_{name}_M{M}"] = {"s": round(t, 4), "TB_s": round(wbytes / t / 1e12, 6),
                                               "sample": f"full {N}x{K}, M={M}"}
    xq = wl.heavy_tailed(4096, 6144, seed=1)
    t = timed(lambda: oracle.quantize(xq))
    rows["quantize_65536x6144"] = {"s": round(t, 4), "GB_s": round(xq.size * 4.5625 / t / 1e9, 3),
                                   "sample": "first 4096 of 65536 rows (the same draw), dynamic scale; "
                                             "GB/s over the two-pass bytes of the sample"}
    for name, (c, s, g, _) in layers.items():
        N, K = c.shape[0], c.shape[1] * 2
        for M in wl.GEMM_M_SWEEP:
            ns = max(16, min(N, ((1 << 30) // (M * K)) // 16 * 16))
            x = wl.activations(M, K, seed=4)
            isc = oracle.global_scale(x)
            t = timed(lambda: oracle.gemm_w4a4(x, isc, c[:ns], s[:ns], g))
            rows[f"gemm_w4a4_{name}_M{M}"] = {"s": round(t, 4), "TFLOPS": round(2.0 * M * ns * K / t / 1e12, 6),
                                              "sample": f"{ns} of {N} weight rows, M={M}, K={K}"}
    moe = host.get("moe")
    if moe is not None:
        x, ids, wts, w = moe["x"], moe["ids"], moe["wts"], moe["w"]
        ts, H, I = x.shape[0], x.shape[1], w[3].shape[2] * 2
        flops = 2.0 * ts * ids.shape[1] * (2 * I * H + H * I)
        for mode in (0, 1):
            kw = {} if mode == 0 else {"a13": moe["a13"], "a2": moe["a2"]}
            t = timed(lambda: oracle.moe(x, ids, wts, *w, mode=mode, **kw))
            rows[f"moe_{'w4a16' if mode == 0 else 'w4a4'}"] = {
                "s": round(t, 4), "TFLOPS": round(flops / t / 1e12, 6),
                "sample": f"{ts} of {moe['tokens']} tokens ({ts * ids.shape[1]} slots over the {moe['experts']} "
                          f"experts they use; the oracle dequantizes each used expert once)"}
    return {"value": round(head, 6), "unit": "TB/s", "cores": int(os.environ.get("OMP_NUM_THREADS", threads)),
            "kind": "oracle", "cpu_model": _cpu_model(),
            "sample": f"headline: W4A16 GEMV o_proj 6144x16384 at M=1 (fp64 oracle incl. its dequantize), "
                      f"{n} calls, {dt:.3f} s per call; rows: the other workloads, one call each on the stated "
                      f"samples", "rows": rows}


if __name__ == "__main__":
    main()
