"""Benchmark of the GEMM hot path on one MI355X.

One step = one BF16 GEMM at M=N=K=4096 (A row-major, B column-major, beta 0.5
on an FP32 C, as in the square 4096^3 workload) followed by one FP8-E4M3
per-token/per-channel scaled GEMM at M=N=K=4096 (bias, GELU, BF16 output).
`value` is the step's throughput: 2MNK flops of both GEMMs over the time of
both, in TFLOP/s, inputs resident in HBM. Buffer sets rotate so that every
call reads operands that are not in the 256 MB MALL.

Also reported (not in `value`): each GEMM's TFLOP/s and fraction of the
dense MFMA peak, the FP8 4096x7168x2048 projection, decode-shaped skinny GEMMs
in achieved HBM GB/s, FFN projection shapes, and the ragged 4093^3 shapes.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from dense_gemm_09_amd.roofline import MI355X_HBM_GBPS, MI355X_PEAK_TFLOPS  # noqa: E402

PEAK = {k: MI355X_PEAK_TFLOPS[k] for k in ("bf16", "fp8")}  # TFLOP/s, MI355X dense
HBM_GBPS = MI355X_HBM_GBPS
ROTATE_BYTES = 600 << 20  # > 2 x (256 MB MALL + 32 MB L2)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-rotate", action="store_true", help="reuse one buffer set (MALL-hot)")
    ap.add_argument("--pmc-run", action="store_true",
                    help="short run for rocprofv3 --pmc: a 256 MiB device copy (counter "
                         "calibration) then 3 launches of each headline GEMM")
    ap.add_argument("--pmc-decode", action="store_true",
                    help="short run for rocprofv3 --pmc: a 256 MiB device copy (counter "
                         "calibration) then the FP8 and BF16 decode GEMMs M=1, N=18432, K=4096 "
                         "over their rotating buffer sets, each set used twice")
    ap.add_argument("--only", default="", help="comma list of extra groups: decode,ffn,ragged,proj,quant,qout,mx,pack")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Workload:
    """A problem resident on the GPU in `copies` rotating buffer sets."""

    def __init__(self, p, copies):
        import torch
        from tests.gpu_util import to_device
        self.p = p
        base = to_device(p)
        self.sets = [base]
        for _ in range(copies - 1):
            self.sets.append({k: (v.clone() if v is not None else None) for k, v in base.items()})
        import dense_gemm_09_amd as g
        need = g.workspace_size(p.M, p.N, p.K, p.kind != "bf16")
        self.ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda") if need else None
        self.i = 0

    def nbytes_per_set(self):
        return sum(v.numel() * v.element_size() for v in self.sets[0].values() if v is not None)

    def __call__(self):
        from tests.gpu_util import call
        d = self.sets[self.i % len(self.sets)]
        self.i += 1
        call(self.p, d, workspace=self.ws)


NO_ROTATE = False


def copies_for(p):
    import numpy as np
    if NO_ROTATE:
        return 1
    per = sum(a.nbytes for a in (p.A, p.B, p.C) if a is not None)
    return int(max(1, min(24, np.ceil(ROTATE_BYTES / max(per, 1)))))


def time_calls(fns, steps, warmup):
    """Run the callables in order per step; per-callable mean ms from HIP events."""
    import torch
    s = torch.cuda.current_stream()
    warm(fns, warmup)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(steps)]
    t0 = time.perf_counter()
    for k in range(steps):
        ev[k][0].record(s)
        for j, f in enumerate(fns):
            f()
            ev[k][j + 1].record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [sum(ev[k][j].elapsed_time(ev[k][j + 1]) for k in range(steps)) / steps
           for j in range(len(fns))]
    total = sum(ev[k][0].elapsed_time(ev[k][-1]) for k in range(steps))
    return per, total, wall


def warm(fns, warmup):
    """`warmup` untimed calls of each callable, and at least one call on each of
    its rotating buffer sets, so that no set is first touched while timed."""
    import torch
    for f in fns:
        for _ in range(max(warmup, len(getattr(f, "sets", ())))):
            f()
    torch.cuda.synchronize()


def time_blocks(fns, steps, warmup):
    """`steps` steps of the callables, run callable by callable: all `steps`
    calls of the first back to back, then of the second, ... (the same work as
    `steps` interleaved steps). HIP events only at block edges on the kernels'
    stream (the current stream, which the calls launch on), so a per-callable
    mean (ms) is its kernels' back-to-back time, with no timing packet between
    launches. Returns (per-callable ms, total ms, wall s)."""
    import torch
    s = torch.cuda.current_stream()
    warm(fns, warmup)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)]
    t0 = time.perf_counter()
    ev[0].record(s)
    for j, f in enumerate(fns):
        for _ in range(steps):
            f()
        ev[j + 1].record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [ev[j].elapsed_time(ev[j + 1]) / steps for j in range(len(fns))]
    return per, ev[0].elapsed_time(ev[-1]), wall


def launch_medians(fns, steps):
    """Median per-launch time (ms) of each callable: an event pair around every
    call (after the callables have been warmed by time_blocks)."""
    import torch
    s = torch.cuda.current_stream()
    out = []
    for f in fns:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for a, b in ev:
            a.record(s)
            f()
            b.record(s)
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) for a, b in ev)
        out.append(t[len(t) // 2])
    return out


def time_graph(fn, calls, reps=5):
    """Mean time per call (ms) of `calls` back-to-back calls captured in one HIP
    graph and replayed `reps` times (launch cost of the host side excluded, as in
    a decode loop that replays a captured graph)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * calls)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(bf16_p, fp8_p, min_seconds=12.0):
    """The oracle as it stands on the host, on the headline step's own inputs: blocks of
    256 rows of the BF16 and of the FP8 4096^3 GEMM (decode from the bit fields,
    the ascending-k float64 triple loop of oracle/triple_loop.c with OpenMP over rows,
    the epilogue and the output rounding), cycling through the rows, until
    min_seconds have passed (a bounded sample)."""
    import numpy as np
    import oracle  # noqa: F401  (the CPU-baseline leg is the one bench path allowed to use it)
    from oracle import native
    from tests.common import reference
    _, threads = native.accumulate(np.zeros((2, 1)), np.zeros((1, 1)), return_threads=True)
    block = 256
    flops = 0
    blocks = 0
    t0 = time.perf_counter()
    while True:
        r0 = (blocks * block) % bf16_p.M
        rows = np.arange(r0, min(r0 + block, bf16_p.M))
        for p in (bf16_p, fp8_p):
            reference(p, rows=rows)
            flops += 2 * len(rows) * p.N * p.K
        blocks += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    steps = blocks * block / bf16_p.M
    return {"value": flops / dt / 1e12, "unit": "TFLOPS", "cores": int(threads), "kind": "oracle",
            "affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
            "timed": "oracle.gemm_bf16 + oracle.gemm_fp8_scaled: bit-field decode, float64 "
                     "i-k-j triple loop (oracle/triple_loop.c, OpenMP over output rows), "
                     "epilogue, output rounding",
            "sample": f"{blocks} blocks of 256 rows of the BF16 and of the FP8 4096^3 GEMM "
                      f"({steps:.3f} steps), {dt:.1f} s, {threads} OpenMP threads"}


def kernel_source_sha():
    """Hash of every library source (csrc/*, include/*): a profile taken on
    another tree does not describe this one."""
    import hashlib
    h = hashlib.sha256()
    files = []
    for d in (os.path.join(ROOT, "dense_gemm_09_amd", "csrc"), os.path.join(ROOT, "include")):
        files += sorted(os.path.join(d, f) for f in os.listdir(d)
                        if f.endswith((".hip", ".hpp", ".cpp", ".h")))
    for path in files:
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the BF16 4096^3 kernel from the committed counter
    summary, or None when the kernel source changed after the counters were taken."""
    path = os.path.join(ROOT, "profiles", "gemm_tile_bf16_4096_traffic.md")
    try:
        text = open(path).read()
    except OSError:
        return None
    rec = dict(line.split(": ", 1) for line in text.splitlines()
               if line.startswith(("kernel_source_sha256: ", "traffic_bytes_per_launch: ")))
    if rec.get("kernel_source_sha256", "").strip() != kernel_source_sha():
        return None
    return int(rec["traffic_bytes_per_launch"])


def pmc_run(p_bf16, p_fp8):
    """Known-size copy (calibrates FETCH_SIZE / WRITE_SIZE), then the GEMMs over
    their rotating buffer sets, as in the timed run: every launch after the
    first round reads operands that are not in the caches."""
    import torch
    src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    w_bf16, w_fp8 = Workload(p_bf16, copies_for(p_bf16)), Workload(p_fp8, copies_for(p_fp8))
    n = 2 * max(len(w_bf16.sets), len(w_fp8.sets))
    for _ in range(n):
        w_bf16()
    for _ in range(n):
        w_fp8()
    torch.cuda.synchronize()
    log(f"[bench] pmc run done: copy 268435456 bytes, {n} x bf16 4096^3 over "
        f"{len(w_bf16.sets)} sets, {n} x fp8 4096^3 over {len(w_fp8.sets)} sets")


def pmc_decode():
    """Known-size copy, then the M=1, N=18432 decode GEMMs over rotating buffer
    sets (after the first round every launch reads weights that are not in the
    caches)."""
    import torch
    from synth import workloads
    src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    for kind in ("fp8", "bf16"):
        p = workloads.decode(kind, 1, 18432)
        w = Workload(p, copies_for(p))
        for _ in range(2 * len(w.sets)):
            w()
        torch.cuda.synchronize()
        log(f"[bench] pmc decode: {2 * len(w.sets)} x {kind} 1x18432x4096 over {len(w.sets)} sets")
        del w
        torch.cuda.empty_cache()


def main():
    args = parse()
    global NO_ROTATE
    NO_ROTATE = args.no_rotate
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(this path has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)
    import torch
    import dense_gemm_09_amd as g
    from synth import workloads
    g.lib()  # fail loudly if the HIP library is missing
    torch.cuda.init()

    if args.pmc_decode:
        pmc_decode()
        return
    log("[bench] generating inputs")
    p_bf16 = workloads.square_bf16(4096)
    p_fp8 = workloads.fp8_projection(4096, 4096, 4096, sub=1)
    if args.pmc_run:
        pmc_run(p_bf16, p_fp8)
        return
    w_bf16 = Workload(p_bf16, copies_for(p_bf16))
    w_fp8 = Workload(p_fp8, copies_for(p_fp8))
    log(f"[bench] rotation: bf16 {len(w_bf16.sets)} sets x {w_bf16.nbytes_per_set() / 1e6:.0f} MB, "
        f"fp8 {len(w_fp8.sets)} x {w_fp8.nbytes_per_set() / 1e6:.0f} MB")

    log(f"[bench] timing {args.steps} steps after {args.warmup} warmup")
    torch.cuda.synchronize()
    per, total_ms, wall = time_blocks([w_bf16, w_fp8], args.steps, args.warmup)
    torch.cuda.synchronize()
    med = launch_medians([w_bf16, w_fp8], args.steps)
    ms_step = total_ms / args.steps
    fl_bf16, fl_fp8 = p_bf16.flops, p_fp8.flops
    tf_bf16 = fl_bf16 / (per[0] * 1e-3) / 1e12
    tf_fp8 = fl_fp8 / (per[1] * 1e-3) / 1e12
    value = (fl_bf16 + fl_fp8) / (ms_step * 1e-3) / 1e12
    log(f"[bench] bf16 {per[0] * 1e3:.1f} us {tf_bf16:.0f} TF ({tf_bf16 / PEAK['bf16']:.1%}) | "
        f"fp8 {per[1] * 1e3:.1f} us {tf_fp8:.0f} TF ({tf_fp8 / PEAK['fp8']:.1%})")

    pl_bf16 = g.plan(4096, 4096, 4096, False)
    roof = {"bound": "mfma", "achieved": round(tf_bf16, 1), "peak": PEAK["bf16"],
            "unit": "TFLOP/s", "frac": round(tf_bf16 / PEAK["bf16"], 4),
            "traffic": measured_traffic(),
            "kernel": f"gemm_tile_kernel<{pl_bf16.tile_m},{pl_bf16.tile_n}> bf16 4096^3",
            "algorithmic_flops_per_launch": fl_bf16, "avg_launch_us": round(per[0] * 1e3, 2)}

    extra = {"bf16_4096": {"us": round(per[0] * 1e3, 2), "tflops": round(tf_bf16, 1),
                           "frac_peak": round(tf_bf16 / PEAK["bf16"], 4),
                           "median_launch_us": round(med[0] * 1e3, 2)},
             "fp8_4096": {"us": round(per[1] * 1e3, 2), "tflops": round(tf_fp8, 1),
                          "frac_peak": round(tf_fp8 / PEAK["fp8"], 4),
                          "median_launch_us": round(med[1] * 1e3, 2)},
             "kernel_source_sha256": kernel_source_sha()}
    del w_bf16, w_fp8
    torch.cuda.empty_cache()

    if not args.no_extras:
        only = set(args.only.split(",")) if args.only else {"decode", "ffn", "ragged", "proj", "quant", "qout", "mx", "pack"}
        extra.update(run_extras(only))

    cpu = None
    if not args.no_cpu:
        log("[bench] cpu baseline (oracle)")
        cpu = cpu_baseline(p_bf16, p_fp8)

    out = {"metric": "GEMM TFLOPS (2MNK/s) bf16 & fp8 at 4096^3; % of MI355X MFMA peak",
           "value": round(value, 1), "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16+fp8", "data": "synthetic",
           "config": {"workload": "bf16 GEMM 4096^3 (A row-major, B col-major, beta 0.5, fp32 C) "
                                  "+ fp8-e4m3 GEMM 4096^3 (per-token/per-channel fp32 scales, "
                                  "bf16 bias, GELU, bf16 out)",
                      "M": 4096, "N": 4096, "K": 4096, "parallelism": "single GPU",
                      "rotating_buffer_sets": True},
           "roofline": roof, "cpu_baseline": cpu, "extra": extra}
    print(json.dumps(out), flush=True)


def run_extras(only):
    import numpy as np
    import torch
    from synth import workloads
    res = {}

    def measure(name, p, steps=30, warmup=5, hbm_bytes=None, graph=False):
        w = Workload(p, copies_for(p))
        if graph:
            us = time_graph(w, calls=4 * len(w.sets)) * 1e3
        else:
            per, _, _ = time_calls([w], steps, warmup)
            us = per[0] * 1e3
        r = {"us": round(us, 2), "tflops": round(p.flops / (us * 1e-6) / 1e12, 1)}
        if hbm_bytes is not None:
            r["gbps"] = round(hbm_bytes / (us * 1e-6) / 1e9, 0)
            r["frac_hbm"] = round(hbm_bytes / (us * 1e-6) / 1e9 / HBM_GBPS, 4)
        res[name] = r
        log(f"[bench] {name}: {r}")
        del w
        torch.cuda.empty_cache()

    if "proj" in only:
        measure("fp8_4096x7168x2048", workloads.fp8_projection())
    if "decode" in only:
        for kind, M, N in workloads.all_decode():
            p = workloads.decode(kind, M, N)
            es = 2 if kind == "bf16" else 1
            by = N * p.K * es + M * p.K * es + M * N * 2 + (8 * (M + N) if kind == "fp8" else 0)
            measure(f"decode_{kind}_{M}x{N}x4096", p, hbm_bytes=by, graph=True)
    if "ffn" in only:
        for M in workloads.FFN_M:
            for N, K in workloads.FFN_SHAPES:
                measure(f"ffn_bf16_{M}x{N}x{K}", workloads.ffn(M, N, K), steps=10, warmup=3)
    if "quant" in only:
        # Per-token FP8 quantisation of BF16 activations (the FP8 GEMM's A
        # operand): the projection's 4096 x 2048 and an FFN's 8192 x 4096.
        # HBM-bound: 2 bytes read + 1 byte written per element + 4 per row.
        import dense_gemm_09_amd as g
        import synth
        for M, K in ((4096, 2048), (8192, 4096)):
            x = synth.to_bf16_bits(synth.normal((M, K), 1.0, 0x5EED9000 + M))
            base = torch.from_numpy(x.view(np.int16)).cuda()
            n = 1 if NO_ROTATE else int(max(1, np.ceil(ROTATE_BYTES / (3 * M * K))))
            xs = [base] + [base.clone() for _ in range(n - 1)]
            qs = [torch.empty((M, K), dtype=torch.uint8, device="cuda") for _ in range(n)]
            ss = [torch.empty(M, dtype=torch.float32, device="cuda") for _ in range(n)]
            state = {"i": 0}

            def call():
                i = state["i"] % n
                state["i"] += 1
                g.quantize_fp8_rows(M, K, xs[i], K, qs[i], K, ss[i])

            us = time_graph(call, calls=4 * n) * 1e3
            by = 3 * M * K + 4 * M
            r = {"us": round(us, 2), "gbps": round(by / (us * 1e-6) / 1e9, 0),
                 "frac_hbm": round(by / (us * 1e-6) / 1e9 / HBM_GBPS, 4)}
            res[f"quant_fp8_rows_{M}x{K}"] = r
            log(f"[bench] quant_fp8_rows_{M}x{K}: {r}")
            del xs, qs, ss
            torch.cuda.empty_cache()
    if "mx" in only:
        # MX FP8 (E8M0 scale per 32 K elements of each row of A / column of B)
        # at 4096^3, BF16 out: the per-group variant of the FP8 GEMM.
        import synth
        p = synth.make_mx_problem(4096, 4096, 4096, seed_base=0x5EEDC000, c_dtype=synth.OUT_BF16,
                                  a_std=1.0, b_std=4096 ** -0.5, name="mxfp8_4096^3")
        measure("mxfp8_4096", p, steps=20, warmup=3)
    if "pack" in only:
        # Pre-laid-out weights: BF16 4096^3 with B row-major (N contiguous), as
        # called directly (register loader) and after one gemm_pack_b into
        # K-major rows (DMA path); and a fused projection (three 4096-column
        # weights concatenated along N) as one launch vs three.
        import dense_gemm_09_amd as g
        from synth import make_problem, ROW, COL, OUT_BF16, OUT_F32
        p = make_problem("bf16", 4096, 4096, 4096, seed_base=0x5EEDD200, layout_b=ROW,
                         c_dtype=OUT_F32, a_std=4096 ** -0.5, b_std=4096 ** -0.5,
                         name="bf16_4096^3_rowB")
        measure("bf16_4096_rowB_direct", p, steps=5, warmup=2)
        w = Workload(p, 1)
        d = w.sets[0]
        Bp = torch.empty((4096, 4096), dtype=torch.int16, device="cuda")

        def do_pack():
            g.pack_b(4096, 4096, d["B"], 4096, ROW, 2, Bp, 4096)

        per, _, _ = time_calls([do_pack], 20, 3)
        res["pack_b_bf16_4096x4096"] = {"us": round(per[0] * 1e3, 2),
                                        "gbps": round(2 * 2 * 4096 * 4096 / (per[0] * 1e-3) / 1e9, 0)}
        log(f"[bench] pack_b_bf16_4096x4096: {res['pack_b_bf16_4096x4096']}")
        import copy
        q = copy.copy(p)
        q.layout_b, q.ldb = COL, 4096
        q.B = Bp.cpu().numpy().view(np.uint16)
        q.name = "bf16_4096^3_packedB"
        del w
        measure("bf16_4096_packedB", q, steps=10, warmup=3)
        M, K, NS = 512, 4096, 4096
        fused = make_problem("bf16", M, 3 * NS, K, seed_base=0x5EEDD300, layout_b=COL,
                             c_dtype=OUT_BF16, a_std=1.0, b_std=0.02, name="proj_fused")
        wf = Workload(fused, copies_for(fused))
        per_f, _, _ = time_calls([wf], 20, 3)
        sets = wf.sets
        Cs = [torch.empty((M, NS), dtype=torch.int16, device="cuda") for _ in range(3)]
        ws = torch.empty(max(1, g.workspace_size(M, NS, K, False)), dtype=torch.uint8, device="cuda")
        st = {"i": 0}

        def three():
            dd = sets[st["i"] % len(sets)]
            st["i"] += 1
            for j in range(3):
                g.gemm_bf16(M, NS, K, 1.0, dd["A"], K, ROW, dd["B"][j * NS:(j + 1) * NS], K, COL,
                            0.0, Cs[j], NS, OUT_BF16, workspace=ws)

        per_3, _, _ = time_calls([three], 20, 3)
        res["proj_512x3x4096x4096"] = {"fused_us": round(per_f[0] * 1e3, 2),
                                       "three_launches_us": round(per_3[0] * 1e3, 2)}
        log(f"[bench] proj_512x3x4096x4096: {res['proj_512x3x4096x4096']}")
        del wf, sets, Cs
        torch.cuda.empty_cache()
    if "qout" in only:
        # The FP8 projection (4096 x 7168 x 2048, bias, GELU) with the
        # quantising epilogue: one byte per output element instead of BF16's
        # two, no separate quantisation pass.
        import dense_gemm_09_amd as g
        p = workloads.fp8_projection()
        w = Workload(p, copies_for(p))
        qs = [torch.empty((p.M, p.N), dtype=torch.uint8, device="cuda") for _ in w.sets]
        osc = torch.full((p.M,), 24.0, dtype=torch.float32, device="cuda")
        ozp = torch.zeros(p.M, dtype=torch.int32, device="cuda")
        for q_dtype, tag in ((g.QOUT_INT8, "int8"), (g.QOUT_E4M3, "e4m3")):
            state = {"i": 0}

            def call():
                i = state["i"] % len(w.sets)
                state["i"] += 1
                d = w.sets[i]
                g.gemm_fp8_scaled_quant(p.M, p.N, p.K, 1.0, d["A"], p.lda, p.layout_a, d["B"],
                                        p.ldb, p.layout_b, d["scale_a"], d["scale_b"], d["bias"],
                                        p.act, osc, ozp if q_dtype == g.QOUT_INT8 else None,
                                        qs[i], p.N, q_dtype, workspace=w.ws)

            per, _, _ = time_calls([call], 30, 5)
            us = per[0] * 1e3
            r = {"us": round(us, 2), "tflops": round(p.flops / (us * 1e-6) / 1e12, 1)}
            res[f"fp8_4096x7168x2048_q{tag}"] = r
            log(f"[bench] fp8_4096x7168x2048_q{tag}: {r}")
        del w, qs
        torch.cuda.empty_cache()
    if "ragged" in only:
        for kind in ("bf16", "fp8"):
            for padded in (False, True):
                p = workloads.ragged(kind, 4093, padded)
                measure(p.name, p, steps=5, warmup=2)
    return res


if __name__ == "__main__":
    main()
