"""Throughput of one decoder layer's linear path (ReSpinQuant online path) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload llama2-7b-prefill-w4a4] [--copies 2] [--no-cpu-baseline]

A step is one pass of the whole path over one batch: two correction sites
(correction + RMSNorm + per-token quantisation), two stand-in activation
quantisations (o_proj and down_proj inputs) and the four quantised linears
(q|k|v, o, gate|up, down). Inputs are resident in HBM before timing starts.
``--copies`` independent copies of every buffer are cycled so that a step
does not find the previous step's data in the 256 MB Infinity Cache.

Prints one JSON line. ``roofline`` describes the dominant kernel (the
quantised GEMM); ``stages`` gives every stage's time and roofline fraction;
``cpu_baseline`` is the CPU oracle timed on a bounded sample of the same
workload.
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
ALONE_COPIES = 16           # buffer copies the stage-alone pass rotates over
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix-core peak
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 matrix-core peak
FP4_PEAK_TOPS = 10100.0        # MI355X dense fp4 (and fp6) matrix-core peak
METRIC = "tokens/s per decoder-layer linear path (W4A4, D=4096, r=32); % HBM / MFMA peak"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    # a workload name from synth.WORKLOADS, or its position there (1-5)
    p.add_argument("--workload", "--config", dest="workload", default="llama2-7b-prefill-w4a4")
    p.add_argument("--copies", type=int, default=2)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample", type=int, default=2048,
                   help="tokens in the CPU oracle sample (capped at the workload; the whole 2048-token batch takes a few s on 16 cores)")
    p.add_argument("--no-dense", action="store_true", help="skip the dense h T comparator")
    p.add_argument("--prep", choices=("device", "host"), default="device",
                   help="where the synthetic sites are prepared (offline step, not timed in the step)")
    p.add_argument("--rank-sweep", action="store_true",
                   help="only the correction at every rank of the workload: its time, its error against dense h T "
                        "and the end-to-end error of the site's linear")
    p.add_argument("--mismatch", choices=("dense", "lowrank"), default="dense",
                   help="the rank sweep's site mismatch: the workload's (dense) or one with T - I of rank <= 64")
    p.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB (calibrates rocprofv3 byte counters) and exit")
    p.add_argument("--mha", action="store_true", help="all-D x D q/k/v projections instead of the GQA shapes")
    p.add_argument("--no-decode", action="store_true", help="skip the decode-size leg (1, 8 and 64 tokens)")
    p.add_argument("--no-workload-legs", action="store_true",
                   help="skip the short legs of the LLaMA-3-8B and LLaMA-2-70B workloads in the default run")
    p.add_argument("--cpu-one-core-sample", type=int, default=256, metavar="TOKENS",
                   help="tokens of the one-thread pass of the CPU oracle (0: skip it)")
    return p.parse_args()


def progress(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def copy_probe(mib: int) -> None:
    """A plain device-to-device copy of known size: under rocprofv3 --pmc its
    FETCH_SIZE / WRITE_SIZE per dispatch give the counters' scale factor."""
    import torch
    nbytes = mib << 20
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": nbytes, "copy_probe_bytes_written": nbytes, "dispatches": 3}))


def capture(fns, reps: int = 1):
    """One HIP graph of `reps` passes over the launches fns (each launched once
    outside the capture first); the launches allocate nothing and set no memory."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for fn in fns:
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(reps):
            for fn in fns:
                fn()
    return graph


def replay_ms(graphs, iters: int, stream) -> float:
    """Mean time of one replay, the graphs replayed in turn (events on the stream around all of them)."""
    import torch
    for i in range(max(3, len(graphs))):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(iters):
        graphs[i % len(graphs)].replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def copy_ceiling(nbytes: int, iters: int = 50):
    """Time of a plain device copy that moves nbytes (half read, half written), cold: the
    copies rotate over more than twice the 256 MB Infinity Cache, launched as one replayed
    HIP graph (as the stages are timed alone). The practical ceiling of a stage that
    streams the same bytes once."""
    import torch
    half = max(nbytes // 2 // 16 * 16, 16)
    nbuf = max(2, int((600 << 20) // (2 * half)) + 1)
    src = [torch.ones(half, dtype=torch.uint8, device="cuda") for _ in range(nbuf)]
    dst = [torch.empty(half, dtype=torch.uint8, device="cuda") for _ in range(nbuf)]
    stream = torch.cuda.current_stream()
    g = capture([lambda i=i: dst[i].copy_(src[i]) for i in range(nbuf)])
    ms = replay_ms([g], max(3, iters // nbuf), stream) / nbuf
    del g, src, dst
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return ms


def _time_ms(fn, iters: int, stream) -> float:
    import torch
    for _ in range(3):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(iters):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def dense_comparator(path, which: str = "A", iters: int = 20):
    """The dense alternative at one junction: h T as a D x D bf16 GEMM (the vendor
    library's, through torch) beside the rank-r correction kernel, and how far
    the correction is from the dense product."""
    import torch
    import rotation_bit_post_amd as B
    t32 = path.mismatch[which]
    h = path.bufs["h"]
    n, d = h.shape
    site = path.sites[which]
    stream = torch.cuda.current_stream()
    t_dev = torch.from_numpy(t32).to(device="cuda", dtype=h.dtype)
    dense = torch.empty_like(h)
    corr = torch.empty_like(h)
    ms_dense = _time_ms(lambda: torch.matmul(h, t_dev, out=dense), iters, stream)
    ms_corr = _time_ms(lambda: B.rsq_subspace_correct(h, corr, site.buf, site.r), iters, stream)
    ref = h.float() @ torch.from_numpy(t32).cuda()
    err_corr = float(torch.linalg.vector_norm(corr.float() - ref) / torch.linalg.vector_norm(ref))
    err_dense = float(torch.linalg.vector_norm(dense.float() - ref) / torch.linalg.vector_norm(ref))
    flops = 2.0 * n * d * d
    return {
        "junction": f"site {which}, {n} tokens, D={d}, r={site.r}, {str(h.dtype).split('.')[-1]}",
        "dense_ms": round(ms_dense, 5),
        "dense_tflops": round(flops / (ms_dense * 1e-3) / 1e12, 1),
        "dense_frac_bf16_peak": round(flops / (ms_dense * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        "correction_ms": round(ms_corr, 5),
        "speedup_vs_dense": round(ms_dense / ms_corr, 2),
        "correction_rel_l2_vs_dense_fp32": round(err_corr, 5),
        "dense_bf16_rel_l2_vs_dense_fp32": round(err_dense, 6),
        "note": "dense h T by the vendor bf16 GEMM (hipBLASLt through torch.matmul), for comparison only; "
                "the rank-r correction's distance from h T is the approximation the method makes",
    }


def rank_sweep(wl, mismatch: str = "dense", iters: int = 20):
    """Per rank of the workload: the correction's time, its distance from the dense h T, and the
    end-to-end error of the site's linear (q|k|v) against an unquantised float64 layer with dense T.

    mismatch: "dense" - the workload's site A (Cayley rotations of dense skew generators, T - I
    of full rank); "lowrank" - rotations whose skew generators have rank 2k = 32 (step 1), so T - I
    has rank at most 64 and the rank-64 correction is exact.
    Rank 0 is the path without a correction (RMSNorm + quantisation of h itself). The float64
    references are plain torch arithmetic on the GPU: they measure the method's error, they are
    not the parity oracle.
    """
    import torch
    import rotation_bit_post_amd as B
    from rotation_bit_post_amd import offline
    from rotation_bit_post_amd.path import make_site, synthetic_mismatch, quantize_weight_on_device
    import synth
    cfg = synth.workload(wl)
    eps = 1e-5
    ranks = cfg.ranks or (cfg.r,)
    progress(f"rank sweep on {cfg.name} ({mismatch} mismatch): ranks {ranks}")
    if mismatch == "lowrank":
        k, step = 16, 1.0
        t = offline.mismatch(offline.synthetic_rotation(synth.low_rank_skew(cfg, "A", "in", k), step),
                             offline.synthetic_rotation(synth.low_rank_skew(cfg, "A", "out", k), step))
    else:
        t = synthetic_mismatch(cfg, "A")
    h = synth.residual(cfg)
    hd = torch.from_numpy(h).cuda()
    hd = hd.to(torch.bfloat16) if cfg.h_dtype == "bf16" else hd
    ref = hd.float() @ torch.from_numpy(t.astype(np.float32)).cuda()
    nrm = torch.linalg.vector_norm

    # the site's linear, unquantised, in float64 with the dense T
    lin = next(l for l in synth.layer_linears(cfg) if l.source == "siteA")
    w = np.concatenate([synth.weight(cfg, part, rows, lin.K) for part, rows in lin.parts], axis=0)
    w64 = torch.from_numpy(w).cuda().double()
    h64 = hd.double()

    def layer64(x):  # RMSNorm (unit weight) and the linear, float64
        return (x * torch.rsqrt((x * x).mean(dim=1, keepdim=True) + eps)) @ w64.T

    y_ref = layer64(h64 @ torch.from_numpy(t).cuda())
    wq = quantize_weight_on_device(w, cfg.bits, lin.name)
    y = torch.empty((cfg.n, lin.N), dtype=torch.bfloat16 if cfg.y_dtype == "bf16" else torch.float32, device="cuda")
    codes = torch.empty((cfg.n, B.rsq_packed_row_bytes(cfg.D, cfg.bits)), dtype=torch.uint8, device="cuda")
    scales = torch.empty(cfg.n, dtype=torch.float32, device="cuda")

    def y_error():
        B.rsq_qgemm(codes, scales, cfg.n, wq.codes, wq.scales, lin.N, lin.K, cfg.bits, y)
        return float(nrm(y.double() - y_ref) / nrm(y_ref))

    stream = torch.cuda.current_stream()
    B.rsq_quant_act(hd, codes, scales, cfg.bits, rmsnorm=True, eps=eps)
    rows = [{"r": 0, "rel_l2_vs_dense_hT": round(float(nrm(hd.float() - ref) / nrm(ref)), 5),
             "y_rel_l2_unquantised": round(float(nrm(layer64(h64) - y_ref) / nrm(y_ref)), 5),
             "y_rel_l2_quantised": round(y_error(), 5)}]
    progress(f"r=0: y error {rows[0]['y_rel_l2_quantised']:.4f}")
    for r in ranks:
        U, M = offline.convert_mismatch(t, r)
        site = make_site(U, M)
        out = torch.empty_like(hd)
        ms_c = _time_ms(lambda: B.rsq_subspace_correct(hd, out, site.buf, r), iters, stream)
        ms_q = _time_ms(lambda: B.rsq_correct_quant(hd, out, site.buf, r, codes, scales, cfg.bits), iters, stream)
        B.rsq_subspace_correct(hd, out, site.buf, r)
        err = float(nrm(out.float() - ref) / nrm(ref))
        u64, m64 = torch.from_numpy(U).cuda().double(), torch.from_numpy(M).cuda().double()
        y_apx = layer64(h64 + ((h64 @ u64) @ m64) @ u64.T)
        B.rsq_correct_quant(hd, out, site.buf, r, codes, scales, cfg.bits, eps=eps)
        rows.append({"r": r, "correction_ms": round(ms_c, 5), "correction_norm_quant_ms": round(ms_q, 5),
                     "rel_l2_vs_dense_hT": round(err, 5),
                     "y_rel_l2_unquantised": round(float(nrm(y_apx - y_ref) / nrm(y_ref)), 5),
                     "y_rel_l2_quantised": round(y_error(), 5)})
        progress(f"r={r}: {ms_c * 1e3:.1f} us, correction error {err:.4f}, y error {rows[-1]['y_rel_l2_quantised']:.4f}")
    print(json.dumps({"rank_sweep": rows, "mismatch": mismatch,
                      "workload": f"{cfg.name}: D={cfg.D}, {cfg.n} tokens, {cfg.h_dtype}, "
                                  f"W{cfg.bits}A{cfg.bits}, linear {lin.name} {lin.N}x{lin.K}",
                      "note": "rel_l2_vs_dense_hT: the corrected residual (GPU) against the dense product h T "
                              "(float32); y_rel_l2_unquantised: the site's linear on the rank-r approximation, "
                              "unquantised float64, against the same with dense T (the approximation alone); "
                              "y_rel_l2_quantised: the GPU path (correction, RMSNorm, per-token quantisation, "
                              "low-bit GEMM with per-channel weight codes) against that float64 reference; "
                              "r = 0: no correction. dense: the synthetic rotations are far from I and "
                              "T - I has full rank, so the approximation error falls slowly with r; "
                              "lowrank: T - I has rank at most 64"}),
          flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "rotation_bit_post_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(name: str, src_hash: str):
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary, if it is current."""
    path = os.path.join(ROOT, "profiles", f"qgemm_traffic_{name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != src_hash:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(path, n_sample: int, min_s: float = 10.0, threads: int = 0):
    """The CPU oracle (unchanged) on the first n_sample tokens of the same workload."""
    import numpy as np
    from oracle import online
    from synth import generators as G
    import threadpoolctl

    cfg, bits = path.cfg, path.cfg.bits
    h = G.residual(cfg, n_sample)
    sites = {w: (s.U.cpu().numpy(), s.M.cpu().numpy()) for w, s in path.sites.items()}
    weights = {name: (lin.codes.cpu().numpy(), lin.scales.cpu().numpy()) for name, lin in path.linears.items()}
    o_in = G.linear_input(cfg, "o_in", n_sample, cfg.D)
    down_in = G.linear_input(cfg, "down_in", n_sample, cfg.F)
    # the host's share of cores (OMP_NUM_THREADS where it is set, else every core)
    limit = threads or int(os.environ.get("OMP_NUM_THREADS") or 0) or os.cpu_count()
    with threadpoolctl.threadpool_limits(limits=limit):
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        # whole passes until at least min_s seconds have run
        passes, t0 = 0, time.perf_counter()
        while True:
            online.layer_linear_path(h, sites["A"], sites["B"], weights, o_in, down_in, cfg.h_dtype, bits,
                                     path.eps, cfg.y_dtype)
            passes += 1
            dt = time.perf_counter() - t0
            if dt >= min_s:
                break
    return {"value": passes * n_sample / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n_sample} tokens of the same workload, whole layer linear path "
                      f"(2 corrections + norms + quantisation + 4 GEMMs with the oracle's packed-code unpacking), "
                      f"float64 numpy; {passes} pass(es) in {dt:.1f} s wall",
            "host": host_cpu()}


def host_cpu() -> dict:
    """The host's processor model and logical CPU count (as the process sees them)."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "logical_cpus": os.cpu_count()}


def decode_leg(sites, ns=(1, 8, 64), copies: int = 12, iters: int = 200):
    """The decode workload (the same layer at 1, 8 and 64 tokens, the prefill workload's
    sites, weights and leading residual rows): one step, and each stage, as replayed HIP
    graphs - an eager decode step is bound by the host's launch rate, not the GPU. Twelve
    copies of every buffer rotate, so that even one stage's weights (25 MB for q|k|v)
    come back to the same copy only after more than the 256 MB Infinity Cache."""
    import torch
    import synth
    from rotation_bit_post_amd.path import LayerPath
    stream = torch.cuda.current_stream()
    out = {}
    for n in ns:
        progress(f"decode leg: {n} token(s)")
        base = LayerPath.build(synth.LLAMA2_7B_DECODE, n=n, sites=sites)
        paths = [base] + [base.clone() for _ in range(copies - 1)]
        # the step as a graph, checked against the eager step first
        base.step()
        torch.cuda.synchronize()
        ref = {k: v.clone() for k, v in base.outputs().items()}
        for v in base.outputs().values():
            v.zero_()
        graphs = [p.capture() for p in paths]
        for v in base.outputs().values():
            v.zero_()
        graphs[0].replay()
        torch.cuda.synchronize()
        same = all(torch.equal(v, ref[k]) for k, v in base.outputs().items())
        ms_step = replay_ms(graphs, iters, stream)
        # each stage cold and alone: one graph launching the stage once for each buffer
        # copy in turn, so that between two launches on the same weights come the other
        # copies' (more than the 256 MB Infinity Cache); time per launch, dispatch included
        stages = {}
        gemm_bytes = gemm_ms = 0.0
        names = [nm for nm, _, _ in base.stages()]
        for j, nm in enumerate(names):
            g = capture([p.stages()[j][2] for p in paths])
            ms = replay_ms([g], max(20, iters // 4), stream) / len(paths)
            byts, ops = base.stage_work(nm)
            stages[nm] = {"ms": round(ms, 5), "alg_bytes": byts,
                          "hbm_frac": round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            if ops:
                gemm_bytes += byts
                gemm_ms += ms
            del g
        out[str(n)] = {
            "ms_per_step": round(ms_step, 5),
            "tokens_per_s": round(n / (ms_step * 1e-3), 1),
            "graph_outputs_identical": same,
            "gemm_hbm_frac": round(gemm_bytes / (gemm_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "stages": stages,
        }
        del paths, graphs, base
        torch.cuda.empty_cache()
    out["note"] = ("decode-size batches of the same layer (llama2-7b shapes, W4A4), replayed as HIP graphs over twelve "
                   "buffer copies, cold: a step, and each stage alone launched once per copy in turn (time per "
                   "launch, graph dispatch included); hbm_frac = algorithmic bytes / time / 8 TB/s")
    return out


def timing_sites(d: int, r: int, seed: int = 0):
    """Seeded sites of the right shapes for a timing run: U an orthonormal d x r basis (QR of a Gaussian
    matrix), M = C - I_r for a Cayley rotation C of r x r. The kernels' work does not depend on the values,
    and these need no d x d solve (minutes on the host at d = 8192)."""
    from rotation_bit_post_amd.offline import cayley_rotation
    out = {}
    for i, which in enumerate(("A", "B")):
        rng = np.random.default_rng([seed, i])
        u, _ = np.linalg.qr(rng.standard_normal((d, r)))
        g = np.triu(rng.standard_normal((r, r)), 1)
        m = cayley_rotation(g - g.T, 0.3) - np.eye(r)
        out[which] = (u.astype(np.float32), m.astype(np.float32))
    return out


def workload_leg(wl, steps: int = 10):
    """A short run of another prefill workload (its weights and batch, seeded timing sites of its shapes):
    eager steps over two buffer copies, events between stages for the GEMMs' matrix-core fraction and
    the sites' HBM fraction."""
    import torch
    import synth
    from rotation_bit_post_amd.path import LayerPath
    progress(f"workload leg: {wl}")
    cfg = synth.workload(wl)
    base = LayerPath.build(wl, sites=timing_sites(cfg.D, cfg.r))
    paths = [base, base.clone()]
    lists = [p.stages() for p in paths]
    stream = torch.cuda.current_stream()
    t0, i = time.perf_counter(), 0
    while i < 3 or time.perf_counter() - t0 < 0.25:
        for _, _, fn in lists[i % 2]:
            fn()
        i += 1
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        for _, _, fn in lists[i % 2]:
            fn()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    names = [nm for nm, _, _ in lists[0]]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        for j, (_, _, fn) in enumerate(lists[i % 2]):
            fn()
            ev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    peak = FP4_PEAK_TOPS if base.fp4 else INT8_PEAK_TOPS
    stages, g_ops, g_ms = {}, 0, 0.0
    for j, nm in enumerate(names):
        t = sum(ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(steps)) / steps
        byts, ops = base.stage_work(nm)
        rec = {"ms": round(t, 5), "hbm_frac": round(byts / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        if ops:
            rec["mfma_frac"] = round(ops / (t * 1e-3) / 1e12 / peak, 4)
            g_ops += ops
            g_ms += t
        stages[nm] = rec
    cfg = base.cfg
    res = {"tokens": base.n, "ms_per_step": round(ms, 5), "tokens_per_s": round(base.n / (ms * 1e-3), 1),
           "gemm_frac_of_peak": round(g_ops / (g_ms * 1e-3) / 1e12 / peak, 4), "peak_tops": peak,
           "dtype": "fp4" if base.fp4 else "int8", "stages": stages,
           "shapes": f"D={cfg.D}, FFN={cfg.F}, r={base.r}, W{cfg.bits}A{cfg.bits}, q|k|v {base.linears['qkv'].N}",
           "sites": "seeded orthonormal subspace sites of the workload's shapes (timing only)"}
    del paths, lists, base
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    torch.cuda.set_device(0)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.rank_sweep:
        rank_sweep(args.workload, args.mismatch)
        return
    from rotation_bit_post_amd.path import LayerPath

    t_build = time.perf_counter()
    progress(f"building workload {args.workload} (sites, weights, inputs)")
    base = LayerPath.build(args.workload, keep_mismatch=not args.no_dense, prep=args.prep, gqa=not args.mha)
    copies = [base] + [base.clone() for _ in range(args.copies - 1)]
    torch.cuda.synchronize()
    t_build = time.perf_counter() - t_build
    progress(f"built in {t_build:.1f} s; warm-up {args.warmup}, timing {args.steps} steps")
    cfg, n = base.cfg, base.n
    stage_lists = [p.stages(correction=True) for p in copies]
    names = [s[0] for s in stage_lists[0]]
    kinds = {s[0]: s[1] for s in stage_lists[0]}

    # untimed warm-up: W steps, continued until 0.25 s of steps have run so
    # that the engine clock has settled (the first few milliseconds of work
    # after set-up run about 10 % slower)
    t_w, i = time.perf_counter(), 0
    while i < args.warmup or time.perf_counter() - t_w < 0.25:
        for _, _, fn in stage_lists[i % len(copies)]:
            fn()
        i += 1
        if i % 50 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    warmup_steps = i
    stream = torch.cuda.current_stream()

    # 1. the step as launched by a caller: K steps back to back, events (on the
    #    stream the library launches on) only around the whole run
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        for _, _, fn in stage_lists[i % len(copies)]:
            fn()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_eager = e0.elapsed_time(e1) / args.steps

    # warm: one buffer set only, so a step finds its inputs in the Infinity Cache
    for _, _, fn in stage_lists[0]:
        fn()
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        for _, _, fn in stage_lists[0]:
            fn()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_warm = e0.elapsed_time(e1) / args.steps

    # 2. the same step as a replayed HIP graph (one per buffer copy), used only
    #    if its outputs are bit-identical to the eager step's
    ms_graph, graph_ok = None, False
    try:
        ref = []
        for p in copies:
            p.step()
            torch.cuda.synchronize()
            ref.append({k: v.clone() for k, v in p.outputs().items()})
            for v in p.outputs().values():
                v.zero_()
        graphs = [p.capture() for p in copies]
        for p in copies:
            for v in p.outputs().values():
                v.zero_()
        for gr in graphs:
            gr.replay()
        torch.cuda.synchronize()
        graph_ok = all(torch.equal(v, r[k]) for p, r in zip(copies, ref) for k, v in p.outputs().items())
        if graph_ok:
            for i in range(args.warmup):
                graphs[i % len(graphs)].replay()
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(args.steps):
                graphs[i % len(graphs)].replay()
            e1.record(stream)
            torch.cuda.synchronize()
            ms_graph = e0.elapsed_time(e1) / args.steps
    except Exception as ex:  # capture unsupported here: report the eager number only
        progress(f"graph capture failed: {ex}")
    ms_per_step = ms_graph if ms_graph is not None and ms_graph < ms_eager else ms_eager

    # 3. per-stage breakdown: events between stages
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        stages = stage_lists[i % len(copies)]
        ev[i][0].record(stream)
        for j, (_, _, fn) in enumerate(stages):
            fn()
            ev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    stage_ms = {nm: [ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(args.steps)] for j, nm in enumerate(names)}
    step_ms = sorted(ev[i][0].elapsed_time(ev[i][-1]) for i in range(args.steps))

    def pct(q):
        return round(step_ms[min(len(step_ms) - 1, int(q * (len(step_ms) - 1) + 0.5))], 5)

    # 4. the step's GEMM launches alone, back to back with events only around the
    #    run (as in 1.): the roofline's per-launch time, free of the event gaps of
    #    the per-stage pass
    gemm_lists = [[fn for nm, kind, fn in sl if kind == "gemm"] for sl in stage_lists]
    for i in range(args.warmup):
        for fn in gemm_lists[i % len(copies)]:
            fn()
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        for fn in gemm_lists[i % len(copies)]:
            fn()
    e1.record(stream)
    torch.cuda.synchronize()
    gemm_pass_ms = e0.elapsed_time(e1) / args.steps

    progress("timed region done; correction-off pass")
    # correction off: each site only normalises and quantises (one global rotation, T = I)
    off_lists = [p.stages(correction=False) for p in copies]
    for i in range(args.warmup):
        for _, _, fn in off_lists[i % len(copies)]:
            fn()
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        for _, _, fn in off_lists[i % len(copies)]:
            fn()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_off = e0.elapsed_time(e1) / args.steps

    # the chained layer: residual adds fused into the o / down GEMMs, site B reads h2
    ms_chain = None
    if "B" in base.sites:
        chain_lists = [p.stages(correction=True, chain=True) for p in copies]
        for i in range(args.warmup):
            for _, _, fn in chain_lists[i % len(copies)]:
                fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.steps):
            for _, _, fn in chain_lists[i % len(copies)]:
                fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms_chain = e0.elapsed_time(e1) / args.steps

    # when the step's value comes from replayed graphs, time the correction-off and the
    # chained steps the same way, so that the overhead compares like with like
    off_graph = chain_graph = None
    if ms_graph is not None and ms_graph < ms_eager:
        off_graph = replay_ms([p.capture(correction=False) for p in copies], args.steps, stream)
        if ms_chain is not None:
            chain_graph = replay_ms([p.capture(correction=True, chain=True) for p in copies], args.steps, stream)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

    # 5. each stage alone and cold: one graph launches it once on each of ALONE_COPIES
    #    buffer copies in turn (so its inputs come back only after more than twice the
    #    Infinity Cache of other copies' traffic), replayed; no events between launches
    alone_ms = {}
    decode_sized = n <= 64
    if decode_sized:
        # a few tokens: an eager step is bound by the host's launch rate, so each stage
        # is timed cold and alone in replayed graphs (decode_leg)
        sites = {w: (st.U.cpu().numpy(), st.M.cpu().numpy()) for w, st in base.sites.items()}
        leg = decode_leg(sites, ns=(n,))
        alone_ms = {nm: leg[str(n)]["stages"][nm]["ms"] for nm in names}
    else:
        progress(f"each stage alone over {ALONE_COPIES} buffer copies (cold, replayed graphs)")
        extra = [base.clone() for _ in range(max(0, ALONE_COPIES - len(copies)))]
        alone_lists = [p.stages() for p in copies + extra]
        for j, nm in enumerate(names):
            g = capture([sl[j][2] for sl in alone_lists])
            alone_ms[nm] = replay_ms([g], 8, stream) / len(alone_lists)
            del g
        del extra, alone_lists
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

    stages_out = {}
    gemm_ops = gemm_ms = gemm_launches = 0
    gemm_peak = FP4_PEAK_TOPS if base.fp4 else INT8_PEAK_TOPS
    for nm in names:
        byts, ops = base.stage_work(nm)
        t_ev = sum(stage_ms[nm]) / args.steps
        t = alone_ms.get(nm, t_ev)
        rec = {"kind": kinds[nm], "ms": round(t, 5), "ms_in_step_with_events": round(t_ev, 5), "alg_bytes": byts}
        rec["hbm_frac"] = round(byts / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        if ops:
            rec["alg_ops"] = ops
            rec["mfma_frac"] = round(ops / (t * 1e-3) / 1e12 / gemm_peak, 4)
            gemm_ops += ops
            gemm_ms += t
            gemm_launches += 1
        stages_out[nm] = rec

    # practical ceiling of the memory-bound stages: a plain device copy moving the same bytes
    progress("copy ceilings of the memory-bound stages")
    ceil_ms = {}
    for nm in names:
        if kinds[nm] in ("site", "quant"):
            byts = stages_out[nm]["alg_bytes"]
            if byts not in ceil_ms:
                ceil_ms[byts] = copy_ceiling(byts)
            stages_out[nm]["copy_ms"] = round(ceil_ms[byts], 5)
            stages_out[nm]["copy_hbm_frac"] = round(byts / (ceil_ms[byts] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
            stages_out[nm]["frac_of_copy"] = round(ceil_ms[byts] / stages_out[nm]["ms"], 4)

    src_hash = kernel_source_hash()
    traffic = measured_traffic(cfg.name, src_hash)
    value = n / (ms_per_step * 1e-3)
    if decode_sized:
        # a few tokens: the GEMMs stream their weights once, so HBM bounds them; their
        # times are the cold replayed-graph times of decode_leg
        gemm_nm = [nm for nm in names if kinds[nm] == "gemm"]
        gemm_bytes = sum(leg[str(n)]["stages"][nm]["alg_bytes"] for nm in gemm_nm)
        gemm_ms = sum(leg[str(n)]["stages"][nm]["ms"] for nm in gemm_nm)
        achieved = gemm_bytes / (gemm_ms * 1e-3) / 1e9
        roofline = {"kernel": "the four quantised-linear launches of a step (weights streamed once; each timed cold "
                              "in a replayed graph)", "bound": "hbm",
                    "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                    "avg_launch_ms": round(gemm_ms / max(gemm_launches, 1), 5)}
    else:
        gemm_ms = gemm_pass_ms
        achieved = gemm_ops / (gemm_ms * 1e-3) / 1e12
        roofline = {
            "kernel": ("qgemm_kernel (3-bit codes as fp4 on v_mfma_scale_f32_32x32x64_f8f6f4)" if base.fp4 else
                       f"qgemm_kernel (int{cfg.bits} codes on v_mfma_i32_32x32x32_i8)") +
                      ", all 4 launches of a step, timed back to back without the other stages",
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": gemm_peak,
            "unit": "TOP/s",
            "frac": round(achieved / gemm_peak, 4),
            "traffic": traffic,
            "avg_launch_ms": round(gemm_ms / max(gemm_launches, 1), 5),
        }
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warmup_steps,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4" if base.fp4 else "int8",
        "data": "synthetic (seeded N(0,1) residual with outlier channels, Hadamard*Cayley rotations, N(0,sigma) weights; no dataset, no trained weights)",
        "config": {
            "workload": f"{cfg.name}: D={cfg.D}, FFN={cfg.F}, r={base.r}, {n} tokens, {cfg.h_dtype} residual, "
                        f"W{cfg.bits}A{cfg.bits}; one layer's linear path = 2 correction sites + 2 stand-in "
                        f"quantisations + GEMMs qkv {base.linears['qkv'].N}x{cfg.D}, o {cfg.D}x{cfg.D}, "
                        f"gate|up {base.linears['gate_up'].N}x{cfg.D}, down {cfg.D}x{cfg.F}",
            "tokens": n, "D": cfg.D, "ffn": cfg.F, "r": base.r, "bits": cfg.bits, "buffer_copies": len(copies),
            "qkv": "all D x D (MHA)" if args.mha else "GQA where the model has it",
        },
        "roofline": roofline,
        "stages": stages_out,
        "correction_overhead": {
            "ms_per_step_correction_off": round(off_graph if off_graph is not None else ms_off, 5),
            "overhead_frac": round((ms_per_step / off_graph if off_graph is not None else ms_eager / ms_off) - 1.0, 4),
            "note": "same path with each site reduced to RMSNorm + quantisation (T = I, a single global rotation); "
                    + ("both replayed as HIP graphs" if off_graph is not None else "both launched eagerly"),
        },
        "layer_chained": None if ms_chain is None else {
            "ms_per_step": round(chain_graph if chain_graph is not None else ms_chain, 5),
            "tokens_per_s": round(n / ((chain_graph if chain_graph is not None else ms_chain) * 1e-3), 1),
            "note": "the same stages with the residual stream carried through: o_proj and down_proj "
                    "outputs added to the corrected residual inside the GEMM epilogue (rsq_qgemm_residual), "
                    "site B reading h2; " + ("replayed as HIP graphs" if chain_graph is not None else
                                             "timed back to back, no events between stages"),
        },
        "timing": {
            "ms_per_step_eager": round(ms_eager, 5),
            "ms_per_step_eager_warm": round(ms_warm, 5),
            "ms_per_step_graph": None if ms_graph is None else round(ms_graph, 5),
            "graph_outputs_identical": graph_ok,
            "value_from": "graph" if ms_per_step != ms_eager else "eager",
            "step_ms_p10_p50_p90": [pct(0.1), pct(0.5), pct(0.9)],
            "note": "eager: the step's launches back to back; graph: the same launches recorded once as a HIP "
                    "graph and replayed (outputs checked bit-identical first); value uses the faster; "
                    "percentiles: single steps of the per-stage pass (events between stages add a little); "
                    "warm: one buffer set, inputs left in the 256 MB Infinity Cache by the previous step (cold, "
                    "the value: buffer copies alternate)",
        },
        "offline_prep": base.prep_info,
        "wall_s_timed": round(wall, 3),
        "setup_s": round(t_build, 1),
        "kernel_source_hash": src_hash,
    }
    if not args.no_dense and "A" in base.mismatch:
        progress("dense h T comparator")
        out["dense_T_comparator"] = dense_comparator(base)
    if decode_sized:
        out["decode"] = leg
    if not args.no_decode and cfg.name == "llama2-7b-prefill-w4a4":
        sites = {w: (st.U.cpu().numpy(), st.M.cpu().numpy()) for w, st in base.sites.items()}
        out["decode"] = decode_leg(sites)
    if not args.no_workload_legs and cfg.name == "llama2-7b-prefill-w4a4":
        out["other_workloads"] = {wl: workload_leg(wl) for wl in ("llama3-8b-prefill-w3a3", "llama2-70b-prefill-w4a4")}
    if not args.no_cpu_baseline:
        progress(f"CPU oracle on a {min(args.cpu_sample, n)}-token sample")
        out["cpu_baseline"] = cpu_baseline(base, min(args.cpu_sample, n))
        if args.cpu_one_core_sample > 0:
            n1 = min(args.cpu_one_core_sample, n)
            progress(f"CPU oracle on one thread, {n1}-token sample")
            one = cpu_baseline(base, n1, min_s=0.0, threads=1)
            out["cpu_baseline"]["one_core"] = {k: one[k] for k in ("value", "unit", "cores", "sample")}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
