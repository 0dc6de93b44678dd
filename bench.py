"""Benchmark of the MAPL boundary hot path on one MI355X.

One step = one pass of the whole hot path over one micro-batch at the 150M
boundary shape (B=8, T=2048 -> N=16384 tokens, d=1024, r=128, V=32000, bf16):

  pack A,P -> compress -> rvq encode -> stream sync -> rvq decode ->
  reconstruct -> reconstruct backward -> compress backward -> spel_step

The residual VQ runs on Z (r=128) as G=4 groups of width 32, K=256, R=2;
spel_step runs on the fp32 1024 x 128 projector with alpha=1e-3, beta=0.9 and
8 Newton-Schulz iterations.  Inputs are seeded synthetic tensors resident in
HBM; before each step a 1 GiB write evicts the caches (L2 and the 256 MB
Infinity Cache), outside the timed region.

`value` is boundary tokens per second of the whole step (N / ms_per_step).
The compress+reconstruct pair alone, the per-kernel times and the roofline of
the dominant codec kernel are reported beside it, each timed with HIP events
on the stream the kernels run on.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # dense bf16 matrix
F32_PEAK_TFLOPS = 157.3      # fp32 matrix


def _only_codec(lac, dev, cfg, r, maps, x_kind="gauss"):
    """The codec maps of one configuration at rank r, on resident inputs."""
    import synth
    c = synth.CONFIGS[cfg]
    N, d = c["B"] * c["T"], c["d"]
    inp = synth.codec_inputs(c["seed"], N, d, r, c["V"], "bf16", x_kind=x_kind)
    g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    pk = lac.mapl_pack(g["P"], g["A"])
    Z = lac.mapl_compress(g["X"], g["tids"], g["E"], g["P"], g["A"], pk=pk, pk_ready=True)
    Xh = torch.empty((N, d), dtype=torch.bfloat16, device=dev)
    gZ, gX = torch.empty_like(Z), torch.empty_like(Xh)
    gA = torch.empty((d, r), dtype=torch.float32, device=dev)
    ws = torch.empty(lac.mapl_bwd_workspace_bytes(c["B"], c["T"], d, r), dtype=torch.uint8, device=dev)
    fns = {
        "compress": lambda: lac.mapl_compress(g["X"], g["tids"], g["E"], g["P"], g["A"], Z=Z, pk=pk, pk_ready=True),
        "reconstruct": lambda: lac.mapl_reconstruct(Z, g["tids"], g["E"], g["P"], g["A"], Xhat=Xh, pk=pk,
                                                    pk_ready=True),
        "reconstruct_bwd": lambda: lac.mapl_reconstruct_bwd(g["gXhat"], Z, g["A"], gZ=gZ, gA=gA, pk=pk,
                                                            pk_ready=True, ws=ws),
        "compress_bwd": lambda: lac.mapl_compress_bwd(gZ, g["X"], g["tids"], g["E"], g["P"], g["A"], gX=gX, gA=gA,
                                                      accumulate=True, pk=pk, pk_ready=True, ws=ws),
    }
    return lambda: [fns[m]() for m in maps]


def _only_rvq(lac, dev, width):
    """RVQ encode at the rvq workload: Z (r = 256) from the codec in 8 groups of width 32, or the
    receiver's gZ in the paper's 128 groups of width 2; K = 256, R = 2."""
    import synth
    c = synth.CONFIGS["rvq"]
    N, d, r, K, R = c["B"] * c["T"], c["d"], c["r"], c["K"], c["R"]
    inp = synth.codec_inputs(c["seed"], N, d, r, c["V"], "bf16")
    g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    Z = lac.mapl_compress(g["X"], g["tids"], g["E"], g["P"], g["A"])
    if width == 2:
        Z, _ = lac.mapl_reconstruct_bwd(g["gXhat"], Z, g["A"])
        G, var = r // 2, 1.0
    else:
        G, var = c["G"], c["codebook_var"]
    C = synth.rvq_codebooks(c["seed"], 1, G, K, r // G, var, sub=1 if width == 2 else 0).to(dev)
    codes = torch.empty((N, R, G), dtype=torch.uint8, device=dev)
    return lambda: lac.rvq_encode(Z, C, G, K, R, codes=codes)


def _only_spel(lac, dev, d, r):
    import synth
    sp = synth.CONFIGS["1b"]["spel"]
    si = synth.spel_inputs(5, d, r, sp["g_var"])
    A, gg, m = si["A"].to(dev), si["g"].to(dev), si["m"].to(dev)
    ws = torch.empty(lac.spel_workspace_bytes(d, r), dtype=torch.uint8, device=dev)
    return lambda: lac.spel_step(A, gg, m, sp["alpha"], sp["beta"], sp["ns_iters"], ws=ws)


def _only_copy(lac, dev):
    """A plain 256 MiB device copy: the known-size reference for the HBM byte counters."""
    src = torch.ones(1 << 26, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    return lambda: dst.copy_(src)


ONLY_CASES = {
    "compress-150m": lambda lac, dev: _only_codec(lac, dev, "150m", 128, ["compress"]),
    "reconstruct-150m": lambda lac, dev: _only_codec(lac, dev, "150m", 128, ["reconstruct"]),
    "bwd-150m": lambda lac, dev: _only_codec(lac, dev, "150m", 128, ["reconstruct_bwd", "compress_bwd"]),
    "pair-r256": lambda lac, dev: _only_codec(lac, dev, "sweep", 256, ["compress", "reconstruct"], "lowrank"),
    "pair-r512": lambda lac, dev: _only_codec(lac, dev, "sweep", 512, ["compress", "reconstruct"], "lowrank"),
    "rvq-w32": lambda lac, dev: _only_rvq(lac, dev, 32),
    "rvq-w2": lambda lac, dev: _only_rvq(lac, dev, 2),
    "spel-1024x128": lambda lac, dev: _only_spel(lac, dev, 1024, 128),
    "spel-2048x256": lambda lac, dev: _only_spel(lac, dev, 2048, 256),
    "copy-256mib": _only_copy,
}


def run_only(lac, dev, case, reps):
    fn = ONLY_CASES[case](lac, dev)
    torch.cuda.synchronize()
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    print(f"only {case}: {reps} runs done", flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-flush", action="store_true", help="do not evict caches between steps")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-tokens", type=int, default=16384, help="token sample of the CPU-oracle baseline")
    p.add_argument("--cpu-reps", type=int, default=3, help="timed repetitions of the CPU-oracle sample (median)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run one plain 256 MiB device copy first (a known-size reference for HBM byte counters)")
    p.add_argument("--cases", metavar="FILE", default=None,
                   help="also time every workload of the measurement table and write them to FILE (JSON)")
    p.add_argument("--only", metavar="CASE", default=None, choices=sorted(ONLY_CASES),
                   help="run one workload --reps times (warm, untimed) and exit: the command that hardware-counter "
                        "profiles (rocprofv3 --pmc) run")
    p.add_argument("--reps", type=int, default=3, help="repetitions of --only")
    return p.parse_args()


class Shape:
    B, T, d, r, V = 8, 2048, 1024, 128, 32000
    G, K, R = 4, 256, 2
    N = B * T
    seed = 2
    alpha, beta, ns = 1e-3, 0.9, 8


def make_inputs(dev):
    import synth
    S = Shape
    inp = synth.codec_inputs(S.seed, S.N, S.d, S.r, S.V, "bf16")
    w = S.r // S.G
    C = synth.rvq_codebooks(S.seed, 1, S.G, S.K, w, 1.0 / 32.0)
    sender = C + torch.from_numpy(synth.gaussian(synth.stream(S.seed, 9), C.shape, 1e-4).astype(np.float32))
    packets = [synth.stream_packets(S.seed, i, sender) for i in range(8)]
    sp = synth.spel_inputs(S.seed, S.d, S.r, 1e-3)
    g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    g["C"] = C.to(dev)
    g["packets"] = [(i.to(dev), v.to(dev)) for i, v in packets]
    g["A32"] = sp["A"].to(dev)
    g["m"] = sp["m"].to(dev)
    return inp, g


def alloc(g, lac):
    S = Shape
    dev = g["X"].device
    bufs = dict(
        pk=torch.empty(lac.mapl_pack_bytes(S.d, S.r), dtype=torch.uint8, device=dev),
        Z=torch.empty((S.N, S.r), dtype=torch.bfloat16, device=dev),
        Zq=torch.empty((S.N, S.r), dtype=torch.bfloat16, device=dev),
        codes=torch.empty((S.N, S.R, S.G), dtype=torch.uint8, device=dev),
        Xh=torch.empty((S.N, S.d), dtype=torch.bfloat16, device=dev),
        gZ=torch.empty((S.N, S.r), dtype=torch.bfloat16, device=dev),
        gX=torch.empty((S.N, S.d), dtype=torch.bfloat16, device=dev),
        gA=torch.empty((S.d, S.r), dtype=torch.float32, device=dev),
        ws=torch.empty(lac.mapl_bwd_workspace_bytes(S.B, S.T, S.d, S.r), dtype=torch.uint8, device=dev),
        sws=torch.empty(lac.spel_workspace_bytes(S.d, S.r), dtype=torch.uint8, device=dev),
    )
    return bufs


def step(lac, g, b, it, ev=None):
    """One pass of the hot path.  ev: optional dict name -> (start, end) events."""
    S = Shape

    def mark(name, i):
        if ev is not None and name in ev:
            ev[name][i].record()

    mark("pack", 0)
    lac.mapl_pack(g["P"], g["A"], pk=b["pk"])
    mark("pack", 1)
    mark("compress", 0)
    lac.mapl_compress(g["X"], g["tids"], g["E"], g["P"], g["A"], Z=b["Z"], pk=b["pk"], pk_ready=True)
    mark("compress", 1)
    mark("rvq_encode", 0)
    lac.rvq_encode(b["Z"], g["C"], S.G, S.K, S.R, codes=b["codes"])
    mark("rvq_encode", 1)
    idx, vals = g["packets"][it % len(g["packets"])]
    mark("rvq_decode", 0)
    # the receiver's codebook sync and decode, one launch
    lac.rvq_stream_decode(g["C"], idx, vals, b["codes"], S.G, S.K, S.R, S.r, Zq=b["Zq"])
    mark("rvq_decode", 1)
    mark("reconstruct", 0)
    lac.mapl_reconstruct(b["Zq"], g["tids"], g["E"], g["P"], g["A"], Xhat=b["Xh"], pk=b["pk"], pk_ready=True)
    mark("reconstruct", 1)
    mark("reconstruct_bwd", 0)
    lac.mapl_reconstruct_bwd(g["gXhat"], b["Zq"], g["A"], gZ=b["gZ"], gA=b["gA"], accumulate=False, pk=b["pk"],
                             pk_ready=True, ws=b["ws"])
    mark("reconstruct_bwd", 1)
    mark("compress_bwd", 0)
    lac.mapl_compress_bwd(b["gZ"], g["X"], g["tids"], g["E"], g["P"], g["A"], gX=b["gX"], gA=b["gA"],
                          accumulate=True, pk=b["pk"], pk_ready=True, ws=b["ws"])
    mark("compress_bwd", 1)
    mark("spel_step", 0)
    lac.spel_step(g["A32"], b["gA"], g["m"], S.alpha, S.beta, S.ns, ws=b["sws"])
    mark("spel_step", 1)


def pair(lac, g, b):
    lac.mapl_compress(g["X"], g["tids"], g["E"], g["P"], g["A"], Z=b["Z"], pk=b["pk"], pk_ready=True)
    lac.mapl_reconstruct(b["Z"], g["tids"], g["E"], g["P"], g["A"], Xhat=b["Xh"], pk=b["pk"], pk_ready=True)


PHASES = ["pack", "compress", "rvq_encode", "rvq_decode", "reconstruct", "reconstruct_bwd", "compress_bwd",
          "spel_step"]


def algorithmic(inp):
    """Algorithmic bytes and flops per launch of the codec kernels at this shape."""
    S = Shape
    n_distinct = int(np.unique(inp["tids"].numpy()).size)
    e_rows = n_distinct * 2 * S.r
    per_tok = 2 * S.d + 4 + 2 * S.r             # X or Xhat (bf16) + tid + Z (bf16)
    comp_bytes = S.N * per_tok + e_rows + 2 * S.d * S.r + 2 * S.r * S.r   # + At + Qn
    reco_bytes = S.N * per_tok + e_rows + 2 * S.d * S.r * 2               # + A + Pt
    comp_flops = S.N * (2 * S.d * S.r + 2 * S.r * S.r)                    # executed: X A + E[t] (P A)
    reco_flops = S.N * 4 * S.d * S.r
    return dict(n_distinct=n_distinct, compress_bytes=comp_bytes, reconstruct_bytes=reco_bytes,
                compress_flops=comp_flops, reconstruct_flops=reco_flops)


def counter_traffic():
    """HBM traffic per compress launch from the committed rocprofv3 counter
    summary, or None once the kernel source differs from the one measured."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "compress_150m_hbm_counters.txt")
    csrc = os.path.join(ROOT, "learned_activation_compression_amd", "csrc")
    try:
        lines = open(path).read().splitlines()
        traffic = int([l for l in lines if l.startswith("traffic_bytes_per_launch:")][0].split(":")[1])
        sha = [l for l in lines if l.startswith("source_sha256")][0].split(":")[1].strip()
        h = hashlib.sha256()
        for f in ("codec_bf16.hip", "common.h"):
            h.update(open(os.path.join(csrc, f), "rb").read())
        if h.hexdigest() != sha:
            return None
        return traffic
    except (OSError, IndexError, ValueError):
        return None


def _device_info():
    """Name, architecture and compute-unit count of cuda:0, as the runtime reports them."""
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", ""), "compute_units": p.multi_processor_count,
            "memory_GiB": round(p.total_memory / 2 ** 30, 1)}


def cpu_baseline(inp, n_tok, reps):
    """The fp64 oracle of the same step on a token sample (host cores): one
    warm-up run, then `reps` timed runs; the rate is the sample's tokens over
    the median time.  BLAS is threaded over the cores this process may run on
    (its affinity mask, capped by OMP_NUM_THREADS when that is set)."""
    from oracle import codec, rvq, spel
    import synth
    S = Shape
    cores = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        cores = max(1, min(cores, int(os.environ["OMP_NUM_THREADS"])))
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=cores)
    except Exception:  # pragma: no cover
        limiter = None
    sl = slice(0, n_tok)
    X = inp["X"][sl].double().numpy()
    t = inp["tids"][sl].numpy()
    E, P, A = inp["E"].double().numpy(), inp["P"].double().numpy(), inp["A"].double().numpy()
    gXh = inp["gXhat"][sl].double().numpy()
    w = S.r // S.G
    C = synth.rvq_codebooks(S.seed, 1, S.G, S.K, w, 1.0 / 32.0).double().numpy()
    sp = synth.spel_inputs(S.seed, S.d, S.r, 1e-3)
    def one():
        Z = codec.compress(X, t, E, P, A)
        enc = rvq.encode(Z, C, S.G, S.K, S.R)
        Zq = rvq.decode(enc["codes"], C, S.G, S.K, S.R)
        codec.reconstruct(Zq, t, E, P, A)
        gZ, gA1 = codec.reconstruct_bwd(gXh, Zq, A)
        _, gA2 = codec.compress_bwd(gZ, X, t, E, P, A)
        spel.spel_step(sp["A"].double().numpy(), gA1 + gA2, sp["m"].double().numpy(), S.alpha, S.beta, S.ns)

    one()  # warm-up
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        one()
        times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    if limiter is not None:
        limiter.restore_original_limits()
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), model)
    except OSError:  # pragma: no cover
        pass
    return {"value": n_tok / dt, "unit": "boundary tokens/s", "cores": int(cores), "kind": "oracle", "cpu": model,
            "sample": f"one full step of the fp64 oracle (codec fwd+bwd, RVQ encode/decode, one spel_step on "
                      f"1024x128) on {n_tok} of the {S.N} tokens: 1 warm-up, median of {reps} runs, {dt:.2f} s per run"}


def _evict(flush):
    """Evict the inputs from L2 and the 256 MB memory-side cache by reading a
    1 GiB buffer.  A read leaves only clean lines behind; an evicting write
    (zero-fill) would leave the memory-side cache full of dirty lines whose
    write-back then runs inside the next timed region."""
    if flush is not None:
        torch.sum(flush)


def _timed(fn, flush, iters=20, warm=3):
    """Median / p10 / p90 (ms) of fn() bracketed by HIP events on the current
    stream, each run after a cache-evicting read (outside the events)."""
    stream = torch.cuda.current_stream()
    for _ in range(warm):
        fn()
    out = []
    for _ in range(iters):
        _evict(flush)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1))
    a = np.array(out)
    return {"ms": round(float(np.median(a)), 5), "p10": round(float(np.percentile(a, 10)), 5),
            "p90": round(float(np.percentile(a, 90)), 5)}


def _codec_counts(N, d, r, n_distinct, ra=None, eye=False):
    """Algorithmic bytes and executed flops of each codec map (whole batch).
    ra is the anchor rank (default r; 0: no anchor); eye marks the full-rank
    anchor (ra = d, P = I), whose rows are added or subtracted directly in
    reconstruct and whose pack has no P sections."""
    ra = r if ra is None else ra
    t4 = 4 if ra > 0 else 0                        # token ids read
    e = n_distinct * 2 * ra                        # distinct anchor rows read
    pt = 0 if eye else 2 * d * ra                  # P^T pack of reconstruct
    rflops = N * 2 * d * r + (0 if eye else N * 2 * d * ra)
    c = dict(
        compress=(N * (2 * d + t4 + 2 * r) + e + 2 * d * r + 2 * r * ra, N * (2 * d * r + 2 * ra * r)),
        reconstruct=(N * (2 * r + t4 + 2 * d) + e + 2 * d * r + pt, rflops),
        reconstruct_bwd=(N * (2 * d + 2 * r + 2 * r) + 2 * d * r + 4 * d * r, N * 4 * d * r),
        compress_bwd=(N * (2 * r + 2 * d + t4 + 2 * d) + e + 2 * 2 * d * r + 2 * 4 * d * r,
                      N * (4 * d * r + 2 * ra * r) + (0 if eye else 2 * d * ra * r)),
    )
    c["pair"] = (c["compress"][0] + c["reconstruct"][0], c["compress"][1] + c["reconstruct"][1])
    return c


def run_cases(lac, dev, flush):
    """Every workload of the measurement table, each timed cold (flushed)."""
    import synth
    res = {"hbm_peak_GBs": HBM_PEAK_GBS, "bf16_peak_TFLOPs": BF16_PEAK_TFLOPS, "f32_peak_TFLOPs": F32_PEAK_TFLOPS,
           "cases": []}

    def add(name, t, nbytes, flops, bound, tokens=None, peak_tf=BF16_PEAK_TFLOPS):
        s = t["ms"] * 1e-3
        row = dict(case=name, **t, bytes=int(nbytes), flops=int(flops), bound=bound,
                   GBs=round(nbytes / s / 1e9, 1), hbm_frac=round(nbytes / s / 1e9 / HBM_PEAK_GBS, 4),
                   TFLOPs=round(flops / s / 1e12, 2), mfma_frac=round(flops / s / 1e12 / peak_tf, 4))
        if tokens:
            row["tokens_per_s"] = round(tokens / s, 1)
        res["cases"].append(row)
        print(f"# {name:34s} {t['ms']*1e3:9.1f} us  {row['GBs']:8.1f} GB/s ({row['hbm_frac']:.3f})  "
              f"{row['TFLOPs']:8.2f} TF/s ({row['mfma_frac']:.3f})", file=sys.stderr, flush=True)

    def codec_case(tag, c, r, x_kind="gauss", ra=None, anchor="factorised"):
        N, d = c["B"] * c["T"], c["d"]
        inp = synth.codec_inputs(c["seed"], N, d, r, c["V"], "bf16", x_kind=x_kind, ra=ra, anchor=anchor)
        g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
        ra = inp["ra"]
        nd = int(np.unique(inp["tids"].numpy()).size)
        eye = anchor == "full"
        cnt = _codec_counts(N, d, r, nd, ra, eye)
        pk = lac.mapl_pack(g["P"], g["A"], ra=ra)
        Z = torch.empty((N, r), dtype=torch.bfloat16, device=dev)
        Xh = torch.empty((N, d), dtype=torch.bfloat16, device=dev)
        gZ = torch.empty_like(Z)
        gX = torch.empty_like(Xh)
        gA = torch.empty((d, r), dtype=torch.float32, device=dev)
        ws = torch.empty(lac.mapl_bwd_workspace_bytes(c["B"], c["T"], d, r, ra=ra), dtype=torch.uint8, device=dev)
        comp = lambda: lac.mapl_compress(g["X"], g["tids"], g["E"], g["P"], g["A"], Z=Z, pk=pk, pk_ready=True)
        reco = lambda: lac.mapl_reconstruct(Z, g["tids"], g["E"], g["P"], g["A"], Xhat=Xh, pk=pk, pk_ready=True)
        rbwd = lambda: lac.mapl_reconstruct_bwd(g["gXhat"], Z, g["A"], gZ=gZ, gA=gA, accumulate=False, pk=pk,
                                                pk_ready=True, ws=ws)
        cbwd = lambda: lac.mapl_compress_bwd(gZ, g["X"], g["tids"], g["E"], g["P"], g["A"], gX=gX, gA=gA,
                                             accumulate=True, pk=pk, pk_ready=True, ws=ws)
        bound = "hbm" if r <= 128 else "mfma"
        add(f"{tag} pair", _timed(lambda: (comp(), reco()), flush), *cnt["pair"], bound, tokens=N)
        add(f"{tag} compress", _timed(comp, flush), *cnt["compress"], bound, tokens=N)
        add(f"{tag} reconstruct", _timed(reco, flush), *cnt["reconstruct"], bound, tokens=N)
        add(f"{tag} reconstruct_bwd", _timed(rbwd, flush), *cnt["reconstruct_bwd"], bound, tokens=N)
        add(f"{tag} compress_bwd", _timed(cbwd, flush), *cnt["compress_bwd"], bound, tokens=N)
        if ra == 0:
            del g, pk, Z, Xh, gZ, gX, gA, ws
            return inp
        # sender's anchor-table gradient from gX (Y read once, P, tids, the whole [V][ra] table written)
        V = c["V"]
        gE = torch.empty((V, ra), dtype=torch.float32, device=dev)
        aws = torch.empty(lac.mapl_anchor_grad_workspace_bytes(c["B"], c["T"], ra, V), dtype=torch.uint8, device=dev)
        agrad = lambda: lac.mapl_anchor_grad(gX, g["tids"], g["P"], V, -1.0, gE=gE, pk=pk, pk_ready=True, r=r,
                                             ws=aws)
        add(f"{tag} anchor_grad", _timed(agrad, flush), 2 * N * d + 4 * N + (0 if eye else 2 * ra * d) + 4 * V * ra,
            0 if eye else 2 * N * d * ra, "hbm", tokens=N)
        del g, pk, Z, Xh, gZ, gX, gA, ws, gE, aws
        return inp

    C = synth.CONFIGS
    codec_case("150m d1024 r128", C["150m"], 128)
    # the anchor variants of the ablation (Table 6) and a separate anchor rank
    codec_case("150m d1024 r128 no-anchor", C["150m"], 128, anchor="none")
    codec_case("150m d1024 r128 full-anchor", C["150m"], 128, anchor="full")
    codec_case("150m d1024 r128 ra256", C["150m"], 128, ra=256)
    for r in C["sweep"]["ranks"]:
        codec_case(f"sweep d1024 r{r}", C["sweep"], r, x_kind="lowrank")
    codec_case("1b d2048 r256", C["1b"], 256)

    # residual VQ at r=256, G=8 x w=32, K=256, R=2 on Z from the codec
    c = C["rvq"]
    N, d, r, G, K, R = c["B"] * c["T"], c["d"], c["r"], c["G"], c["K"], c["R"]
    inp = synth.codec_inputs(c["seed"], N, d, r, c["V"], "bf16")
    g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    Z = lac.mapl_compress(g["X"], g["tids"], g["E"], g["P"], g["A"])
    Cb = synth.rvq_codebooks(c["seed"], 1, G, K, r // G, c["codebook_var"]).to(dev)
    codes = torch.empty((N, R, G), dtype=torch.uint8, device=dev)
    Zq = torch.empty((N, r), dtype=torch.float32, device=dev)
    enc = lambda: lac.rvq_encode(Z, Cb, G, K, R, codes=codes)
    dec = lambda: lac.rvq_decode(codes, Cb, G, K, R, r, Zq=Zq)
    # w = 32 >= 16: two bf16 matrix-core scans of the K codewords (w dims each; the norm starts the
    # accumulator) and a few exact fp64 distances; the executed flops are the scans', 4 r K R per token,
    # against the bf16 peak (the method's count is 2 r K R = 262144 flops per token)
    add("rvq r256 G8 K256 R2 encode (bf16 scan)", _timed(enc, flush), N * (2 * r + R * G) + Cb.numel() * 4,
        N * G * R * 2 * 2 * (r // G) * K, "alu", tokens=N, peak_tf=BF16_PEAK_TFLOPS)
    add("rvq r256 G8 K256 R2 decode (fp32)", _timed(dec, flush), N * (R * G + 4 * r) + Cb.numel() * 4,
        N * r * R, "hbm", tokens=N, peak_tf=F32_PEAK_TFLOPS)
    # the backward gradient gZ = gXhat A in the paper's grouping: 128 groups of width 2, K = 256, R = 2
    # (256 code bytes per token); the distance loop is vector-ALU work, not matrix-core work
    gZ, _ = lac.mapl_reconstruct_bwd(g["gXhat"], Z, g["A"])
    G2 = r // 2
    C2 = synth.rvq_codebooks(c["seed"], 1, G2, K, 2, 1.0, sub=1).to(dev)
    codes2 = torch.empty((N, R, G2), dtype=torch.uint8, device=dev)
    enc2 = lambda: lac.rvq_encode(gZ, C2, G2, K, R, codes=codes2)
    dec2 = lambda: lac.rvq_decode(codes2, C2, G2, K, R, r, Zq=Zq)
    add("rvq gZ r256 G128 (w2) K256 R2 encode", _timed(enc2, flush), N * (2 * r + R * G2) + C2.numel() * 4,
        N * 2 * r * K * R, "alu", tokens=N, peak_tf=F32_PEAK_TFLOPS)
    add("rvq gZ r256 G128 (w2) K256 R2 decode", _timed(dec2, flush), N * (R * G2 + 4 * r) + C2.numel() * 4,
        N * r * R, "hbm", tokens=N, peak_tf=F32_PEAK_TFLOPS)
    del g, Z, Cb, codes, Zq, gZ, C2, codes2

    # one spel_step on the fp32 2048 x 256 and 1024 x 128 projectors, flops executed.  r <= 256 (the r x r
    # iteration): the tangent projection's Gram and product and, per polar map, a Gram and X M, 2 d r^2 each
    # (12 d r^2); per polar map 8 row products (2 r^2 flops per row) for each exchanged S_k after S_0,
    # floor((n - 1) / 2) of them, and about 4 for each of the ceil(n / 2) Q steps.  r > 256 (the d x r
    # iteration): 4 d r^2 per step and the projection's.
    def ns_flops(d, r, n):
        if r <= 256:
            return 12 * d * r * r + 4 * r ** 3 * (8 * ((n - 1) // 2) + 4 * ((n + 1) // 2))
        return 4 * d * r * r * (1 + 2 * n)
    c = C["1b"]
    d, r, sp = c["d"], c["r"], c["spel"]
    si = synth.spel_inputs(c["seed"], d, r, sp["g_var"])
    A, gg, m = si["A"].to(dev), si["g"].to(dev), si["m"].to(dev)
    sws = torch.empty(lac.spel_workspace_bytes(d, r), dtype=torch.uint8, device=dev)
    # repeated steps from the same gradient: A stays on the manifold, m keeps accumulating
    spel_fn = lambda: lac.spel_step(A, gg, m, sp["alpha"], sp["beta"], sp["ns_iters"], ws=sws)
    flops = ns_flops(d, r, sp["ns_iters"])
    add("spel_step d2048 r256 NS8", _timed(spel_fn, flush), 4 * 4 * d * r, flops, "mfma", peak_tf=F32_PEAK_TFLOPS)
    # the Polar Express polar map (5 LMO / 7 retraction steps): per step a Gram (2 d r^2 with
    # both triangles), S^2 (2 r^3) and X M (2 d r^2)
    pe_fn = lambda: lac.spel_step_polar_express(A, gg, m, sp["alpha"], sp["beta"], 5, 7, ws=sws)
    pe_flops = 4 * d * r * r + 12 * (4 * d * r * r + 2 * r * r * r)
    add("spel_step d2048 r256 Polar Express 5/7", _timed(pe_fn, flush), 4 * 4 * d * r, pe_flops, "mfma",
        peak_tf=F32_PEAK_TFLOPS)
    d2, r2 = C["150m"]["d"], C["150m"]["r"]
    si2 = synth.spel_inputs(c["seed"], d2, r2, sp["g_var"])
    A2, g2, m2 = si2["A"].to(dev), si2["g"].to(dev), si2["m"].to(dev)
    sws2 = torch.empty(lac.spel_workspace_bytes(d2, r2), dtype=torch.uint8, device=dev)
    ns2 = lambda: lac.spel_step(A2, g2, m2, sp["alpha"], sp["beta"], sp["ns_iters"], ws=sws2)
    pe2 = lambda: lac.spel_step_polar_express(A2, g2, m2, sp["alpha"], sp["beta"], 5, 7, ws=sws2)
    add("spel_step d1024 r128 NS8", _timed(ns2, flush), 4 * 4 * d2 * r2, ns_flops(d2, r2, sp["ns_iters"]), "mfma",
        peak_tf=F32_PEAK_TFLOPS)
    add("spel_step d1024 r128 Polar Express 5/7", _timed(pe2, flush), 4 * 4 * d2 * r2,
        4 * d2 * r2 * r2 + 12 * (4 * d2 * r2 * r2 + 2 * r2 * r2 * r2), "mfma", peak_tf=F32_PEAK_TFLOPS)
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the boundary codec has no multi-GPU path here "
              f"(got --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import learned_activation_compression_amd as lac
    lac.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.only:
        run_only(lac, dev, args.only, max(1, args.reps))
        return
    S = Shape
    inp, g = make_inputs(dev)
    b = alloc(g, lac)
    flush = None if args.no_flush else torch.zeros(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
    stream = torch.cuda.current_stream()

    if args.copy_calibration:
        src = torch.ones(1 << 26, dtype=torch.float32, device=dev)  # 256 MiB read, 256 MiB written
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for i in range(args.warmup):
        step(lac, g, b, i)
    torch.cuda.synchronize()

    # The timed steps carry no event marker besides the step's own pair (every event record is a
    # marker the GPU waits at, a few us each).  The compress kernel, which the roofline is measured
    # on, is launched with an event pair of its own that takes the kernel's begin and end time
    # stamps (mapl_time_next_compress_kernel); the per-phase breakdown comes from a second,
    # instrumented run of the same steps.
    kc = [torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
    for e in kc:
        e.record(stream)  # torch creates an event at its first record
    step_ms, comp_ms = [], []
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        _evict(flush)
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        lac.mapl_time_next_compress_kernel(kc[0], kc[1])
        step(lac, g, b, args.warmup + i)
        s1.record(stream)
        torch.cuda.synchronize()
        step_ms.append(s0.elapsed_time(s1))
        comp_ms.append(kc[0].elapsed_time(kc[1]))
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ev = {p: [torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for p in PHASES}
    phase_ms, inst_ms = {p: [] for p in PHASES}, []
    for i in range(args.steps):
        _evict(flush)
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        step(lac, g, b, args.warmup + args.steps + i, ev)
        s1.record(stream)
        torch.cuda.synchronize()
        inst_ms.append(s0.elapsed_time(s1))
        for p in PHASES:
            phase_ms[p].append(ev[p][0].elapsed_time(ev[p][1]))

    # compress+reconstruct pair, cold (flushed) and warm
    pair_cold, pair_warm = [], []
    for i in range(args.steps):
        _evict(flush)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        pair(lac, g, b)
        e1.record(stream)
        torch.cuda.synchronize()
        pair_cold.append(e0.elapsed_time(e1))
    for i in range(args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        pair(lac, g, b)
        e1.record(stream)
        torch.cuda.synchronize()
        pair_warm.append(e0.elapsed_time(e1))

    ms = float(np.mean(step_ms))
    med = {p: float(np.median(v)) for p, v in phase_ms.items()}
    alg = algorithmic(inp)
    # the metric's dominant kernel: compress (Eq. 1), one launch per step, timed cold by its own
    # kernel events in the timed steps
    dom_bytes = alg["compress_bytes"]
    comp_med = float(np.median(comp_ms))
    dom_s = comp_med * 1e-3
    achieved = dom_bytes / dom_s / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": counter_traffic(),
                "kernel": "compress (k_tok_reduce_dma<1, 6, 2, true, false>)", "algorithmic_bytes": dom_bytes,
                "ms": round(comp_med, 5), "timing": "kernel begin/end stamps (hipExtLaunchKernelGGL events)",
                "ms_between_event_markers": round(med["compress"], 5)}
    pc = float(np.median(pair_cold))
    pw = float(np.median(pair_warm))
    pair_bytes = alg["compress_bytes"] + alg["reconstruct_bytes"]
    pair_flops = alg["compress_flops"] + alg["reconstruct_flops"]

    out = {
        "metric": "boundary tokens/s compress+reconstruct (d=1024,r=128) and % HBM/MFMA roofline",
        "value": round(S.N / (ms * 1e-3), 1),
        "unit": "boundary tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "150M-shaped boundary, whole hot path per step (codec fwd+bwd, RVQ G=4xw32 K=256 "
                               "R=2, stream sync, spel_step 1024x128 NS8)",
                   "B": S.B, "T": S.T, "N": S.N, "d": S.d, "r": S.r, "V": S.V, "flush_between_steps": flush is not None},
        "roofline": roofline,
        "pair": {"tokens_per_s": round(S.N / (pc * 1e-3), 1), "ms": round(pc, 5), "ms_warm": round(pw, 5),
                 "hbm_frac": round(pair_bytes / (pc * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                 "mfma_frac": round(pair_flops / (pc * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                 "algorithmic_bytes": pair_bytes, "flops": pair_flops},
        "phase_ms": {p: round(v, 5) for p, v in med.items()},
        "phase_run_ms_per_step": round(float(np.mean(inst_ms)), 5),
        "wall_s_timed_loop": round(wall, 3),
        "device": _device_info(),
        "distinct_tids": alg["n_distinct"],
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, min(args.cpu_tokens, S.N), max(1, args.cpu_reps))
    if args.cases:
        res = run_cases(lac, dev, flush)
        with open(args.cases, "w") as f:
            json.dump(res, f, indent=1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
