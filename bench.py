"""Throughput of block-diffusion attention over a cached prefix on one MI355X.

Default workload (the metric's configuration): bf16, batch 4, 28 q-heads /
4 kv-heads, head_dim 128, prefix P = 32768, block Bq = 32, 1 % of the prefix
key rows scaled by 4; one step = one blkattn_full call (prefix partials over
the key splits, the block tile, and the log-sum-exp merge). Inputs are
generated on the host from fixed seeds, uploaded once and resident in HBM
before timing; two copies are rotated so no step finds the previous step's
K/V in the 256 MB Infinity Cache.

Prints one JSON line: throughput (algorithmic TFLOP/s over the whole step),
the attention kernel's achieved HBM GB/s against the 8 TB/s peak (timed with
HIP events around that kernel on its stream), and the fp64 CPU oracle timed on
the same workload.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--path full|cached]
  python bench.py --extra          # also one JSON line per secondary path
  python bench.py --copy-probe     # plain device copy of known size (counter scale)
  python bench.py --record-traffic DIR   # write the traffic record from rocprofv3 runs
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import datagen  # noqa: E402

METRIC = "cached-prefix block-attention TFLOP/s and HBM GB/s vs roofline at P=32K, Bq=32"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
FP32_VALU_PEAK_TFLOPS = 157.3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(sh: datagen.Shape, with_block: bool = True):
    """Flops and bytes of one call: QK^T + PV over N_k keys; K/V read once per
    kv-head, Q read, O and LSE written (split partials are not counted)."""
    nk = sh.prefix_keys + (sh.block_len if with_block else 0)
    B, Hq, Hkv, Bq, d, e = sh.batch, sh.q_heads, sh.kv_heads, sh.block_len, sh.head_dim, sh.elt_bytes
    flops = 4.0 * B * Hq * Bq * nk * d
    kv = 2.0 * B * Hkv * nk * d * e
    q = B * Hq * Bq * d * e
    out = B * Hq * Bq * d * e + 4.0 * B * Hq * Bq
    idx = 4.0 * B * Hkv * sh.prefix_keys if sh.n_keep is not None else 0.0
    return dict(flops=flops, bytes=kv + q + out + idx,
                # the attention kernel's own launch: K/V (+ indices) and Q in
                kernel_bytes=kv + q + idx, units=B * Hkv,
                unit_bytes=(kv + q + idx) / (B * Hkv))


def measured_traffic(path, sh: datagen.Shape, fn_path: str):
    """HBM bytes per attention-kernel launch from the committed counter record
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy), or None when the record
    is for another workload or the kernel sources changed since it was taken."""
    if not path or not os.path.exists(path) or sh.name != "dream_gqa" or fn_path != "full":
        return None
    with open(path) as f:
        rec = json.load(f)
    srcs = rec.get("kernel_sources", [])
    if not srcs or not all(os.path.exists(os.path.join(ROOT, x)) for x in srcs):
        return None
    if sources_sha256(srcs) != rec.get("kernel_sources_sha256"):
        return None
    return rec.get("bytes_per_launch")


def sources_sha256(paths) -> str:
    """SHA-256 over the concatenated contents of the given repository files."""
    import hashlib
    h = hashlib.sha256()
    for x in paths:
        with open(os.path.join(ROOT, x), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def up(x, torch):
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def cpu_baseline(sh: datagen.Shape, inp, budget_s: float = 10.0):
    """The fp64 oracle (as it stands) over the whole workload, repeated until
    about `budget_s` seconds of CPU work; rate in the metric's unit."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    flops = algorithmic(sh)["flops"]
    times = []
    t_all = time.perf_counter()
    while not times or (time.perf_counter() - t_all < budget_s and len(times) < 10):
        t0 = time.perf_counter()
        oracle.full(inp.q, inp.k_pre, inp.v_pre, inp.k_blk, inp.v_blk, sh.scale, idx=inp.idx)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"the whole {sh.name} workload (all {sh.batch * sh.q_heads} (batch, q-head) pairs), "
                      f"{len(times)} passes, median {t:.2f} s per pass, numpy float64"}


KERNEL_SOURCES = ("cached_block_attention_amd/csrc/attn_bf16.hip", "cached_block_attention_amd/csrc/gfx950.h",
                  "cached_block_attention_amd/csrc/launch.h")


def attention_kernel_name(sh: datagen.Shape) -> str:
    """Name of the attention kernel a blkattn_full call of this workload runs:
    eight-wave workgroups with at most 224 packed rows (129 to 224 rows per
    kv-head chunk) run the ping-pong kernel with its dedicated DMA wave, fp32
    workloads the fp32 kernel, everything else the sequential bf16 kernel."""
    if sh.dtype != datagen.BF16:
        return "attn_f32_kernel"
    rows = sh.q_heads // sh.kv_heads * sh.block_len
    chunks = -(-rows // 256) if rows > 256 else 1
    per_wg = 32 * -(-(-(-rows // chunks)) // 32)
    return "attn_bf16_pp_kernel" if 128 < per_wg <= 224 else "attn_bf16_kernel"


def record_traffic(top: str, out_path: str):
    """Traffic record of the metric workload's attention kernel from four
    rocprofv3 counter runs under `top`: pmc_fetch / pmc_write (FETCH_SIZE /
    WRITE_SIZE of `bench.py --steps 5 --warmup 2 --no-cpu-baseline`) and
    pmc_cfetch / pmc_cwrite (the same counters over `bench.py --copy-probe`).
    The copy moves a known number of bytes, which gives each counter's scale."""
    import csv
    import glob

    def per_dispatch(run, kernel):
        files = glob.glob(os.path.join(top, run, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter CSV under {os.path.join(top, run)}")
        vals = []
        for f in files:
            for r in csv.DictReader(open(f)):
                if kernel in r.get("Kernel_Name", ""):
                    vals.append(float(r["Counter_Value"]))
        if not vals:
            raise SystemExit(f"kernel {kernel!r} not found in {run}")
        return sum(vals) / len(vals)

    sh = datagen.WORKLOADS["dream_gqa"]
    kern = attention_kernel_name(sh)
    copy_bytes = 1024 * 1024 * 1024
    cf = per_dispatch("pmc_cfetch", "copyBuffer")
    cw = per_dispatch("pmc_cwrite", "copyBuffer")
    fetch_scale = copy_bytes / (cf * 1024.0)
    write_scale = copy_bytes / (cw * 1024.0)
    f = per_dispatch("pmc_fetch", kern)
    w = per_dispatch("pmc_write", kern)
    rec = {
        "kernel": kern,
        "workload": "dream_gqa: bf16 B4 Hq28/Hkv4 d128 P32768 Bq32, 16 key splits",
        "kernel_sources": list(KERNEL_SOURCES),
        "kernel_sources_sha256": sources_sha256(KERNEL_SOURCES),
        "fetch_size_kib_per_dispatch": round(f, 1),
        "write_size_kib_per_dispatch": round(w, 1),
        "copy_probe": {"bytes": copy_bytes, "fetch_size_kib": round(cf, 1), "write_size_kib": round(cw, 1),
                       "fetch_scale": fetch_scale, "write_scale": write_scale},
        "bytes_per_launch": int(round(f * 1024.0 * fetch_scale + w * 1024.0 * write_scale)),
        "commands": [
            "rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT -o run -- python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline",
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT -o run -- python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline",
            "rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT -o run -- python3 bench.py --copy-probe",
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT -o run -- python3 bench.py --copy-probe",
        ],
    }
    with open(out_path, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    print(json.dumps(rec))


def copy_probe(mib: int = 1024):
    """A plain device copy of known size, for scaling memory counters."""
    import torch
    n = mib * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n * 4, "launches": 5}))


def _median_ms(fn, reps: int, warm: int = 3):
    """Median device time (ms) of fn() over `reps` calls, HIP events around each."""
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in evs]))


EXTRA_PATHS = ("prefix", "llada", "reuse", "retention", "large", "sequence")


def extra_lines(reps: int, paths=EXTRA_PATHS):
    """Timings of the other paths (one JSON line each): the prefix partial at the
    metric workload, dense attention at the LLaDA slice, the reuse path over 8
    steps, the retained-row pipeline at the sparse workload, large blocks and the
    full-sequence FACache step; `paths` picks a subset."""
    import torch
    import cached_block_attention_amd as ba

    def emit(**kw):
        print(json.dumps(kw), flush=True)

    def upl(inp):
        d = {k: up(getattr(inp, k), torch) for k in ("q", "k_pre", "v_pre", "k_blk", "v_blk")}
        d["idx"] = up(inp.idx, torch) if inp.idx is not None else None
        return d

    if "prefix" in paths:
        # prefix partial at the metric workload (the state FACache stores)
        sh = datagen.WORKLOADS["dream_gqa"]
        t = upl(datagen.make_inputs(sh))
        alg = algorithmic(sh, with_block=False)
        pp = ba.empty_partial(sh.batch, sh.q_heads, sh.block_len, sh.head_dim, "cuda")
        ms = _median_ms(lambda: ba.blkattn_prefix_partial(t["q"], t["k_pre"], t["v_pre"], pp), reps)
        emit(path="blkattn_prefix_partial", workload="dream_gqa P32768", ms=round(ms, 4),
             tflops=round(alg["flops"] / ms / 1e9, 1), hbm_gbps=round(alg["bytes"] / ms / 1e6, 1))
        del t, pp
        torch.cuda.empty_cache()

    if "llada" in paths:
        # dense attention at the LLaDA slice (fits the 256 MB MALL: timed as is)
        sh = datagen.WORKLOADS["llada_bf16"]
        t = upl(datagen.make_inputs(sh))
        alg = algorithmic(sh)
        ms = _median_ms(lambda: ba.attention(t["q"], t["k_pre"], t["v_pre"], t["k_blk"], t["v_blk"]), reps)
        emit(path="blkattn_full", workload="llada_bf16 P4096", ms=round(ms, 4),
             tflops=round(alg["flops"] / ms / 1e9, 1), hbm_gbps=round(alg["bytes"] / ms / 1e6, 1))
        del t
        torch.cuda.empty_cache()

    if "reuse" in paths:
        # reuse over 8 denoising steps: prefix partial once, then per step the fused
        # block step, or block partial + merge, against recomputing full attention
        sh = datagen.WORKLOADS["reuse_bf16"]
        inp = datagen.make_inputs(sh)
        t = upl(inp)
        steps = [(t["q"], t["k_blk"], t["v_blk"])]
        for i in range(1, sh.steps):
            qn, kn, vn = datagen.step_inputs(sh, i)
            steps.append((up(qn, torch), up(kn, torch), up(vn, torch)))
        pp = ba.empty_partial(sh.batch, sh.q_heads, sh.block_len, sh.head_dim, "cuda")
        o = torch.empty_like(t["q"])
        lse = torch.empty(sh.batch, sh.q_heads, sh.block_len, dtype=torch.float32, device="cuda")
        pb = ba.empty_partial(sh.batch, sh.q_heads, sh.block_len, sh.head_dim, "cuda")
        ms_prefix = _median_ms(lambda: ba.blkattn_prefix_partial(t["q"], t["k_pre"], t["v_pre"], pp), max(3, reps // 10))
        ms_step = float(np.median([_median_ms(lambda s=s: ba.blkattn_block_step(s[0], s[1], s[2], pp, o, lse), reps)
                                   for s in steps]))
        def two_launch(s):
            ba.blkattn_block_partial(s[0], s[1], s[2], pb)
            ba.blkattn_merge(pp, pb, o=o, lse=lse)
        ms_two = float(np.median([_median_ms(lambda s=s: two_launch(s), reps) for s in steps]))
        wsf = torch.empty(ba.workspace_bytes(ba.make_dims(t["q"], sh.kv_heads, sh.prefix_len), ba.OP_FULL) + 16,
                          dtype=torch.uint8, device="cuda")
        ms_full = _median_ms(lambda: ba.blkattn_full(steps[1][0], t["k_pre"], t["v_pre"], steps[1][1], steps[1][2], o, lse,
                                                     workspace=wsf), max(3, reps // 10))
        n = sh.steps
        emit(path="reuse", workload=f"reuse_bf16 B8 H32 P16384 Bq32, {n} steps", prefix_partial_ms=round(ms_prefix, 4),
             block_step_ms=round(ms_step, 4), block_partial_plus_merge_ms=round(ms_two, 4),
             full_recompute_ms=round(ms_full, 4),
             amortized_ms_per_step=round((ms_prefix + n * ms_step) / n, 4),
             reuse_gain=round(ms_full / ((ms_prefix + n * ms_step) / n), 2),
             prefix_partial_hbm_gbps=round(algorithmic(sh, with_block=False)["bytes"] / ms_prefix / 1e6, 1))
        del t, steps, pp, pb, inp
        torch.cuda.empty_cache()

    if "retention" in paths:
        # retained rows at the sparse workload: mass over all 131072 rows, top-k,
        # standalone gather, and the fused-gather attention over the kept rows
        sh = datagen.WORKLOADS["sparse_gqa"]
        inp = datagen.make_inputs(sh)
        t = upl(inp)
        _, lse = ba.attention(t["q"], t["k_pre"], t["v_pre"], t["k_blk"], t["v_blk"])
        mass = torch.empty(sh.batch, sh.kv_heads, sh.prefix_len, dtype=torch.float32, device="cuda")
        idx = torch.empty(sh.batch, sh.kv_heads, sh.n_keep, dtype=torch.int32, device="cuda")
        ms_mass = _median_ms(lambda: ba.blkattn_prefix_mass(t["q"], t["k_pre"], lse, mass), reps)
        sel_dims = ba.Dims(sh.batch, sh.kv_heads, sh.kv_heads, 64, 1, sh.n_keep, sh.prefix_len, ba.F32, 1.0, 0, 0)
        sel_ws = torch.empty(ba.workspace_bytes(sel_dims, ba.OP_SELECT), dtype=torch.uint8, device="cuda")
        ms_sel = _median_ms(lambda: ba.blkattn_select_retained(mass, idx, workspace=sel_ws), reps)
        ko = torch.empty(sh.batch, sh.kv_heads, sh.n_keep, sh.head_dim, dtype=t["k_pre"].dtype, device="cuda")
        vo = torch.empty_like(ko)
        ms_gather = _median_ms(lambda: ba.blkattn_gather_prefix(t["k_pre"], t["v_pre"], t["idx"], ko, vo), reps)
        ms_fused = _median_ms(lambda: ba.attention(t["q"], t["k_pre"], t["v_pre"], t["k_blk"], t["v_blk"], idx=t["idx"]), reps)
        G = sh.q_heads // sh.kv_heads
        mass_flops = 2.0 * sh.batch * sh.kv_heads * G * sh.block_len * sh.prefix_len * sh.head_dim
        mass_bytes = 2.0 * sh.batch * sh.kv_heads * sh.prefix_len * sh.head_dim + 4.0 * sh.batch * sh.kv_heads * sh.prefix_len
        alg = algorithmic(sh)
        gather_bytes = 2 * 2.0 * 2 * sh.batch * sh.kv_heads * sh.n_keep * sh.head_dim
        emit(path="retention", workload="sparse_gqa B2 Hq28/Hkv4 P_full131072 keep8192 Bq64",
             mass_ms=round(ms_mass, 4), mass_tflops=round(mass_flops / ms_mass / 1e9, 1),
             mass_hbm_gbps=round(mass_bytes / ms_mass / 1e6, 1), select_ms=round(ms_sel, 4),
             gather_ms=round(ms_gather, 4), gather_gbps=round(gather_bytes / ms_gather / 1e6, 1),
             fused_gather_full_ms=round(ms_fused, 4), fused_tflops=round(alg["flops"] / ms_fused / 1e9, 1))
        del t, inp, mass, idx, ko, vo
        torch.cuda.empty_cache()

    if "large" in paths:
        # a large block (square, compute-bound bidirectional tile): block partial
        for bq in (256, 1024):
            sh = datagen.scaled_shape("llada_bf16", block_len=bq, prefix_len=0)
            t = upl(datagen.make_inputs(sh))
            pbq = ba.empty_partial(sh.batch, sh.q_heads, bq, sh.head_dim, "cuda")
            ms = _median_ms(lambda: ba.blkattn_block_partial(t["q"], t["k_blk"], t["v_blk"], pbq), reps)
            fl = 4.0 * sh.batch * sh.q_heads * bq * bq * sh.head_dim
            emit(path="blkattn_block_partial", workload=f"large block Bq{bq} B1 H32 d128", ms=round(ms, 4),
                 tflops=round(fl / ms / 1e9, 1), mfma_frac=round(fl / ms / 1e9 / BF16_MFMA_PEAK_TFLOPS, 4))
            del t, pbq
            torch.cuda.empty_cache()

    if "sequence" in paths:
        # full-sequence FACache step (LLaDA-like: 4096 rows, block at rows 2048..2079):
        # the block's first step builds the cache, later steps reuse it; against
        # plain attention of every row over every row at each step
        sh = datagen.WORKLOADS["llada_seq"]
        B, Hq, N, d, Bq, c0 = sh.batch, sh.q_heads, sh.prefix_len, sh.head_dim, sh.block_len, sh.block_start
        q, k, v = (up(x, torch) for x in datagen.sequence_inputs(sh, 0))
        cache = ba.empty_partial(B, Hq, N, d, "cuda")
        o = torch.empty_like(q)
        lse = torch.empty(B, Hq, N, dtype=torch.float32, device="cuda")
        dims = ba.Dims(B, Hq, sh.kv_heads, d, Bq, 0, N, ba.BF16, float(sh.scale), 0, 0)
        ws = torch.empty(max(1, ba.workspace_bytes(dims, ba.OP_SEQUENCE)), dtype=torch.uint8, device="cuda")
        ms_gen = _median_ms(lambda: ba.blkattn_sequence_step(q, k, v, c0, Bq, cache, True, o, lse, workspace=ws), reps)
        ms_step = _median_ms(lambda: ba.blkattn_sequence_step(q, k, v, c0, Bq, cache, False, o, lse, workspace=ws), reps)
        full = ba.empty_partial(B, Hq, N, d, "cuda")
        ms_full = _median_ms(lambda: ba.blkattn_prefix_partial(q, k, v, full), reps)
        nu = N - Bq
        fl_gen = 4.0 * B * Hq * (nu * nu + nu * Bq + Bq * N) * d
        fl_step = 4.0 * B * Hq * (nu * Bq + Bq * N) * d
        fl_full = 4.0 * B * Hq * N * N * d
        # a reuse step reads q, the cached (o, m, l) of the other rows and the whole
        # sequence's k, v (for the block queries), and writes o and lse
        step_bytes = (2.0 * B * Hq * N * d + 4.0 * B * Hq * nu * (d + 2) + 2 * 2.0 * B * sh.kv_heads * N * d
                      + 2.0 * B * Hq * N * d + 4.0 * B * Hq * N)
        n = sh.steps
        amort = (ms_gen + (n - 1) * ms_step) / n
        emit(path="blkattn_sequence_step", workload=f"llada_seq B1 H32 d128 N{N} block [{c0},{c0 + Bq}), {n} steps",
             first_step_ms=round(ms_gen, 4), first_step_tflops=round(fl_gen / ms_gen / 1e9, 1),
             reuse_step_ms=round(ms_step, 4), reuse_step_tflops=round(fl_step / ms_step / 1e9, 1),
             reuse_step_hbm_gbps=round(step_bytes / ms_step / 1e6, 1),
             full_attention_ms=round(ms_full, 4), full_attention_tflops=round(fl_full / ms_full / 1e9, 1),
             amortized_ms_per_step=round(amort, 4), facache_gain=round(ms_full / amort, 2))
        del q, k, v, cache, o, lse, ws, full
        torch.cuda.empty_cache()


def power_line(step, seconds: float, sh: datagen.Shape):
    """Run `step` back to back for `seconds` while another thread samples the
    board (amd-smi metric -p -c) every 0.2 s; print the step time and the
    median socket power and graphics clock of the samples."""
    import subprocess
    import threading
    import torch

    samples, stop = [], [False]

    def sample():
        r = subprocess.run(["amd-smi", "metric", "-p", "-c", "--json"], capture_output=True, text=True)
        try:
            d = json.loads(r.stdout)
            g = d[0] if isinstance(d, list) else d
            g = g["gpu_data"][0] if "gpu_data" in g else g
            clocks = [v["clk"]["value"] for k, v in g["clock"].items()
                      if k.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict)
                      and isinstance(v["clk"].get("value"), (int, float))]
            return float(g["power"]["socket_power"]["value"]), float(np.mean(clocks))
        except (ValueError, KeyError, TypeError, IndexError):
            return None

    def sampler():
        while not stop[0]:
            x = sample()
            if x is not None:
                samples.append(x)
            time.sleep(0.2)

    th = threading.Thread(target=sampler)
    th.start()
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(100):
            step(n)
            n += 1
        torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    stop[0] = True
    th.join()
    tail = samples[len(samples) // 3:]  # after the first third, once power has settled
    print(json.dumps({
        "power_run": sh.name, "seconds": round(dt, 2), "steps": n, "ms_per_step": round(dt / n * 1e3, 5),
        "samples": len(tail),
        "socket_power_w_median": float(np.median([x[0] for x in tail])) if tail else None,
        "gfx_clock_mhz_median": float(np.median([x[1] for x in tail])) if tail else None,
    }), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=400,
                    help="untimed steps first; the GPU clock needs some 300 back-to-back calls to ramp up "
                         "from idle, so the timed steps see the steady state")
    ap.add_argument("--workload", default="dream_gqa",
                    choices=sorted(k for k, w in datagen.WORKLOADS.items() if w.block_start is None))
    ap.add_argument("--path", default="full", choices=["full", "cached"],
                    help="full: blkattn_full; cached: prefix partial + block partial + merge")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--power", type=float, metavar="SECONDS",
                    help="after the warmup, run the step back to back for SECONDS while sampling board power "
                         "and clocks with amd-smi; print one JSON line and exit")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--record-traffic", metavar="DIR",
                    help="write the --traffic record from the four rocprofv3 counter runs under DIR")
    ap.add_argument("--extra-path", choices=EXTRA_PATHS, action="append",
                    help="with --extra: only this secondary path (repeatable)")
    ap.add_argument("--extra", action="store_true",
                    help="time the other paths (prefix partial, LLaDA slice, reuse steps, retention, "
                         "large blocks, full-sequence step) instead of the metric line")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "attn_bf16_dream_gqa_traffic.json"),
                    help="JSON record of the attention kernel's measured HBM bytes per launch "
                         "(used only while its kernel-source hash matches the current source)")
    args = ap.parse_args()

    if args.record_traffic:
        record_traffic(args.record_traffic, args.traffic)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for {max(args.gpus, world)}): the path would shard "
              "over (batch, kv-head) groups with no communication", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_probe:
        copy_probe()
        return
    if args.extra:
        extra_lines(max(10, args.steps // 10), tuple(args.extra_path or EXTRA_PATHS))
        return
    import cached_block_attention_amd as ba
    ba.library()

    sh = datagen.WORKLOADS[args.workload]
    log(f"generating {sh.name} inputs")
    inp = datagen.make_inputs(sh)
    copies = []
    for c in range(2):
        d = {k: up(getattr(inp, k), torch) for k in ("q", "k_pre", "v_pre", "k_blk", "v_blk")}
        d["idx"] = up(inp.idx, torch) if inp.idx is not None else None
        copies.append(d)
    B, Hq, Bq, dh = inp.q.shape
    dtype = copies[0]["q"].dtype
    o = torch.empty(B, Hq, Bq, dh, dtype=dtype, device="cuda")
    lse = torch.empty(B, Hq, Bq, dtype=torch.float32, device="cuda")
    dims = ba.make_dims(copies[0]["q"], sh.kv_heads, sh.prefix_len,
                        sh.n_keep or 0)
    ws = torch.empty(max(ba.workspace_bytes(dims, ba.OP_FULL),
                         ba.workspace_bytes(dims, ba.OP_PREFIX_PARTIAL), 16),
                     dtype=torch.uint8, device="cuda")
    pp = ba.empty_partial(B, Hq, Bq, dh, "cuda")
    pb = ba.empty_partial(B, Hq, Bq, dh, "cuda")
    splits = ba.plan_splits(dims, ba.OP_FULL if args.path == "full" else ba.OP_PREFIX_PARTIAL)

    def step(i, ev=None):
        t = copies[i % 2]
        if ev is not None:
            ba.set_kernel_events(*ev)
        if args.path == "full":
            ba.blkattn_full(t["q"], t["k_pre"], t["v_pre"], t["k_blk"], t["v_blk"], o, lse,
                            idx=t["idx"], workspace=ws)
        else:
            ba.blkattn_prefix_partial(t["q"], t["k_pre"], t["v_pre"], pp, idx=t["idx"], workspace=ws)
            ba.blkattn_block_partial(t["q"], t["k_blk"], t["v_blk"], pb)
            ba.blkattn_merge(pp, pb, o=o, lse=lse)

    log(f"warmup {args.warmup} steps")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if args.power:
        power_line(step, args.power, sh)
        return

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in evs:   # create the HIP events before the timed region
        a.record()
        b.record()
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    # The K timed steps run exactly as a caller runs them. Events around
    # every attention launch would stretch each step (the stream waits on
    # them between kernels), so the kernel's own duration comes from a second
    # pass of K steps with per-launch events.
    log(f"timing {args.steps} steps")
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(args.steps):
        step(i)
    t_stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_stop) / args.steps
    log(f"timing the attention kernel over {args.steps} more steps")
    t_start.record()
    for i in range(args.steps):
        step(i, evs[i])
    t_stop.record()
    torch.cuda.synchronize()
    ms_step_ev = t_start.elapsed_time(t_stop) / args.steps
    k_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))

    alg = algorithmic(sh, with_block=(args.path == "full"))
    full_alg = algorithmic(sh)
    tflops = full_alg["flops"] / (ms_step * 1e-3) / 1e12
    achieved = alg["kernel_bytes"] / (k_ms * 1e-3) / 1e9
    traffic = measured_traffic(args.traffic, sh, args.path)

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on the host")
        cpu = cpu_baseline(sh, inp)

    line = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if sh.dtype == datagen.BF16 else "f32",
        "data": "synthetic: seeded N(0,1) inputs rounded to bf16 (datagen.py); no dataset or weights",
        "config": {
            "workload": (f"{sh.name}: {sh.dtype} B{sh.batch} Hq{sh.q_heads}/Hkv{sh.kv_heads} "
                         f"d{sh.head_dim} P{sh.prefix_len}"
                         + (f" keep{sh.n_keep}" if sh.n_keep else "")
                         + f" Bq{sh.block_len}"),
            "function": "blkattn_full" if args.path == "full" else
                        "blkattn_prefix_partial+blkattn_block_partial+blkattn_merge",
            "key_splits": splits,
            "batch": sh.batch, "prefix_len": sh.prefix_len, "block_len": sh.block_len,
        },
        "hbm_gbps_step": round(full_alg["bytes"] / (ms_step * 1e-3) / 1e9, 1),
        "mfma_frac_step": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
        "roofline": {
            "bound": "hbm",
            "kernel": attention_kernel_name(sh),
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel_ms": round(k_ms, 6),
            "kernel_ms_from": f"HIP events of each attention launch over a second pass of {args.steps} steps "
                              f"({ms_step_ev:.6f} ms per step with the events)",
            "algorithmic_bytes_per_launch": alg["kernel_bytes"],
        },
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 4),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
