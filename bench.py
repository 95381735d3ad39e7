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
  python bench.py --copy-probe     # plain device copy of known size (counter scale)
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
    is for another workload or the kernel source changed since it was taken."""
    import hashlib
    if not path or not os.path.exists(path) or sh.name != "dream_gqa" or fn_path != "full":
        return None
    with open(path) as f:
        rec = json.load(f)
    src = os.path.join(ROOT, rec.get("kernel_source", ""))
    if not os.path.exists(src):
        return None
    with open(src, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != rec.get("kernel_source_sha256"):
            return None
    return rec.get("bytes_per_launch")


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="dream_gqa", choices=sorted(datagen.WORKLOADS))
    ap.add_argument("--path", default="full", choices=["full", "cached"],
                    help="full: blkattn_full; cached: prefix partial + block partial + merge")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "attn_bf16_dream_gqa_traffic.json"),
                    help="JSON record of the attention kernel's measured HBM bytes per launch "
                         "(used only while its kernel-source hash matches the current source)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for {max(args.gpus, world)}): the path shards "
              "over (batch, kv-head) groups with no communication, see DESIGN.md", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_probe:
        copy_probe()
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

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in evs:   # create the HIP events before the timed region
        a.record()
        b.record()
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(args.steps):
        step(i, evs[i])
    t_stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_start.elapsed_time(t_stop)
    ms_step = ms_total / args.steps
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
            "kernel": "attn_bf16_kernel" if sh.dtype == datagen.BF16 else "attn_f32_kernel",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel_ms": round(k_ms, 6),
            "algorithmic_bytes_per_launch": alg["kernel_bytes"],
        },
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 4),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
