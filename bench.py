"""Benchmark of the block-sparse attention path on one MI355X.

One step = the whole path on one batch: plan (pool Q and K, pooled scores, per-row top-k)
and forward (INT8/FP8 quantization, block-sparse attention). Inputs are seeded synthetic
3-D grid Q/K/V resident in HBM before the timed region. Prints one JSON line.

The step is two library calls: sparse_attn_plan_prepare (block means, pooled scores and top-k,
and the INT8/FP8 quantization, with one pass over Q, K and V) and sparse_attn_attend.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config 720p] [--cold] [--graph]
                    [--no-cpu-baseline] [--calibrate-copy]

Default workload: the 720p-shaped quantized case, B=1 H=40 L=75600 (21x45x80 grid), d=128,
block_q=128, block_k=64, keep 0.10 (119 of 1182 key blocks per query block).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "ms/call + dense-equiv TFLOP/s, sparse attn L=75600 H=40 d=128 keep=10%"
PEAKS = {"int8fp8": 5.0e15, "fp8": 5.0e15, "bf16": 2.5e15}  # dense MFMA peaks of MI355X (ops/s)
COUNTERS = os.path.join(ROOT, "profiles", "attn_i8f8_720p_traffic.json")
ATTN_SRC = os.path.join(ROOT, "dynamic_block_sparse_mean_amd", "csrc", "attn.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="720p", choices=["720p", "480p", "long", "long_dense", "sweep", "tiny"])
    ap.add_argument("--keep", type=float, default=None, help="override the keep ratio")
    ap.add_argument("--heads", type=int, default=None,
                    help="run only the first H heads (5: one GPU's share of the 40 heads over 8 GPUs)")
    ap.add_argument("--all-keeps", action="store_true",
                    help="also time plan_prepare and attend at every keep ratio of the workload (keep sweep)")
    ap.add_argument("--mode", default=None, choices=["int8fp8", "fp8", "bf16"],
                    help="override the workload's arithmetic (fp8: Q, K and V all in E4M3)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip timing the CPU oracle and the workload statistics it comes with")
    ap.add_argument("--graph", action="store_true",
                    help="capture plan_prepare and attend once as two HIP graphs and replay them each "
                         "step (for the launch-bound small workloads)")
    ap.add_argument("--cold", action="store_true",
                    help="write 512 MB of scratch before every timed step so no input stays in the "
                         "caches (for the small workloads; the step time then comes from HIP events)")
    ap.add_argument("--no-prologue", action="store_true",
                    help="skip timing plan_prepare with the fused Q/K prologue (RMSNorm + 3-D RoPE)")
    ap.add_argument("--no-gemm", action="store_true",
                    help="skip timing the NVFP4 block-scaled GEMM at the 720p FFN shape")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the 1.5 s attend loop that samples the shader clock (for profiled runs)")
    ap.add_argument("--ulysses", type=int, default=8, metavar="P",
                    help="also time one peer's Light-Ulysses FP8 pack/unpack kernels for P peers at the "
                         "workload's shape (0 skips)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (for counter calibration)")
    ap.add_argument("--summarize-traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR", "CAL_WRITE_DIR"),
                    help="write the attention kernel's per-launch HBM traffic from four rocprofv3 --pmc "
                         "output folders (FETCH_SIZE and WRITE_SIZE of a bench run, then of --calibrate-copy)")
    return ap.parse_args()


def workload(name, keep_override, heads=None):
    import dataclasses

    from synth import CONFIGS

    if name == "long_dense":
        cfg, keep = CONFIGS["long"], 1.0
    else:
        cfg = CONFIGS[name]
        keep = cfg.keep
    if keep_override is not None:
        keep = keep_override
    if heads:  # the first `heads` heads of the workload (e.g. one GPU's share of a head split)
        cfg = dataclasses.replace(cfg, H=heads)
    return cfg, keep


def upload(cfg):
    import numpy as np
    import torch

    from synth import head_qkv

    dev = torch.device("cuda:0")
    B, H, L, d = cfg.B, cfg.H, cfg.L, cfg.d
    qkv = [torch.empty((B, H, L, d), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    for b in range(B):
        sigma = cfg.sigmas[b % len(cfg.sigmas)]
        for h in range(H):
            for t, x in zip(qkv, head_qkv(cfg.seed, b, h, cfg.grid, d, sigma)):
                t[b, h].copy_(torch.from_numpy(np.ascontiguousarray(x)))
    torch.cuda.synchronize()
    return qkv


def valid_pairs(plan_np, L, bq, bk):
    """Number of (query, key) pairs inside the kept tiles, padding excluded."""
    import numpy as np

    nQ = plan_np.shape[2]
    qrows = np.full(nQ, bq, dtype=np.int64)
    qrows[-1] = L - bq * (nQ - 1)
    last = (L + bk - 1) // bk - 1
    kcols = np.where(plan_np == last, L - bk * last, bk).astype(np.int64).sum(axis=-1)  # [B,H,nQ]
    return int((kcols * qrows[None, None, :]).sum())


def _counter_rows(folder, counter):
    """(kernel name, value) rows of one rocprofv3 --pmc csv output folder."""
    import csv
    import glob

    rows = []
    for path in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    if not rows:
        raise SystemExit(f"no {counter} rows under {folder}")
    return rows


def summarize_traffic(fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, kernel="attn_i8f8_kernel"):
    """Per-launch HBM bytes of `kernel` from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each
    scaled by what the same counter reads for a plain copy of known size."""
    n = 1 << 30  # bytes read and written by --calibrate-copy
    cal_f = [v for name, v in _counter_rows(cal_fetch_dir, "FETCH_SIZE") if "copyBuffer" in name]
    cal_w = [v for name, v in _counter_rows(cal_write_dir, "WRITE_SIZE") if "copyBuffer" in name]
    f_scale = n / (sum(cal_f) / len(cal_f) * 1024)
    w_scale = n / (sum(cal_w) / len(cal_w) * 1024)
    fk = [v for name, v in _counter_rows(fetch_dir, "FETCH_SIZE") if kernel in name]
    wk = [v for name, v in _counter_rows(write_dir, "WRITE_SIZE") if kernel in name]
    fetch = sum(fk) / len(fk) * 1024 * f_scale
    write = sum(wk) / len(wk) * 1024 * w_scale
    rec = {
        "kernel": kernel,
        "workload": "720p",
        "attn_source_sha256": hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest(),
        "fetch_size_kib_per_dispatch": sum(fk) / len(fk),
        "write_size_kib_per_dispatch": sum(wk) / len(wk),
        "dispatches": [len(fk), len(wk)],
        "copy_calibration": {"bytes": n, "fetch_scale": f_scale, "write_scale": w_scale},
        "bytes_per_launch": fetch + write,
    }
    os.makedirs(os.path.dirname(COUNTERS), exist_ok=True)
    with open(COUNTERS, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def traffic_from_profile():
    """HBM bytes per attend launch from the committed counter summary, if it was taken on
    the current attention source; else None."""
    if not os.path.exists(COUNTERS):
        return None
    with open(COUNTERS) as f:
        rec = json.load(f)
    src = hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()
    if rec.get("attn_source_sha256") != src:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(cfg, keep, dense_flops, mode="int8fp8", heads_sampled=4, blocks_per_head=150):
    """The oracle, untuned, on a bounded sample of the same workload, scaled to it: the full
    plan and quantization of `heads_sampled` heads, and the attention of `blocks_per_head`
    evenly spaced query blocks of each (about 15-25 s on 16 host cores). In bf16 mode the
    oracle is exact attention over the kept blocks, computed for one whole head."""
    import numpy as np
    import torch

    import oracle
    from synth import head_qkv

    try:
        from threadpoolctl import threadpool_info

        pools = threadpool_info()
        threads = max([i.get("num_threads", 1) for i in pools] or [1])
        blas = sorted({f"{i.get('internal_api', '?')}:{i.get('num_threads', '?')}" for i in pools})
    except Exception:  # pragma: no cover
        threads, blas = 1, []
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    bq, bk = cfg.block_q, cfg.block_k
    heads = cfg.B * cfg.H
    if mode == "bf16":
        heads_sampled = 1
    sampled = [int(x) for x in np.linspace(0, heads - 1, heads_sampled)]
    qk_quant = oracle.quantize_fp8_blocks if mode == "fp8" else oracle.quantize_int8_blocks
    t_plan = t_quant = t_att = 0.0
    n_blocks = 0
    nQ = None
    for bh in sampled:
        b, h = divmod(bh, cfg.H)
        q, k, v = head_qkv(cfg.seed, b, h, cfg.grid, cfg.d, cfg.sigmas[b % len(cfg.sigmas)])
        q, k, v = (torch.from_numpy(x).to(torch.bfloat16).float().numpy()[None, None] for x in (q, k, v))
        t0 = time.perf_counter()
        pl = oracle.plan(q, k, bq, bk, keep)
        t1 = time.perf_counter()
        nQ = pl.shape[2]
        if mode == "bf16":
            t2 = t1
            oracle.attend_exact(q, k, v, pl, bq, bk)
            rows = range(nQ)
        else:
            Qh, sq = qk_quant(q, bq)
            Kh, sk = qk_quant(k, bk)
            Vq, sv = oracle.quantize_fp8_blocks(v, bk)
            t2 = time.perf_counter()
            rows = [(0, 0, int(i)) for i in np.linspace(0, nQ - 1, min(blocks_per_head, nQ))]
            oracle.attend_quantized(Qh, sq, Kh, sk, Vq, sv, pl, bq, bk, rows=rows)
        t3 = time.perf_counter()
        t_plan += t1 - t0
        t_quant += t2 - t1
        t_att += t3 - t2
        n_blocks += len(rows)
    per_head = (t_plan + t_quant) / len(sampled) + nQ * t_att / n_blocks
    total = heads * per_head
    what = "exact attention" if mode == "bf16" else "quantized attention"
    return {
        "value": dense_flops / total / 1e12,
        "unit": "dense-equiv TFLOP/s",
        "ms_per_call": total * 1e3,
        "cores": threads,
        "kind": "oracle",
        "host": {"cpu_model": cpu_model, "os_cpu_count": os.cpu_count(), "thread_pools": blas},
        "sample": (f"{len(sampled)} of {heads} heads: full plan ({t_plan:.1f} s) and quantization "
                   f"({t_quant:.1f} s), {what} of {n_blocks} query blocks "
                   f"({n_blocks // len(sampled)} of {nQ} per head, {t_att:.1f} s); scaled to "
                   f"{heads} heads x {nQ} blocks"),
    }


def workload_stats(cfg, keep, heads_sampled=4, blocks_per_head=4, rows_per_block=32):
    """How peaked the workload's attention is, on a sample of rows: the mean entropy (nats) of a
    query's dense softmax over all L keys, against log(L) for a uniform row, and the mean share
    of that softmax's mass that falls in the key blocks the oracle's plan keeps for the row's
    query block. Computed in fp64 on the host from the same seeded bf16 inputs."""
    import numpy as np
    import torch

    import oracle
    from synth import head_qkv

    bq, bk, d, L = cfg.block_q, cfg.block_k, cfg.d, cfg.L
    sm = 1.0 / math.sqrt(d)
    heads = cfg.B * cfg.H
    ent, kept, n = 0.0, 0.0, 0
    for bh in [int(x) for x in np.linspace(0, heads - 1, min(heads_sampled, heads))]:
        b, h = divmod(bh, cfg.H)
        q, k, _ = head_qkv(cfg.seed, b, h, cfg.grid, d, cfg.sigmas[b % len(cfg.sigmas)])
        q, k = (torch.from_numpy(x).to(torch.bfloat16).double().numpy() for x in (q, k))
        pl = oracle.plan(q[None, None], k[None, None], bq, bk, keep)[0, 0]
        nQ = pl.shape[0]
        for i in [int(x) for x in np.linspace(0, nQ - 1, min(blocks_per_head, nQ))]:
            r0, r1 = i * bq, min((i + 1) * bq, L)
            rows = np.linspace(r0, r1 - 1, min(rows_per_block, r1 - r0)).astype(np.int64)
            z = sm * (q[rows] @ k.T)
            z -= z.max(axis=1, keepdims=True)
            w = np.exp(z)
            w /= w.sum(axis=1, keepdims=True)
            ent += float(-(w * np.log(np.where(w > 0, w, 1.0))).sum())
            mask = np.zeros(L, dtype=bool)
            for j in pl[i]:
                mask[int(j) * bk:min((int(j) + 1) * bk, L)] = True
            kept += float(w[:, mask].sum())
            n += len(rows)
    return {"mean_row_entropy_nats": ent / n, "uniform_entropy_nats": math.log(L),
            "kept_softmax_mass": kept / n, "rows_sampled": n}


def current_sclk_mhz(text):
    """The current shader clock in a pp_dpm_sclk listing: the MHz of the line marked '*' (None
    when no line is marked)."""
    import re
    for line in text.splitlines():
        m = re.search(r"(\d+)\s*mhz\s*\*\s*$", line.strip(), re.I)
        if m:
            return int(m.group(1))
    return None


def sclk_under_load(torch, fn, seconds=1.5):
    """Median shader clock (MHz) while fn runs back to back for `seconds`, sampled every 20 ms
    from the amdgpu driver's pp_dpm_sclk of the first card (the one GPU this benchmark runs on;
    the line marked '*' carries the current clock), with
    the number of samples; None where the file cannot be read. The published peaks assume
    2.4 GHz; under sustained MFMA load the chip holds a lower clock."""
    import glob
    import threading
    paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    if not paths:
        return None
    samples, stop = [], threading.Event()

    def reader():
        while not stop.is_set():
            try:
                with open(paths[0]) as f:
                    text = f.read()
            except OSError:
                return
            mhz = current_sclk_mhz(text)
            if mhz is not None:
                samples.append(mhz)
            stop.wait(0.02)

    fn()
    torch.cuda.synchronize()
    th = threading.Thread(target=reader, daemon=True)
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    if not samples:
        return None
    return {"mhz_median": float(sorted(samples)[len(samples) // 2]), "samples": len(samples),
            "source": paths[0]}


def keep_sweep(sa, torch, np, cfg, mode, q, k, v, steps, warmup):
    """plan_prepare and attend at every keep ratio of the workload: times, and the attention
    kernel's algorithmic MFMA fraction (valid pairs x 4d / time / peak)."""
    B, H, L, d, bq, bk = cfg.B, cfg.H, cfg.L, cfg.d, cfg.block_q, cfg.block_k
    out = torch.empty_like(q)
    rows = []
    for keep in cfg.keeps:
        nK = sa.num_blocks(L, bk)
        nk = sa.n_keep(nK, keep)
        plan, ws = sa.plan_prepare(q, k, v, bq, bk, keep, mode)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for _ in range(warmup):
            sa.plan_prepare(q, k, v, bq, bk, keep, mode, out=plan, workspace=ws)
            sa.attend(q, plan, ws, bq, bk, mode, out=out)
        torch.cuda.synchronize()
        for e in ev:
            e[0].record()
            sa.plan_prepare(q, k, v, bq, bk, keep, mode, out=plan, workspace=ws)
            e[1].record()
            sa.attend(q, plan, ws, bq, bk, mode, out=out)
            e[2].record()
        torch.cuda.synchronize()
        t = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2])] for e in ev])
        pp, att = np.median(t, axis=0)
        pairs = valid_pairs(plan.cpu().numpy(), L, bq, bk)
        achieved = 4.0 * d * pairs / (att * 1e-3)
        rows.append({"keep": keep, "n_keep": nk, "plan_prepare_ms": float(pp), "attend_ms": float(att),
                     "attend_dense_equiv_tflops": 4.0 * B * H * L * L * d / (att * 1e-3) / 1e12,
                     "attend_algorithmic_tflops": achieved / 1e12, "mfma_frac": achieved / PEAKS[mode]})
        del plan, ws
    return rows


def prologue_stage(sa, torch, cfg, keep, mode, q, k, v, plan, ws_fwd, steps, warmup):
    """plan_prepare with the Q/K prologue (RMSNorm + 3-D RoPE fused into the same pass over Q, K,
    V) on the workload's inputs, against the plain plan_prepare timed in the step. Gains are
    seeded uniform(0.5, 1.5); eps 1e-6; theta 10000; the workload's token grid."""
    import numpy as np

    if mode == "bf16":
        return None
    B, H, L, d = q.shape
    r = np.random.default_rng(1234)
    pro = {"q_gain": torch.from_numpy(r.uniform(0.5, 1.5, (H, d)).astype(np.float32)).cuda(),
           "k_gain": torch.from_numpy(r.uniform(0.5, 1.5, (H, d)).astype(np.float32)).cuda(),
           "eps": 1e-6, "grid": cfg.grid, "theta": 10000.0}
    pws = torch.empty(sa.plan_prologue_workspace_bytes(B, H, L, d, cfg.block_q, cfg.block_k, cfg.grid),
                      dtype=torch.uint8, device=q.device)

    def run():
        sa.plan_prepare(q, k, v, cfg.block_q, cfg.block_k, keep, mode, out=plan, plan_workspace=pws,
                        workspace=ws_fwd, prologue=pro)

    for _ in range(warmup):
        run()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    evs[0].record()
    for _ in range(steps):
        run()
    evs[1].record()
    torch.cuda.synchronize()
    ms = evs[0].elapsed_time(evs[1]) / steps
    return {"plan_prepare_ms": ms, "grid": list(cfg.grid),
            "note": "RMSNorm (per head; fp32 operations on the exact fp64 sum of squares) + 3-D RoPE of Q and K fused into the quantization and "
                    "block-means pass; an unfused norm+rotation pass would read and write Q and K once more"}


def hbm_stages(sa, torch, q, k, v, bq, bk, mode, steps, warmup):
    """The HBM-bound passes on the workload's inputs, each timed alone with HIP events: the
    standalone block-mean pooling of Q and of K (the plan entry point's first two launches) and
    the quantization pass (prepare: INT8/FP8 codes and scales of Q, K, V, no block means).
    Algorithmic bytes: every input element read once, every output byte (pad rows of the code
    tiles included, which the pass writes as zeros) written once."""
    B, H, L, d = q.shape
    nQ, nK = sa.num_blocks(L, bq), sa.num_blocks(L, bk)
    ws = sa.prepare(q, k, v, bq, bk, mode)
    in_b = B * H * L * d * 2
    code_b = 1 if mode != "bf16" else 2
    calls = {
        "pool_q": (lambda: sa.pool(q, bq), in_b + B * H * nQ * d * 8),
        "pool_k": (lambda: sa.pool(k, bk), in_b + B * H * nK * d * 8),
        "quantize": (lambda: sa.prepare(q, k, v, bq, bk, mode, workspace=ws),
                     3 * in_b + B * H * (nQ * bq + 2 * nK * bk) * d * code_b
                     + (B * H * (nQ + 2 * nK) * 4 if mode != "bf16" else 0)),
    }
    if mode == "bf16":
        # the bf16 prepare pass only lays out K and V (Q is read by the attention kernel itself)
        calls["quantize"] = (calls["quantize"][0], 2 * in_b + 2 * B * H * nK * bk * d * 2)
    out = {}
    for name, (fn, nbytes) in calls.items():
        for _ in range(warmup):
            fn()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        evs[0].record()
        for _ in range(steps):
            fn()
        evs[1].record()
        torch.cuda.synchronize()
        ms = evs[0].elapsed_time(evs[1]) / steps
        out[name] = {"us": ms * 1e3, "bytes": nbytes, "GB/s": nbytes / (ms * 1e-3) / 1e9,
                     "frac_hbm": nbytes / (ms * 1e-3) / 8e12}
    del ws
    return out


def nvfp4_stage(sa, torch, steps, warmup, M=75600, N=13824, K=5120):
    """The block-scaled 4-bit GEMM at the FFN up-projection shape of the 720p latent (75600
    tokens, hidden 5120 -> 13824): activations and weights quantized to NVFP4 by the library,
    then the GEMM with a bf16 bias. Seeded N(0, 1) activations, N(0, 0.02^2) weights."""
    g = torch.Generator(device="cuda").manual_seed(11)
    a = torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16)
    w = (torch.randn((N, K), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    b = (torch.randn(N, generator=g, device="cuda") * 0.1).to(torch.bfloat16)
    qa = sa.nvfp4_quantize(a)
    qw = sa.nvfp4_quantize(w)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def timed(fn, n):
        for _ in range(warmup):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(n):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / n

    gemm_ms = timed(lambda: sa.nvfp4_gemm(qa, qw, b, out=y), steps)
    quant_ms = timed(lambda: sa.nvfp4_quantize(a, out=qa), steps)
    flops = 2.0 * M * N * K
    achieved = flops / (gemm_ms * 1e-3) / 1e12
    qbytes = M * K * 2 * 2 + M * K // 2 + M * K // 16  # input read twice (tensor max, blocks); codes, scales
    del a, w, y
    return {"shape": {"M": M, "N": N, "K": K},
            "gemm_ms": gemm_ms, "gemm_tflops": achieved,
            "quantize_activations_ms": quant_ms, "quantize_GB/s": qbytes / (quant_ms * 1e-3) / 1e9,
            "roofline": {"bound": "mfma", "kernel": "nvfp4_gemm_kernel", "achieved": achieved, "peak": 2500.0,
                         "unit": "TFLOP/s", "frac": achieved / 2500.0,
                         "note": "exactly dequantized fp16 operands on the fp16 MFMA (E2M1 x E4M3 needs 6 "
                                 "significant bits; the FP4 matrix path takes only power-of-two scales per 32); "
                                 "against the FP4 peak of 10100 TFLOP/s the fraction is %.3f" % (achieved / 10100.0)}}


def ulysses_stages(sa, torch, q, k, v, P, steps, warmup):
    """One peer's share of the sequence-parallel exchange around attention, at the workload's
    shape: pack its token shard of Q, K, V (sequence to head), unpack a received payload into its
    H/P heads, pack its attention output (head to sequence), unpack the returned output shard.
    The all-to-all between them needs P GPUs and is not timed; the payload it would deliver is
    stood in for by the peer's own send buffer (same size and layout). HBM-bound kernels: the
    algorithmic bytes are the bf16 rows read or written plus the payload (codes + scale bytes)."""
    B, H, L, d = q.shape
    if P < 2 or H % P:
        return None
    hp = H // P
    lmax = -(-L // P)
    if (P - 1) * lmax >= L:
        return None
    lr = lmax  # rank 0 holds a full shard
    shard = [x[:, :, :lr] for x in (q, k, v)]
    chunk, total = sa.ulysses_payload_bytes(B, hp, L, P, 3)
    chunk1, total1 = sa.ulysses_payload_bytes(B, hp, L, P, 1)
    pay3 = torch.empty(total, dtype=torch.uint8, device=q.device)
    pay1 = torch.empty(total1, dtype=torch.uint8, device=q.device)
    heads = [torch.empty((B, hp, L, d), dtype=torch.bfloat16, device=q.device) for _ in range(3)]
    back = torch.empty((B, H, lr, d), dtype=torch.bfloat16, device=q.device)
    rows3, rows1 = B * lmax * hp * 3, B * lmax * hp
    calls = {
        "pack_seq": (lambda: sa.ulysses_pack_seq(shard, L, P, 0, payload=pay3),
                     3 * B * H * lr * d * 2 + P * rows3 * (d + 1)),
        "unpack_head": (lambda: sa.ulysses_unpack_head(pay3, P, heads),
                        P * rows3 * (d + 1) + 3 * B * hp * L * d * 2),
        "pack_head": (lambda: sa.ulysses_pack_head([heads[0]], P, payload=pay1),
                      B * hp * L * d * 2 + P * rows1 * (d + 1)),
        "unpack_seq": (lambda: sa.ulysses_unpack_seq(pay1, L, P, 0, [back]),
                       P * rows1 * (d + 1) + B * H * lr * d * 2),
    }
    out = {}
    for name, (fn, nbytes) in calls.items():
        for _ in range(warmup):
            fn()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        evs[0].record()
        for _ in range(steps):
            fn()
        evs[1].record()
        torch.cuda.synchronize()
        ms = evs[0].elapsed_time(evs[1]) / steps
        out[name] = {"us": ms * 1e3, "bytes": nbytes, "GB/s": nbytes / (ms * 1e-3) / 1e9,
                     "frac_hbm": nbytes / (ms * 1e-3) / 8e12}
    # context: a plain device copy moving the same bytes as the Q/K/V pack (half read, half written)
    src = torch.empty(calls["pack_seq"][1] // 2, dtype=torch.uint8, device=q.device)
    dst = torch.empty_like(src)
    for _ in range(warmup):
        dst.copy_(src)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    evs[0].record()
    for _ in range(steps):
        dst.copy_(src)
    evs[1].record()
    torch.cuda.synchronize()
    copy_gbs = 2 * src.numel() / (evs[0].elapsed_time(evs[1]) / steps * 1e-3) / 1e9
    del src, dst
    tot_us = sum(x["us"] for x in out.values())
    tot_b = sum(x["bytes"] for x in out.values())
    return {"peers": P, "per_peer": f"B={B} H={H} L={L}: token shard {lr}, {hp} heads, Q/K/V then the output",
            "payload_bytes": {"qkv": total, "out": total1}, "kernels": out,
            "total_us": tot_us, "total_GB/s": tot_b / (tot_us * 1e-6) / 1e9, "device_copy_GB/s": copy_gbs,
            "roofline": {"bound": "hbm", "achieved": tot_b / (tot_us * 1e-6) / 1e9, "peak": 8000.0,
                         "unit": "GB/s", "frac": tot_b / (tot_us * 1e-6) / 8e12}}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: only --gpus 1 is supported (the kernels and the timed step run on one GPU; got {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic)
        return
    import numpy as np
    import torch

    if args.calibrate_copy:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n}))
        return

    import dynamic_block_sparse_mean_amd as sa

    cfg, keep = workload(args.config, args.keep, args.heads)
    mode = args.mode or ("bf16" if cfg.mode == "bf16" else "int8fp8")
    B, H, L, d, bq, bk = cfg.B, cfg.H, cfg.L, cfg.d, cfg.block_q, cfg.block_k
    print(f"[bench] generating {cfg.name}: B={B} H={H} L={L} d={d} keep={keep} mode={mode}",
          file=sys.stderr, flush=True)
    q, k, v = upload(cfg)
    nQ, nK = sa.num_blocks(L, bq), sa.num_blocks(L, bk)
    nk = sa.n_keep(nK, keep)
    plan = torch.empty((B, H, nQ, nk), dtype=torch.int32, device=q.device)
    ws_plan = torch.empty(sa.plan_workspace_bytes(B, H, L, d, bq, bk), dtype=torch.uint8, device=q.device)
    ws_fwd = torch.empty(sa.forward_workspace_bytes(B, H, L, d, bq, bk, mode), dtype=torch.uint8,
                         device=q.device)
    out = torch.empty_like(q)

    def plan_call():
        # plan (pool, score, select) and prepare (quantize) in one pass over Q, K, V
        sa.plan_prepare(q, k, v, bq, bk, keep, mode, out=plan, plan_workspace=ws_plan, workspace=ws_fwd)

    def attend_call():
        sa.attend(q, plan, ws_fwd, bq, bk, mode, out=out)

    if args.graph:  # the same calls, captured once and replayed (the library only launches kernels)
        graphs = []
        for fn in (plan_call, attend_call):
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                fn()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            graphs.append(g)
        plan_call, attend_call = graphs[0].replay, graphs[1].replay

    def step(ev=None):
        if ev: ev[0].record()
        plan_call()
        if ev: ev[1].record()
        attend_call()
        if ev: ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps); timing {args.steps}", file=sys.stderr, flush=True)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    # cold runs: 512 MB written between steps, twice the 256 MB last-level cache
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=q.device) if args.cold else None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        if flush is not None:
            flush.fill_(s & 0xFF)
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2])] for e in evs])  # ms
    # warm: wall clock over the K steps; cold: the steps' own HIP-event spans (the flushes between
    # them are not part of the work)
    ms_step = float(stage.sum(axis=1).mean()) if args.cold else wall * 1e3 / args.steps
    pp_ms, att_ms = stage.mean(axis=0)
    stage_stats = {name: {"median": float(np.median(stage[:, c])), "min": float(stage[:, c].min()),
                          "p90": float(np.quantile(stage[:, c], 0.9))}
                   for c, name in enumerate(("plan_prepare", "attend"))}
    dense_flops = 4.0 * B * H * L * L * d
    pairs = valid_pairs(plan.cpu().numpy(), L, bq, bk)
    alg_flops = 4.0 * d * pairs
    exec_flops = 4.0 * d * B * H * nQ * nk * bq * bk
    achieved = alg_flops / (att_ms * 1e-3)
    peak = PEAKS[mode]
    traffic = traffic_from_profile() if (cfg.name == "720p" and mode == "int8fp8") else None
    result = {
        "metric": METRIC,
        "value": dense_flops / (ms_step * 1e-3) / 1e12,
        "unit": "dense-equiv TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"int8fp8": "int8+fp8", "fp8": "fp8", "bf16": "bf16"}[mode],
        "data": "synthetic",
        "config": {
            "workload": (f"{cfg.name}: B={B} H={H} L={L} d={d} grid {'x'.join(map(str, cfg.grid))}, "
                         f"block_q={bq} block_k={bk} keep={keep} ({nk} of {nK} key blocks), "
                         + {"int8fp8": "INT8 Q/K + FP8 V", "fp8": "FP8 Q/K/V", "bf16": "bf16"}[mode]),
            "global_batch": B, "seq_len": L, "heads": H, "head_dim": d, "keep": keep,
            "parallelism": ("single GPU" if not args.heads else
                            f"single GPU; {H} heads, one GPU's share of a head split of the workload"),
            "caches": "cold (512 MB written before each step)" if args.cold else "warm",
            "launch": "HIP graphs (plan_prepare and attend captured once)" if args.graph else "eager",
        },
        "stages_ms": {"plan_prepare": pp_ms, "attend": att_ms},
        "stages_ms_stats": stage_stats,
        "attend": {"dense_equiv_tflops": dense_flops / (att_ms * 1e-3) / 1e12,
                   "executed_tflops": exec_flops / (att_ms * 1e-3) / 1e12,
                   "algorithmic_tflops": achieved / 1e12},
        "roofline": {"bound": "mfma", "kernel": "attn_bf16_kernel" if mode == "bf16" else "attn_i8f8_kernel",
                     "achieved": achieved / 1e12, "peak": peak / 1e12, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": traffic},
    }
    clk = None
    if not args.no_clock:
        print("[bench] shader clock under a sustained attend loop", file=sys.stderr, flush=True)
        clk = sclk_under_load(torch, attend_call)
    if clk:
        # the same algorithmic rate against the peak at the clock the chip held
        result["roofline"]["clock_mhz"] = clk["mhz_median"]
        result["roofline"]["frac_at_clock"] = achieved / (peak * clk["mhz_median"] / 2400.0)
        result["clock"] = clk
    if args.all_keeps and len(cfg.keeps) > 1:
        print(f"[bench] keep sweep {cfg.keeps}", file=sys.stderr, flush=True)
        result["keep_sweep"] = keep_sweep(sa, torch, np, cfg, mode, q, k, v, args.steps, args.warmup)
    print("[bench] HBM-bound passes alone (pooling, quantization)", file=sys.stderr, flush=True)
    result["hbm_passes"] = hbm_stages(sa, torch, q, k, v, bq, bk, mode, args.steps, args.warmup)
    if not args.no_prologue:
        print("[bench] plan_prepare with the Q/K prologue", file=sys.stderr, flush=True)
        result["prologue"] = prologue_stage(sa, torch, cfg, keep, mode, q, k, v, plan, ws_fwd, args.steps,
                                            args.warmup)
        if result["prologue"]:
            result["prologue"]["plain_plan_prepare_ms"] = pp_ms
    if not args.no_gemm:
        print("[bench] NVFP4 GEMM at the 720p FFN shape", file=sys.stderr, flush=True)
        result["nvfp4_gemm"] = nvfp4_stage(sa, torch, args.steps, args.warmup)
    if args.ulysses:
        print(f"[bench] Light-Ulysses pack/unpack, {args.ulysses} peers", file=sys.stderr, flush=True)
        result["ulysses"] = ulysses_stages(sa, torch, q, k, v, args.ulysses, args.steps, args.warmup)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(cfg, keep, dense_flops, mode)
        print("[bench] workload statistics on sampled rows", file=sys.stderr, flush=True)
        result["workload_stats"] = workload_stats(cfg, keep)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
