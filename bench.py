"""Benchmark: Prism estimator + block-sparse causal prefill for one attention
layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole path over one layer's inputs, resident in
HBM: prism_estimate (block means and energies, temperatures, scores, Top-P,
union) followed by prism_block_sparse_attn over the resulting mask. Before
each step a 512 MB scratch buffer is read so that the 256 MB Infinity Cache
holds none of Q, K, V from the previous step. (Reading rather than writing
it: a write would leave the cache full of dirty lines whose write-back then
falls inside the timed region, traffic that is not the step's; the estimator
after a written flush is reported beside the line for comparison.) HIP events
around each call (on
the stream the kernels run on) time the phases; `value` is the median over the
K timed steps of estimator + attention. The K steps run back to back between
device synchronisations; their wall time per step (scratch reads included)
is reported too. Prints one JSON line.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "estimator ms + block-sparse prefill ms/layer at 128K; speedup vs dense"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
ATTN_SRC = os.path.join(ROOT, "block_sparse_attention_band_amd", "csrc", "sparse_attn.hip")
def traffic_file(workload):
    """rocprofv3 traffic summary of the attention kernel on this workload"""
    return os.path.join(ROOT, "profiles", f"sparse_attn_bf16_{workload}_traffic.txt")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def attention_flops(mask, block, head_dim):
    """Algorithmic FLOPs of causal block-sparse attention for a uint8 mask
    [b, H, nb, nb] on the device: 4 B^2 d per selected block below the
    diagonal, 2 B^2 d per selected diagonal block."""
    import torch
    nb = mask.shape[-1]
    m = mask.bool()
    diag = torch.diagonal(m, dim1=-2, dim2=-1).sum().item()
    below = torch.tril(m, diagonal=-1).sum().item()
    return 4.0 * block * block * head_dim * below + 2.0 * block * block * head_dim * diag, below + diag


def traffic_from_profile(workload):
    """HBM bytes per launch measured by rocprofv3 counters for the current
    attention kernel source on this workload, or None when absent, taken on
    other source or on another workload."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != attn_build_sha() or "hbm_bytes_per_launch" not in vals:
        return None
    return float(vals["hbm_bytes_per_launch"])


def attn_build_sha():
    """sha256 over the attention kernel's code (comments and whitespace
    stripped, so a comment edit keeps a measurement valid) and the hipcc
    flags it is built with"""
    from block_sparse_attention_band_amd import build
    src = open(ATTN_SRC).read()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    h = hashlib.sha256(" ".join(src.split()).encode())
    flags = [f for f in build.flags() if not f.startswith("/")] + build.EXTRA.get("sparse_attn.hip", [])
    h.update(" ".join(flags).encode())
    return h.hexdigest()


def machine_microbench():
    """Context for the roofline fractions, measured on this GPU: a plain
    device-to-device copy of 1 GiB (GB/s of bytes read + written) and a large
    bf16 GEMM through torch.matmul (the vendor BLAS), best of 5 each."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def best(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            ev[0].record()
            fn()
            ev[1].record()
            torch.cuda.synchronize()
            ts.append(ev[0].elapsed_time(ev[1]))
        return min(ts)

    src = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    copy_ms = best(lambda: dst.copy_(src))
    del src, dst
    n = 8192
    a = torch.randn(n, n, dtype=torch.bfloat16, device="cuda")
    b = torch.randn(n, n, dtype=torch.bfloat16, device="cuda")
    c = torch.empty(n, n, dtype=torch.bfloat16, device="cuda")
    gemm_ms = best(lambda: torch.matmul(a, b, out=c))
    del a, b, c
    return {"copy_gbs": round(2 * (1 << 30) / (copy_ms * 1e-3) / 1e9, 1),
            "gemm_bf16_8192_tflops": round(2 * n ** 3 / (gemm_ms * 1e-3) / 1e12, 1)}


def cpu_baseline(q, k, v, mask_np, out_bits, w, budget_s=24.0):
    """The CPU oracle on a bounded sample of the same layer, extrapolated to
    ms per layer: the estimator head by head (KV group by KV group) and the
    attention on 16 query-block rows per head, head by head, each until about
    half of `budget_s` is spent. The oracle's results are then compared with
    the GPU's (outside the timed calls): the mask of every head it estimated,
    under the GPU tests' mask rule, and the attention rows against the GPU's
    sparse output `out_bits` (as stored: bf16 bits or fp32)."""
    import oracle.prism_oracle as po
    from synth import to_f64
    from tests.parity import compare_masks
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    cpu_model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    t_est = 0.0
    heads_done = 0
    per_head = {}
    mask_check = {}
    for g in range(w.hkv):
        t0 = time.perf_counter()
        kbar = po.mean_pool(to_f64(k[0, :, g, :], w.dtype), w.block)
        t_est += time.perf_counter() - t0
        for h in range(w.hq):
            if po.kv_head(h, w.hq, w.hkv) != g:
                continue
            t0 = time.perf_counter()
            r = po.estimate_head(to_f64(q[0, :, h, :], w.dtype), None, block=w.block, d_high=w.d_high,
                                 d_low=w.d_low, p=w.p, causal=True, kbar=kbar)
            t_est += time.perf_counter() - t0
            per_head[(0, h)] = r
            heads_done += 1
        stats = compare_masks(mask_np, per_head, w.p, True)  # untimed; frees the per-head arrays
        per_head.clear()
        for key in ("blocks", "mismatch", "mass_tie", "score_tie", "unexcused"):
            mask_check[key] = mask_check.get(key, 0) + stats[key]
        if t_est > budget_s / 2:
            break
    est_ms = t_est / heads_done * w.hq * 1e3
    mask_check["heads"] = heads_done
    # attention: 16 query-block rows spread over the causal length, head after
    # head, until half the budget is spent
    nb = w.nb
    rows = sorted({min(nb - 1, max(0, (nb * f) // 16)) for f in range(16, 0, -1)}, reverse=True)
    t_attn = 0.0
    blocks_done = 0
    used = []
    max_abs = rel_norm = 0.0
    for h in range(w.hq):
        g = po.kv_head(h, w.hq, w.hkv)
        t0 = time.perf_counter()
        qh, kh, vh = to_f64(q[0, :, h, :], w.dtype), to_f64(k[0, :, g, :], w.dtype), to_f64(v[0, :, g, :], w.dtype)
        t_attn += time.perf_counter() - t0
        for i in rows:
            t0 = time.perf_counter()
            oo = po.attention_block_row(qh, kh, vh, mask_np[0, h, i], i, block=w.block, causal=True)
            t_attn += time.perf_counter() - t0
            blocks_done += int(mask_np[0, h, i, : i + 1].sum())
            used.append((h, i))
            og = to_f64(out_bits[0, i * w.block: min((i + 1) * w.block, w.seq), h, :], w.dtype)
            max_abs = max(max_abs, float(np.abs(og - oo).max()))
            rel_norm = max(rel_norm, float(np.linalg.norm(og - oo) / max(np.linalg.norm(oo), 1e-30)))
        if t_attn > budget_s / 2:
            break
    total_blocks = int(np.tril(mask_np[0]).sum())
    attn_ms = t_attn / max(1, blocks_done) * total_blocks * 1e3
    return {
        "value": round(est_ms + attn_ms, 1), "unit": "ms", "cores": int(threads), "cpu_model": cpu_model, "kind": "oracle",
        "sample": (f"float64 numpy oracle; estimator on {heads_done} of {w.hq} query heads ({t_est:.1f} s), "
                   f"attention on query-block rows {rows} of heads 0..{used[-1][0]} ({len(used)} rows, "
                   f"{blocks_done} selected blocks, {t_attn:.1f} s); both extrapolated linearly to the whole "
                   f"layer ({w.hq} heads; {total_blocks} selected blocks over all heads) -- estimator {est_ms:.0f} ms "
                   f"+ attention {attn_ms:.0f} ms"),
        "estimator_ms": round(est_ms, 1), "attention_ms": round(attn_ms, 1),
    }, {"mask": dict(mask_check), "attention": {"rows": len(used), "max_abs": max_abs, "rel_norm": rel_norm,
                                                "tolerance": "max_abs <= 2e-2 and rel_norm <= 1e-2 (bf16)"}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3_8b_128k")
    ap.add_argument("--mask-bits", action="store_true", help="bit-packed block mask (one bit per block)")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense baselines")
    ap.add_argument("--no-machine", action="store_true", help="skip the copy / GEMM microbenchmarks")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--density-sweep", default="",
                    help="comma-separated block densities: after the line's measurement, time the attention on "
                         "seeded random causal block masks of these densities (diagonal blocks kept), reported "
                         "beside the line as `density_sweep`")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run one plain 1 GiB device-to-device copy (reads 1 GiB, writes 1 GiB), the "
                         "reference dispatch for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path is per head and shards "
              f"by KV group without any collective -- run one process per GPU on its own heads.", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_attention_band_amd as prism
    from synth import WORKLOADS, make_qkv

    if args.calibrate_copy:
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: 1073741824 bytes read, 1073741824 bytes written")
        del src, dst

    w = WORKLOADS[args.workload]
    log(f"workload {w.name}: seq={w.seq} hq={w.hq} hkv={w.hkv} {w.dtype}; generating inputs")
    t = time.perf_counter()
    q, k, v = make_qkv(w)
    log(f"inputs ready in {time.perf_counter() - t:.1f}s; uploading")

    def dev(x):
        if w.dtype == "bf16":
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(x).cuda()

    qd, kd, vd = dev(q), dev(k), dev(v)
    cfg = prism.EstimatorConfig(block_size=w.block, d_high=w.d_high, d_low=w.d_low, p=w.p, causal=True)
    ws = prism.new_workspace(qd, kd, cfg)
    nb = w.nb
    if args.mask_bits:
        mask = torch.empty((w.batch, w.hq, nb, (nb + 31) // 32), dtype=torch.int32, device="cuda")
    else:
        mask = torch.empty((w.batch, w.hq, nb, nb), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(qd)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        prism.estimate(qd, kd, cfg, workspace=ws, mask_out=mask)
        if ev is not None:
            ev[1].record()
        prism.block_sparse_attn(qd, kd, vd, mask, out=out)
        if ev is not None:
            ev[2].record()

    scratch = torch.ones(128 << 20, dtype=torch.float32, device="cuda")  # 512 MB

    def flush():  # evict Q, K, V and the previous step's data from the Infinity Cache (reads only)
        scratch.sum()

    for i in range(args.warmup):
        flush()
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps); timing {args.steps} steps")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        flush()
        step(evs[i])
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    est = [e[0].elapsed_time(e[1]) for e in evs]
    attn = [e[1].elapsed_time(e[2]) for e in evs]
    step_ms = float(np.median([a + b for a, b in zip(est, attn)]))
    est_ms, attn_ms = float(np.median(est)), float(np.median(attn))
    log(f"timed: {step_ms:.3f} ms/step (median), estimator {est_ms:.3f} ms, attention {attn_ms:.3f} ms, "
        f"{wall_ms:.3f} ms/step wall incl. cache flush")

    # context: the estimator after a *written* 512 MB flush, whose dirty lines are written back
    # during the call (reported beside `value`, not in it)
    est_w = []
    for _ in range(args.steps):
        scratch.fill_(1.0)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        prism.estimate(qd, kd, cfg, workspace=ws, mask_out=mask)
        ev[1].record()
        torch.cuda.synchronize()
        est_w.append(ev[0].elapsed_time(ev[1]))
    est_written_flush_ms = float(np.median(est_w))

    # context: the same estimator as one persistent launch (grid barrier instead of kernel
    # boundaries), read-flushed like the timed steps; its mask must equal theirs bit for bit
    single = None
    if nb <= 1024:
        cfg1 = dataclasses.replace(cfg, single_launch=True)
        ws1 = prism.new_workspace(qd, kd, cfg1)
        m1 = torch.empty_like(mask)
        ts = []
        for i in range(args.warmup + args.steps):
            flush()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record()
            prism.estimate(qd, kd, cfg1, workspace=ws1, mask_out=m1)
            ev[1].record()
            torch.cuda.synchronize()
            if i >= args.warmup:
                ts.append(ev[0].elapsed_time(ev[1]))
        single = {"estimator_ms": round(float(np.median(ts)), 3), "mask_identical": bool(torch.equal(m1, mask))}
        log(f"single-launch estimator: {single}")
        del ws1, m1

    # the sparse output as stored, kept on the host before the dense baselines overwrite `out`
    out_bits = (out.view(torch.int16).cpu().numpy().view(np.uint16) if w.dtype == "bf16"
                else out.cpu().numpy()) if not args.no_cpu_baseline else None
    mask_u8 = mask
    if args.mask_bits:  # unpack (outside the timed region) for the FLOP count and the CPU baseline
        shifts = torch.arange(32, device="cuda", dtype=torch.int32)
        mask_u8 = ((mask.unsqueeze(-1) >> shifts) & 1).to(torch.uint8).flatten(-2)[..., :nb].contiguous()
    flops, nsel = attention_flops(mask_u8, w.block, w.head_dim)
    total_blocks = w.batch * w.hq * nb * (nb + 1) // 2
    density = nsel / total_blocks
    achieved = flops / (attn_ms * 1e-3) / 1e12
    elem = 2 if w.dtype == "bf16" else 4
    est_bytes = (q.size + k.size) * elem + mask.numel() * mask.element_size()
    est_gbs = est_bytes / (est_ms * 1e-3) / 1e9

    result = {
        "metric": METRIC, "value": round(step_ms, 3), "unit": "ms", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_ms, 3), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": w.seq, "q_heads": w.hq, "kv_heads": w.hkv,
                   "head_dim": w.head_dim, "block": w.block, "d_high": w.d_high, "d_low": w.d_low, "p": w.p,
                   "rope_theta": w.theta, "causal": True, "parallelism": "none",
                   "mask_format": "bits" if args.mask_bits else "u8"},
        "estimator_ms": round(est_ms, 3), "attention_ms": round(attn_ms, 3),
        "estimator_ms_after_written_flush": round(est_written_flush_ms, 3),
        "estimator_single_launch": single,
        "wall_ms_per_step_incl_cache_flush": round(wall_ms, 3),
        "mask_density": round(density, 4),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic_from_profile(w.name),
                     "kernel": "attn_bf16_kernel", "flops_per_launch": flops},
        "estimator_roofline": {"bound": "hbm", "achieved": round(est_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                               "frac": round(est_gbs / PEAK_HBM_GBS, 4), "bytes_per_step": est_bytes},
    }

    if not args.no_dense:
        dense = {}
        ones = torch.tril(torch.ones((nb, nb), dtype=torch.uint8, device="cuda")).expand(w.batch, w.hq, nb, nb).contiguous()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        prism.block_sparse_attn(qd, kd, vd, ones, out=out)
        e[0].record()
        for _ in range(2):
            prism.block_sparse_attn(qd, kd, vd, ones, out=out)
        e[1].record()
        torch.cuda.synchronize()
        dense["own_kernel_all_blocks_ms"] = round(e[0].elapsed_time(e[1]) / 2, 3)
        try:
            from torch.nn.attention import SDPBackend, sdpa_kernel
            G = w.hq // w.hkv
            qt = qd.permute(0, 2, 1, 3).contiguous()
            kt = kd.permute(0, 2, 1, 3).repeat_interleave(G, dim=1).contiguous()
            vt = vd.permute(0, 2, 1, 3).repeat_interleave(G, dim=1).contiguous()
            with sdpa_kernel([SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION]):
                torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
                e[0].record()
                for _ in range(2):
                    torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
                e[1].record()
                torch.cuda.synchronize()
            dense["torch_sdpa_ms"] = round(e[0].elapsed_time(e[1]) / 2, 3)
            del qt, kt, vt
        except Exception as ex:  # no fused SDPA backend for this shape / arch
            dense["torch_sdpa_ms"] = None
            dense["torch_sdpa_error"] = str(ex)[:160]
        best = min(x for x in (dense.get("own_kernel_all_blocks_ms"), dense.get("torch_sdpa_ms")) if x)
        dense["faster"] = "own_kernel" if best == dense["own_kernel_all_blocks_ms"] else "torch_sdpa"
        result["dense_ms"] = dense
        result["speedup_vs_dense"] = round(best / step_ms, 3)
        log(f"dense: {dense}")

    if args.density_sweep:
        # context, not the metric: the same attention kernel on random causal block masks (each block
        # kept with probability d, the diagonal always), read-flushed like the timed steps, median of 3
        from synth import random_mask
        dense_own = result.get("dense_ms", {}).get("own_kernel_all_blocks_ms")
        sweep = []
        for si, d in enumerate(float(x) for x in args.density_sweep.split(",")):
            m = random_mask(w.batch, w.hq, nb, d, seed=2000 + si, causal=True)
            m[..., np.arange(nb), np.arange(nb)] = 1
            md = torch.from_numpy(m).cuda()
            del m
            f, ns = attention_flops(md, w.block, w.head_dim)
            ts = []
            for r in range(4):
                flush()
                e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                e[0].record()
                prism.block_sparse_attn(qd, kd, vd, md, out=out)
                e[1].record()
                torch.cuda.synchronize()
                if r:
                    ts.append(e[0].elapsed_time(e[1]))
            ms = float(np.median(ts))
            tf = f / (ms * 1e-3) / 1e12
            sweep.append({"density": round(ns / total_blocks, 4), "attention_ms": round(ms, 3),
                          "tflops": round(tf, 1), "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                          "speedup_vs_dense_own_kernel": round(dense_own / ms, 3) if dense_own else None})
            log(f"density sweep: {sweep[-1]}")
            del md
        result["density_sweep"] = sweep

    if not args.no_machine:
        result["machine"] = machine_microbench()
        log(f"machine: {result['machine']}")

    if not args.no_cpu_baseline:
        log("CPU oracle baseline (bounded sample)")
        result["cpu_baseline"], result["oracle_check"] = cpu_baseline(q, k, v, mask_u8.cpu().numpy(), out_bits, w)
        log(f"oracle check: {result['oracle_check']}")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
