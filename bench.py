#!/usr/bin/env python3
"""Throughput of the fused ragged paged attention call on one MI355X.

One step = one ra_forward call over one batch (KV-cache update + attention
for every request, with the plan, prefill and decode kernels it needs),
inputs resident in HBM.  Default workload: the Llama-3-8B-shaped
decode batch (128 requests x 1 new token, contexts U[1024, 8192], Hq=32,
Hkv=8, head_dim=128, page 16, bf16).  Prints ONE JSON line on stdout.

  python bench.py [--steps K] [--warmup W] [--config NAME] [--variant V]
                  [--extra-configs A,B,...|none]

Roofline: the dominant kernel's algorithmic bytes (HBM-bound decode) or
FLOPs (MFMA-bound prefill) per launch divided by its average launch time,
measured with hipEvents the library records on its own stream around each
stage.  The oracle (fp64 CPU) is timed on a bounded sample of the same
workload as the CPU baseline.

After the headline workload the same measurement runs for the other
workloads (causal and non-causal prefill, the mixed batch, and the
head_dim-256 decode and prefill batches), each under the line's "configs"
key with its own roofline and a shorter CPU baseline; a mixed batch also
reports max(B / 8 TB/s, F / bf16 peak) over its overlapped step time.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from ragged_paged_attention_amd import binding  # noqa: E402
from ragged_paged_attention_amd.inputs import Batch, CONFIGS, config  # noqa: E402

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2516.6  # 256 CU x 4096 FLOP/clk x 2.4 GHz, dense bf16
# Least untimed time per workload before its timed calls (after --warmup calls).
WARMUP_MIN_MS = 100.0

WORKLOADS = {
    "tiny": "tiny mixed batch: 2 decode (context 37, 100) + prefill 20 (context 0) + 33 (context 50), Hq=4 Hkv=2 D=64",
    "decode": "decode: 128 requests x 1 new token, context U[1024,8192], Hq=32 Hkv=8 D=128, page 16, bf16",
    "prefill": "prefill: 4 x 2048 new tokens, no context, causal, Hq=32 Hkv=8 D=128, page 16, bf16",
    "prefill_noncausal": "prefill: 4 x 2048 new tokens, no context, non-causal, Hq=32 Hkv=8 D=128, page 16, bf16",
    "mixed": "mixed: 96 decode (context U[512,8192]) + 8 x 512-token chunks (context U[0,4096]), shuffled, Hq=32 Hkv=8 D=128, page 16, bf16",
    "decode_d256": "decode: 128 requests x 1 new token, context U[1024,4096], Hq=16 Hkv=8 D=256, page 16, bf16",
    "prefill_d256": "prefill: 4 x 2048 new tokens, no context, causal, Hq=16 Hkv=8 D=256, page 16, bf16",
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# Algorithmic work (what the method must move / compute, nothing else)
# ---------------------------------------------------------------------------
def algorithmic_bytes(b: Batch, requests=None) -> int:
    """Prior KV read + new KV read and written + q read + out written + page ids + metadata."""
    cu = b.cu_q_lens.numpy().astype(np.int64)
    ctx = b.context_lens.numpy().astype(np.int64)
    rs = range(b.num_reqs) if requests is None else requests
    Hq, Hkv, D, S = b.num_q_heads, b.num_kv_heads, b.head_dim, b.page_size
    total = 0
    for r in rs:
        q = int(cu[r + 1] - cu[r])
        c = int(ctx[r])
        L = c + q
        total += c * Hkv * D * 2 * 2          # prior K and V
        total += q * Hkv * D * 2 * 2 * 2      # new K and V: read once, written once
        total += q * Hq * D * 2 * 2           # q read, out written
        total += 4 * ((L + S - 1) // S)       # page ids
        total += 4 * (2 + q)                  # cu_q_lens, context_lens, slot_mapping
    return total + 4


def algorithmic_flops(b: Batch, requests=None) -> int:
    """4*D FLOPs per visible (query, key) pair per q head (QK^T and PV)."""
    cu = b.cu_q_lens.numpy().astype(np.int64)
    ctx = b.context_lens.numpy().astype(np.int64)
    rs = range(b.num_reqs) if requests is None else requests
    pairs = 0
    for r in rs:
        q = int(cu[r + 1] - cu[r])
        c = int(ctx[r])
        if b.causal:
            pairs += q * c + q * (q + 1) // 2
        else:
            pairs += q * (c + q)
    return pairs * b.num_q_heads * 4 * b.head_dim


def decode_requests(b: Batch):
    ql = b.q_lens
    return [r for r in range(b.num_reqs) if ql[r] == 1]


def prefill_requests(b: Batch):
    ql = b.q_lens
    return [r for r in range(b.num_reqs) if ql[r] > 1]


# ---------------------------------------------------------------------------
# HBM traffic from rocprofv3 counters, valid only for the kernel source they
# were taken on.
# ---------------------------------------------------------------------------
def kernel_source_hash(stage: str) -> str:
    """Hash of the sources the stage's kernel is compiled from (its file and
    the device headers it includes)."""
    names = ({"decode": "decode.hip", "prefill": "prefill.hip"}[stage], "common.hpp", "plan.hpp")
    h = hashlib.sha256()
    for name in names:
        h.update(open(os.path.join(ROOT, "ragged_paged_attention_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(stage: str, workload: str):
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(f"{workload}/{stage}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256_16") != kernel_source_hash(stage):
        return None
    return rec.get("bytes_per_launch")


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the same workload
# ---------------------------------------------------------------------------
def counter_means(directory: str, counter: str):
    """Mean value of `counter` per dispatch, per kernel name, from the
    counter_collection.csv that `rocprofv3 --pmc` wrote under `directory`."""
    import csv
    import glob
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {directory}")
    acc = {}
    for f in files:
        for row in csv.DictReader(open(f)):
            if row["Counter_Name"] != counter:
                continue
            tot, n = acc.get(row["Kernel_Name"], (0.0, 0))
            acc[row["Kernel_Name"]] = (tot + float(row["Counter_Value"]), n + 1)
    return {k: (tot / n, n) for k, (tot, n) in acc.items()}


def ingest_counters(args):
    """HBM bytes per launch of the decode and prefill kernels from two
    FETCH_SIZE / WRITE_SIZE passes over a workload, each scaled by what the
    same counter reads for a device-to-device copy of known size."""
    fetch_dir, write_dir, cal_fetch_dir, cal_write_dir = args.ingest_counters
    copy_kib = args.copy_calibration_mib * 1024.0
    factors = {}
    for ctr, d in (("FETCH_SIZE", cal_fetch_dir), ("WRITE_SIZE", cal_write_dir)):
        means = counter_means(d, ctr)
        name, (val, n) = max(means.items(), key=lambda kv: kv[1][1])  # the copy: most dispatches
        factors[ctr] = copy_kib / val
        print(f"calibration {ctr}: {name} x{n}, {val:.0f} KiB per dispatch for a "
              f"{copy_kib:.0f} KiB copy -> factor {factors[ctr]:.4f}")
    fetch, write = counter_means(fetch_dir, "FETCH_SIZE"), counter_means(write_dir, "WRITE_SIZE")
    path = os.path.join(ROOT, "profiles", "traffic.json")
    db = json.load(open(path)) if os.path.exists(path) else {}
    for stage, knames in (("decode", ("decode_kernel",)), ("prefill", ("prefill_pp_kernel",))):
        keys = [k for k in fetch if k.split("<")[0].split("(")[0].strip() in knames]
        if not keys:
            continue
        k = keys[0]
        f_kib, n = fetch[k]
        w_kib = write.get(k, (0.0, 0))[0]
        total = (f_kib * factors["FETCH_SIZE"] + w_kib * factors["WRITE_SIZE"]) * 1024.0
        db[f"{args.config}/{stage}"] = {
            "kernel": k, "dispatches": n, "fetch_kib_raw": f_kib, "write_kib_raw": w_kib,
            "fetch_factor": factors["FETCH_SIZE"], "write_factor": factors["WRITE_SIZE"],
            "bytes_per_launch": total, "source_sha256_16": kernel_source_hash(stage)}
        print(f"{args.config}/{stage}: {k} x{n}: FETCH {f_kib:.0f} KiB, WRITE {w_kib:.0f} KiB raw "
              f"-> {total / 1e9:.4f} GB per launch")
    with open(path, "w") as fh:
        json.dump(db, fh, indent=1, sort_keys=True)
        fh.write("\n")


def copy_calibration(mib: int):
    """Device-to-device copies of `mib` MiB: the known-size kernel that the
    HBM counters are scaled by."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "copies": 5}))


def sub_batch(b: Batch, reqs) -> Batch:
    cu = b.cu_q_lens.tolist()
    toks = [t for r in reqs for t in range(cu[r], cu[r + 1])]
    qlens = [cu[r + 1] - cu[r] for r in reqs]
    ncu = torch.tensor([0] + list(np.cumsum(qlens)), dtype=torch.int32)
    idx = torch.tensor(toks, dtype=torch.int64)
    return Batch(q=b.q[idx], k_new=b.k_new[idx], v_new=b.v_new[idx], k_cache=b.k_cache,
                 v_cache=b.v_cache, page_table=b.page_table[list(reqs)], cu_q_lens=ncu,
                 context_lens=b.context_lens[list(reqs)], slot_mapping=b.slot_mapping[idx],
                 causal=b.causal, scale=b.scale)


def cpu_baseline(b: Batch, kind: str, budget_s: float):
    import oracle
    from ragged_paged_attention_amd.inputs import u16

    def run(reqs):
        sb = sub_batch(b, reqs)
        t = time.perf_counter()
        oracle.forward(u16(sb.q), u16(sb.k_new), u16(sb.v_new), u16(sb.k_cache), u16(sb.v_cache),
                       sb.page_table.numpy(), sb.cu_q_lens.numpy(), sb.context_lens.numpy(),
                       sb.slot_mapping.numpy(), scale=b.effective_scale(), causal=b.causal)
        return time.perf_counter() - t

    order = list(range(b.num_reqs))
    # Cost model from one- and two-request probes (a call has a fixed part,
    # the cache copy, and a per-request part); then the whole workload,
    # repeated to fill the budget, when one pass fits, else the first n.
    t1 = run(order[:1])
    t2 = run(order[:2]) if b.num_reqs > 1 else t1
    per_req = max(t2 - t1, 1e-4)
    fixed = max(t1 - per_req, 0.0)
    est_all = fixed + per_req * b.num_reqs
    if est_all <= budget_s:
        reqs, n = order, b.num_reqs
        reps = int(max(1, min(20, budget_s // max(est_all, 1e-3))))
        secs = sum(run(order) for _ in range(reps)) / reps
    else:
        n = int(max(1, min(len(order), (budget_s - fixed) / per_req)))
        reqs, reps = order[:n], 1
        secs = run(reqs)
    toks = sum(b.q_lens[r] for r in reqs)
    if kind == "hbm":
        value, unit = algorithmic_bytes(b, reqs) / secs / 1e9, "GB/s"
    else:
        value, unit = algorithmic_flops(b, reqs) / secs / 1e12, "TFLOP/s"
    cpu_model = next((ln.split(":", 1)[1].strip() for ln in open("/proc/cpuinfo")
                      if ln.startswith("model name")), "unknown")
    return {"value": value, "unit": unit, "cores": oracle.num_threads(), "kind": "oracle",
            "cpu_model": cpu_model, "nproc": os.cpu_count(),
            "sample": (f"{'all' if n == b.num_reqs else f'first {n} of'} {b.num_reqs} requests "
                       f"({toks} new tokens) x {reps} pass(es), {secs:.2f} s per pass, fp64, "
                       f"OpenMP over (token, q head), cache copy + scatter included"),
            "tokens_per_s": toks / secs, "seconds": secs}


def warm_up(call, stream, n: int, min_ms: float = 40.0) -> int:
    """n untimed calls, then more until at least min_ms have passed: the
    part's clock settles over tens of milliseconds of back-to-back work, which
    a fixed count of short calls (50 calls of a 20-60 us batch) does not
    cover, so a sweep point measured right after a change of batch read up to
    14 % slow.  Returns the number of untimed calls made."""
    t0 = time.perf_counter()
    done = 0
    for _ in range(n):
        call(stream)
    done += n
    torch.cuda.synchronize()
    while (time.perf_counter() - t0) * 1e3 < min_ms:
        for _ in range(10):
            call(stream)
        done += 10
        torch.cuda.synchronize()
    return done


def sweep_decode(args):
    """Decode bandwidth against context length: 128 requests x 1 new token,
    every request at the same context c; Llama-3-8B shapes (Hq=32, Hkv=8,
    head_dim 128) or, with --head-dim 256, Hq=16, Hkv=8, head_dim 256."""
    from ragged_paged_attention_amd.inputs import build_batch
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev).cuda_stream
    D = args.head_dim
    Hq = 32 if D == 128 else 16
    for c in (128, 256, 512, 1024, 2048, 4096, 8192):
        b = build_batch([1] * 128, [c] * 128, num_q_heads=Hq, num_kv_heads=8, head_dim=D,
                        seed=2000 + c, name=f"decode_c{c}")
        dt = [t.to(dev) for t in (b.q, b.k_new, b.v_new, b.k_cache, b.v_cache, b.page_table,
                                  b.cu_q_lens, b.context_lens, b.slot_mapping)]
        call = binding.Prepared(*dt, causal=True, scale=None, variant=args.variant,
                                cu_q_lens_host=b.cu_q_lens, context_lens_host=b.context_lens)
        warm_up(call, stream, args.warmup)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            call(stream)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / args.steps * 1e3
        timers = [binding.StageTimer() for _ in range(args.steps)]
        for t in timers:
            call(stream, t)
        torch.cuda.synchronize()
        dec_us = float(np.mean([t.stage_ms()["decode"] for t in timers])) * 1e3
        for t in timers:
            t.close()
        B = algorithmic_bytes(b)
        print(json.dumps({"sweep": "decode_context", "context": c, "requests": 128, "head_dim": D,
                          "step_us": us, "GB_per_s": B / us / 1e3, "frac_of_8TBs": B / us / 1e3 / HBM_PEAK_GBS,
                          "decode_kernel_us": dec_us, "kernel_GB_per_s": B / dec_us / 1e3,
                          "algorithmic_bytes": B, "tokens_per_s": 128 / (us * 1e-6)}), flush=True)
        del call, dt


def sweep_short_chunks(args):
    """Short prefill chunks (a few new tokens after a long context, as in
    speculative verification or chunked-prefill tails): K/V bandwidth with
    the chunks in the decode kernel (q G <= 32 query columns per kv head, in
    blocks of 16) and, with RA_SHORT_CHUNKS=0, in the prefill kernel."""
    from ragged_paged_attention_amd.inputs import build_batch
    cases = [  # (requests, new tokens, context, Hq, Hkv, D)
        (128, 4, 4096, 32, 8, 128), (128, 2, 4096, 32, 8, 128), (128, 16, 2048, 8, 8, 128),
        (128, 8, 2048, 32, 8, 128), (64, 16, 2048, 32, 8, 128), (64, 32, 2048, 16, 8, 128),
        (128, 8, 2048, 16, 8, 256)]
    for n, q, c, hq, hkv, d in cases:
        b = build_batch([q] * n, [c] * n, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                        seed=5000 + q + c, name="short")
        B = algorithmic_bytes(b)
        for routed in ("1", "0"):
            os.environ["RA_SHORT_CHUNKS"] = routed
            us, st = time_call(b, args)
            print(json.dumps({"sweep": "short_chunks", "requests": n, "new_tokens": q, "context": c,
                              "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": d,
                              "rows_per_kv_head": q * hq // hkv,
                              "kernel": "decode" if routed == "1" and q * hq // hkv <= 32 else "prefill",
                              "column_blocks": (q * hq // hkv + 15) // 16 if routed == "1" and q * hq // hkv <= 32 else 0,
                              "step_us": us, "GB_per_s": B / us / 1e3,
                              "frac_of_8TBs": B / us / 1e3 / HBM_PEAK_GBS,
                              "kernel_us": {k: v * 1e3 for k, v in st.items()}}), flush=True)
        os.environ.pop("RA_SHORT_CHUNKS", None)
        del b


def time_call(b: Batch, args):
    """Mean step time (us) of plain calls, and the per-stage event means."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev).cuda_stream
    dt = [t.to(dev) for t in (b.q, b.k_new, b.v_new, b.k_cache, b.v_cache, b.page_table,
                              b.cu_q_lens, b.context_lens, b.slot_mapping)]
    call = binding.Prepared(*dt, causal=b.causal, scale=None, variant=args.variant,
                            cu_q_lens_host=b.cu_q_lens, context_lens_host=b.context_lens)
    warm_up(call, stream, args.warmup)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        call(stream)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / args.steps * 1e3
    timers = [binding.StageTimer() for _ in range(args.steps)]
    for t in timers:
        call(stream, t)
    torch.cuda.synchronize()
    stages = {s: float(np.mean([t.stage_ms()[s] for t in timers])) * 1e3 for s in binding.STAGES}
    for t in timers:
        t.close()
    return us, stages


def sweep_prefill_length(args):
    """Prefill throughput against chunk length at a fixed 16384 new tokens per
    call: 16384 / L requests of L tokens, no context, causal and non-causal;
    Llama-3-8B shapes (Hq=32, Hkv=8, head_dim 128).  Short chunks pay the
    per-item start and end and the partial diagonal tiles; long ones converge
    to the key-tile loop's rate."""
    from ragged_paged_attention_amd.inputs import build_batch
    for causal in (True, False):
        for L in (128, 256, 512, 1024, 2048, 4096, 8192, 16384):
            n = 16384 // L
            b = build_batch([L] * n, [0] * n, num_q_heads=32, num_kv_heads=8, head_dim=128, causal=causal,
                            seed=6000 + L, name="prefill_len")
            us, st = time_call(b, args)
            F = algorithmic_flops(b)
            print(json.dumps({"sweep": "prefill_length", "causal": causal, "chunk_tokens": L, "requests": n,
                              "step_us": us, "TFLOP_per_s": F / us / 1e6,
                              "frac_of_peak": F / us / 1e6 / MFMA_BF16_PEAK_TFLOPS,
                              "prefill_kernel_us": st["prefill"],
                              "kernel_TFLOP_per_s": F / st["prefill"] / 1e6}), flush=True)
            del b


def sweep_shapes(args):
    """head_dim x page_size: a decode batch (128 requests x 1 token, context
    4096) and a causal prefill batch (4 x 2048 tokens), Hkv = 8, G = 4 at
    head_dim 64 / 128 and G = 2 at 256."""
    from ragged_paged_attention_amd.inputs import build_batch
    for D in (64, 128, 256):
        hq = 16 if D == 256 else 32
        for S in (16, 32, 64):
            dec = build_batch([1] * 128, [4096] * 128, num_q_heads=hq, num_kv_heads=8, head_dim=D,
                              page_size=S, seed=3000 + D + S, name="decode")
            us, st = time_call(dec, args)
            B = algorithmic_bytes(dec)
            print(json.dumps({"sweep": "shapes", "kind": "decode", "head_dim": D, "page_size": S,
                              "step_us": us, "GB_per_s": B / us / 1e3, "frac_of_8TBs": B / us / 1e3 / HBM_PEAK_GBS,
                              "decode_kernel_us": st["decode"]}), flush=True)
            del dec
            pre = build_batch([2048] * 4, [0] * 4, num_q_heads=hq, num_kv_heads=8, head_dim=D,
                              page_size=S, seed=4000 + D + S, name="prefill")
            us, st = time_call(pre, args)
            F = algorithmic_flops(pre)
            print(json.dumps({"sweep": "shapes", "kind": "prefill_causal", "head_dim": D, "page_size": S,
                              "step_us": us, "TFLOP_per_s": F / us / 1e6,
                              "frac_of_peak": F / us / 1e6 / MFMA_BF16_PEAK_TFLOPS,
                              "prefill_kernel_us": st["prefill"]}), flush=True)
            del pre


# ---------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # 400 untimed calls per workload: the part's clock settles over tens of
    # milliseconds of back-to-back work, after the process starts GPU work
    # (the head_dim-256 decode kernel from 425 to 549 us and back to ~440)
    # and again when the work changes from HBM-bound decode to MFMA-bound
    # prefill.  Fifty calls (8 ms of causal prefill) left the prefill lines
    # 3-8 % slow (168.4 against 155.0 us per step, same machine); 400 cost well
    # under a second in all.
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--config", default="decode", choices=[c for c in CONFIGS])
    ap.add_argument("--variant", default="auto", choices=list(binding.VARIANTS))
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU-baseline budget (0 disables the oracle leg)")
    ap.add_argument("--extra-configs", default="prefill,prefill_noncausal,mixed,decode_d256,prefill_d256",
                    help="workloads timed after the headline one, under the line's 'configs' key "
                         "(comma-separated; 'none' for the headline only)")
    ap.add_argument("--extra-cpu-seconds", type=float, default=4.0,
                    help="CPU-baseline budget of each extra workload")
    ap.add_argument("--sweep-decode", action="store_true",
                    help="instead of the contract line: one JSON line per decode context length "
                         "(128 requests x 1 token, context 128 .. 8192), HBM fraction against context")
    ap.add_argument("--head-dim", type=int, default=128, choices=[128, 256],
                    help="head_dim of --sweep-decode (128: Hq=32 Hkv=8; 256: Hq=16 Hkv=8)")
    ap.add_argument("--sweep-shapes", action="store_true",
                    help="instead of the contract line: one JSON line per head_dim x page_size "
                         "(64/128/256 x 16/32/64) for a decode batch and a causal prefill batch")
    ap.add_argument("--sweep-prefill-length", action="store_true",
                    help="prefill TFLOP/s against chunk length (16384 new tokens per call)")
    ap.add_argument("--sweep-short-chunks", action="store_true",
                    help="instead of the contract line: one JSON line per short-chunk batch (a few new "
                         "tokens after long contexts), decode-kernel routing against the prefill kernel")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run 5 device-to-device copies of this many MiB (counter calibration)")
    ap.add_argument("--ingest-counters", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR", "CAL_WRITE_DIR"),
                    help="CPU only: turn rocprofv3 FETCH_SIZE / WRITE_SIZE passes over --config (and over "
                         "--copy-calibration-mib) into profiles/traffic.json")
    args = ap.parse_args()
    if args.ingest_counters:
        ingest_counters(args)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)
        return

    if args.sweep_decode:
        sweep_decode(args)
        return
    if args.sweep_shapes:
        sweep_shapes(args)
        return
    if args.sweep_short_chunks:
        sweep_short_chunks(args)
        return
    if args.sweep_prefill_length:
        sweep_prefill_length(args)
        return

    extras = [] if args.extra_configs in ("", "none") else args.extra_configs.split(",")
    for name in extras:
        if name not in CONFIGS:
            raise SystemExit(f"unknown config {name!r} in --extra-configs")
    res = measure(args.config, args, cpu_budget=args.cpu_seconds, per_call=True)
    line = {
        "metric": res["metric"], "value": res["value"], "unit": res["unit"], "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
    }
    line.update({k: v for k, v in res.items() if k not in line and k not in ("metric", "value", "unit")})
    line["context"] = {"pages_decode_mbu_tpu7x": 0.86, "pages_prefill_mfu_tpu7x": 0.73,
                       "pages_prefill_mfu_causal_tpu7x": 0.63}
    if extras:
        line["configs"] = {}
        for name in extras:
            if name == args.config:
                continue
            r = measure(name, args, cpu_budget=args.extra_cpu_seconds, per_call=False)
            line["configs"][name] = r
    print(json.dumps(line), flush=True)


def measure(name: str, args, cpu_budget: float, per_call: bool) -> dict:
    """Times one workload: --steps plain calls between events (the step), the
    same number of calls with stage events (per-kernel times), and for the
    headline also single calls and an L2/MALL-flushed pass; then the dominant
    kernel's roofline and the oracle on a bounded sample."""
    log(f"[bench] building inputs for {name}")
    b = config(name)
    dev = torch.device("cuda:0")
    dt = [t.to(dev) for t in (b.q, b.k_new, b.v_new, b.k_cache, b.v_cache, b.page_table,
                              b.cu_q_lens, b.context_lens, b.slot_mapping)]
    call = binding.Prepared(*dt, causal=b.causal, scale=b.scale or None, variant=args.variant,
                            cu_q_lens_host=b.cu_q_lens, context_lens_host=b.context_lens)
    stream = torch.cuda.current_stream(dev).cuda_stream
    log(f"[bench] {name}: R={b.num_reqs} T={b.total_tokens} pages={b.num_pages} "
        f"workspace={call.workspace.numel()} B; warmup {args.warmup}")
    # --warmup untimed calls, then more until WARMUP_MIN_MS have passed on this
    # workload: the clock settles over tens of milliseconds whenever the work
    # changes between HBM-bound decode and MFMA-bound prefill, so a handful of
    # untimed calls left the prefill lines several per cent slow.
    warm_calls = warm_up(call, stream, args.warmup, WARMUP_MIN_MS)

    # Timed region: exactly K plain calls between events on the call's stream.
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        call(stream)
    stop.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(stop) / args.steps

    # Per-kernel durations: K more calls whose kernels each carry a start and
    # a stop hipEvent in their launch (recorded at the kernel's own start and
    # end); these calls are not the ones `value` is timed on (a mixed batch
    # runs its kernels one after the other in them, so each is timed alone).
    timers = [binding.StageTimer() for _ in range(args.steps)]
    for k in range(args.steps):
        call(stream, timers[k])
    torch.cuda.synchronize()
    stages = {s: float(np.mean([t.stage_ms()[s] for t in timers])) for s in binding.STAGES}
    for t in timers:
        t.close()
    log(f"[bench] {name}: {ms_per_step * 1e3:.1f} us/step; kernels (us): "
        + ", ".join(f"{k}={v * 1e3:.1f}" for k, v in stages.items()))

    # Distribution of single calls (an event pair around each call), and for
    # a decode-dominated batch the same with a 512 MiB write between calls,
    # which evicts L2 and the MALL (the cache bytes then all come from HBM).
    def per_call_us(n, between=None):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for e0, e1 in evs:
            if between is not None:
                between()
            e0.record()
            call(stream)
            e1.record()
        torch.cuda.synchronize()
        return np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in evs])

    def pctl(x):
        return {"p10": float(np.percentile(x, 10)), "p50": float(np.median(x)),
                "p90": float(np.percentile(x, 90))}

    single = per_call_us(args.steps)
    flushed = None
    if per_call and stages["decode"] >= stages["prefill"]:
        junk = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        fl = per_call_us(args.steps, between=junk.zero_)
        del junk
        flushed = {"us": pctl(fl), "GB_per_s_p50": algorithmic_bytes(b) / (np.median(fl) * 1e-6) / 1e9,
                   "note": "512 MiB written between calls (L2 and MALL evicted)"}

    B = algorithmic_bytes(b)
    F = algorithmic_flops(b)
    T = b.total_tokens
    dec, pre = decode_requests(b), prefill_requests(b)
    step_s = ms_per_step / 1e3
    if args.variant == "generic":
        dominant = "prefill"  # the generic kernel runs in the prefill slot
        bound = "hbm" if not pre else "mfma"
    else:
        dominant = "decode" if stages["decode"] >= stages["prefill"] else "prefill"
        bound = "hbm" if dominant == "decode" else "mfma"
    kern_s = stages[dominant] / 1e3
    if bound == "hbm":
        units = algorithmic_bytes(b, dec if args.variant != "generic" else None)
        achieved = units / kern_s / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS,
                "traffic": measured_traffic("decode", name) if dominant == "decode" else None,
                "kernel": "decode_kernel" if args.variant != "generic" else "generic_kernel",
                "algorithmic_bytes_per_launch": units, "kernel_us": kern_s * 1e6,
                "note": "decode bytes over the decode kernel alone; its merge kernel is timed "
                        "separately (kernel_us_merge)",
                "kernel_us_merge": stages["merge"] * 1e3}
    else:
        units = algorithmic_flops(b, pre)
        achieved = units / kern_s / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                "traffic": measured_traffic("prefill", name),
                "kernel": "generic_kernel" if args.variant == "generic" else "prefill_pp_kernel",
                "algorithmic_flops_per_launch": units, "kernel_us": kern_s * 1e6}

    if pre and not dec:
        metric, unit, value = "prefill TFLOP/s (% bf16 MFMA peak)", "TFLOP/s", F / step_s / 1e12
        frac_step = value / MFMA_BF16_PEAK_TFLOPS
    else:
        metric, unit, value = "decode HBM GB/s (% of 8 TB/s)", "GB/s", B / step_s / 1e9
        frac_step = value / HBM_PEAK_GBS
    res = {"metric": metric, "value": value, "unit": unit, "ms_per_step": ms_per_step,
           "config": {"workload": WORKLOADS[name], "name": name, "requests": b.num_reqs,
                      "total_tokens": T, "context_tokens": int(b.context_lens.sum()),
                      "num_q_heads": b.num_q_heads, "num_kv_heads": b.num_kv_heads,
                      "head_dim": b.head_dim, "page_size": b.page_size, "causal": b.causal,
                      "variant": args.variant},
           "tokens_per_s": T / step_s, "frac_of_peak_whole_step": frac_step,
           "untimed_calls": warm_calls,
           "algorithmic_bytes": B, "algorithmic_flops": F,
           "kernel_us": {k: v * 1e3 for k, v in stages.items()},
           "step_us_single_calls": pctl(single)}
    if dec and pre:
        # Both rooflines on the whole (overlapped) call: the time the call
        # would take at 8 TB/s for its bytes or at the bf16 peak for its
        # FLOPs, whichever is longer, over the measured step.
        t_min = max(B / (HBM_PEAK_GBS * 1e9), F / (MFMA_BF16_PEAK_TFLOPS * 1e12))
        res["mixed_roofline"] = {
            "formula": "max(B / 8 TB/s, F / 2516.6 TFLOP/s) / t_step", "B": B, "F": F,
            "t_us": ms_per_step * 1e3, "t_roofline_us": t_min * 1e6, "frac": t_min / step_s,
            "frac_single_call_p50": t_min / (np.median(single) * 1e-6)}
    if per_call:
        res["flushed"] = flushed
    res["roofline"] = roof
    cpu = None
    if cpu_budget > 0:
        log(f"[bench] {name}: CPU baseline: oracle on a sample (~{cpu_budget:.0f} s)")
        cpu = cpu_baseline(b, "hbm" if unit == "GB/s" else "mfma", cpu_budget)
    res["cpu_baseline"] = cpu
    del call, dt
    torch.cuda.synchronize()
    return res


if __name__ == "__main__":
    main()
