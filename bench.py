"""Paged decode attention on one MI355X: effective KV GB/s and seq-steps/s.

One step = one decode step of the whole batch through one layer:
  host   libpa block manager reserves each sequence's next slot (a new block
         when the position starts one) and exports tables / lengths into a
         pinned staging buffer;
  H2D    slots, lengths and block tables (one async copy each);
  GPU    pa_reshape_and_cache (new K/V rows into their slots),
         pa_decode_partition (one workgroup per sequence x KV head x 512-token
         partition), pa_decode_reduce (log-sum-exp merge of partitions).
The host work of step s+1 overlaps the GPU work of step s (double-buffered
staging). Inputs (pools, q, new k/v) are resident in HBM before timing.

Metric: effective KV GB/s = sum over steps of (sum_i L_i * 2 * Hkv * D * 2 B)
divided by the timed wall time; L_i counts the tokens each decode attends to.
The roofline line uses the partition kernel's own time from HIP events.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention: effective KV GB/s (% of HBM peak) + seq-steps/s"
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_llama3_8b.json")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def storage_np(t):
    """Host numpy copy in storage form (float32, or uint16 bf16 bits)."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("pa_kernels.hip", "pa_api.cpp", "pa_internal.h"):
        with open(os.path.join(ROOT, "paged_kv_cache_343_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(variant_name: str):
    """HBM bytes per partition-kernel launch measured with rocprofv3 counters
    for the current kernel source, or None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as fh:
        rec = json.load(fh)
    if rec.get("source_hash") != kernel_source_hash() or rec.get("variant") != variant_name:
        return None
    return rec.get("bytes_per_launch")


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama3_8b")
    ap.add_argument("--variant", default="auto", choices=["auto", "valu", "mfma"])
    ap.add_argument("--partition-tokens", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "the path shards by sequence or KV head with no exchange, see the design notes.",
              file=sys.stderr)
        return 2

    import torch
    import paged_kv_cache_343_amd as P
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    P.lib()  # fail loudly if libpa.so is missing
    dev = torch.device("cuda", 0)
    w = W.get(args.workload)
    if "prefix" in w.lengths[0]:
        print("bench.py times the plain decode workloads", file=sys.stderr)
        return 1
    variant = {"auto": P.PA_VARIANT_AUTO, "valu": P.PA_VARIANT_VALU, "mfma": P.PA_VARIANT_MFMA}[args.variant]
    B, hq, hkv, d, bs = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    ptok = args.partition_tokens if args.partition_tokens is not None else w.partition_tokens
    nsteps = args.warmup + args.steps
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    eb = 2 if w.dtype == "bf16" else 4

    # ---- inputs (seeded, synthetic) ------------------------------------
    rng = np.random.default_rng(w.seed)
    ctx = W.draw_lengths(w, rng)                       # tokens cached before the first step
    final = ctx + nsteps
    occupied = int(sum(-(-int(L) // bs) for L in ctx + 1))
    nb = max(W.pool_blocks(w, occupied), int(sum(-(-int(L) // bs) for L in final)))
    order = W.free_order(nb, rng)
    maxb = int(-(-int(final.max()) // bs))
    max_len = int(final.max())
    k_pool = W.normal_device((nb, hkv, bs, d), w.seed * 1000 + 1, w.dtype, dev)
    v_pool = W.normal_device((nb, hkv, bs, d), w.seed * 1000 + 2, w.dtype, dev)
    q_all = W.normal_device((nsteps, B, hq, d), w.seed * 1000 + 3, w.dtype, dev)
    kn_all = W.normal_device((nsteps, B, hkv, d), w.seed * 1000 + 4, w.dtype, dev)
    vn_all = W.normal_device((nsteps, B, hkv, d), w.seed * 1000 + 5, w.dtype, dev)
    out = torch.empty((B, hq, d), dtype=tdt, device=dev)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    kp_host = vp_host = None
    if not args.no_cpu_baseline:
        kp_host, vp_host = storage_np(k_pool), storage_np(v_pool)
    log(f"inputs ready: {B} sequences, {nb} blocks, {k_pool.numel() * eb * 2 / 1e9:.2f} GB of KV pool")

    bm = P.BlockManager(nb, bs, order)
    for i, L in enumerate(ctx):
        bm.add_seq(i, int(L))
    seq_ids = np.arange(B, dtype=np.int32)
    # double-buffered pinned staging and device copies
    stage = [dict(slots=torch.empty(B, dtype=torch.int64, pin_memory=True),
                  pairs=torch.empty(2 * B, dtype=torch.int64, pin_memory=True),
                  tables=torch.empty((B, maxb), dtype=torch.int32, pin_memory=True),
                  lens=torch.empty(B, dtype=torch.int32, pin_memory=True)) for _ in range(2)]
    devbuf = [dict(slots=torch.empty(B, dtype=torch.int64, device=dev),
                   tables=torch.empty((B, maxb), dtype=torch.int32, device=dev),
                   lens=torch.empty(B, dtype=torch.int32, device=dev)) for _ in range(2)]
    copied = [None, None]
    shape = P.DecodeShape(B, hq, hkv, d, bs, nb, maxb, max_len, ptok,
                          P.PA_BF16 if w.dtype == "bf16" else P.PA_F32, variant)
    ws = torch.empty(max(P.pa_decode_workspace_bytes(shape), 16), dtype=torch.uint8, device=dev)
    step_bytes = []
    ev = []  # per step: (reshape start, partition start, partition end, reduce end)

    def host_step(s: int, b: int):
        if copied[b] is not None:
            copied[b].synchronize()          # the staging buffer's last copy has landed
        st = stage[b]
        ncow = bm.append_slots_into(seq_ids, st["slots"].numpy(), st["pairs"].numpy())
        if ncow:
            raise RuntimeError("no copy-on-write expected in this workload")
        bm.export(seq_ids, maxb, st["tables"].numpy(), st["lens"].numpy())
        step_bytes.append(int(st["lens"].numpy().astype(np.int64).sum()) * 2 * hkv * d * eb)

    def gpu_step(s: int, b: int, timed: bool):
        st, db = stage[b], devbuf[b]
        for k in ("slots", "tables", "lens"):
            db[k].copy_(st[k], non_blocking=True)
        e = torch.cuda.Event()
        e.record()
        copied[b] = e
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if timed else None
        if timed:
            evs[0].record()
        P.pa_reshape_and_cache(kn_all[s], vn_all[s], db["slots"], k_pool, v_pool)
        if timed:
            evs[1].record()
        P.pa_decode_partition(q_all[s], k_pool, v_pool, db["tables"], db["lens"], scale, out,
                              max_seq_len=max_len, partition_tokens=ptok, variant=variant,
                              workspace=ws)
        if timed:
            evs[2].record()
        P.pa_decode_reduce(q_all[s], k_pool, db["tables"], db["lens"], out, max_seq_len=max_len,
                           partition_tokens=ptok, variant=variant, workspace=ws)
        if timed:
            evs[3].record()
            ev.append(evs)

    for s in range(args.warmup):
        host_step(s, s % 2)
        gpu_step(s, s % 2, False)
    torch.cuda.synchronize()
    log("warmup done")
    if P.pa_device_errors() != 0:
        raise RuntimeError("device index error during warmup")
    step_bytes.clear()
    t0 = time.perf_counter()
    for s in range(args.warmup, nsteps):
        host_step(s, s % 2)
        gpu_step(s, s % 2, True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if P.pa_device_errors() != 0:
        raise RuntimeError("device index error during the timed steps")

    log(f"timed {args.steps} steps in {t1 - t0:.3f} s")
    wall = t1 - t0
    K = args.steps
    total_bytes = sum(step_bytes)
    gbs = total_bytes / wall / 1e9
    part_ms = [a.elapsed_time(b) for _, a, b, _ in ev]
    red_ms = [a.elapsed_time(b) for _, _, a, b in ev]
    cache_ms = [a.elapsed_time(b) for a, b, _, _ in ev]
    part_avg_s = float(np.mean(part_ms)) / 1e3
    bytes_per_launch = total_bytes / K
    achieved = bytes_per_launch / part_avg_s / 1e9
    vname = {0: "auto", 1: "valu", 2: "mfma"}[variant]
    if variant == P.PA_VARIANT_AUTO:
        vname = "mfma" if (w.dtype == "bf16" and d == 128 and hq // hkv in (1, 2, 4)) else "valu"
    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": B, "num_q_heads": hq, "num_kv_heads": hkv,
                   "head_dim": d, "block_size": bs, "partition_tokens": ptok,
                   "context_tokens": f"U{{{w.lengths[1]}..{w.lengths[2]}}}+step",
                   "kernel": vname, "parallelism": "single GPU"},
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "seq_steps_per_s": round(B * K / wall, 1),
        "kernels_us": {"partition": round(1e3 * float(np.mean(part_ms)), 2),
                       "reduce": round(1e3 * float(np.mean(red_ms)), 2),
                       "reshape_and_cache": round(1e3 * float(np.mean(cache_ms)), 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(vname),
                     "kernel": "decode_partition_" + vname,
                     "algorithmic_bytes_per_launch": int(bytes_per_launch)},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline(w, kp_host, vp_host, storage_np(q_all[nsteps - 1]),
                                              ctx, order, nb, nsteps, scale, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


def cpu_baseline(w, kp_host, vp_host, q_host, ctx, order, nb, nsteps, scale, seconds, n_seq=32):
    """The float64 C oracle on the host cores, on a bounded sample: the first
    `n_seq` sequences of the workload at their last timed step (block tables
    from the oracle's own allocator mirror, replayed through every step),
    repeated for about `seconds` of wall time."""
    from oracle import pa_oracle as O
    from oracle import ref as R

    bs = w.block_size
    obm = O.OracleBlockManager(nb, bs, order)
    seqs = list(range(len(ctx)))
    for i, L in enumerate(ctx):
        obm.add_seq(i, int(L))
    for _ in range(nsteps):
        obm.append_slots(seqs)
    sample = seqs[:n_seq]
    maxb = max(len(obm.table(i)) for i in sample)
    tables, lens = obm.export(sample, maxb)
    threads = min(16, len(os.sched_getaffinity(0)))
    R.decode(q_host[:n_seq], kp_host, vp_host, tables, lens, scale, w.dtype, num_threads=threads)
    reps, t0 = 0, time.perf_counter()
    while True:
        R.decode(q_host[:n_seq], kp_host, vp_host, tables, lens, scale, w.dtype, num_threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 1000:
            break
    kv_bytes = int(lens.astype(np.int64).sum()) * 2 * w.num_kv_heads * w.head_dim * w.elem_bytes
    return {"value": round(n_seq * reps / el, 2), "unit": "seq-steps/s", "cores": threads,
            "kind": "oracle",
            "kv_gb_per_s": round(kv_bytes * reps / el / 1e9, 3),
            "sample": (f"first {n_seq} of {len(ctx)} {w.name} sequences at the last timed step "
                       f"(sum of lengths {int(lens.sum())}), plain C float64 oracle, "
                       f"{reps} repetitions in {el:.1f} s")}


if __name__ == "__main__":
    sys.exit(main())
