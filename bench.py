"""Paged decode attention on one MI355X: effective KV GB/s and seq-steps/s.

One step = one decode step of the whole batch through one layer:
  host   libpa block manager reserves each sequence's next slot (a new block
         when the position starts one) and exports tables / lengths into a
         pinned staging buffer;
  H2D    slots, lengths and block tables, packed, in one async copy on a
         side stream (ordered before the step's kernels by an event);
  GPU    pa_reshape_and_cache (new K/V rows into their slots),
         pa_decode_partition (one workgroup per sequence x KV head x 512-token
         partition), pa_decode_reduce (log-sum-exp merge of partitions).
The host work and the H2D copy of step s+1 overlap the GPU work of step s
(double-buffered staging). Inputs (pools, q, new k/v) are resident in HBM before timing.

Metric: effective KV GB/s = sum over steps of (sum_i L_i * 2 * Hkv * D * 2 B)
divided by the timed wall time; L_i counts the tokens each decode attends to.
The roofline line uses the partition kernel's own time from HIP events.
"""
from __future__ import annotations

import argparse
import ctypes
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
_KEEP_ALIVE = []   # device allocations made outside torch, held until the process ends
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


def recorded_traffic(variant_name: str, workload: str = "llama3_8b"):
    """The traffic record (HBM bytes per partition-kernel launch measured
    with rocprofv3 counters, and the algorithmic K/V bytes of the same
    launches) for the current kernel source and this workload in the bench's
    default launch configuration, or None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as fh:
        rec = json.load(fh)
    if (rec.get("source_hash") != kernel_source_hash() or rec.get("variant") != variant_name
            or rec.get("workload") != workload):
        return None
    return rec


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama3_8b")
    ap.add_argument("--variant", default="auto", choices=["auto", "valu", "mfma"])
    ap.add_argument("--partition-tokens", type=int, default=None)
    ap.add_argument("--block-size", type=int, default=None,
                    help="override the workload's block size (tokens per block)")
    ap.add_argument("--kv-dtype", default="native", choices=["native", "e4m3"],
                    help="KV pool storage: the workload's dtype, or FP8 E4M3 codes with one "
                         "scale per pool (q and out stay bf16)")
    ap.add_argument("--block-order", default="shuffled", choices=["shuffled", "identity"],
                    help="free-list order: a seeded permutation (scattered blocks, the "
                         "default) or 0, 1, 2, ... (each sequence's blocks contiguous)")
    ap.add_argument("--upload-tables", action="store_true",
                    help="upload whole block tables and lengths every step instead of keeping "
                         "them on the device (pa_append_tokens)")
    ap.add_argument("--gpu-wait-upload", action="store_true",
                    help="order each step's kernels after its upload with a stream wait "
                         "instead of on the host")
    ap.add_argument("--prefix-decode", default="auto", choices=["auto", "pa_decode", "shared"],
                    help="shared-prefix workloads: decode with pa_decode over a work plan, or "
                         "with pa_decode_shared_prefix (each shared prompt block read once per "
                         "group, the walks after the prompts over a work plan); auto = the "
                         "latter")
    ap.add_argument("--half-partials", action="store_true",
                    help="store partial outputs in bf16 (PA_DECODE_HALF_PARTIALS; an option "
                         "with a looser error bound, off by default)")
    ap.add_argument("--workspace-memory", default="default",
                    choices=["default", "finegrained", "uncached"],
                    help="device memory kind of the decode workspace (partials): a torch "
                         "tensor, or hipExtMallocWithFlags fine-grained or uncached memory "
                         "(never freed: the process ends after the run)")
    ap.add_argument("--no-plan", action="store_true",
                    help="launch pa_decode's full grid instead of a host work plan")
    ap.add_argument("--event-every", type=int, default=5,
                    help="record the partition kernel's timing events on every n-th timed step")
    ap.add_argument("--done-every", type=int, default=2,
                    help="record the step-completion event (buffer reuse) every n-th step (n <= 4)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the timed steps, run pa_copy_blocks over this many MiB per "
                         "pool (read and written) so that rocprofv3 counters of the decode "
                         "kernel can be scaled by those of a copy of known size")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) of "
                         "this script with --copy-calibration-mib into a traffic record")
    ap.add_argument("--traffic-out", default=None)
    ap.add_argument("--configs", default="auto", choices=["auto", "on", "off"],
                    help="after the headline workload, run the other workloads (single_fp32, "
                         "small_mha, llama2_13b, shared_prefix, shared_prefix_long) through the "
                         "same step loop and report them under 'configs'; auto = on for the "
                         "default headline launch")
    ap.add_argument("--config-steps", type=int, default=50,
                    help="timed steps per workload under 'configs' (5 warm-up steps each)")
    ap.add_argument("--side-rows", default="on", choices=["on", "off"],
                    help="measure the rows outside the step (block copies, fork, multi-token "
                         "queries, group 8, swapping, the read probe) after the timed steps")
    ap.add_argument("--scrub", action="store_true",
                    help="also time the step's decode alone with 512 MiB written between "
                         "iterations (outside the timed region), and without")
    args = ap.parse_args()
    if args.configs == "auto":
        args.configs = ("on" if (args.workload == "llama3_8b" and args.variant == "auto" and
                                 args.partition_tokens is None and args.block_size is None and
                                 args.kv_dtype == "native" and args.block_order == "shuffled" and
                                 not args.upload_tables and not args.no_plan and
                                 not args.half_partials and args.copy_calibration_mib == 0)
                        else "off")
    args.configs = args.configs == "on"
    if args.traffic_from:
        return summarise_traffic(args)
    if args.event_every < 1 or not 1 <= args.done_every <= 4 or args.steps < 1 or args.warmup < 0:
        print("need --event-every >= 1, 1 <= --done-every <= 4, --steps >= 1, --warmup >= 0",
              file=sys.stderr)
        return 2
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
    result = run_workload(args, torch, P, W, dev, side_rows=args.side_rows == "on")
    if args.configs:
        result["configs"] = other_configs(args, torch, P, W, dev, result)
    result["run"] = run_metadata(torch, W.get(args.workload), result)
    print(json.dumps(result), flush=True)
    return 0


def run_workload(args, torch, P, W, dev, side_rows=True) -> dict:
    """Build one workload, run its warm-up and timed steps and return the
    result record (the JSON line's fields for this workload). side_rows adds
    the measurements of the rows outside the step (block copies, fork,
    multi-token queries, group 8, swapping, the read-bandwidth probe, the CPU
    baseline)."""
    w = W.get(args.workload)
    prefix = w.lengths[0] == "prefix_suffix"
    variant = {"auto": P.PA_VARIANT_AUTO, "valu": P.PA_VARIANT_VALU, "mfma": P.PA_VARIANT_MFMA}[args.variant]
    B, hq, hkv, d, bs = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    if args.block_size:
        bs = args.block_size
    fp8 = args.kv_dtype == "e4m3"
    # 8-bit pools: partitions of the same bytes as the workload's bf16 ones
    # (twice the positions; the library's automatic choice)
    ptok = (args.partition_tokens if args.partition_tokens is not None
            else (2 * w.partition_tokens if fp8 else w.partition_tokens))
    nsteps = args.warmup + args.steps
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    eb = 2 if w.dtype == "bf16" else 4
    if fp8 and (w.dtype != "bf16" or d != 128):
        print("8-bit pools need a bf16 workload with head dim 128", file=sys.stderr)
        return 1
    pool_eb = 1 if fp8 else eb          # bytes per stored K/V element
    k_scale = v_scale = 0.05            # 8-bit pools: scale per pool

    # ---- inputs (seeded, synthetic) ------------------------------------
    rng = np.random.default_rng(w.seed)
    if prefix:
        # prompt groups: one parent holds the shared prompt, the other samples
        # fork it, then every sample appends its private suffix (the first
        # write into a shared partial block copies it) before timing starts
        suffix = W.draw_lengths(w, rng)
        ngroups, nsamp = w.extra["groups"], w.extra["samples"]
        plen = w.lengths[1]
        n_long = w.extra.get("long_seqs", 0)
        ctx = np.concatenate([plen + suffix[:ngroups * nsamp],
                              np.full(n_long, w.extra.get("long_len", 0))]).astype(np.int64)
        args.no_cpu_baseline = True      # the CPU baseline leg times the headline workload
        unique_prompt = ngroups * -(-plen // bs)
        occupied = unique_prompt + int(sum(-(-int(L) // bs) - plen // bs for L in ctx[:ngroups * nsamp] + 1))
        occupied += int(sum(-(-int(L) // bs) for L in ctx[ngroups * nsamp:] + 1))
    else:
        ctx = W.draw_lengths(w, rng)                   # tokens cached before the first step
        occupied = int(sum(-(-int(L) // bs) for L in ctx + 1))
    final = ctx + nsteps
    nb = max(W.pool_blocks(w, occupied), occupied + B * (-(-nsteps // bs) + 1))
    order = W.free_order(nb, rng)
    if args.block_order == "identity":
        order = np.arange(nb, dtype=np.int32)
    maxb = int(-(-int(final.max()) // bs))
    max_len = int(final.max())
    if fp8:
        k_pool = W.random_e4m3_codes_device((nb, hkv, bs, d), w.seed * 1000 + 1, dev)
        v_pool = W.random_e4m3_codes_device((nb, hkv, bs, d), w.seed * 1000 + 2, dev)
        args.no_cpu_baseline = True      # the CPU baseline leg times the native pools
    else:
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
    cow_setup = 0
    if prefix:
        for gi in range(ngroups):
            bm.add_seq(gi * nsamp, plen)
            for k in range(1, nsamp):
                bm.fork(gi * nsamp, gi * nsamp + k)
        for k in range(n_long):
            bm.add_seq(ngroups * nsamp + k, int(ctx[ngroups * nsamp + k]))
        kz = torch.zeros((B, hkv, d), dtype=tdt, device=dev)
        for step in range(int(suffix[:ngroups * nsamp].max())):
            batch = np.array([sq for sq in range(ngroups * nsamp) if suffix[sq] > step], dtype=np.int32)
            slots, pairs = bm.append_slots(batch)
            if pairs.shape[0]:
                cow_setup += pairs.shape[0]
                P.pa_copy_blocks(k_pool, v_pool, torch.from_numpy(pairs).to(dev))
            sl = torch.from_numpy(slots).to(dev)
            n = len(batch)
            if fp8:
                P.pa_reshape_and_cache_e4m3(kz[:n], kz[:n], sl, k_pool, v_pool, k_scale, v_scale)
            else:
                P.pa_reshape_and_cache(kz[:n], kz[:n], sl, k_pool, v_pool)
        torch.cuda.synchronize()
        log(f"shared prompts forked, suffixes written ({cow_setup} copy-on-write blocks)")
    else:
        for i, L in enumerate(ctx):
            bm.add_seq(i, int(L))
    seq_ids = np.arange(B, dtype=np.int32)
    # Per step the host produces slots (int64 [B]) and the work plan; they
    # travel in one packed pinned buffer and one H2D copy on a side stream.
    # Block tables and lengths stay on the device: pa_append_tokens applies
    # each step's append to them (the host block manager still decides every
    # slot and block; the device copies are checked against it at the end).
    # With --upload-tables the host exports tables (int32 [B, maxb]) and
    # lengths (int32 [B]) into the same buffer every step instead. NBUF
    # staging/device buffer pairs let the host run up to NBUF - 1 steps
    # ahead, so host jitter never leaves the GPU waiting, and the copy of
    # step s+1 overlaps the kernels of step s.
    NBUF = 4
    upload = args.upload_tables
    tab0, len0 = bm.export(list(range(B)), maxb)
    lens_host = len0.astype(np.int32).copy()        # the host's lengths, kept by the loop
    tables_dev = torch.from_numpy(tab0).to(dev)
    lens_dev = torch.from_numpy(len0).to(dev)
    # forked samples share their prompt blocks: say so to the library
    shape = P.DecodeShape(B, hq, hkv, d, bs, nb, maxb, max_len, ptok,
                          P.PA_BF16 if w.dtype == "bf16" else P.PA_F32,
                          variant | (P.PA_DECODE_SHARED_KV if prefix else 0) |
                          (P.PA_DECODE_HALF_PARTIALS if args.half_partials else 0))
    # Work plan (pa_decode_plan): the host lists the step's (sequence,
    # partition) units from the lengths it just exported, into the same
    # staging buffer; the partition kernel's grid then holds only those.
    plan_cap = 0
    if not args.no_plan and (ptok != 0 or not fp8):
        try:
            P.pa_decode_plan(shape, np.minimum(ctx + 1, max_len).astype(np.int32))
            plan_cap = P.pa_decode_plan_capacity(shape)
        except P.PaError:
            plan_cap = 0                 # a shape on the per-tile kernel: full grid
    # layout: slots | plan (16-byte aligned) | lengths | tables
    n_slots, n_lens, n_tab = 8 * B, 4 * B, 4 * B * maxb
    plan_off = -(-n_slots // 16) * 16
    lens_off = plan_off + 16 * plan_cap
    tab_off = lens_off + n_lens
    pack_bytes = tab_off + n_tab

    def views(buf):
        return dict(slots=buf[:n_slots].view(torch.int64),
                    plan=buf[plan_off:lens_off].view(torch.int32),
                    lens=buf[lens_off:tab_off].view(torch.int32),
                    tables=buf[tab_off:pack_bytes].view(torch.int32).view(B, maxb))

    stage_raw = [torch.empty(pack_bytes, dtype=torch.uint8, pin_memory=True) for _ in range(NBUF)]
    dev_raw = [torch.empty(pack_bytes, dtype=torch.uint8, device=dev) for _ in range(NBUF)]
    stage = [views(x) for x in stage_raw]
    devbuf = [views(x) for x in dev_raw]
    pairs_host = np.empty(2 * B, dtype=np.int64)
    # Two non-default streams (default priority): on ROCm an H2D copy issued
    # on the null stream, or ordered after null-stream work, blocks the host
    # until the GPU drains, which would serialise host and GPU work.
    compute = torch.cuda.Stream(dev)
    copier = torch.cuda.Stream(dev)
    torch.cuda.synchronize(dev)      # inputs drawn on the null stream are ready
    copied = [None] * NBUF    # H2D copy of staging buffer b done
    done_step = [-1] * NBUF   # step whose completion event sits in done_ev[step % NBUF]
    n_units = [0] * NBUF      # work-plan units in staging / device buffer b
    ws = torch.empty(max(P.pa_decode_workspace_bytes(shape), 16), dtype=torch.uint8, device=dev)
    # Shared-prefix decode in the step (shared-prefix workloads): the prompt
    # groups and each sample's shared positions (the whole prompt blocks; a
    # half-filled prompt block was copied on write at setup) stay fixed.
    sp_mode = prefix and not fp8 and args.prefix_decode in ("shared", "auto")
    walk_start_ptr = None           # host prefix lengths: the plan's walk starts
    if sp_mode:
        shared = (plen // bs) * bs
        sp_gs = torch.arange(0, ngroups * nsamp + 1, nsamp, dtype=torch.int32, device=dev)
        sp_prefix_host = np.zeros(B, dtype=np.int32)
        sp_prefix_host[:ngroups * nsamp] = shared
        sp_prefix = torch.from_numpy(sp_prefix_host).to(dev)
        walk_start_ptr = sp_prefix_host.ctypes.data
        sp_ws = torch.empty(max(16, P.pa_decode_shared_prefix_workspace_bytes(shape, nsamp, shared)),
                            dtype=torch.uint8, device=dev)
        sp_args = (ngroups, sp_gs.data_ptr(), sp_prefix.data_ptr(), nsamp, shared)
        sp_ws_args = (sp_ws.data_ptr(), sp_ws.numel())
        sp_ptrs = (sp_gs, sp_prefix, sp_ws)  # kept alive for the raw calls
    step_bytes = []
    host_s = [0.0]  # host time per timed step, waits excluded
    step_lens = []  # shared-prefix workloads: lengths per step, for the unique bytes
    bm_s = [0.0]    # block manager (append + export) time
    plan_s = [0.0]  # work plan time
    nunits_c = ctypes.c_int32(0)
    shape_ref = ctypes.byref(shape)
    ev = []  # per step: (reshape start, partition start, partition end, reduce end)

    # Host side of a step through the raw C ABI (block manager: append one
    # token per sequence, then export tables and lengths straight into the
    # pinned staging buffer), pointers resolved once.
    Lh = P.lib()
    ids_ptr = seq_ids.ctypes.data
    pairs_ptr = pairs_host.ctypes.data
    ncow = ctypes.c_int32(0)
    stage_ptr = [{k: v.data_ptr() for k, v in st.items()} for st in stage]
    lens_np = [st["lens"].numpy() for st in stage]

    def host_step(s: int, b: int):
        if copied[b] is not None:
            w0 = time.perf_counter()
            copied[b].synchronize()          # the staging buffer's last copy has landed
            host_s[0] -= time.perf_counter() - w0
        sp = stage_ptr[b]
        t_bm = time.perf_counter()
        st = Lh.pa_bm_append_slots(bm._h, ids_ptr, B, sp["slots"], pairs_ptr, ctypes.byref(ncow))
        if st != 0:
            raise P.PaError(st, "pa_bm_append_slots")
        if ncow.value:
            raise RuntimeError("no copy-on-write expected in this workload")
        if upload:
            st = Lh.pa_bm_export(bm._h, ids_ptr, B, maxb, sp["tables"], sp["lens"])
            if st != 0:
                raise P.PaError(st, "pa_bm_export")
        bm_s[0] += time.perf_counter() - t_bm
        lens_host[:] += 1                    # every sequence appended one token
        if not upload:
            lens_np[b][:] = lens_host
        if plan_cap:
            # (pa_decode_shared_prefix: the walks after each prefix)
            t_pl = time.perf_counter()
            st = Lh.pa_decode_plan(shape_ref, sp["lens"], walk_start_ptr, sp["plan"], plan_cap,
                                   ctypes.byref(nunits_c))
            if st != 0:
                raise P.PaError(st, "pa_decode_plan")
            n_units[b] = nunits_c.value
            plan_s[0] += time.perf_counter() - t_pl
        step_bytes.append(int(lens_np[b].sum(dtype=np.int64)) * 2 * hkv * d * pool_eb)
        if prefix:
            step_lens.append(lens_np[b].copy())

    # Raw C-ABI calls with pointers resolved once: the step's host cost stays
    # far below its GPU time, so the GPU never waits for the host.
    L = P.lib()
    c_scale = ctypes.c_float(scale)
    c_kscale, c_vscale = ctypes.c_float(k_scale), ctypes.c_float(v_scale)
    ws_ptr, ws_bytes = ws.data_ptr(), ws.numel()
    if args.workspace_memory != "default":
        # the partials in fine-grained or uncached device memory; uncached
        # memory is kept to the end of the process once a kernel has used it
        hipx = ctypes.CDLL("libamdhip64.so")
        hipx.hipExtMallocWithFlags.restype = ctypes.c_int
        hipx.hipExtMallocWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t,
                                               ctypes.c_uint]
        wsp = ctypes.c_void_p()
        flag = {"finegrained": 0x1, "uncached": 0x3}[args.workspace_memory]
        if hipx.hipExtMallocWithFlags(ctypes.byref(wsp), ws_bytes, flag) != 0 or not wsp.value:
            raise RuntimeError("hipExtMallocWithFlags failed")
        ws_ptr = wsp.value
        _KEEP_ALIVE.append(wsp)
    kp_ptr, vp_ptr, out_ptr = k_pool.data_ptr(), v_pool.data_ptr(), out.data_ptr()
    dt_code = P.PA_BF16 if w.dtype == "bf16" else P.PA_F32
    cs = compute.cuda_stream
    dptr = [{k: v.data_ptr() for k, v in db.items()} for db in devbuf]
    def check(st, what):
        if st != 0:
            raise P.PaError(st, what)

    copy_ev = [torch.cuda.Event() for _ in range(NBUF)]
    done_ev = [torch.cuda.Event() for _ in range(NBUF)]
    # Timed steps carry two events each, around the partition kernel (its
    # duration feeds the roofline); every event recorded between kernels
    # costs the step ~5 us, so the slot write and the merge are timed in a
    # separate loop afterwards.
    time_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]

    # The upload is one hipMemcpyAsync on the side stream, called directly
    # (torch's stream-switching context costs tens of microseconds per use).
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpyAsync.restype = ctypes.c_int
    hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                   ctypes.c_void_p]
    HIP_H2D = 1
    copier_handle = copier.cuda_stream
    stage_base = [x.data_ptr() for x in stage_raw]
    dev_base = [x.data_ptr() for x in dev_raw]

    tab_dev_ptr, len_dev_ptr = tables_dev.data_ptr(), lens_dev.data_ptr()

    def gpu_step(s: int, b: int, timed: bool):
        db = dict(dptr[b])
        if not upload:
            db["tables"], db["lens"] = tab_dev_ptr, len_dev_ptr
        # step s-NBUF must no longer read device buffer b: wait (on the host; a
        # GPU-side wait would make the runtime run the copy synchronously) on
        # the first completion event recorded at or after that step, normally
        # long since complete
        for t in range(max(0, s - NBUF), s):
            if done_step[t % NBUF] == t:
                done_ev[t % NBUF].synchronize()
                break
        nbytes = pack_bytes if upload else plan_off + 16 * n_units[b]
        if hip.hipMemcpyAsync(dev_base[b], stage_base[b], nbytes, HIP_H2D, copier_handle):
            raise RuntimeError("hipMemcpyAsync failed")
        copied[b] = copy_ev[b]
        copied[b].record(copier)
        if args.gpu_wait_upload:
            compute.wait_event(copied[b])
        else:
            # ordered on the host: the kernels that read buffer b are enqueued
            # once its copy has landed (the host is steps ahead of the GPU, so
            # this costs it ~10-20 us of slack and spares the compute stream a
            # cross-stream wait, ~7 us per step)
            w0 = time.perf_counter()
            copied[b].synchronize()
            host_s[0] -= time.perf_counter() - w0
        evs = time_ev[s - args.warmup] if timed else None
        if not upload and fp8:
            check(L.pa_append_tokens_e4m3(kn_all[s].data_ptr(), vn_all[s].data_ptr(), db["slots"],
                                          kp_ptr, vp_ptr, db["tables"], db["lens"], B, maxb, hkv,
                                          d, bs, nb, c_kscale, c_vscale, cs),
                  "pa_append_tokens_e4m3")
        elif not upload:
            check(L.pa_append_tokens(kn_all[s].data_ptr(), vn_all[s].data_ptr(), db["slots"],
                                     kp_ptr, vp_ptr, db["tables"], db["lens"], B, maxb, hkv, d,
                                     bs, nb, dt_code, cs), "pa_append_tokens")
        elif fp8:
            check(L.pa_reshape_and_cache_e4m3(kn_all[s].data_ptr(), vn_all[s].data_ptr(),
                                              db["slots"], kp_ptr, vp_ptr, B, hkv, d, bs, nb,
                                              c_kscale, c_vscale, cs), "pa_reshape_and_cache_e4m3")
        else:
            check(L.pa_reshape_and_cache(kn_all[s].data_ptr(), vn_all[s].data_ptr(), db["slots"],
                                         kp_ptr, vp_ptr, B, hkv, d, bs, nb, dt_code, cs),
                  "pa_reshape_and_cache")
        if timed:
            evs[0].record(compute)
        plan_ptr, plan_n = (db["plan"], n_units[b]) if plan_cap else (None, 0)
        if sp_mode:
            # prefix pass and per-sequence walks in one launch, then the merge
            check(L.pa_decode_shared_prefix(q_all[s].data_ptr(), kp_ptr, vp_ptr, db["tables"],
                                            db["lens"], c_scale, out_ptr, shape_ref, *sp_args,
                                            plan_ptr, plan_n, *sp_ws_args, cs),
                  "pa_decode_shared_prefix")
        elif fp8:
            check(L.pa_decode_partition_e4m3(q_all[s].data_ptr(), kp_ptr, vp_ptr, db["tables"],
                                             db["lens"], c_scale, c_kscale, c_vscale, out_ptr,
                                             shape_ref, plan_ptr, plan_n, ws_ptr, ws_bytes, cs),
                  "pa_decode_partition_e4m3")
        else:
            check(L.pa_decode_partition(q_all[s].data_ptr(), kp_ptr, vp_ptr, db["tables"],
                                        db["lens"], c_scale, out_ptr, shape_ref, plan_ptr,
                                        plan_n, ws_ptr, ws_bytes, cs), "pa_decode_partition")
        if timed:
            evs[1].record(compute)
            ev.append(evs)
        if not sp_mode:
            check(L.pa_decode_reduce(db["lens"], out_ptr, shape_ref, ws_ptr, ws_bytes, cs),
                  "pa_decode_reduce")
        if s % args.done_every == 0 or s == nsteps - 1:
            done_ev[s % NBUF].record(compute)
            done_step[s % NBUF] = s

    for s in range(args.warmup):
        host_step(s, s % NBUF)
        gpu_step(s, s % NBUF, False)
    torch.cuda.synchronize()
    log("warmup done")
    if P.pa_device_errors() != 0:
        raise RuntimeError("device index error during warmup")
    step_bytes.clear()
    step_lens.clear()
    bm_s[0] = 0.0
    plan_s[0] = 0.0
    t0 = time.perf_counter()
    for s in range(args.warmup, nsteps):
        h0 = time.perf_counter()
        host_step(s, s % NBUF)
        gpu_step(s, s % NBUF, (s - args.warmup) % args.event_every == 0)
        host_s[0] += time.perf_counter() - h0
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if P.pa_device_errors() != 0:
        raise RuntimeError("device index error during the timed steps")
    b_last = (nsteps - 1) % NBUF
    if not upload:
        # the device tables and lengths must be the host block manager's
        st_last = stage[b_last]
        bm.export(list(range(B)), maxb, st_last["tables"].numpy(), st_last["lens"].numpy())
        if not (np.array_equal(tables_dev.cpu().numpy(), st_last["tables"].numpy()) and
                np.array_equal(lens_dev.cpu().numpy(), st_last["lens"].numpy())):
            raise RuntimeError("device block tables / lengths differ from the host block manager")
        devbuf[b_last]["tables"].copy_(tables_dev)
        devbuf[b_last]["lens"].copy_(lens_dev)
        torch.cuda.synchronize()
        log("device tables and lengths match the host block manager")

    log(f"timed {args.steps} steps in {t1 - t0:.3f} s; host enqueue {1e6 * host_s[0] / args.steps:.0f} us/step")
    wall = t1 - t0
    K = args.steps
    total_bytes = sum(step_bytes)
    gbs = total_bytes / wall / 1e9
    part_ms = [a.elapsed_time(b) for a, b in ev]
    # the slot write and the merge, timed separately on the last step's inputs
    # (the slot write rewrites the same slots with the same rows; the table and
    # length upkeep of pa_append_tokens is left out there, since repeating it
    # would advance the lengths): 5 batches of 20 back-to-back launches, one
    # event pair per batch, so that the events' own cost (a few µs per pair)
    # does not land on kernels of a few µs
    db = dptr[b_last]

    def slot_write():
        if fp8:
            check(L.pa_reshape_and_cache_e4m3(kn_all[nsteps - 1].data_ptr(), vn_all[nsteps - 1].data_ptr(),
                                              db["slots"], kp_ptr, vp_ptr, B, hkv, d, bs, nb,
                                              c_kscale, c_vscale, cs), "pa_reshape_and_cache_e4m3")
        else:
            check(L.pa_reshape_and_cache(kn_all[nsteps - 1].data_ptr(), vn_all[nsteps - 1].data_ptr(),
                                         db["slots"], kp_ptr, vp_ptr, B, hkv, d, bs, nb, dt_code, cs),
                  "pa_reshape_and_cache")

    def merge():
        check(L.pa_decode_reduce(db["lens"], out_ptr, shape_ref, ws_ptr, ws_bytes, cs),
              "pa_decode_reduce")

    def per_launch_ms(fn, batches=5, n=20):
        out = []
        for _ in range(batches):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(compute)
            for _ in range(n):
                fn()
            e1.record(compute)
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) / n)
        return out

    cache_ms = per_launch_ms(slot_write)
    # (the shared-prefix call merges itself)
    red_ms = [0.0] if sp_mode else per_launch_ms(merge)
    scrub_us = None
    if args.scrub:
        # the last step's decode again on its own inputs, timed alone: after
        # 512 MiB were written (L2 and the 256 MB MALL then hold other
        # lines, so K/V come from HBM), and back to back without that
        tabs_p = db["tables"] if upload else tab_dev_ptr
        lens_p = db["lens"] if upload else len_dev_ptr
        qp = q_all[nsteps - 1].data_ptr()

        def decode_last():
            plan_ptr, plan_n = (db["plan"], n_units[b_last]) if plan_cap else (None, 0)
            if sp_mode:
                check(L.pa_decode_shared_prefix(qp, kp_ptr, vp_ptr, tabs_p, lens_p, c_scale,
                                                out_ptr, shape_ref, *sp_args, plan_ptr, plan_n,
                                                *sp_ws_args, cs), "pa_decode_shared_prefix")
                return
            if fp8:
                check(L.pa_decode_partition_e4m3(qp, kp_ptr, vp_ptr, tabs_p, lens_p, c_scale,
                                                 c_kscale, c_vscale, out_ptr, shape_ref,
                                                 plan_ptr, plan_n, ws_ptr, ws_bytes, cs),
                      "partition")
            else:
                check(L.pa_decode_partition(qp, kp_ptr, vp_ptr, tabs_p, lens_p, c_scale, out_ptr,
                                            shape_ref, plan_ptr, plan_n, ws_ptr, ws_bytes, cs),
                      "partition")
            check(L.pa_decode_reduce(lens_p, out_ptr, shape_ref, ws_ptr, ws_bytes, cs),
                  "pa_decode_reduce")

        junk = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        scrub_us = {}
        for mode in ("unscrubbed", "scrubbed"):
            ts = []
            for k in range(22):
                if mode == "scrubbed":
                    junk.fill_(k + 1)
                torch.cuda.synchronize()
                e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                e[0].record(compute)
                decode_last()
                e[1].record(compute)
                torch.cuda.synchronize()
                ts.append(e[0].elapsed_time(e[1]))
            scrub_us[mode] = 1e3 * float(np.median(ts[2:]))
        del junk
        if P.pa_device_errors() != 0:
            raise RuntimeError("device index error in the scrub measurement")
    period_ms = [ev[k][0].elapsed_time(ev[k + 1][0]) / args.event_every
                 for k in range(len(ev) - 1)]
    log(f"GPU step period {1e3 * np.mean(period_ms):.1f} us")
    part_avg_s = float(np.mean(part_ms)) / 1e3
    bytes_per_launch = total_bytes / K
    achieved = bytes_per_launch / part_avg_s / 1e9
    # the counters were taken in the default launch configuration only
    default_launch = (not fp8 and args.block_size is None and args.block_order == "shuffled"
                      and args.partition_tokens is None and not args.no_plan
                      and not args.upload_tables and args.variant == "auto"
                      and not args.half_partials and args.workspace_memory == "default")
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
        "dtype": w.dtype if not fp8 else "bf16 q/out, e4m3 K/V",
        "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": B, "num_q_heads": hq, "num_kv_heads": hkv,
                   "head_dim": d, "block_size": bs,
                   "partition_tokens": ptok if ptok else "automatic (library)",
                   "context_tokens": (f"U{{{w.lengths[1]}..{w.lengths[2]}}}+step"
                                      if w.lengths[0] == "uniform" else f"{w.lengths}+step"),
                   "kernel": vname, "block_order": args.block_order,
                   "work_plan": bool(plan_cap) and not sp_mode,
                   "decode_call": "pa_decode_shared_prefix" if sp_mode else "pa_decode",
                   "device_tables": not upload,
                   "kv_storage": "e4m3" if fp8 else w.dtype,
                   "partial_outputs": "bf16" if args.half_partials else "fp32",
                   "workspace_memory": args.workspace_memory,
                   "parallelism": "single GPU"},
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "seq_steps_per_s": round(B * K / wall, 1),
        "kernels_us": {"partition": round(1e3 * float(np.mean(part_ms)), 2),
                       "reduce": None if sp_mode else round(1e3 * float(np.mean(red_ms)), 2),
                       "reshape_and_cache": round(1e3 * float(np.mean(cache_ms)), 2),
                       # spread of the sampled partition launches and step periods
                       "partition_p10_p50_p90": [round(1e3 * float(x), 2) for x in
                                                 np.percentile(part_ms, [10, 50, 90])],
                       "step_period_p10_p50_p90": ([round(1e3 * float(x), 2) for x in
                                                    np.percentile(period_ms, [10, 50, 90])]
                                                   if period_ms else None),
                       "partition_samples": len(part_ms)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None,
                     "kernel": ("shared_prefix_decode + decode_reduce (one call)" if sp_mode else
                                "decode_partition_" + vname + ("_e4m3" if fp8 else "")),
                     "algorithmic_bytes_per_launch": int(bytes_per_launch)},
    }
    avg_len = total_bytes / K / (2 * hkv * d * pool_eb) / B
    result["sum_L_per_step"] = round(avg_len * B, 1)
    rec = recorded_traffic(vname, w.name) if default_launch else None
    if rec is not None:
        # the counters' run had its own step mix (its steps and warm-up): its
        # traffic is set against its own algorithmic bytes
        rf = result["roofline"]
        rf["traffic"] = rec["bytes_per_launch"]
        if rec.get("algorithmic_bytes_per_launch"):
            rf["traffic_run_algorithmic_bytes"] = rec["algorithmic_bytes_per_launch"]
            rf["traffic_over_algorithmic"] = round(
                rec["bytes_per_launch"] / rec["algorithmic_bytes_per_launch"], 4)
    parts = float(np.mean([-(-int(x) // ptok) for x in stage[0]["lens"].numpy()])) if ptok > 0 else 1.0
    pe = 2 if (args.half_partials and eb == 2) else 4      # bytes per partial-output element
    red_bytes = B * hq * (parts * d * pe + d * eb) + B * hkv * parts * 128 if parts > 1 else 0
    cache_bytes = B * 2 * hkv * d * (eb + pool_eb)
    result["rows"] = {
        "a1_block_manager_host_us": round(1e6 * bm_s[0] / K, 1),
        "work_plan_host_us": round(1e6 * plan_s[0] / K, 1),
        "a2_reshape_and_cache": {"us": round(1e3 * float(np.mean(cache_ms)), 2),
                                 "timed": SMALL_KERNEL_TIMING,
                                 "bytes_moved": cache_bytes,
                                 "GBps": round(cache_bytes / (float(np.mean(cache_ms)) / 1e3) / 1e9, 1)},
        "a3_decode_partition": {"us": round(1e3 * float(np.mean(part_ms)), 2),
                                "GBps": round(achieved, 1), "mean_len": round(avg_len, 1)},
        "a4_decode_reduce": ({"us": None, "note": "merged inside the pa_decode_shared_prefix call "
                                                  "(its time is in kernels_us.partition)"}
                             if sp_mode else
                             {"us": round(1e3 * float(np.mean(red_ms)), 2), "timed": SMALL_KERNEL_TIMING,
                              "bytes_moved": int(red_bytes),
                              "GBps": round(red_bytes / (float(np.mean(red_ms)) / 1e3) / 1e9, 1)}),
    }
    if side_rows:
        result["rows"].update({
            "a5_copy_blocks": copy_blocks_rate(P, torch, dev),
            "a6_fork_cow_host_us": fork_cow_host_us(P),
            "n2_multi_query": multi_query_rate(P, torch, dev, W),
            "decode_group8": group8_decode_rate(P, torch, dev, W),
            "n3_swap_blocks": swap_rate(P, torch, dev),
            "mfma_valu_overlap": mfma_valu_overlap(torch, dev),
        })
        peak = stream_read_peak(torch, dev)
        result["practical_peak"] = dict(peak, partition_frac=round(achieved / peak["GBps"], 4),
                                        partition_frac_of_random_4k=round(
                                            achieved / peak["random_4k_GBps"], 4))
    if prefix:
        # bytes of distinct cached rows read per step: a shared prompt block is
        # read once per step however many sequences point at it
        tab_last = stage[(nsteps - 1) % NBUF]["tables"].numpy()
        uniq = []
        for lens_s in step_lens:
            rows = np.zeros(nb, dtype=np.int64)
            nblk = -(-lens_s.astype(np.int64) // bs)
            for i in range(B):
                k = np.arange(nblk[i])
                np.maximum.at(rows, tab_last[i, :nblk[i]], np.minimum(bs, lens_s[i] - k * bs))
            uniq.append(int(rows.sum()) * 2 * hkv * d * pool_eb)
        ub = float(np.mean(uniq))
        cascade = None if fp8 else shared_prefix_rate(P, torch, dev, w, q_all[nsteps - 1], k_pool, v_pool,
                                     devbuf[(nsteps - 1) % NBUF], plen, bs, max_len, scale,
                                     uniq[-1], int(step_lens[-1].sum()) * 2 * hkv * d * pool_eb)
        result["shared_prefix"] = {
            "pa_decode_shared_prefix": cascade,
            "logical_bytes_per_step": int(total_bytes / K), "unique_bytes_per_step": int(ub),
            "unique_GBps": round(ub / (wall / K) / 1e9, 1),
            "pct_of_hbm_peak_unique": round(100.0 * ub / (wall / K) / 1e9 / HBM_PEAK_GBS, 2),
            "partition_unique_GBps": round(ub / part_avg_s / 1e9, 1),
            "copy_on_write_blocks_at_setup": cow_setup}
        # A shared prompt block is fetched from HBM once per step however many
        # sequences read it, so the roofline of the partition kernel counts the
        # distinct K/V rows (unique bytes); the logical rate stays beside it.
        rf = result["roofline"]
        uach = ub / part_avg_s / 1e9
        rf.update({"achieved": round(uach, 1), "frac": round(uach / HBM_PEAK_GBS, 4),
                   "algorithmic_bytes_per_launch": int(ub), "bytes": "unique K/V rows",
                   "logical_achieved": round(achieved, 1)})
        if "practical_peak" in result:
            result["practical_peak"]["partition_frac"] = round(
                uach / result["practical_peak"]["GBps"], 4)
    if scrub_us is not None:
        nbytes = int(uniq[-1]) if prefix else int(step_bytes[-1])
        result["scrub"] = {
            "decode_us_unscrubbed": round(scrub_us["unscrubbed"], 2),
            "decode_us_scrubbed": round(scrub_us["scrubbed"], 2),
            "bytes": nbytes, "bytes_kind": "unique K/V rows" if prefix else "K/V rows",
            "GBps_unscrubbed": round(nbytes / scrub_us["unscrubbed"] / 1e3, 1),
            "GBps_scrubbed": round(nbytes / scrub_us["scrubbed"] / 1e3, 1),
            "frac_scrubbed": round(nbytes / scrub_us["scrubbed"] / 1e3 / HBM_PEAK_GBS, 4),
            "what": "the last step's decode (partition + merge) timed alone, median of 20, "
                    "with 512 MiB written between iterations outside the timed region, and "
                    "back to back without"}
    if args.copy_calibration_mib > 0:
        result["copy_calibration"] = copy_calibration(P, torch, dev, args.copy_calibration_mib,
                                                      hkv * bs * d * eb)
    if side_rows and not args.no_cpu_baseline:
        log("timing the CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline(w, kp_host, vp_host, storage_np(q_all[nsteps - 1]),
                                              ctx, order, nb, nsteps, scale, args.cpu_seconds)
    return result


SMALL_KERNEL_TIMING = ("per launch: 5 batches of 20 back-to-back launches on the last step's "
                       "inputs, one HIP event pair per batch, mean")

# The workloads reported under 'configs' beside the headline, with their tags.
OTHER_CONFIGS = (("single_fp32", "C1"), ("small_mha", "C2"), ("llama2_13b", "C3"),
                 ("shared_prefix", "C5"), ("shared_prefix_long", "C5-long"))
# cache-resident working sets (below the 256 MB MALL, or near it): also timed
# with the caches scrubbed
SCRUBBED_CONFIGS = ("small_mha", "shared_prefix")


def other_configs(args, torch, P, W, dev, head: dict) -> dict:
    """Every other workload through the same step loop (fewer steps), one
    summary row each."""
    out = {}
    for name, tag in OTHER_CONFIGS:
        sub = argparse.Namespace(**vars(args))
        sub.workload, sub.steps, sub.warmup = name, args.config_steps, 5
        sub.no_cpu_baseline, sub.copy_calibration_mib = True, 0
        sub.scrub = name in SCRUBBED_CONFIGS
        log(f"config {tag}: {name}")
        r = run_workload(sub, torch, P, W, dev, side_rows=False)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        rf = r["roofline"]
        row = {"config": tag, "workload": name, "dtype": r["dtype"], "steps": sub.steps,
               "decode_call": r["config"]["decode_call"], "ms_per_step": r["ms_per_step"],
               "step_GBps": r["value"], "seq_steps_per_s": r["seq_steps_per_s"],
               "partition_us": r["kernels_us"]["partition"], "reduce_us": r["kernels_us"]["reduce"],
               "kernel_GBps": rf["achieved"], "frac": rf["frac"],
               "bytes": rf.get("bytes", "K/V rows"), "sum_L_per_step": r["sum_L_per_step"]}
        if "shared_prefix" in r:
            sp = r["shared_prefix"]
            row["logical_kernel_GBps"] = rf.get("logical_achieved")
            row["shared_prefix"] = {k: sp[k] for k in (
                "logical_bytes_per_step", "unique_bytes_per_step", "unique_GBps",
                "pct_of_hbm_peak_unique", "partition_unique_GBps")}
        if "scrub" in r:
            row["scrub"] = r["scrub"]
        if "practical_peak" in head:
            row["practical_frac"] = round(rf["achieved"] / head["practical_peak"]["GBps"], 4)
        out[name] = row
    return out


def run_metadata(torch, w, result: dict) -> dict:
    """Versions, device and host facts, and the draw seed of the run."""
    props = torch.cuda.get_device_properties(0)
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as fh:
            rocm = fh.read().strip()
    except OSError:
        pass
    with open(os.path.abspath(__file__), "rb") as fh:
        bench_sha = hashlib.sha256(fh.read()).hexdigest()[:16]
    return {"gpu": props.name, "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "hbm_bytes": int(props.total_memory),
            "rocm": rocm, "hip_runtime": torch.version.hip, "torch": torch.__version__,
            "host_cpu": cpu_model(), "host_affinity_cpus": len(os.sched_getaffinity(0)),
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "workload_seed": w.seed, "sum_L_per_step": result.get("sum_L_per_step"),
            "kernel_source_hash": kernel_source_hash(), "bench_sha16": bench_sha}


PROBE_PATTERNS = {0: ("stride", (1, 2, 4, 8)), 1: ("wavetile", (1, 2, 4, 8)),
                  2: ("random4k", (4, 8))}


def stream_read_peak(torch, dev) -> dict:
    """Practical HBM read ceiling: the read probe (libpa_probe.so) over a
    4 GiB buffer, best over a sweep of launch shapes (workgroups of 256
    threads from 4 to 64 per CU; 1 to 8 independent 16-byte loads in flight
    per lane; plain and streaming cache policy) and access patterns
    (grid-stride, consecutive tiles per wave, random 4 KiB tiles of two
    pools), 10 timed launches each. The best random-tile rate, the pattern of
    paged decode's gather, is reported beside the overall best."""
    path = os.path.join(ROOT, "paged_kv_cache_343_amd", "libpa_probe.so")
    lib = ctypes.CDLL(path)
    lib.pa_probe_stream_read.restype = ctypes.c_int
    lib.pa_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_void_p, ctypes.c_void_p]
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    s = torch.cuda.current_stream(dev).cuda_stream
    sweep = {}
    for pattern, (pname, loads_set) in PROBE_PATTERNS.items():
        for grid in (1024, 2048, 4096, 8192, 16384):
            for loads in loads_set:
                for nt in (0, 1):
                    args = (buf.data_ptr(), nbytes, grid, loads, nt, pattern, sink.data_ptr(), s)
                    for _ in range(2):
                        if lib.pa_probe_stream_read(*args):
                            raise RuntimeError("probe launch failed")
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record()
                    for _ in range(10):
                        lib.pa_probe_stream_read(*args)
                    e1.record()
                    torch.cuda.synchronize()
                    # (4 GiB splits into two halves of 2^19 4-KiB tiles, all read)
                    sweep[f"{pname}_wg{grid}_loads{loads}_{'nt' if nt else 'plain'}"] = round(
                        nbytes / (e0.elapsed_time(e1) / 10 / 1e3) / 1e9, 1)
    del buf
    best = max(sweep, key=sweep.get)
    rnd = max((k for k in sweep if k.startswith("random4k")), key=sweep.get)
    return {"GBps": sweep[best], "bytes": nbytes, "kernel": "pa_probe_stream_read",
            "best_launch": best, "random_4k_GBps": sweep[rnd], "random_4k_best_launch": rnd,
            "sweep_GBps": sweep}


OVERLAP_MODES = {0: "mfma_only", 1: "fma_only", 2: "both_in_every_wave",
                 3: "mfma_waves_beside_fma_waves", 4: "mfma_one_chain", 5: "exp2_only"}


def mfma_valu_overlap(torch, dev) -> dict:
    """How far matrix-core and vector work overlap on one SIMD: the overlap
    probe of libpa_probe.so (16 independent v_mfma_f32_16x16x32_bf16 and/or
    64 fp32 FMAs per iteration, by mode), 1024 workgroups of 8 waves x 2000
    iterations (8 waves per SIMD), 5 timed launches per mode. Reported per
    mode: milliseconds, and SIMD cycles at 2.4 GHz per iteration of the
    waves that run it. The two ratios compare running both kinds of work
    against running them one after the other (1.0: no overlap, 0.5: full
    overlap of equal halves)."""
    lib = ctypes.CDLL(os.path.join(ROOT, "paged_kv_cache_343_amd", "libpa_probe.so"))
    lib.pa_probe_mfma_valu.restype = ctypes.c_int
    lib.pa_probe_mfma_valu.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_void_p]
    grid, iters = 1024, 2000
    out = torch.empty(grid * 512, dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream(dev).cuda_stream
    wave_iters = grid * 8 * iters / 1024            # per SIMD (1024 SIMDs)
    res = {}
    for mode, name in OVERLAP_MODES.items():
        args = (mode, grid, iters, out.data_ptr(), s)
        if lib.pa_probe_mfma_valu(*args):
            raise RuntimeError("overlap probe launch failed")
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            lib.pa_probe_mfma_valu(*args)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 5
        waves = wave_iters / 2 if mode == 3 else wave_iters
        res[name] = {"ms": round(ms, 3),
                     "simd_cycles_per_iteration": round(ms * 1e-3 * 2.4e9 / waves, 1)}
    m, f = res["mfma_only"]["ms"], res["fma_only"]["ms"]
    res["both_in_every_wave_vs_serial"] = round(res["both_in_every_wave"]["ms"] / (m + f), 3)
    # mode 3 does half of each kind of work
    res["beside_vs_serial"] = round(res["mfma_waves_beside_fma_waves"]["ms"] / ((m + f) / 2), 3)
    del out
    return res


def copy_blocks_rate(P, torch, dev) -> dict:
    """pa_copy_blocks on the shared-prefix workload's copy-on-write set (64
    prompt groups x 3 diverging samples = 192 blocks of 32 tokens, 8 KV
    heads, D 128, bf16: 64 KiB per block per pool) and on 4096 blocks, timed
    with HIP events on a pool pair of its own."""
    hkv, bs, d = 8, 32, 128
    nb = 8192
    kp = torch.zeros((nb, hkv, bs, d), dtype=torch.bfloat16, device=dev)
    vp = torch.zeros_like(kp)
    block_bytes = hkv * bs * d * 2
    out = {}
    for npairs in (192, 4096):
        perm = np.random.default_rng(7).permutation(nb)
        pairs = torch.from_numpy(np.stack([perm[:npairs], perm[npairs:2 * npairs]], 1).astype(np.int64)).to(dev)
        for _ in range(3):
            P.pa_copy_blocks(kp, vp, pairs)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            P.pa_copy_blocks(kp, vp, pairs)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / 20 / 1e3
        moved = 2 * 2 * npairs * block_bytes        # K and V, read and written
        out[f"{npairs}_pairs"] = {"us": round(t * 1e6, 2), "bytes_moved": moved,
                                  "GBps": round(moved / t / 1e9, 1)}
    return out


def swap_rate(P, torch, dev) -> dict:
    """pa_swap_blocks between a device pool pair and a pinned host pool pair:
    1024 blocks of the headline shape (8 KV heads x 16 tokens x D 128, bf16:
    32 KiB per block per pool), out and back in, timed with HIP events."""
    nb, n = 4096, 1024
    shape = (nb, 8, 16, 128)
    kp = torch.randn(shape, device=dev).to(torch.bfloat16)
    vp = torch.randn(shape, device=dev).to(torch.bfloat16)
    hk = torch.empty((n,) + shape[1:], dtype=torch.bfloat16, pin_memory=True)
    hv = torch.empty_like(hk, pin_memory=True)
    perm = np.random.default_rng(11).permutation(nb)[:n]
    out_pairs = torch.from_numpy(np.stack([perm, np.arange(n)], 1).astype(np.int64)).to(dev)
    in_pairs = torch.from_numpy(np.stack([np.arange(n), perm], 1).astype(np.int64)).to(dev)
    res = {}
    for name, args in (("device_to_host", (kp, vp, hk, hv, out_pairs)),
                       ("host_to_device", (hk, hv, kp, vp, in_pairs))):
        for _ in range(2):
            P.pa_swap_blocks(*args)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            P.pa_swap_blocks(*args)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / 5 / 1e3
        moved = 2 * n * kp[0].numel() * 2
        res[name] = {"us": round(t * 1e6, 1), "bytes": moved, "GBps": round(moved / t / 1e9, 1)}
    return res


def shared_prefix_rate(P, torch, dev, w, q, k_pool, v_pool, db, plen, bs, max_len, scale,
                       unique_bytes, logical_bytes) -> dict:
    """The last timed step of a shared-prefix workload decoded three ways:
    pa_decode with and without the shared-blocks hint, and
    pa_decode_shared_prefix (the prompt groups passed as groups; the blocks
    they share are the whole prompt blocks, the partial one having been
    copied on write), all on the compute path alone."""
    ngroups, nsamp = w.extra["groups"], w.extra["samples"]
    B = q.shape[0]
    shared = (plen // bs) * bs
    gs = torch.arange(0, ngroups * nsamp + 1, nsamp, dtype=torch.int32, device=dev)
    prefix = torch.zeros(B, dtype=torch.int32, device=dev)
    prefix[:ngroups * nsamp] = shared
    out = torch.empty_like(q)
    tables, lens = db["tables"], db["lens"]
    shape = P.DecodeShape(B, q.shape[1], k_pool.shape[1], q.shape[2], bs, k_pool.shape[0],
                          tables.shape[1], max_len, 0, P.PA_BF16, P.PA_VARIANT_AUTO)
    ws_c = torch.empty(P.pa_decode_shared_prefix_workspace_bytes(shape, nsamp, shared),
                       dtype=torch.uint8, device=dev)
    ws_d = torch.empty(max(16, P.pa_decode_workspace_bytes(shape)), dtype=torch.uint8, device=dev)
    res = {}
    for name, fn in (
            ("pa_decode", lambda: P.pa_decode(q, k_pool, v_pool, tables, lens, scale, out,
                                              max_seq_len=max_len, workspace=ws_d,
                                              variant=P.PA_DECODE_SHARED_KV)),
            ("pa_decode_no_hint", lambda: P.pa_decode(q, k_pool, v_pool, tables, lens, scale,
                                                      out, max_seq_len=max_len, workspace=ws_d)),
            ("pa_decode_shared_prefix", lambda: P.pa_decode_shared_prefix(
                q, k_pool, v_pool, tables, lens, scale, out, group_start=gs, prefix_lens=prefix,
                max_group_size=nsamp, max_prefix_len=shared, max_seq_len=max_len,
                workspace=ws_c))):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            fn()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / 20 / 1e3
        res[name] = {"us": round(t * 1e6, 1), "logical_GBps": round(logical_bytes / t / 1e9, 1),
                     "unique_GBps": round(unique_bytes / t / 1e9, 1),
                     "pct_of_hbm_peak_unique": round(100.0 * unique_bytes / t / 1e9 / HBM_PEAK_GBS, 2)}
    if P.pa_device_errors() != 0:
        raise RuntimeError("device error flags set by the shared-prefix decode")
    return res


def group8_decode_rate(P, torch, dev, W) -> dict:
    """pa_decode at 8 query heads per KV head (64 query / 8 KV heads, D 128,
    bf16, block size 16, scattered blocks; 256 sequences of U{512..4096}):
    the matrix-core default (full grid and over a work plan) and the
    vector-ALU kernel."""
    hq, hkv, d, bs = 64, 8, 128, 16
    rng = np.random.default_rng(19)
    lens = rng.integers(512, 4097, 256)
    B = len(lens)
    nblk = [-(-int(L) // bs) for L in lens]
    nb = int(sum(nblk) * 1.1) + 1
    order = rng.permutation(nb)
    tab = np.full((B, max(nblk)), -1, dtype=np.int32)
    p0 = 0
    for i, n in enumerate(nblk):
        tab[i, :n] = order[p0:p0 + n]
        p0 += n
    kp = W.normal_device((nb, hkv, bs, d), 911, "bf16", dev)
    vp = W.normal_device((nb, hkv, bs, d), 912, "bf16", dev)
    q = W.normal_device((B, hq, d), 913, "bf16", dev)
    tabd, lensd = torch.from_numpy(tab).to(dev), torch.from_numpy(lens.astype(np.int32)).to(dev)
    kv = int(lens.sum()) * 2 * hkv * d * 2
    res = {}
    ml = int(lens.max())
    shape = P._decode_shape(q, kp, tabd, ml, 0, P.PA_VARIANT_AUTO)
    plan = torch.from_numpy(P.pa_decode_plan(shape, lens.astype(np.int32))).to(dev)
    for name, variant, wp in (("matrix_cores", P.PA_VARIANT_AUTO, None),
                              ("matrix_cores_planned", P.PA_VARIANT_AUTO, plan),
                              ("vector_alu", P.PA_VARIANT_VALU, None)):
        out = torch.empty_like(q)
        ws = torch.empty(max(16, P.pa_decode_workspace_bytes(
            P._decode_shape(q, kp, tabd, ml, 0, variant))), dtype=torch.uint8, device=dev)

        def call():
            P.pa_decode(q, kp, vp, tabd, lensd, 1.0 / math.sqrt(d), out, max_seq_len=ml,
                        variant=variant, workspace=ws, work_plan=wp)
        for _ in range(2):
            call()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            call()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / 10 / 1e3
        res[name] = {"us": round(t * 1e6, 1), "kv_GBps": round(kv / t / 1e9, 1),
                     "seq_steps_per_s": round(B / t, 1)}
    del kp, vp
    return res


def multi_query_rate(P, torch, dev, W) -> dict:
    """pa_multi_query on the headline head shape (32 query / 8 KV heads, D 128,
    bf16, block size 16, scattered blocks): a 512-token prefill chunk at the
    end of 4096-token contexts for 16 sequences, and 4 speculative tokens for
    each of the 256 headline sequences (lengths U{512..4096}). Matrix-core
    bound: flops = 4 * D * Hq * (positions each query token attends)."""
    hq, hkv, d, bs = 32, 8, 128, 16
    res = {}
    rng = np.random.default_rng(17)
    spec_lens = rng.integers(512, 4097, 256)
    # (lengths, query tokens, split the context into 512-position partitions)
    cases = {"prefill_chunk_512_of_4096_x16": (np.full(16, 4096), np.full(16, 512), False),
             "speculative_4_x256": (spec_lens, np.full(256, 4), False),
             "speculative_4_x256_split": (spec_lens, np.full(256, 4), True)}
    for name, (lens, tqs, split) in cases.items():
        B = len(lens)
        nblk = [-(-int(L) // bs) for L in lens]
        nb = int(sum(nblk) * 1.1) + 1
        order = rng.permutation(nb)
        maxb = max(nblk)
        tab = np.full((B, maxb), -1, dtype=np.int32)
        p0 = 0
        for i, n in enumerate(nblk):
            tab[i, :n] = order[p0:p0 + n]
            p0 += n
        kp = W.normal_device((nb, hkv, bs, d), 901, "bf16", dev)
        vp = W.normal_device((nb, hkv, bs, d), 902, "bf16", dev)
        qs = np.concatenate([[0], np.cumsum(tqs)]).astype(np.int32)
        T = int(qs[-1])
        q = W.normal_device((T, hq, d), 903, "bf16", dev)
        out = torch.empty_like(q)
        args = (q, kp, vp, torch.from_numpy(tab).to(dev),
                torch.from_numpy(lens.astype(np.int32)).to(dev), torch.from_numpy(qs).to(dev),
                1.0 / math.sqrt(d), out)
        kw = dict(max_seq_len=int(lens.max()), max_query_len=int(tqs.max()), split=split)
        if split:
            shape = P.MultiQueryShape(B, hq, hkv, d, bs, nb, maxb, int(lens.max()),
                                      int(tqs.max()), T, P.PA_BF16)
            kw["workspace"] = torch.empty(max(16, P.pa_multi_query_workspace_bytes(shape)),
                                          dtype=torch.uint8, device=dev)
        for _ in range(2):
            P.pa_multi_query(*args, **kw)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            P.pa_multi_query(*args, **kw)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / 10 / 1e3
        attended = sum(int(tq) * (int(L) - int(tq)) + int(tq) * (int(tq) + 1) // 2
                       for L, tq in zip(lens, tqs))
        flops = 4 * d * hq * attended
        kv = int(lens.sum()) * 2 * hkv * d * 2
        res[name] = {"us": round(t * 1e6, 1), "TFLOPs": round(flops / t / 1e12, 1),
                     "mfma_bf16_frac": round(flops / t / 2.5e15, 4),
                     "kv_GBps": round(kv / t / 1e9, 1), "query_tokens": T}
        del kp, vp
    return res


def fork_cow_host_us(P) -> float:
    """Host time of the shared-prefix workload's sharing decisions: 64 prompt
    groups of 1040 tokens at block size 32, three forks each, then the first
    private token of all 256 samples (192 copy-on-write pairs)."""
    groups, samples, bs, prefix = 64, 4, 32, 1040
    nb = groups * (prefix // bs + 1) + groups * samples * 2 + 64
    bm = P.BlockManager(nb, bs)
    t0 = time.perf_counter()
    for gi in range(groups):
        bm.add_seq(gi * samples, prefix)
        for k in range(1, samples):
            bm.fork(gi * samples, gi * samples + k)
    _, pairs = bm.append_slots(np.arange(groups * samples, dtype=np.int32))
    el = time.perf_counter() - t0
    if pairs.shape[0] != groups * (samples - 1):
        raise RuntimeError("unexpected copy-on-write count")
    return round(el * 1e6, 1)


CALIBRATION_LAUNCHES = 3


def copy_calibration(P, torch, dev, mib: int, block_bytes: int) -> dict:
    """pa_copy_blocks over a fresh pair of pools: n blocks copied to n other
    blocks in each of the K and V pools, so that exactly 2 * n * block_bytes
    bytes are read and as many written. Its FETCH_SIZE / WRITE_SIZE readings
    calibrate the counters (KiB per dispatch) against a known byte count."""
    n = max(1, mib * 2**20 // block_bytes)
    kp = torch.zeros((2 * n, block_bytes // 2), dtype=torch.int16, device=dev)
    vp = torch.zeros_like(kp)
    pairs = torch.stack([torch.arange(n), torch.arange(n, 2 * n)], dim=1).to(
        device=dev, dtype=torch.int64).contiguous()
    for _ in range(CALIBRATION_LAUNCHES):
        P.pa_copy_blocks(kp.view(2 * n, 1, 1, block_bytes // 2), vp.view(2 * n, 1, 1, block_bytes // 2),
                         pairs)
    torch.cuda.synchronize()
    return {"pairs": n, "block_bytes": block_bytes, "read_bytes": 2 * n * block_bytes,
            "write_bytes": 2 * n * block_bytes, "launches": CALIBRATION_LAUNCHES}


def _counter_rows(directory: str, counter: str):
    """(kernel name, value) per dispatch from a rocprofv3 --pmc csv run."""
    import csv
    import glob
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *counter_collection.csv under {directory}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                if r.get("Counter_Name") == counter:
                    rows.append((int(r.get("Dispatch_Id") or len(rows)), r["Kernel_Name"],
                                 float(r["Counter_Value"])))
    rows.sort(key=lambda x: x[0])                 # dispatch order
    return [(k, v) for _, k, v in rows]


def summarise_traffic(args) -> int:
    """HBM bytes per partition-kernel launch from two rocprofv3 --pmc runs.

    Each counter (KiB per dispatch) is scaled by copy-bytes / counter-reading
    of the calibration copy kernel (pa_copy_blocks of a known size) in the
    same run, then averaged over the partition kernel's dispatches."""
    fetch_dir, write_dir = args.traffic_from
    out = {"source_hash": kernel_source_hash(), "workload": args.workload}
    per_launch = 0.0
    for counter, directory in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(directory, counter)
        # the step loop's partition kernel is the run's first decode_partition
        # dispatch; later side measurements launch other instances
        main = next((k for k, _ in rows if "decode_partition" in k), None)
        part = [v for k, v in rows if k == main]
        cal = [v for k, v in rows if "copy_blocks_kernel" in k]
        if not part or not cal:
            raise RuntimeError(f"{counter}: need partition and copy dispatches in {directory}")
        # warm-up dispatches first, then the timed steps
        part = part[args.warmup:args.warmup + args.steps] if args.steps else part
        variant = "mfma" if "decode_partition_mfma" in main else "valu"
        # the calibration copies are the run's last copy dispatches (the
        # copy-on-write and swap measurements use the same kernel earlier)
        cal_kib = float(np.median(cal[-CALIBRATION_LAUNCHES:]))
        out[counter] = {"partition_kib_mean": float(np.mean(part)), "dispatches": len(part),
                        "copy_kib_median": cal_kib}
        out["variant"] = variant
    return _finish_traffic(args, out)


def _finish_traffic(args, out) -> int:
    cal = args.copy_calibration_mib
    if cal <= 0:
        raise SystemExit("--copy-calibration-mib must give the calibration size used in the runs")
    w_ = __import__("workloads").get(args.workload)
    block_bytes = w_.num_kv_heads * w_.block_size * w_.head_dim * w_.elem_bytes
    n = max(1, cal * 2**20 // block_bytes)
    known_kib = 2 * n * block_bytes / 1024.0
    total = 0.0
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        c = out[counter]
        c["scale"] = known_kib / c["copy_kib_median"]
        c["partition_bytes"] = c["partition_kib_mean"] * c["scale"] * 1024.0
        total += c["partition_bytes"]
    out["bytes_per_launch"] = round(total)
    out["calibration_bytes_each_way"] = int(2 * n * block_bytes)
    # algorithmic K/V bytes of the same launches: the seeded lengths plus one
    # token per step, at the counted (timed) steps
    if w_.lengths[0] != "prefix_suffix":
        ctx = __import__("workloads").draw_lengths(
            w_, np.random.default_rng(w_.seed)).astype(np.int64)
        per_tok = 2 * w_.num_kv_heads * w_.head_dim * w_.elem_bytes
        steps = range(args.warmup, args.warmup + args.steps)
        out["algorithmic_bytes_per_launch"] = round(float(np.mean(
            [int((ctx + s + 1).sum()) * per_tok for s in steps])))
        out["steps"], out["warmup"] = args.steps, args.warmup
        out["traffic_over_algorithmic"] = round(total / out["algorithmic_bytes_per_launch"], 4)
    text = json.dumps(out, indent=1)
    print(text)
    if args.traffic_out:
        with open(args.traffic_out, "w") as fh:
            fh.write(text + "\n")
    return 0


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


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
    # all the cores this process may run on, but no more than the host's
    # share for it (OMP_NUM_THREADS, set to the machine's CPU share)
    affinity = len(os.sched_getaffinity(0))
    share = int(os.environ.get("OMP_NUM_THREADS") or affinity)
    threads = max(1, min(affinity, share))
    R.decode(q_host[:n_seq], kp_host, vp_host, tables, lens, scale, w.dtype, num_threads=threads)
    # three timed runs of about seconds / 3 each; the median rate is reported
    runs, reps, el = [], 0, 0.0
    for _ in range(3):
        r, t0 = 0, time.perf_counter()
        while True:
            R.decode(q_host[:n_seq], kp_host, vp_host, tables, lens, scale, w.dtype,
                     num_threads=threads)
            r += 1
            dt = time.perf_counter() - t0
            if dt >= seconds / 3 or r >= 400:
                break
        runs.append(n_seq * r / dt)
        reps, el = reps + r, el + dt
    kv_bytes = int(lens.astype(np.int64).sum()) * 2 * w.num_kv_heads * w.head_dim * w.elem_bytes
    # the same oracle on one thread, for a third of the time
    reps1, t1 = 0, time.perf_counter()
    while True:
        R.decode(q_host[:n_seq], kp_host, vp_host, tables, lens, scale, w.dtype, num_threads=1)
        reps1 += 1
        el1 = time.perf_counter() - t1
        if el1 >= seconds / 3 or reps1 >= 1000:
            break
    med = float(np.median(runs))
    return {"value": round(med, 2), "unit": "seq-steps/s", "cores": threads,
            "kind": "oracle", "affinity_cpus": affinity,
            "thread_rule": ("OpenMP over (sequence, query head) pairs on min(affinity set, "
                            "OMP_NUM_THREADS) threads"),
            "runs_seq_steps_per_s": [round(x, 2) for x in runs],
            "kv_gb_per_s": round(kv_bytes * med / n_seq / 1e9, 3),
            "cpu_model": cpu_model(),
            "single_thread": {"value": round(n_seq * reps1 / el1, 2), "unit": "seq-steps/s",
                              "repetitions": reps1, "seconds": round(el1, 1)},
            "sample": (f"first {n_seq} of {len(ctx)} {w.name} sequences at the last timed step "
                       f"(sum of lengths {int(lens.sum())}), plain C float64 oracle, "
                       f"median of 3 runs, {reps} repetitions in {el:.1f} s")}


if __name__ == "__main__":
    sys.exit(main())
