"""Python binding of libpa, the gfx950 paged decode attention library.

Argument marshalling only: every computation runs in libpa.so (HIP kernels
for the GPU calls, C++ for the host block manager). torch tensors supply
device memory and the current stream. There is no fallback: if libpa.so has
not been built, importing the binding's functions raises.

Calls mirror the C ABI in include/pa.h:
    pa_decode, pa_decode_partition, pa_decode_reduce, pa_decode_workspace_bytes,
    pa_decode_plan_capacity, pa_decode_plan (the decode calls take its plan as work_plan),
    pa_reshape_and_cache, pa_append_tokens, pa_copy_blocks, pa_swap_blocks, pa_device_errors,
    BlockManager (pa_bm_*).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

__all__ = [
    "LIB_PATH", "PaError", "lib", "PA_F32", "PA_BF16", "PA_DEVERR_BLOCK_ID", "PA_DEVERR_SEQ_LEN",
    "PA_DEVERR_SLOT", "PA_DEVERR_COPY_PAIR", "PA_DEVERR_QUERY", "PA_DEVERR_PREFIX",
    "pa_decode_shared_prefix", "pa_decode_shared_prefix_workspace_bytes", "MultiQueryShape", "pa_multi_query", "pa_multi_query_workspace_bytes",
    "pa_decode_e4m3", "pa_reshape_and_cache_e4m3", "PA_DEVERR_PLAN",
    "pa_decode_plan_capacity", "pa_decode_plan",
    "pa_append_tokens",
    "PA_VARIANT_AUTO", "PA_VARIANT_VALU", "PA_VARIANT_MFMA", "PA_DECODE_SHARED_KV", "DecodeShape",
    "pa_decode_workspace_bytes", "pa_decode", "pa_decode_partition", "pa_decode_reduce",
    "pa_reshape_and_cache", "pa_copy_blocks", "pa_swap_blocks", "pa_device_errors",
    "BlockManager", "EXPORTED_SYMBOLS", "PA_DECODE_HALF_PARTIALS", "pa_decode_noalloc",
    "PA_NOALLOC_SCRATCH_BYTES",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa.so")

PA_F32, PA_BF16 = 0, 1
# device error word bits (include/pa.h PA_DEVERR_*)
PA_DEVERR_BLOCK_ID, PA_DEVERR_SEQ_LEN, PA_DEVERR_SLOT, PA_DEVERR_COPY_PAIR = 0x1, 0x2, 0x4, 0x8
PA_DEVERR_QUERY = 0x10
PA_DEVERR_PREFIX = 0x20
PA_DEVERR_PLAN = 0x40
PA_VARIANT_AUTO, PA_VARIANT_VALU, PA_VARIANT_MFMA = 0, 1, 2
# hint OR-ed into `variant`: the batch's sequences share blocks (pa.h)
PA_DECODE_SHARED_KV = 0x100
# option OR-ed into `variant`: bf16 partial outputs (pa.h; off by default)
PA_DECODE_HALF_PARTIALS = 0x200
# size of the device array pa_decode_noalloc keeps its partials in (pa.h)
PA_NOALLOC_SCRATCH_BYTES = 64 << 20
_STATUS = {0: "PA_OK", 1: "PA_EINVAL", 2: "PA_EUNSUPPORTED", 3: "PA_EWORKSPACE",
           4: "PA_ENOBLOCKS", 5: "PA_EREFCOUNT", 6: "PA_EHIP", 7: "PA_EDEVICE"}

# Every function include/pa.h declares.
EXPORTED_SYMBOLS = (
    "pa_decode_workspace_bytes", "pa_decode", "pa_decode_partition", "pa_decode_reduce",
    "pa_decode_noalloc",
    "pa_reshape_and_cache", "pa_copy_blocks", "pa_swap_blocks", "pa_device_errors",
    "pa_status_str", "pa_last_hip_error", "pa_multi_query", "pa_multi_query_workspace_bytes",
    "pa_multi_query_split", "pa_decode_shared_prefix", "pa_decode_shared_prefix_workspace_bytes",
    "pa_decode_e4m3", "pa_decode_partition_e4m3",
    "pa_reshape_and_cache_e4m3",
    "pa_decode_plan_capacity", "pa_decode_plan",
    "pa_append_tokens", "pa_append_tokens_e4m3",
    "pa_bm_create", "pa_bm_destroy", "pa_bm_add_seq", "pa_bm_append_slots", "pa_bm_fork",
    "pa_bm_free_seq", "pa_bm_export", "pa_bm_num_free", "pa_bm_refcount", "pa_bm_num_tokens",
    "pa_bm_set_swap_space", "pa_bm_swap_out", "pa_bm_swap_in", "pa_bm_num_free_swap",
    "pa_bm_is_swapped",
)


class PaError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        self.name = _STATUS.get(status, str(status))
        msg = f"{what}: {self.name}" if what else self.name
        if self.name == "PA_EHIP" and _lib is not None:
            # the HIP error behind it (the calling thread's most recent one)
            msg += f" ({_lib.pa_last_hip_error().decode()})"
        super().__init__(msg)


class DecodeShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_seqs", "num_q_heads", "num_kv_heads", "head_dim", "block_size", "num_blocks",
        "max_blocks_per_seq", "max_seq_len", "partition_tokens", "dtype", "variant")]


class MultiQueryShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_seqs", "num_q_heads", "num_kv_heads", "head_dim", "block_size", "num_blocks",
        "max_blocks_per_seq", "max_seq_len", "max_query_len", "num_tokens", "dtype")]


_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_SIGS = {
    "pa_decode_workspace_bytes": (_sz, [ctypes.POINTER(DecodeShape)]),
    "pa_decode": (_i32, [_vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp,
                         ctypes.POINTER(DecodeShape), _vp, _i32, _vp, _sz, _vp]),
    "pa_decode_partition": (_i32, [_vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp,
                                   ctypes.POINTER(DecodeShape), _vp, _i32, _vp, _sz, _vp]),
    "pa_decode_reduce": (_i32, [_vp, _vp, ctypes.POINTER(DecodeShape), _vp, _sz, _vp]),
    "pa_decode_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp,
                                 ctypes.POINTER(DecodeShape), _vp]),
    "pa_decode_plan_capacity": (_i64, [ctypes.POINTER(DecodeShape)]),
    "pa_decode_plan": (_i32, [ctypes.POINTER(DecodeShape), _vp, _vp, _vp, _i64,
                              ctypes.POINTER(_i32)]),
    "pa_reshape_and_cache": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                    _i32, _vp]),
    "pa_copy_blocks": (_i32, [_vp, _vp, _vp, _i32, _i64, _i32, _vp]),
    "pa_swap_blocks": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i64, _i32, _i32, _vp]),
    "pa_multi_query": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp,
                              ctypes.POINTER(MultiQueryShape), _vp]),
    "pa_multi_query_workspace_bytes": (_sz, [ctypes.POINTER(MultiQueryShape), _i32]),
    "pa_decode_shared_prefix_workspace_bytes": (_sz, [ctypes.POINTER(DecodeShape), _i32, _i32]),
    "pa_decode_shared_prefix": (_i32, [_vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp,
                                       ctypes.POINTER(DecodeShape), _i32, _vp, _vp, _i32, _i32,
                                       _vp, _i32, _vp, _sz, _vp]),
    "pa_multi_query_split": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp,
                                    ctypes.POINTER(MultiQueryShape), _i32, _vp, _sz, _vp]),
    "pa_decode_e4m3": (_i32, [_vp, _vp, _vp, _vp, _vp, ctypes.c_float, ctypes.c_float,
                              ctypes.c_float, _vp, ctypes.POINTER(DecodeShape), _vp, _i32, _vp,
                              _sz, _vp]),
    "pa_decode_partition_e4m3": (_i32, [_vp, _vp, _vp, _vp, _vp, ctypes.c_float, ctypes.c_float,
                                        ctypes.c_float, _vp, ctypes.POINTER(DecodeShape), _vp,
                                        _i32, _vp, _sz, _vp]),
    "pa_append_tokens": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                _i32, _i32, _vp]),
    "pa_append_tokens_e4m3": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                     _i32, _i32, ctypes.c_float, ctypes.c_float, _vp]),
    "pa_reshape_and_cache_e4m3": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                         ctypes.c_float, ctypes.c_float, _vp]),
    "pa_device_errors": (_i32, [ctypes.POINTER(ctypes.c_uint32), _vp]),
    "pa_status_str": (ctypes.c_char_p, [_i32]),
    "pa_last_hip_error": (ctypes.c_char_p, []),
    "pa_bm_create": (_i32, [_i32, _i32, _vp, ctypes.POINTER(_vp)]),
    "pa_bm_destroy": (None, [_vp]),
    "pa_bm_add_seq": (_i32, [_vp, _i32, _i32]),
    "pa_bm_append_slots": (_i32, [_vp, _vp, _i32, _vp, _vp, ctypes.POINTER(_i32)]),
    "pa_bm_fork": (_i32, [_vp, _i32, _i32]),
    "pa_bm_free_seq": (_i32, [_vp, _i32]),
    "pa_bm_export": (_i32, [_vp, _vp, _i32, _i32, _vp, _vp]),
    "pa_bm_num_free": (_i32, [_vp]),
    "pa_bm_refcount": (_i32, [_vp, _i32]),
    "pa_bm_num_tokens": (_i32, [_vp, _i32]),
    "pa_bm_set_swap_space": (_i32, [_vp, _i32]),
    "pa_bm_swap_out": (_i32, [_vp, _i32, _vp, _i32, ctypes.POINTER(_i32)]),
    "pa_bm_swap_in": (_i32, [_vp, _i32, _vp, _i32, ctypes.POINTER(_i32)]),
    "pa_bm_num_free_swap": (_i32, [_vp]),
    "pa_bm_is_swapped": (_i32, [_vp, _i32]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libpa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -c 'import __graft_entry__ as g; g.build()'`")
        # libpa.so takes whichever HIP runtime (soname libamdhip64.so.7) the
        # process has loaded. torch ships its own copy, which owns the device
        # memory and streams handed to libpa: load it first, or libpa would
        # bring in a second runtime to which torch's pointers mean nothing
        import torch  # noqa: F401
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(handle, name)
            f.restype = res
            f.argtypes = args
        _lib = handle
    return _lib


def _check(status: int, what: str) -> None:
    if status != 0:
        raise PaError(status, what)


# --------------------------------------------------------------------------
# GPU calls (torch tensors in, pointers out)
# --------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream_ptr(stream, device) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return s.cuda_stream


def _need(t, name, dtype=None, dim=None, device=None):
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dims")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}")


def _decode_shape(q, k_pool, block_tables, max_seq_len, partition_tokens, variant):
    B, hq, d = q.shape
    nb, hkv, bs, d2 = k_pool.shape
    if d2 != d:
        raise ValueError("head_dim mismatch between q and the pools")
    return DecodeShape(B, hq, hkv, d, bs, nb, block_tables.shape[1], int(max_seq_len),
                       int(partition_tokens), _dtype_code(q), int(variant))


def pa_decode_workspace_bytes(shape: DecodeShape) -> int:
    return int(lib().pa_decode_workspace_bytes(ctypes.byref(shape)))


def pa_decode_plan_capacity(shape: DecodeShape) -> int:
    return int(lib().pa_decode_plan_capacity(ctypes.byref(shape)))


def pa_decode_plan(shape: DecodeShape, seq_lens_host, walk_start=None) -> np.ndarray:
    """Host work plan of a decode call (include/pa.h pa_decode_plan):
    int32 [num_units, 4] entries (sequence, partition, length, walk start),
    built from the host lengths (int32 array-like [B]) and, for
    pa_decode_shared_prefix, the host prefix lengths as walk_start."""
    lens = np.ascontiguousarray(np.asarray(seq_lens_host, dtype=np.int32))
    if lens.shape != (shape.num_seqs,):
        raise ValueError("seq_lens must hold num_seqs lengths")
    starts = None
    if walk_start is not None:
        starts = np.ascontiguousarray(np.asarray(walk_start, dtype=np.int32))
        if starts.shape != lens.shape:
            raise ValueError("walk_start must hold num_seqs positions")
    cap = pa_decode_plan_capacity(shape)
    plan = np.zeros((max(cap, 1), 4), dtype=np.int32)
    n = ctypes.c_int32(0)
    _check(lib().pa_decode_plan(ctypes.byref(shape), lens.ctypes.data,
                                None if starts is None else starts.ctypes.data,
                                plan.ctypes.data, cap, ctypes.byref(n)), "pa_decode_plan")
    return plan[:n.value].copy()


def _plan_args(work_plan, dev):
    """(pointer, unit count) of an optional device work plan."""
    if work_plan is None:
        return None, 0
    torch = _torch()
    _need(work_plan, "work_plan", dtype=torch.int32, dim=2, device=dev)
    if work_plan.shape[1] != 4:
        raise ValueError("work_plan must be [num_units, 4]")
    return work_plan.data_ptr(), int(work_plan.shape[0])


def _decode_call(fn_name, q, k_pool, v_pool, block_tables, seq_lens, scale, out, *,
                 max_seq_len, partition_tokens=0, variant=PA_VARIANT_AUTO, workspace=None,
                 stream=None, work_plan=None):
    torch = _torch()
    dev = q.device
    _need(q, "q", dim=3)
    _need(k_pool, "k_pool", dtype=q.dtype, dim=4, device=dev)
    _need(v_pool, "v_pool", dtype=q.dtype, dim=4, device=dev)
    _need(block_tables, "block_tables", dtype=torch.int32, dim=2, device=dev)
    _need(seq_lens, "seq_lens", dtype=torch.int32, dim=1, device=dev)
    _need(out, "out", dtype=q.dtype, device=dev)
    if tuple(v_pool.shape) != tuple(k_pool.shape) or tuple(out.shape) != tuple(q.shape):
        raise ValueError("shape mismatch")
    if block_tables.shape[0] != q.shape[0] or seq_lens.shape[0] != q.shape[0]:
        raise ValueError("batch mismatch")
    shape = _decode_shape(q, k_pool, block_tables, max_seq_len, partition_tokens, variant)
    need = pa_decode_workspace_bytes(shape)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    plan_args = _plan_args(work_plan, dev)
    st = getattr(lib(), fn_name)(
        q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), block_tables.data_ptr(),
        seq_lens.data_ptr(), ctypes.c_float(scale), out.data_ptr(), ctypes.byref(shape),
        *plan_args, workspace.data_ptr(), ws_bytes, _stream_ptr(stream, dev))
    _check(st, fn_name)
    return out


def pa_decode(q, k_pool, v_pool, block_tables, seq_lens, scale, out, *, max_seq_len,
              partition_tokens=0, variant=PA_VARIANT_AUTO, workspace=None, stream=None,
              work_plan=None):
    """Paged decode attention (include/pa.h pa_decode). q [B,Hq,D]; pools
    [NB,Hkv,bs,D]; block_tables int32 [B,maxb]; seq_lens int32 [B]; out
    [B,Hq,D]; work_plan: None, or the pa_decode_plan output as a device int32
    tensor [num_units, 4]. Enqueues on `stream` (default: torch's current
    stream)."""
    return _decode_call("pa_decode", q, k_pool, v_pool, block_tables, seq_lens, scale, out,
                        max_seq_len=max_seq_len, partition_tokens=partition_tokens,
                        variant=variant, workspace=workspace, stream=stream,
                        work_plan=work_plan)


def pa_decode_noalloc(q, k_pool, v_pool, block_tables, seq_lens, scale, out, *, max_seq_len,
                      partition_tokens=0, variant=PA_VARIANT_AUTO, stream=None):
    """pa_decode with its partials in libpa's own device array instead of a
    caller workspace (include/pa.h pa_decode_noalloc): allocates nothing.
    Calls that may overlap on one GPU race."""
    torch = _torch()
    dev = q.device
    _need(q, "q", dim=3)
    _need(k_pool, "k_pool", dtype=q.dtype, dim=4, device=dev)
    _need(v_pool, "v_pool", dtype=q.dtype, dim=4, device=dev)
    _need(block_tables, "block_tables", dtype=torch.int32, dim=2, device=dev)
    _need(seq_lens, "seq_lens", dtype=torch.int32, dim=1, device=dev)
    _need(out, "out", dtype=q.dtype, device=dev)
    if tuple(v_pool.shape) != tuple(k_pool.shape) or tuple(out.shape) != tuple(q.shape):
        raise ValueError("shape mismatch")
    if block_tables.shape[0] != q.shape[0] or seq_lens.shape[0] != q.shape[0]:
        raise ValueError("batch mismatch")
    shape = _decode_shape(q, k_pool, block_tables, max_seq_len, partition_tokens, variant)
    st = lib().pa_decode_noalloc(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                 block_tables.data_ptr(), seq_lens.data_ptr(),
                                 ctypes.c_float(scale), out.data_ptr(), ctypes.byref(shape),
                                 _stream_ptr(stream, dev))
    _check(st, "pa_decode_noalloc")
    return out


def pa_decode_shared_prefix_workspace_bytes(shape: DecodeShape, max_group_size: int,
                                            max_prefix_len: int) -> int:
    return int(lib().pa_decode_shared_prefix_workspace_bytes(
        ctypes.byref(shape), int(max_group_size), int(max_prefix_len)))


def pa_decode_shared_prefix(q, k_pool, v_pool, block_tables, seq_lens, scale, out, *,
                            group_start, prefix_lens, max_group_size, max_prefix_len,
                            max_seq_len, partition_tokens=0, workspace=None, stream=None,
                            work_plan=None):
    """pa_decode for groups of sequences sharing a prompt (include/pa.h
    pa_decode_shared_prefix). group_start int32 [G+1] and prefix_lens int32
    [B] on the device; the workspace is allocated here unless given;
    work_plan: None, or a pa_decode_plan output built with walk_start = the
    host prefix lengths, as a device int32 tensor [num_units, 4]."""
    torch = _torch()
    dev = q.device
    _need(q, "q", dtype=torch.bfloat16, dim=3)
    _need(k_pool, "k_pool", dtype=q.dtype, dim=4, device=dev)
    _need(v_pool, "v_pool", dtype=q.dtype, dim=4, device=dev)
    _need(block_tables, "block_tables", dtype=torch.int32, dim=2, device=dev)
    _need(seq_lens, "seq_lens", dtype=torch.int32, dim=1, device=dev)
    _need(group_start, "group_start", dtype=torch.int32, dim=1, device=dev)
    _need(prefix_lens, "prefix_lens", dtype=torch.int32, dim=1, device=dev)
    _need(out, "out", dtype=q.dtype, device=dev)
    if tuple(v_pool.shape) != tuple(k_pool.shape) or tuple(out.shape) != tuple(q.shape):
        raise ValueError("shape mismatch")
    B = q.shape[0]
    if block_tables.shape[0] != B or seq_lens.shape[0] != B or prefix_lens.shape[0] != B:
        raise ValueError("batch mismatch")
    shape = _decode_shape(q, k_pool, block_tables, max_seq_len, partition_tokens,
                          PA_VARIANT_AUTO)
    need = pa_decode_shared_prefix_workspace_bytes(shape, max_group_size, max_prefix_len)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", device=dev)
    st = lib().pa_decode_shared_prefix(
        q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), block_tables.data_ptr(),
        seq_lens.data_ptr(), ctypes.c_float(scale), out.data_ptr(), ctypes.byref(shape),
        group_start.shape[0] - 1, group_start.data_ptr(), prefix_lens.data_ptr(),
        int(max_group_size), int(max_prefix_len), *_plan_args(work_plan, dev),
        workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream_ptr(stream, dev))
    _check(st, "pa_decode_shared_prefix")
    return out


def pa_decode_partition(q, k_pool, v_pool, block_tables, seq_lens, scale, out, *, max_seq_len,
                        partition_tokens=0, variant=PA_VARIANT_AUTO, workspace, stream=None,
                        work_plan=None):
    """First half of pa_decode (per-partition kernel); pa_decode_reduce
    completes it."""
    return _decode_call("pa_decode_partition", q, k_pool, v_pool, block_tables, seq_lens, scale,
                        out, max_seq_len=max_seq_len, partition_tokens=partition_tokens,
                        variant=variant, workspace=workspace, stream=stream,
                        work_plan=work_plan)


def pa_decode_reduce(q, k_pool, block_tables, seq_lens, out, *, max_seq_len, partition_tokens=0,
                     variant=PA_VARIANT_AUTO, workspace, stream=None):
    """Second half of pa_decode (partition merge). q/k_pool/block_tables only
    describe the shape."""
    shape = _decode_shape(q, k_pool, block_tables, max_seq_len, partition_tokens, variant)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().pa_decode_reduce(seq_lens.data_ptr(), out.data_ptr(), ctypes.byref(shape),
                                workspace.data_ptr(), ws_bytes, _stream_ptr(stream, out.device))
    _check(st, "pa_decode_reduce")
    return out


def pa_decode_e4m3(q, k_pool, v_pool, block_tables, seq_lens, scale, k_scale, v_scale, out, *,
                   max_seq_len, partition_tokens=0, variant=PA_VARIANT_MFMA, workspace=None,
                   stream=None, work_plan=None):
    """pa_decode over 8-bit pools (include/pa.h pa_decode_e4m3): q, out bf16
    [B,Hq,D]; pools uint8 [NB,Hkv,bs,D] of FP8 E4M3 codes. `variant` may carry
    PA_DECODE_SHARED_KV (the kernel is always the matrix-core one). With
    `work_plan` (device int32 [num_units, 4] from pa_decode_plan, built with
    the same explicit partition_tokens) the grid follows the plan."""
    torch = _torch()
    dev = q.device
    _need(q, "q", dtype=torch.bfloat16, dim=3)
    _need(k_pool, "k_pool", dtype=torch.uint8, dim=4, device=dev)
    _need(v_pool, "v_pool", dtype=torch.uint8, dim=4, device=dev)
    _need(block_tables, "block_tables", dtype=torch.int32, dim=2, device=dev)
    _need(seq_lens, "seq_lens", dtype=torch.int32, dim=1, device=dev)
    _need(out, "out", dtype=q.dtype, device=dev)
    if tuple(v_pool.shape) != tuple(k_pool.shape) or tuple(out.shape) != tuple(q.shape):
        raise ValueError("shape mismatch")
    shape = _decode_shape(q, k_pool, block_tables, max_seq_len, partition_tokens, variant)
    need = pa_decode_workspace_bytes(shape)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    fn, plan_args = "pa_decode_e4m3", _plan_args(work_plan, dev)
    st = getattr(lib(), fn)(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                            block_tables.data_ptr(), seq_lens.data_ptr(), ctypes.c_float(scale),
                            ctypes.c_float(k_scale), ctypes.c_float(v_scale), out.data_ptr(),
                            ctypes.byref(shape), *plan_args, workspace.data_ptr(),
                            workspace.numel() * workspace.element_size(), _stream_ptr(stream, dev))
    _check(st, fn)
    return out


def pa_reshape_and_cache_e4m3(k, v, slot_mapping, k_pool, v_pool, k_scale, v_scale, stream=None):
    """Quantized slot write: k/v bf16 [T,Hkv,D] into uint8 pools of FP8 E4M3 codes."""
    torch = _torch()
    dev = k_pool.device
    _need(k, "k", dtype=torch.bfloat16, dim=3, device=dev)
    _need(v, "v", dtype=torch.bfloat16, dim=3, device=dev)
    _need(slot_mapping, "slot_mapping", dtype=torch.int64, dim=1, device=dev)
    _need(k_pool, "k_pool", dtype=torch.uint8, dim=4)
    _need(v_pool, "v_pool", dtype=torch.uint8, device=dev)
    nb, hkv, bs, d = k_pool.shape
    T = k.shape[0]
    if tuple(k.shape) != (T, hkv, d) or tuple(v.shape) != (T, hkv, d) or slot_mapping.shape[0] != T:
        raise ValueError("shape mismatch")
    st = lib().pa_reshape_and_cache_e4m3(k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(),
                                         k_pool.data_ptr(), v_pool.data_ptr(), T, hkv, d, bs, nb,
                                         ctypes.c_float(k_scale), ctypes.c_float(v_scale),
                                         _stream_ptr(stream, dev))
    _check(st, "pa_reshape_and_cache_e4m3")


def pa_multi_query_workspace_bytes(shape: MultiQueryShape, partition_tokens: int = 0) -> int:
    return int(lib().pa_multi_query_workspace_bytes(ctypes.byref(shape), int(partition_tokens)))


def pa_multi_query(q, k_pool, v_pool, block_tables, seq_lens, query_start, scale, out, *,
                   max_seq_len, max_query_len, stream=None, split=False, partition_tokens=0,
                   workspace=None):
    """Attention of several query tokens per sequence (include/pa.h
    pa_multi_query; with split=True, pa_multi_query_split over context
    partitions of partition_tokens positions, the workspace allocated here
    unless a large enough uint8 device tensor is passed).
    q, out [T, Hq, D] bf16; query_start int32 [B+1]."""
    torch = _torch()
    dev = q.device
    _need(q, "q", dtype=torch.bfloat16, dim=3)
    _need(k_pool, "k_pool", dtype=q.dtype, dim=4, device=dev)
    _need(v_pool, "v_pool", dtype=q.dtype, dim=4, device=dev)
    _need(block_tables, "block_tables", dtype=torch.int32, dim=2, device=dev)
    _need(seq_lens, "seq_lens", dtype=torch.int32, dim=1, device=dev)
    _need(query_start, "query_start", dtype=torch.int32, dim=1, device=dev)
    _need(out, "out", dtype=q.dtype, device=dev)
    T, hq, d = q.shape
    nb, hkv, bs, d2 = k_pool.shape
    B = seq_lens.shape[0]
    if d2 != d or tuple(out.shape) != tuple(q.shape) or tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError("shape mismatch")
    if block_tables.shape[0] != B or query_start.shape[0] != B + 1:
        raise ValueError("batch mismatch")
    shape = MultiQueryShape(B, hq, hkv, d, bs, nb, block_tables.shape[1], int(max_seq_len),
                            int(max_query_len), T, PA_BF16)
    if not split:
        st = lib().pa_multi_query(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                  block_tables.data_ptr(), seq_lens.data_ptr(),
                                  query_start.data_ptr(), ctypes.c_float(scale), out.data_ptr(),
                                  ctypes.byref(shape), _stream_ptr(stream, dev))
        _check(st, "pa_multi_query")
        return out
    need = pa_multi_query_workspace_bytes(shape, partition_tokens)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", dtype=torch.uint8, device=dev)
    st = lib().pa_multi_query_split(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                    block_tables.data_ptr(), seq_lens.data_ptr(),
                                    query_start.data_ptr(), ctypes.c_float(scale), out.data_ptr(),
                                    ctypes.byref(shape), int(partition_tokens),
                                    workspace.data_ptr(), workspace.numel(),
                                    _stream_ptr(stream, dev))
    _check(st, "pa_multi_query_split")
    return out


def pa_reshape_and_cache(k, v, slot_mapping, k_pool, v_pool, stream=None):
    """Write k/v [T,Hkv,D] into the pools at slot_mapping (int64 [T]);
    slot < 0 writes nothing."""
    torch = _torch()
    dev = k_pool.device
    _need(k, "k", dtype=k_pool.dtype, dim=3, device=dev)
    _need(v, "v", dtype=k_pool.dtype, dim=3, device=dev)
    _need(slot_mapping, "slot_mapping", dtype=torch.int64, dim=1, device=dev)
    _need(k_pool, "k_pool", dim=4)
    _need(v_pool, "v_pool", dtype=k_pool.dtype, device=dev)
    nb, hkv, bs, d = k_pool.shape
    T = k.shape[0]
    if tuple(k.shape) != (T, hkv, d) or tuple(v.shape) != (T, hkv, d) or slot_mapping.shape[0] != T:
        raise ValueError("shape mismatch")
    st = lib().pa_reshape_and_cache(k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(),
                                    k_pool.data_ptr(), v_pool.data_ptr(), T, hkv, d, bs, nb,
                                    _dtype_code(k_pool), _stream_ptr(stream, dev))
    _check(st, "pa_reshape_and_cache")


def pa_append_tokens(k, v, slot_mapping, k_pool, v_pool, block_tables, seq_lens, stream=None,
                     kv_scales=None):
    """One token per sequence (include/pa.h pa_append_tokens): k/v [B,Hkv,D]
    written at slot_mapping (int64 [B]), and the device block_tables (int32
    [B,maxb]) and seq_lens (int32 [B]) updated in place. With uint8 pools of
    FP8 codes pass kv_scales=(k_scale, v_scale) (pa_append_tokens_e4m3)."""
    torch = _torch()
    dev = k_pool.device
    fp8 = k_pool.dtype == torch.uint8
    _need(k, "k", dtype=torch.bfloat16 if fp8 else k_pool.dtype, dim=3, device=dev)
    _need(v, "v", dtype=k.dtype, dim=3, device=dev)
    _need(slot_mapping, "slot_mapping", dtype=torch.int64, dim=1, device=dev)
    _need(k_pool, "k_pool", dim=4)
    _need(v_pool, "v_pool", dtype=k_pool.dtype, device=dev)
    _need(block_tables, "block_tables", dtype=torch.int32, dim=2, device=dev)
    _need(seq_lens, "seq_lens", dtype=torch.int32, dim=1, device=dev)
    nb, hkv, bs, d = k_pool.shape
    B = k.shape[0]
    if (tuple(k.shape) != (B, hkv, d) or tuple(v.shape) != (B, hkv, d) or
            slot_mapping.shape[0] != B or block_tables.shape[0] != B or seq_lens.shape[0] != B):
        raise ValueError("shape mismatch")
    common = (k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(), k_pool.data_ptr(),
              v_pool.data_ptr(), block_tables.data_ptr(), seq_lens.data_ptr(), B,
              block_tables.shape[1], hkv, d, bs, nb)
    if fp8:
        if kv_scales is None:
            raise ValueError("8-bit pools need kv_scales")
        st = lib().pa_append_tokens_e4m3(*common, ctypes.c_float(kv_scales[0]),
                                         ctypes.c_float(kv_scales[1]), _stream_ptr(stream, dev))
    else:
        st = lib().pa_append_tokens(*common, _dtype_code(k_pool), _stream_ptr(stream, dev))
    _check(st, "pa_append_tokens")


def pa_copy_blocks(k_pool, v_pool, pairs, stream=None):
    """Copy whole blocks (src, dst) = pairs[n] in both pools; pairs int64 [N,2]."""
    torch = _torch()
    dev = k_pool.device
    _need(k_pool, "k_pool", dim=4)
    _need(v_pool, "v_pool", dtype=k_pool.dtype, device=dev)
    _need(pairs, "pairs", dtype=torch.int64, device=dev)
    n = pairs.numel() // 2
    block_bytes = k_pool[0].numel() * k_pool.element_size()
    st = lib().pa_copy_blocks(k_pool.data_ptr(), v_pool.data_ptr(), pairs.data_ptr(), n,
                              block_bytes, k_pool.shape[0], _stream_ptr(stream, dev))
    _check(st, "pa_copy_blocks")


def pa_swap_blocks(src_k, src_v, dst_k, dst_v, pairs, stream=None):
    """Move whole blocks (src, dst) = pairs[n] from (src_k, src_v) to (dst_k,
    dst_v); one side is normally a pinned host pool. pairs int64 [N,2] on the
    device; block shapes must match."""
    torch = _torch()
    dev = pairs.device
    for name, t in (("src_k", src_k), ("src_v", src_v), ("dst_k", dst_k), ("dst_v", dst_v)):
        _need(t, name, dim=4)
        if t.device.type == "cpu" and not t.is_pinned():
            raise ValueError(f"{name} is host memory that is not pinned")
    _need(pairs, "pairs", dtype=torch.int64)
    if pairs.device.type != "cuda":
        raise ValueError("pairs must be device memory")
    if (tuple(src_k.shape[1:]) != tuple(dst_k.shape[1:]) or src_k.shape != src_v.shape or
            dst_k.shape != dst_v.shape or src_k.dtype != dst_k.dtype):
        raise ValueError("block shape or dtype mismatch")
    block_bytes = src_k[0].numel() * src_k.element_size()
    st = lib().pa_swap_blocks(src_k.data_ptr(), src_v.data_ptr(), dst_k.data_ptr(),
                              dst_v.data_ptr(), pairs.data_ptr(), pairs.numel() // 2, block_bytes,
                              src_k.shape[0], dst_k.shape[0], _stream_ptr(stream, dev))
    _check(st, "pa_swap_blocks")


def pa_device_errors(stream=None, device=None) -> int:
    """Synchronise the stream and return (and clear) the device error word."""
    torch = _torch()
    dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    flags = ctypes.c_uint32(0)
    st = lib().pa_device_errors(ctypes.byref(flags), _stream_ptr(stream, dev))
    if st not in (0, 7):
        raise PaError(st, "pa_device_errors")
    return int(flags.value)


# --------------------------------------------------------------------------
# Host block manager
# --------------------------------------------------------------------------

class BlockManager:
    """pa_bm_*: free pool, block tables, reference counts, fork, CoW."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        self._l = lib()
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)
        h = ctypes.c_void_p()
        order = None
        if free_order is not None:
            order = np.ascontiguousarray(free_order, dtype=np.int32)
            if order.shape != (num_blocks,):
                raise ValueError("free_order must list every block once")
        st = self._l.pa_bm_create(num_blocks, block_size,
                                  None if order is None else order.ctypes.data, ctypes.byref(h))
        _check(st, "pa_bm_create")
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            self._l.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def add_seq(self, seq_id: int, num_tokens: int) -> None:
        _check(self._l.pa_bm_add_seq(self._h, seq_id, num_tokens), "pa_bm_add_seq")

    def append_slots(self, seq_ids):
        """Returns (slots int64 [n], cow_pairs int64 [k, 2])."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int32)
        n = ids.shape[0]
        slots = np.empty(max(n, 1), dtype=np.int64)
        pairs = np.empty(max(2 * n, 2), dtype=np.int64)
        ncow = ctypes.c_int32(0)
        st = self._l.pa_bm_append_slots(self._h, ids.ctypes.data, n, slots.ctypes.data,
                                        pairs.ctypes.data, ctypes.byref(ncow))
        _check(st, "pa_bm_append_slots")
        return slots[:n], pairs[: 2 * ncow.value].reshape(-1, 2)

    def append_slots_into(self, seq_ids, slots_out, pairs_out) -> int:
        """append_slots writing into caller arrays (e.g. pinned host memory);
        returns the number of copy pairs."""
        ncow = ctypes.c_int32(0)
        st = self._l.pa_bm_append_slots(self._h, seq_ids.ctypes.data, seq_ids.shape[0],
                                        slots_out.ctypes.data, pairs_out.ctypes.data,
                                        ctypes.byref(ncow))
        _check(st, "pa_bm_append_slots")
        return ncow.value

    def fork(self, parent: int, child: int) -> None:
        _check(self._l.pa_bm_fork(self._h, parent, child), "pa_bm_fork")

    def free_seq(self, seq_id: int) -> None:
        _check(self._l.pa_bm_free_seq(self._h, seq_id), "pa_bm_free_seq")

    def export(self, seq_ids, max_blocks: int, tables_out=None, lens_out=None):
        ids = np.ascontiguousarray(seq_ids, dtype=np.int32)
        n = ids.shape[0]
        tab = tables_out if tables_out is not None else np.empty((n, max_blocks), dtype=np.int32)
        lens = lens_out if lens_out is not None else np.empty(n, dtype=np.int32)
        st = self._l.pa_bm_export(self._h, ids.ctypes.data, n, max_blocks, tab.ctypes.data,
                                  lens.ctypes.data)
        _check(st, "pa_bm_export")
        return tab, lens

    def set_swap_space(self, num_cpu_blocks: int) -> None:
        _check(self._l.pa_bm_set_swap_space(self._h, num_cpu_blocks), "pa_bm_set_swap_space")

    def _swap(self, fn, seq_id: int):
        cap = 1 << 16
        pairs = np.empty(2 * cap, dtype=np.int64)
        n = ctypes.c_int32(0)
        _check(getattr(self._l, fn)(self._h, seq_id, pairs.ctypes.data, cap, ctypes.byref(n)), fn)
        return pairs[: 2 * n.value].reshape(-1, 2)

    def swap_out(self, seq_id: int):
        """(device block, swap block) pairs, int64 [k, 2]."""
        return self._swap("pa_bm_swap_out", seq_id)

    def swap_in(self, seq_id: int):
        """(swap block, device block) pairs, int64 [k, 2]."""
        return self._swap("pa_bm_swap_in", seq_id)

    def num_free_swap(self) -> int:
        return int(self._l.pa_bm_num_free_swap(self._h))

    def is_swapped(self, seq_id: int) -> bool:
        v = int(self._l.pa_bm_is_swapped(self._h, seq_id))
        if v < 0:
            raise KeyError(seq_id)
        return bool(v)

    def num_free(self) -> int:
        return int(self._l.pa_bm_num_free(self._h))

    def refcount(self, block: int) -> int:
        return int(self._l.pa_bm_refcount(self._h, block))

    def num_tokens(self, seq_id: int) -> int:
        return int(self._l.pa_bm_num_tokens(self._h, seq_id))
