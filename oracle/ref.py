"""ctypes wrapper of the plain-C float64 oracle (test infrastructure only)."""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import LIB, build

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        lib = ctypes.CDLL(LIB)
        lib.pa_oracle_decode.restype = ctypes.c_int
        lib.pa_oracle_decode.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_int]
        lib.pa_oracle_decode_e4m3.restype = ctypes.c_int
        lib.pa_oracle_decode_e4m3.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_float,
            ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_int]
        lib.pa_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return _load().pa_oracle_max_threads()


def decode(q, k_pool, v_pool, block_tables, seq_lens, scale, dtype, num_threads=0):
    """Same contract as pa_oracle.decode(); inputs in storage form (float32
    arrays, or uint16 bf16 bit patterns). Returns float64 [B, Hq, D]."""
    lib = _load()
    want = np.float32 if dtype == "f32" else np.uint16
    q = np.ascontiguousarray(q).view(want) if dtype == "bf16" else np.ascontiguousarray(q, dtype=want)
    k_pool = np.ascontiguousarray(k_pool)
    v_pool = np.ascontiguousarray(v_pool)
    if dtype == "bf16":
        k_pool, v_pool = k_pool.view(np.uint16), v_pool.view(np.uint16)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    B, hq, d = q.shape
    nb, hkv, bs, d2 = k_pool.shape
    assert d == d2 and v_pool.shape == k_pool.shape and bt.shape[0] == B and sl.shape == (B,)
    out = np.zeros((B, hq, d), dtype=np.float64)
    rc = lib.pa_oracle_decode(
        q.ctypes.data, k_pool.ctypes.data, v_pool.ctypes.data, 0 if dtype == "f32" else 1,
        bt.ctypes.data, bt.shape[1], sl.ctypes.data, B, hq, hkv, d, bs, nb,
        ctypes.c_float(scale), out.ctypes.data, int(num_threads))
    if rc != 0:
        raise RuntimeError(f"pa_oracle_decode failed: {rc}")
    return out


def decode_e4m3(q, k_codes, v_codes, k_scale, v_scale, block_tables, seq_lens, scale,
                num_threads=0):
    """pa_oracle.decode over 8-bit pools: q as uint16 bf16 bit patterns
    [B, Hq, D], pools of FP8 E4M3 codes (uint8) read as code value times their
    pool's float32 scale. Returns float64 [B, Hq, D]."""
    lib = _load()
    q = np.ascontiguousarray(q).view(np.uint16)
    k_codes = np.ascontiguousarray(k_codes, dtype=np.uint8)
    v_codes = np.ascontiguousarray(v_codes, dtype=np.uint8)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    B, hq, d = q.shape
    nb, hkv, bs, d2 = k_codes.shape
    assert d == d2 and v_codes.shape == k_codes.shape and bt.shape[0] == B and sl.shape == (B,)
    out = np.zeros((B, hq, d), dtype=np.float64)
    rc = lib.pa_oracle_decode_e4m3(
        q.ctypes.data, k_codes.ctypes.data, v_codes.ctypes.data, ctypes.c_float(k_scale),
        ctypes.c_float(v_scale), bt.ctypes.data, bt.shape[1], sl.ctypes.data, B, hq, hkv, d, bs,
        nb, ctypes.c_float(scale), out.ctypes.data, int(num_threads))
    if rc != 0:
        raise RuntimeError(f"pa_oracle_decode_e4m3 failed: {rc}")
    return out
