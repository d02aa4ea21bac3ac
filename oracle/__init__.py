"""Plain FP32 CPU oracle for QSA sparse main-attention prefill.

TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product package never does, and
the two share no code.  The arithmetic lives in ``qsa_oracle.c`` (plain C,
FP32, ``-O2`` without fast-math); this module only builds, loads and
marshals numpy arrays for it.

The page followed is "Qwen4-Exp QSA comes to Huawei's Ascend: inside SGLang's
opt-in CANN prefill PR": the layout-embedding paragraph of section "What the
pull request actually adds" (plain softmax(scale * Q K^T) V over the selected
slots), its "Sizing bounds" bullet (-1 entries, zero output for empty rows) and
section "Nine tests that passed, ..." (FP32 CPU reference from the same BF16
inputs).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qsa_oracle.c")
_LIB = os.path.join(_HERE, "libqsa_oracle.so")

OK, BAD_SLOT, BAD_SHAPE, NO_MEMORY = 0, 1, 2, 3

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with the host C compiler (gcc, -O2, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        lib.qsa_oracle_compact.argtypes = [vp, i64, i64, i64, i64, vp, vp, vp]
        lib.qsa_oracle_compact.restype = ctypes.c_int
        lib.qsa_oracle_prefill.argtypes = [
            vp, i64, i64, vp, i64, i64, vp, i64, i64, vp, i64, i64, i64,
            i32, i32, i32, ctypes.c_float, vp, i64, vp, i32]
        lib.qsa_oracle_prefill.restype = ctypes.c_int
        lib.qsa_oracle_prefill_fp8kv.argtypes = [
            vp, i64, i64, vp, i64, i64, vp, i64, i64, ctypes.c_float, ctypes.c_float,
            vp, i64, i64, i64, i32, i32, i32, ctypes.c_float, vp, i64, vp, i32]
        lib.qsa_oracle_prefill_fp8kv.restype = ctypes.c_int
        lib.qsa_oracle_e4m3_to_float.argtypes = [ctypes.c_uint8]
        lib.qsa_oracle_e4m3_to_float.restype = ctypes.c_float
        lib.qsa_oracle_indexer_scores.argtypes = [vp, i64, i64, vp, i64, i64, i64, i32, i32,
                                                  vp, i32]
        lib.qsa_oracle_indexer_scores.restype = ctypes.c_int
        lib.qsa_oracle_indexer_select.argtypes = [vp, i64, i64, vp, vp, i64, i32, vp]
        lib.qsa_oracle_indexer_select.restype = ctypes.c_int
        lib.qsa_oracle_default_threads.argtypes = []
        lib.qsa_oracle_default_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.__array_interface__["data"][0]


def _elem_strides(a: np.ndarray):
    st = [s // a.itemsize for s in a.strides]
    if any(s * a.itemsize != b for s, b in zip(st, a.strides)):
        raise ValueError("strides must be whole elements")
    return st


def default_threads() -> int:
    return int(_load().qsa_oracle_default_threads())


def compact(slot_idx: np.ndarray, S: int):
    """Stable filter of each selection row.

    Returns ``(lists, counts, n_bad)``: ``lists[t][:counts[t]]`` are the
    entries of row t that lie in [0, S), in their original order; ``n_bad[t]``
    counts entries that are neither -1 nor a valid slot.
    """
    if slot_idx.dtype != np.int32 or slot_idx.ndim != 2:
        raise TypeError("slot_idx must be a 2-D int32 array")
    T, W = slot_idx.shape
    st = _elem_strides(slot_idx)
    if W > 1 and st[1] != 1:
        raise ValueError("slot_idx rows must be contiguous")
    lists = np.full((T, max(W, 1)), -1, dtype=np.int32)
    counts = np.zeros(T, dtype=np.int64)
    n_bad = np.zeros(T, dtype=np.int64)
    rc = _load().qsa_oracle_compact(_ptr(slot_idx), st[0], T, W, S,
                                    _ptr(lists), _ptr(counts), _ptr(n_bad))
    if rc != OK:
        raise ValueError(f"oracle compact failed with status {rc}")
    return lists[:, :W], counts, n_bad


def expand_blocks(block_idx: np.ndarray, block_size: int) -> np.ndarray:
    """Micro-block selections as slot selections: entry b becomes the slots
    b*block_size .. b*block_size + block_size - 1, in that order; -1 stays
    -1 (block_size copies); other negative entries stay invalid."""
    b = np.asarray(block_idx, dtype=np.int64)
    offs = np.arange(block_size, dtype=np.int64)
    slots = np.where(b[..., None] >= 0, b[..., None] * block_size + offs, b[..., None])
    # an invalid negative entry other than -1 must remain invalid after expansion
    slots = np.where((b[..., None] < -1), -2, slots)
    return slots.reshape(b.shape[0], -1).astype(np.int32)


def prefill_blocks(q, k_cache, v_cache, block_idx, block_size, scale, rows=None, nthreads=0):
    """FP32 sparse prefill where each selection entry names a micro-block of
    block_size consecutive cache slots (reading: block b = slots
    b*block_size .. b*block_size + block_size - 1)."""
    return prefill(q, k_cache, v_cache, expand_blocks(block_idx, block_size), scale, rows=rows,
                   nthreads=nthreads)


def e4m3_to_float(code: int) -> float:
    """The oracle's decoding of one FP8 E4M3 byte."""
    return float(_load().qsa_oracle_e4m3_to_float(int(code)))


def prefill(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
            slot_idx: np.ndarray, scale: float, rows=None,
            nthreads: int = 0) -> np.ndarray:
    """FP32 sparse prefill for token ``rows`` (default: all tokens).

    q is [T, Hq, D], k_cache/v_cache are [S, Hkv, D], all numpy views of
    uint16 BF16 bit patterns with unit innermost stride (other strides free);
    slot_idx is [T, W] int32 with -1 meaning "no slot".  ``scale`` must be
    given explicitly.  Returns float32 [len(rows), Hq, D].
    """
    return _prefill(q, k_cache, v_cache, slot_idx, scale, rows, nthreads, None)


def prefill_fp8kv(q: np.ndarray, k8: np.ndarray, v8: np.ndarray, k_scale: float,
                  v_scale: float, slot_idx: np.ndarray, scale: float, rows=None,
                  nthreads: int = 0) -> np.ndarray:
    """FP32 sparse prefill with an FP8 E4M3 KV cache: k8/v8 are [S, Hkv, D]
    uint8 codes meaning decode(code) * k_scale (resp. v_scale)."""
    return _prefill(q, k8, v8, slot_idx, scale, rows, nthreads, (k_scale, v_scale))


def _prefill(q, k_cache, v_cache, slot_idx, scale, rows, nthreads, fp8_scales):
    kv_dtype = np.uint16 if fp8_scales is None else np.uint8
    for name, a, dt in (("q", q, np.uint16), ("k_cache", k_cache, kv_dtype),
                        ("v_cache", v_cache, kv_dtype)):
        if a.dtype != dt or a.ndim != 3:
            raise TypeError(f"{name} must be a 3-D {np.dtype(dt).name} array")
        if a.shape[2] > 1 and a.strides[2] != a.itemsize:
            raise ValueError(f"{name} must have unit stride over D")
    if slot_idx.dtype != np.int32 or slot_idx.ndim != 2:
        raise TypeError("slot_idx must be a 2-D int32 array")
    T, Hq, D = q.shape
    S, Hkv, Dk = k_cache.shape
    if v_cache.shape != k_cache.shape or Dk != D:
        raise ValueError("cache shapes disagree")
    if slot_idx.shape[0] != T:
        raise ValueError("slot_idx must have one row per token")
    W = slot_idx.shape[1]
    if W > 1 and slot_idx.strides[1] != 4:
        raise ValueError("slot_idx rows must be contiguous")
    if rows is None:
        rows_arr = np.arange(T, dtype=np.int64)
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        if rows_arr.size and (rows_arr.min() < 0 or rows_arr.max() >= T):
            raise IndexError("row index out of range")
    out = np.empty((rows_arr.size, Hq, D), dtype=np.float32)
    qs, ks, vs, ss = (_elem_strides(a) for a in (q, k_cache, v_cache, slot_idx))
    if fp8_scales is None:
        rc = _load().qsa_oracle_prefill(
            _ptr(q), qs[0], qs[1], _ptr(k_cache), ks[0], ks[1],
            _ptr(v_cache), vs[0], vs[1], _ptr(slot_idx), ss[0], S, W,
            Hq, Hkv, D, float(scale), _ptr(rows_arr), rows_arr.size, _ptr(out),
            int(nthreads))
    else:
        rc = _load().qsa_oracle_prefill_fp8kv(
            _ptr(q), qs[0], qs[1], _ptr(k_cache), ks[0], ks[1],
            _ptr(v_cache), vs[0], vs[1], float(fp8_scales[0]), float(fp8_scales[1]),
            _ptr(slot_idx), ss[0], S, W, Hq, Hkv, D, float(scale), _ptr(rows_arr),
            rows_arr.size, _ptr(out), int(nthreads))
    if rc == BAD_SLOT:
        raise ValueError("slot_idx holds an entry that is neither -1 nor in [0, S)")
    if rc != OK:
        raise ValueError(f"oracle prefill failed with status {rc}")
    return out


def indexer_scores(iq: np.ndarray, ik: np.ndarray, nthreads: int = 0) -> np.ndarray:
    """score[t, c] = sum_h max(0, iq[t,h] . ik[c]) in FP32.  iq is [T, H, D] and
    ik [C, D] (or [C, 1, D]), both uint16 BF16 bits with unit inner stride."""
    if ik.ndim == 3:
        ik = ik[:, 0, :]
    if iq.dtype != np.uint16 or ik.dtype != np.uint16 or iq.ndim != 3 or ik.ndim != 2:
        raise TypeError("iq must be [T, H, D] and ik [C, D] uint16 (bf16 bits)")
    T, H, D = iq.shape
    C = ik.shape[0]
    if ik.shape[1] != D:
        raise ValueError("head dims disagree")
    out = np.empty((T, C), dtype=np.float32)
    qs, ks = _elem_strides(iq), _elem_strides(ik)
    if (D > 1 and (qs[2] != 1 or ks[1] != 1)):
        raise ValueError("unit inner stride required")
    rc = _load().qsa_oracle_indexer_scores(_ptr(iq), qs[0], qs[1], _ptr(ik), ks[0], T, C, H, D,
                                           _ptr(out), int(nthreads))
    if rc != OK:
        raise ValueError(f"oracle indexer scores failed with status {rc}")
    return out


def indexer_select(scores: np.ndarray, positions: np.ndarray, slot_of_pos: np.ndarray,
                   budget: int) -> np.ndarray:
    """Top-`budget` complete causal blocks per query (ties to the lower block),
    expanded to slots with the causal tail; returns int32 [T, 4*budget + 3]."""
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    positions = np.ascontiguousarray(positions, dtype=np.int32)
    slot_of_pos = np.ascontiguousarray(slot_of_pos, dtype=np.int32)
    T, C = scores.shape
    out = np.empty((T, 4 * budget + 3), dtype=np.int32)
    rc = _load().qsa_oracle_indexer_select(_ptr(scores), T, C, _ptr(positions),
                                           _ptr(slot_of_pos), slot_of_pos.size, int(budget),
                                           _ptr(out))
    if rc != OK:
        raise ValueError(f"oracle indexer select failed with status {rc}")
    return out
