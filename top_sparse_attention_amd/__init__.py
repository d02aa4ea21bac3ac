"""Python binding of libqsa: QSA sparse main-attention prefill on MI355X.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of ``libqsa.so`` (built in-tree by ``_build.py``); torch supplies the
device memory and the current stream.  If the library is missing the calls
raise instead of computing anything some other way.

The operation is the one on the page "Qwen4-Exp QSA comes to Huawei's Ascend:
inside SGLang's opt-in CANN prefill PR" (section "What the pull request
actually adds"): ``out[t,h] = softmax(scale * q[t,h] . k[s]) . v[s]`` over the
slots ``s`` of ``slot_idx[t]`` that are not -1, with query head ``h`` reading
KV head ``h // (Hq // Hkv)``; rows with nothing selected are exactly zero.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

__all__ = [
    "QsaError", "library_path", "load_library", "version", "workspace_bytes",
    "workspace_layout", "new_workspace", "compact_slots", "compacted_lists",
    "sparse_attend", "sparse_prefill", "check_status", "gather_only",
    "compact_slot_range", "partials_bytes", "new_partials", "sparse_attend_partial",
    "merge_partials", "decode_splits", "decode_workspace_bytes", "sparse_decode",
    "sparse_attend_fp8kv", "sparse_prefill_fp8kv", "sparse_decode_fp8kv", "gather_only_fp8kv",
    "compact_blocks", "sparse_prefill_blocks", "indexer_scores", "indexer_select",
    "indexer_topk", "indexer_topk_fused", "indexer_topk_fused_bytes", "indexer_scores_bytes", "stream_read", "sparse_prefill_noalloc", "noalloc_scratch_bytes",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libqsa.so")
HEAD_DIM = 256

QSA_OK = 0
STATUS_NAMES = {
    0: "QSA_OK", 1: "QSA_ERR_NULL", 2: "QSA_ERR_SHAPE", 3: "QSA_ERR_STRIDE",
    4: "QSA_ERR_SCALE", 5: "QSA_ERR_WORKSPACE", 6: "QSA_ERR_SLOT_RANGE",
    7: "QSA_ERR_UNSUPPORTED", 8: "QSA_ERR_HIP", 9: "QSA_ERR_ALIAS",
}


class QsaError(RuntimeError):
    """A non-OK qsa_status; ``status`` holds the code."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class BF16View(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("size", ctypes.c_int64 * 3),
                ("stride", ctypes.c_int64 * 3)]


class I32View(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("size", ctypes.c_int64 * 2),
                ("stride", ctypes.c_int64 * 2)]


class WorkspaceMap(ctypes.Structure):
    _fields_ = [("list_offset", ctypes.c_int64), ("row_stride", ctypes.c_int64),
                ("count_offset", ctypes.c_int64), ("bad_offset", ctypes.c_int64),
                ("share_offset", ctypes.c_int64), ("total_bytes", ctypes.c_int64)]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libqsa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it with `python -m top_sparse_attention_amd._build` "
            "or __graft_entry__.build(); there is no fallback implementation")
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER
    vp, i64, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.qsa_version.restype = ctypes.c_char_p
    lib.qsa_version.argtypes = []
    lib.qsa_status_string.restype = ctypes.c_char_p
    lib.qsa_status_string.argtypes = [ctypes.c_int]
    lib.qsa_last_error.restype = ctypes.c_char_p
    lib.qsa_last_error.argtypes = []
    lib.qsa_workspace_bytes.restype = sz
    lib.qsa_workspace_bytes.argtypes = [i64, i64]
    lib.qsa_sparse_prefill_workspace_bytes.restype = sz
    lib.qsa_sparse_prefill_workspace_bytes.argtypes = [i64, i64]
    lib.qsa_workspace_layout.restype = ctypes.c_int
    lib.qsa_workspace_layout.argtypes = [i64, i64, P(WorkspaceMap)]
    lib.qsa_compact_slots.restype = ctypes.c_int
    lib.qsa_compact_slots.argtypes = [P(I32View), i64, vp, sz, vp]
    lib.qsa_sparse_attend.restype = ctypes.c_int
    lib.qsa_sparse_attend.argtypes = [P(BF16View), P(BF16View), P(BF16View), i64, f32,
                                      vp, sz, P(BF16View), vp]
    lib.qsa_sparse_prefill.restype = ctypes.c_int
    lib.qsa_sparse_prefill.argtypes = [P(BF16View), P(BF16View), P(BF16View), P(I32View),
                                       f32, P(BF16View), vp, sz, vp]
    lib.qsa_check_status.restype = ctypes.c_int
    lib.qsa_check_status.argtypes = [vp, sz, i64, i64, vp, P(i64)]
    lib.qsa_gather_only.restype = ctypes.c_int
    lib.qsa_gather_only.argtypes = [P(BF16View), P(BF16View), i64, i64, vp, sz, vp, vp]
    lib.qsa_compact_slot_range.restype = ctypes.c_int
    lib.qsa_compact_slot_range.argtypes = [P(I32View), i64, i64, i64, vp, sz, vp]
    lib.qsa_partials_bytes.restype = sz
    lib.qsa_partials_bytes.argtypes = [i64, i64, i64]
    lib.qsa_sparse_attend_partial.restype = ctypes.c_int
    lib.qsa_sparse_attend_partial.argtypes = [P(BF16View), P(BF16View), P(BF16View), i64, f32,
                                              vp, sz, ctypes.c_int32, i64, i64, vp, sz, vp]
    lib.qsa_merge_partials.restype = ctypes.c_int
    lib.qsa_merge_partials.argtypes = [vp, sz, i64, i64, i64, P(BF16View), vp]
    lib.qsa_decode_splits.restype = ctypes.c_int32
    lib.qsa_decode_splits.argtypes = [i64, i64, ctypes.c_int32, ctypes.c_int32]
    lib.qsa_decode_workspace_bytes.restype = sz
    lib.qsa_decode_workspace_bytes.argtypes = [i64, i64, ctypes.c_int32, ctypes.c_int32]
    lib.qsa_sparse_decode.restype = ctypes.c_int
    lib.qsa_sparse_decode.argtypes = [P(BF16View), P(BF16View), P(BF16View), P(I32View), f32,
                                      P(BF16View), vp, sz, vp]
    lib.qsa_sparse_attend_fp8kv.restype = ctypes.c_int
    lib.qsa_sparse_attend_fp8kv.argtypes = [P(BF16View), P(BF16View), P(BF16View), f32, f32,
                                            i64, f32, vp, sz, P(BF16View), vp]
    lib.qsa_sparse_prefill_fp8kv.restype = ctypes.c_int
    lib.qsa_sparse_prefill_fp8kv.argtypes = [P(BF16View), P(BF16View), P(BF16View), f32, f32,
                                             P(I32View), f32, P(BF16View), vp, sz, vp]
    lib.qsa_sparse_decode_fp8kv.restype = ctypes.c_int
    lib.qsa_sparse_decode_fp8kv.argtypes = [P(BF16View), P(BF16View), P(BF16View), f32, f32,
                                            P(I32View), f32, P(BF16View), vp, sz, vp]
    lib.qsa_prefill_blocks_workspace_bytes.restype = sz
    lib.qsa_prefill_blocks_workspace_bytes.argtypes = [i64, i64, ctypes.c_int32]
    lib.qsa_compact_blocks.restype = ctypes.c_int
    lib.qsa_compact_blocks.argtypes = [P(I32View), i64, ctypes.c_int32, vp, sz, vp]
    lib.qsa_sparse_prefill_blocks.restype = ctypes.c_int
    lib.qsa_sparse_prefill_blocks.argtypes = [P(BF16View), P(BF16View), P(BF16View), P(I32View),
                                              ctypes.c_int32, f32, P(BF16View), vp, sz, vp]
    lib.qsa_indexer_scores_bytes.restype = sz
    lib.qsa_indexer_scores_bytes.argtypes = [i64, i64]
    lib.qsa_indexer_scores.restype = ctypes.c_int
    lib.qsa_indexer_scores.argtypes = [P(BF16View), P(BF16View), vp, vp, sz, vp]
    lib.qsa_indexer_select.restype = ctypes.c_int
    lib.qsa_indexer_select.argtypes = [vp, sz, i64, i64, vp, vp, i64, ctypes.c_int32,
                                       P(I32View), vp]
    lib.qsa_indexer_topk.restype = ctypes.c_int
    lib.qsa_indexer_topk.argtypes = [P(BF16View), P(BF16View), vp, vp, i64, ctypes.c_int32, vp,
                                     sz, P(I32View), vp]
    lib.qsa_indexer_topk_fused_bytes.restype = sz
    lib.qsa_indexer_topk_fused_bytes.argtypes = [i64, i64]
    lib.qsa_indexer_topk_fused.restype = ctypes.c_int
    lib.qsa_indexer_topk_fused.argtypes = [P(BF16View), P(BF16View), vp, vp, i64, ctypes.c_int32,
                                           vp, sz, P(I32View), vp]
    lib.qsa_noalloc_scratch_bytes.restype = sz
    lib.qsa_noalloc_scratch_bytes.argtypes = []
    lib.qsa_sparse_prefill_noalloc.restype = ctypes.c_int
    lib.qsa_sparse_prefill_noalloc.argtypes = [P(BF16View), P(BF16View), P(BF16View),
                                               P(I32View), f32, P(BF16View), vp]
    lib.qsa_stream_read.restype = ctypes.c_int
    lib.qsa_stream_read.argtypes = [vp, sz, sz, i64, vp, vp]
    lib.qsa_gather_only_fp8kv.restype = ctypes.c_int
    lib.qsa_gather_only_fp8kv.argtypes = [P(BF16View), P(BF16View), i64, i64, vp, sz, vp, vp]
    _lib = lib
    return lib


def _raise_on(status: int) -> None:
    if status != QSA_OK:
        raise QsaError(status, load_library().qsa_last_error().decode())


def version() -> str:
    return load_library().qsa_version().decode()


def _bf16_view(t: torch.Tensor, name: str) -> BF16View:
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if t.dim() != 3:
        raise ValueError(f"{name} must be 3-D, got shape {tuple(t.shape)}")
    if t.numel() and not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    return BF16View(t.data_ptr() if t.numel() else 0, (ctypes.c_int64 * 3)(*t.shape),
                    (ctypes.c_int64 * 3)(*t.stride()))


def _i32_view(t: torch.Tensor, name: str) -> I32View:
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32, got {t.dtype}")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    if t.numel() and not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    return I32View(t.data_ptr() if t.numel() else 0, (ctypes.c_int64 * 2)(*t.shape),
                   (ctypes.c_int64 * 2)(*t.stride()))


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def workspace_bytes(T: int, W: int) -> int:
    return int(load_library().qsa_workspace_bytes(T, W))


def workspace_layout(T: int, W: int) -> dict:
    m = WorkspaceMap()
    _raise_on(load_library().qsa_workspace_layout(T, W, ctypes.byref(m)))
    return {f: getattr(m, f) for f, _ in WorkspaceMap._fields_}


def new_workspace(T: int, W: int, device="cuda") -> torch.Tensor:
    """A uint8 device buffer large enough for T tokens of width W."""
    return torch.empty(max(workspace_bytes(T, W), 1), dtype=torch.uint8, device=device)


def compact_slots(slot_idx: torch.Tensor, S: int,
                  workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Enqueue the validation/compaction pass; returns the workspace."""
    T, W = slot_idx.shape
    if workspace is None:
        workspace = new_workspace(T, W, slot_idx.device)
    sv = _i32_view(slot_idx, "slot_idx")
    _raise_on(load_library().qsa_compact_slots(
        ctypes.byref(sv), S, workspace.data_ptr(), workspace.numel(), _stream(workspace.device)))
    return workspace


def compacted_lists(workspace: torch.Tensor, T: int, W: int):
    """Views of a compacted workspace: (list [T, row_stride], count [T], n_bad [T])."""
    m = workspace_layout(T, W)
    ws32 = workspace.view(torch.int32)
    lst = ws32[m["list_offset"] // 4: m["list_offset"] // 4 + T * m["row_stride"]]
    cnt = ws32[m["count_offset"] // 4: m["count_offset"] // 4 + T]
    bad = ws32[m["bad_offset"] // 4: m["bad_offset"] // 4 + T]
    return lst.view(T, m["row_stride"]), cnt, bad


def _default_scale(scale: Optional[float], D: int) -> float:
    return 1.0 / math.sqrt(D) if scale is None else float(scale)


def sparse_attend(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                  workspace: torch.Tensor, W: int, scale: Optional[float] = None,
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Gather attention over an already compacted workspace."""
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    qv, kv, vv, ov = (_bf16_view(q, "q"), _bf16_view(k_cache, "k_cache"),
                      _bf16_view(v_cache, "v_cache"), _bf16_view(out, "out"))
    _raise_on(load_library().qsa_sparse_attend(
        ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv), W,
        _default_scale(scale, q.shape[-1]), workspace.data_ptr(), workspace.numel(),
        ctypes.byref(ov), _stream(q.device)))
    return out


def sparse_prefill(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   slot_idx: torch.Tensor, scale: Optional[float] = None,
                   out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None,
                   check: bool = False) -> torch.Tensor:
    """QSA sparse prefill: compaction + gather attention, on the current stream.

    q [T, Hq, 256], k_cache/v_cache [S, Hkv, 256] bfloat16 (strided views are
    fine), slot_idx [T, W] int32 with -1 for "no slot".  ``scale`` None means
    1/sqrt(256).  ``check=True`` synchronizes and raises if any entry was
    neither -1 nor a valid slot.
    """
    T, W = slot_idx.shape
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if workspace is None:
        workspace = new_workspace(T, W, q.device)
    qv, kv, vv, ov = (_bf16_view(q, "q"), _bf16_view(k_cache, "k_cache"),
                      _bf16_view(v_cache, "v_cache"), _bf16_view(out, "out"))
    sv = _i32_view(slot_idx, "slot_idx")
    stream = _stream(q.device)
    _raise_on(load_library().qsa_sparse_prefill(
        ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv), ctypes.byref(sv),
        _default_scale(scale, q.shape[-1]), ctypes.byref(ov), workspace.data_ptr(),
        workspace.numel(), stream))
    if check:
        check_status(workspace, T, W)
    return out


def noalloc_scratch_bytes() -> int:
    """Size of the fixed scratch array qsa_sparse_prefill_noalloc works in."""
    return int(load_library().qsa_noalloc_scratch_bytes())


def sparse_prefill_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                           slot_idx: torch.Tensor, scale: Optional[float] = None,
                           out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """sparse_prefill without a workspace argument: the library works in its
    fixed per-GPU scratch array and allocates nothing (calls that overlap on
    one GPU race on that array).  ``out`` must be given to allocate nothing
    here either."""
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    qv, kv, vv, ov = (_bf16_view(q, "q"), _bf16_view(k_cache, "k_cache"),
                      _bf16_view(v_cache, "v_cache"), _bf16_view(out, "out"))
    sv = _i32_view(slot_idx, "slot_idx")
    _raise_on(load_library().qsa_sparse_prefill_noalloc(
        ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv), ctypes.byref(sv),
        _default_scale(scale, q.shape[-1]), ctypes.byref(ov), _stream(q.device)))
    return out


def check_status(workspace: torch.Tensor, T: int, W: int) -> int:
    """Synchronize the current stream and raise QsaError if the last
    compaction into ``workspace`` dropped invalid entries; returns 0."""
    n_bad = ctypes.c_int64(0)
    status = load_library().qsa_check_status(
        workspace.data_ptr(), workspace.numel(), T, W, _stream(workspace.device),
        ctypes.byref(n_bad))
    _raise_on(status)
    return n_bad.value


def gather_only(k_cache: torch.Tensor, v_cache: torch.Tensor, workspace: torch.Tensor,
                T: int, W: int, sink: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Run the gather-only measurement kernel; returns sink [T * Hkv] (int32 bits)."""
    Hkv = k_cache.shape[1]
    if sink is None:
        sink = torch.empty(max(T * Hkv, 1), dtype=torch.int32, device=k_cache.device)
    kv, vv = _bf16_view(k_cache, "k_cache"), _bf16_view(v_cache, "v_cache")
    _raise_on(load_library().qsa_gather_only(
        ctypes.byref(kv), ctypes.byref(vv), T, W, workspace.data_ptr(), workspace.numel(),
        sink.data_ptr(), _stream(k_cache.device)))
    return sink


def stream_read(buf: torch.Tensor, footprint_bytes: int, bytes_per_workgroup: int,
                workgroups: int, sink: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Run the streaming-read measurement kernel over the first
    ``footprint_bytes`` of ``buf``; returns sink [workgroups] (int32 bits)."""
    if footprint_bytes > buf.numel() * buf.element_size():
        raise ValueError("footprint larger than the buffer")
    if sink is None:
        sink = torch.empty(max(workgroups, 1), dtype=torch.int32, device=buf.device)
    _raise_on(load_library().qsa_stream_read(
        buf.data_ptr(), footprint_bytes, bytes_per_workgroup, workgroups, sink.data_ptr(),
        _stream(buf.device)))
    return sink


# ---------------------------------------------------------------- split attention

def compact_slot_range(slot_idx: torch.Tensor, S: int, lo: int, hi: int,
                       workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Compaction for the cache shard [lo, hi): kept slots are stored as slot - lo."""
    T, W = slot_idx.shape
    if workspace is None:
        workspace = new_workspace(T, W, slot_idx.device)
    sv = _i32_view(slot_idx, "slot_idx")
    _raise_on(load_library().qsa_compact_slot_range(
        ctypes.byref(sv), S, lo, hi, workspace.data_ptr(), workspace.numel(),
        _stream(workspace.device)))
    return workspace


def partials_bytes(n_parts: int, T: int, Hq: int) -> int:
    return int(load_library().qsa_partials_bytes(n_parts, T, Hq))


def new_partials(n_parts: int, T: int, Hq: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(partials_bytes(n_parts, T, Hq), 1), dtype=torch.uint8, device=device)


def sparse_attend_partial(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                          workspace: torch.Tensor, W: int, splits: int, part_base: int,
                          n_parts: int, partials: torch.Tensor,
                          scale: Optional[float] = None) -> torch.Tensor:
    """Write `splits` shares of each item into parts [part_base, part_base + splits)."""
    qv, kv, vv = _bf16_view(q, "q"), _bf16_view(k_cache, "k_cache"), _bf16_view(v_cache, "v_cache")
    _raise_on(load_library().qsa_sparse_attend_partial(
        ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv), W,
        _default_scale(scale, q.shape[-1]), workspace.data_ptr(), workspace.numel(),
        splits, part_base, n_parts, partials.data_ptr(), partials.numel(), _stream(q.device)))
    return partials


def merge_partials(partials: torch.Tensor, n_parts: int, T: int, Hq: int,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    if out is None:
        out = torch.empty((T, Hq, HEAD_DIM), dtype=torch.bfloat16, device=partials.device)
    ov = _bf16_view(out, "out")
    _raise_on(load_library().qsa_merge_partials(
        partials.data_ptr(), partials.numel(), n_parts, T, Hq, ctypes.byref(ov),
        _stream(partials.device)))
    return out


def decode_splits(T: int, W: int, Hq: int, Hkv: int) -> int:
    return int(load_library().qsa_decode_splits(T, W, Hq, Hkv))


def decode_workspace_bytes(T: int, W: int, Hq: int, Hkv: int) -> int:
    return int(load_library().qsa_decode_workspace_bytes(T, W, Hq, Hkv))


def sparse_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                  slot_idx: torch.Tensor, scale: Optional[float] = None,
                  out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Sparse attention for few tokens: split attention over the raw selection
    rows (no compaction pass), then the merge."""
    T, W = slot_idx.shape
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if workspace is None:
        nbytes = decode_workspace_bytes(T, W, q.shape[1], k_cache.shape[1])
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    qv, kv, vv, ov = (_bf16_view(q, "q"), _bf16_view(k_cache, "k_cache"),
                      _bf16_view(v_cache, "v_cache"), _bf16_view(out, "out"))
    sv = _i32_view(slot_idx, "slot_idx")
    _raise_on(load_library().qsa_sparse_decode(
        ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv), ctypes.byref(sv),
        _default_scale(scale, q.shape[-1]), ctypes.byref(ov), workspace.data_ptr(),
        workspace.numel(), _stream(q.device)))
    return out


# ---------------------------------------------------------------- FP8 KV cache

def _fp8_view(t: torch.Tensor, name: str) -> BF16View:
    """An FP8 E4M3 cache tensor (uint8 codes or torch.float8_e4m3fn), 3-D.
    qsa_fp8_view has the layout of qsa_bf16_view, so the same struct is used."""
    if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise TypeError(f"{name} must hold FP8 E4M3 codes (uint8 or float8_e4m3fn), got {t.dtype}")
    if t.dim() != 3:
        raise ValueError(f"{name} must be 3-D, got shape {tuple(t.shape)}")
    if t.numel() and not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    return BF16View(t.data_ptr() if t.numel() else 0, (ctypes.c_int64 * 3)(*t.shape),
                    (ctypes.c_int64 * 3)(*t.stride()))


def sparse_attend_fp8kv(q: torch.Tensor, k8: torch.Tensor, v8: torch.Tensor, k_scale: float,
                        v_scale: float, workspace: torch.Tensor, W: int,
                        scale: Optional[float] = None,
                        out: Optional[torch.Tensor] = None) -> torch.Tensor:
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    qv, kv, vv, ov = (_bf16_view(q, "q"), _fp8_view(k8, "k_cache"), _fp8_view(v8, "v_cache"),
                      _bf16_view(out, "out"))
    _raise_on(load_library().qsa_sparse_attend_fp8kv(
        ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv), float(k_scale), float(v_scale), W,
        _default_scale(scale, q.shape[-1]), workspace.data_ptr(), workspace.numel(),
        ctypes.byref(ov), _stream(q.device)))
    return out


def sparse_prefill_fp8kv(q: torch.Tensor, k8: torch.Tensor, v8: torch.Tensor, k_scale: float,
                         v_scale: float, slot_idx: torch.Tensor, scale: Optional[float] = None,
                         out: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Sparse prefill over an FP8 E4M3 KV cache (element = decode(code) * scale)."""
    T, W = slot_idx.shape
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if workspace is None:
        workspace = new_workspace(T, W, q.device)
    qv, kv, vv, ov = (_bf16_view(q, "q"), _fp8_view(k8, "k_cache"), _fp8_view(v8, "v_cache"),
                      _bf16_view(out, "out"))
    sv = _i32_view(slot_idx, "slot_idx")
    _raise_on(load_library().qsa_sparse_prefill_fp8kv(
        ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv), float(k_scale), float(v_scale),
        ctypes.byref(sv), _default_scale(scale, q.shape[-1]), ctypes.byref(ov),
        workspace.data_ptr(), workspace.numel(), _stream(q.device)))
    return out


def sparse_decode_fp8kv(q: torch.Tensor, k8: torch.Tensor, v8: torch.Tensor, k_scale: float,
                        v_scale: float, slot_idx: torch.Tensor, scale: Optional[float] = None,
                        out: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """sparse_decode over an FP8 E4M3 KV cache (element = decode(code) * scale)."""
    T, W = slot_idx.shape
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if workspace is None:
        nbytes = decode_workspace_bytes(T, W, q.shape[1], k8.shape[1])
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    qv, kv, vv, ov = (_bf16_view(q, "q"), _fp8_view(k8, "k_cache"), _fp8_view(v8, "v_cache"),
                      _bf16_view(out, "out"))
    sv = _i32_view(slot_idx, "slot_idx")
    _raise_on(load_library().qsa_sparse_decode_fp8kv(
        ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv), float(k_scale), float(v_scale),
        ctypes.byref(sv), _default_scale(scale, q.shape[-1]), ctypes.byref(ov),
        workspace.data_ptr(), workspace.numel(), _stream(q.device)))
    return out


def gather_only_fp8kv(k8: torch.Tensor, v8: torch.Tensor, workspace: torch.Tensor, T: int,
                      W: int, sink: Optional[torch.Tensor] = None) -> torch.Tensor:
    Hkv = k8.shape[1]
    if sink is None:
        sink = torch.empty(max(T * Hkv, 1), dtype=torch.int32, device=k8.device)
    kv, vv = _fp8_view(k8, "k_cache"), _fp8_view(v8, "v_cache")
    _raise_on(load_library().qsa_gather_only_fp8kv(
        ctypes.byref(kv), ctypes.byref(vv), T, W, workspace.data_ptr(), workspace.numel(),
        sink.data_ptr(), _stream(k8.device)))
    return sink


# ---------------------------------------------------------------- micro-blocks

def compact_blocks(block_idx: torch.Tensor, S: int, block_size: int,
                   workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Compaction of micro-block selections into a workspace of width
    W * block_size (block b = slots b*block_size .. +block_size-1)."""
    T, W = block_idx.shape
    if workspace is None:
        workspace = new_workspace(T, W * block_size, block_idx.device)
    bv = _i32_view(block_idx, "block_idx")
    _raise_on(load_library().qsa_compact_blocks(
        ctypes.byref(bv), S, block_size, workspace.data_ptr(), workspace.numel(),
        _stream(workspace.device)))
    return workspace


def prefill_blocks_workspace_bytes(T: int, W: int, block_size: int) -> int:
    """Workspace bytes for sparse_prefill_blocks with room for the aligned
    block lists (a workspace of workspace_bytes(T, W * block_size) also works,
    with plain lists)."""
    return int(load_library().qsa_prefill_blocks_workspace_bytes(T, W, block_size))


def sparse_prefill_blocks(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                          block_idx: torch.Tensor, block_size: int,
                          scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    T, W = block_idx.shape
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if workspace is None:
        nbytes = prefill_blocks_workspace_bytes(T, W, block_size)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    qv, kv, vv, ov = (_bf16_view(q, "q"), _bf16_view(k_cache, "k_cache"),
                      _bf16_view(v_cache, "v_cache"), _bf16_view(out, "out"))
    bv = _i32_view(block_idx, "block_idx")
    _raise_on(load_library().qsa_sparse_prefill_blocks(
        ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv), ctypes.byref(bv), block_size,
        _default_scale(scale, q.shape[-1]), ctypes.byref(ov), workspace.data_ptr(),
        workspace.numel(), _stream(q.device)))
    return out


# ---------------------------------------------------------------- indexer + Top-K

def _bf16_any(t: torch.Tensor, name: str) -> BF16View:
    if t.dtype != torch.bfloat16 or t.dim() != 3:
        raise TypeError(f"{name} must be a 3-D bfloat16 tensor")
    return BF16View(t.data_ptr() if t.numel() else 0, (ctypes.c_int64 * 3)(*t.shape),
                    (ctypes.c_int64 * 3)(*t.stride()))


def _check_i32_1d(t: torch.Tensor, name: str) -> None:
    if t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous 1-D int32 tensor")


def indexer_scores(iq: torch.Tensor, ik: torch.Tensor, positions: torch.Tensor,
                   scores: Optional[torch.Tensor] = None) -> torch.Tensor:
    """FP32 [T, C] scores sum_h max(0, iq[t,h] . ik[c]); iq [T,4,128], ik [C,1,128]."""
    _check_i32_1d(positions, "positions")
    T, C = iq.shape[0], ik.shape[0]
    if scores is None:
        scores = torch.empty((T, C), dtype=torch.float32, device=iq.device)
    _raise_on(load_library().qsa_indexer_scores(
        ctypes.byref(_bf16_any(iq, "iq")), ctypes.byref(_bf16_any(ik, "ik")),
        positions.data_ptr(), scores.data_ptr(), scores.numel() * 4, _stream(iq.device)))
    return scores


def indexer_select(scores: torch.Tensor, positions: torch.Tensor, slot_of_pos: torch.Tensor,
                   budget: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Top-`budget` complete causal blocks per query, expanded to slots with
    the causal tail: int32 [T, 4*budget + 3], -1 padded."""
    _check_i32_1d(positions, "positions")
    _check_i32_1d(slot_of_pos, "slot_of_pos")
    T, C = scores.shape
    if out is None:
        out = torch.empty((T, 4 * budget + 3), dtype=torch.int32, device=scores.device)
    ov = _i32_view(out, "slot_idx")
    _raise_on(load_library().qsa_indexer_select(
        scores.data_ptr(), scores.numel() * 4, T, C, positions.data_ptr(), slot_of_pos.data_ptr(),
        slot_of_pos.numel(), budget, ctypes.byref(ov), _stream(scores.device)))
    return out


def indexer_scores_bytes(T: int, C: int) -> int:
    """Bytes of the [T, C] float32 scores (the scratch of indexer_topk)."""
    return int(load_library().qsa_indexer_scores_bytes(T, C))


def indexer_topk_fused_bytes(T: int, C: int) -> int:
    """Scratch bytes of indexer_topk_fused."""
    return int(load_library().qsa_indexer_topk_fused_bytes(T, C))


def _topk_call(fn, iq, ik, positions, slot_of_pos, budget, scratch, out):
    _check_i32_1d(positions, "positions")
    _check_i32_1d(slot_of_pos, "slot_of_pos")
    if out is None:
        out = torch.empty((iq.shape[0], 4 * budget + 3), dtype=torch.int32, device=iq.device)
    ov = _i32_view(out, "slot_idx")
    _raise_on(fn(
        ctypes.byref(_bf16_any(iq, "iq")), ctypes.byref(_bf16_any(ik, "ik")),
        positions.data_ptr(), slot_of_pos.data_ptr(), slot_of_pos.numel(), budget,
        scratch.data_ptr(), scratch.numel() * scratch.element_size(), ctypes.byref(ov),
        _stream(iq.device)))
    return out


def indexer_topk(iq: torch.Tensor, ik: torch.Tensor, positions: torch.Tensor,
                 slot_of_pos: torch.Tensor, budget: int, scores: Optional[torch.Tensor] = None,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Indexer scores and Top-K selection in one call.  ``scores`` is the
    [T, C] float32 scratch (allocated when None); it holds the scores
    afterwards."""
    if scores is None:
        scores = torch.empty((iq.shape[0], ik.shape[0]), dtype=torch.float32, device=iq.device)
    return _topk_call(load_library().qsa_indexer_topk, iq, ik, positions, slot_of_pos, budget,
                      scores, out)


def indexer_topk_fused(iq: torch.Tensor, ik: torch.Tensor, positions: torch.Tensor,
                       slot_of_pos: torch.Tensor, budget: int,
                       scratch: Optional[torch.Tensor] = None,
                       out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The same selection without the full score matrix (sampled threshold,
    candidates, exact selection; budgets up to 512).  ``scratch`` is device
    memory of indexer_topk_fused_bytes(T, C) bytes (allocated when None)."""
    if scratch is None:
        scratch = torch.empty(max(indexer_topk_fused_bytes(iq.shape[0], ik.shape[0]), 1),
                              dtype=torch.uint8, device=iq.device)
    return _topk_call(load_library().qsa_indexer_topk_fused, iq, ik, positions, slot_of_pos,
                      budget, scratch, out)
