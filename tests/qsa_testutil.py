"""Helpers shared by the GPU tests, the smoke check and the benchmark.

The gate is the one the page "Qwen4-Exp QSA comes to Huawei's Ascend: inside
SGLang's opt-in CANN prefill PR" states in section "Nine tests that passed,
...": atol = 0.025, rtol = 0.025 (elementwise |y - r| <= atol + rtol |r|),
relative L2 error below 0.008, and rows with nothing selected exactly zero.
"""
from __future__ import annotations

import numpy as np

ATOL = 0.025
RTOL = 0.025
REL_L2_MAX = 0.008


def upload(case, device="cuda"):
    """Copy a qsa_inputs.Case to the GPU keeping every view's strides.

    Returns torch views (q, k_cache, v_cache, slot_idx).
    """
    import torch

    dev = {}
    for b in case.bases.values():
        if b.dtype == np.uint16:
            dev[id(b)] = torch.from_numpy(b.view(np.int16)).to(device).view(torch.bfloat16)
        else:
            dev[id(b)] = torch.from_numpy(b).to(device)

    def view_of(arr):
        base = case.base_of(arr)
        off_bytes = arr.__array_interface__["data"][0] - base.__array_interface__["data"][0]
        return torch.as_strided(dev[id(base)], arr.shape,
                                [s // arr.itemsize for s in arr.strides],
                                off_bytes // arr.itemsize)

    return view_of(case.q), view_of(case.k_cache), view_of(case.v_cache), view_of(case.slot_idx)


def upload_fp8(case, device="cuda"):
    """The FP8 K/V codes of a case made by qsa_inputs.with_fp8_kv, as uint8
    device views with the same strides.  Returns (k8, v8, k_scale, v_scale)."""
    import torch

    out = []
    for name in ("k", "v"):
        base, view = case.info[f"{name}8_base"], case.info[f"{name}8"]
        dev = torch.from_numpy(np.ascontiguousarray(base)).to(device)
        off = view.__array_interface__["data"][0] - base.__array_interface__["data"][0]
        out.append(torch.as_strided(dev, view.shape, list(view.strides), off))
    return out[0], out[1], case.info["k_scale"], case.info["v_scale"]


def bf16_tensor_to_f32(t) -> np.ndarray:
    """A (CPU or GPU) torch bfloat16 tensor as float32 numpy."""
    return t.detach().float().cpu().numpy()


def bf16_tensor_bits(t) -> np.ndarray:
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def gate(got: np.ndarray, want: np.ndarray, empty_rows: np.ndarray) -> dict:
    """Apply the page's gate to GPU output `got` (float32 from bf16) against
    oracle output `want` (float32), both [R, Hq, D].  `empty_rows` [R] marks
    rows with nothing selected, which must be exactly +0.0.  Returns metrics and
    raises AssertionError on failure."""
    assert got.shape == want.shape
    full = ~empty_rows
    metrics = {"rows": int(got.shape[0]), "empty_rows": int(empty_rows.sum())}
    if empty_rows.any():
        e = got[empty_rows]
        assert np.all(e == 0) and not np.any(np.signbit(e)), "empty rows must be exactly +0.0"
    if full.any():
        y = got[full].astype(np.float64)
        r = want[full].astype(np.float64)
        assert np.all(np.isfinite(y)), "non-finite output"
        err = np.abs(y - r)
        bound = ATOL + RTOL * np.abs(r)
        worst = float((err - bound).max())
        rel = float(np.linalg.norm(err.ravel()) / max(np.linalg.norm(r.ravel()), 1e-300))
        metrics.update(max_abs_err=float(err.max()), rel_l2=rel, worst_margin=worst)
        assert worst <= 0, f"elementwise gate failed: max excess {worst:.3g}"
        assert rel < REL_L2_MAX, f"relative L2 {rel:.4g} >= {REL_L2_MAX}"
    return metrics


def empty_row_mask(slot_idx: np.ndarray, S: int, rows=None) -> np.ndarray:
    sel = slot_idx if rows is None else slot_idx[rows]
    return ~np.any((sel >= 0) & (sel < S), axis=1)
