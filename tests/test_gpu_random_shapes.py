"""GPU parity over seeded random shapes: the prefill, the decode path and the
FP8 prefill against the FP32 oracle, under the gate of the page's section
"Nine tests that passed, ..." (empty rows exactly +0.0).

The shapes are drawn once from a fixed seed: 1 to 24 query heads per KV head
(up to 64 with one KV head: up to four head blocks), 1 to 4 KV heads, widths
from 0 to 2,100 with tail or interior -1 padding, caches from a handful of
slots to 20,000, default and explicit scales.  Sizes are capped so that the
oracle finishes each case in about a second.
"""
import numpy as np
import pytest
import torch

import oracle
import qsa_inputs as qi
import top_sparse_attention_amd as qsa
from qsa_testutil import bf16_tensor_to_f32, empty_row_mask, gate, upload, upload_fp8

pytestmark = pytest.mark.gpu

DEV = "cuda"
N_CASES = 16


def draw_cases():
    rng = np.random.Generator(np.random.PCG64(2024))
    cases = []
    while len(cases) < N_CASES:
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.integers(1, 65 if Hkv == 1 else 25))
        Hq = Hkv * G
        if Hq > 64:
            continue
        r = [int(x) for x in rng.integers(2, 2101, size=4)]
        W = int(rng.choice([0, 1, 16, 17] + r))
        T = int(rng.integers(1, 300))
        if T * max(W, 1) * Hq > 12_000_000:
            continue
        pad = float(rng.choice([0.0, 0.2, 0.6, 0.95]))
        n_valid = W - int(round(pad * W))
        S = int(rng.integers(max(n_valid, 1), 20001))
        scale = None if rng.random() < 0.5 else float(rng.uniform(-0.2, 0.3))
        cases.append(dict(seed=3000 + len(cases), T=T, S=S, Hq=Hq, Hkv=Hkv, W=W,
                          pad_frac=pad, interior=bool(rng.random() < 0.5), scale=scale))
    return cases


CASES = draw_cases()


def case_id(c):
    return f"T{c['T']}-S{c['S']}-{c['Hq']}x{c['Hkv']}-W{c['W']}-p{c['pad_frac']}"


def build(c):
    return qi.random_case(c["seed"], T=c["T"], S=c["S"], Hq=c["Hq"], Hkv=c["Hkv"], W=c["W"],
                          scale=c["scale"], pad_frac=c["pad_frac"], interior=c["interior"])


def want_of(case):
    scale = case.scale if case.scale is not None else 1.0 / 16.0
    return oracle.prefill(case.q, case.k_cache, case.v_cache, case.slot_idx, scale)


@pytest.mark.parametrize("c", CASES, ids=case_id)
def test_prefill_and_decode_on_random_shapes(c):
    case = build(c)
    q, k, v, sl = upload(case, DEV)
    want = want_of(case)
    empty = empty_row_mask(case.slot_idx, case.S)
    out = qsa.sparse_prefill(q, k, v, sl, scale=case.scale)
    dec = qsa.sparse_decode(q, k, v, sl, scale=case.scale)
    torch.cuda.synchronize()
    print(case_id(c), "prefill", gate(bf16_tensor_to_f32(out), want, empty), flush=True)
    print(case_id(c), "decode", gate(bf16_tensor_to_f32(dec), want, empty), flush=True)


@pytest.mark.parametrize("c", CASES[::2], ids=case_id)
def test_fp8_prefill_on_random_shapes(c):
    case = qi.with_fp8_kv(build(c))
    q, _, _, sl = upload(case, DEV)
    k8, v8, ks, vs = upload_fp8(case, DEV)
    out = qsa.sparse_prefill_fp8kv(q, k8, v8, ks, vs, sl, scale=case.scale)
    torch.cuda.synchronize()
    scale = case.scale if case.scale is not None else 1.0 / 16.0
    want = oracle.prefill_fp8kv(case.q, case.info["k8"], case.info["v8"], ks, vs, case.slot_idx,
                                scale)
    print(case_id(c), "fp8", gate(bf16_tensor_to_f32(out), want,
                                  empty_row_mask(case.slot_idx, case.S)), flush=True)
