"""qsa_sparse_prefill_noalloc (the entry point for callers that cannot
allocate) against qsa_sparse_prefill with a caller-owned workspace, through
the C ABI: the same kernels on the same lists, so the outputs must agree bit
for bit, on two calls in a row (the second smaller, so stale scratch contents
from the first would show), and both within the page's gate of the oracle.
Also the refusal of a selection too large for the scratch array."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import qsa_inputs as qi
import top_sparse_attention_amd as qsa
from qsa_testutil import bf16_tensor_to_f32, empty_row_mask, gate, upload

pytestmark = pytest.mark.gpu

DEV = "cuda"


def one_call(case):
    q, k, v, sl = upload(case, DEV)
    out_ref = torch.full_like(q, 3.0)
    out_na = torch.full_like(q, -5.0)
    ws = qsa.new_workspace(case.T, case.W, DEV)
    qsa.sparse_prefill(q, k, v, sl, scale=case.scale, out=out_ref, workspace=ws)
    torch.cuda.synchronize()
    print(f"case {case.name}: T {case.T} W {case.W} S {case.S} heads ({case.Hq},{case.Hkv})",
          flush=True)
    qsa.sparse_prefill_noalloc(q, k, v, sl, scale=case.scale, out=out_na)
    torch.cuda.synchronize()
    assert torch.equal(out_na.view(torch.int16), out_ref.view(torch.int16)), \
        "no-allocation prefill differs from the workspace prefill"
    want = oracle.prefill(case.q, case.k_cache, case.v_cache, case.slot_idx,
                          case.scale if case.scale is not None else 1.0 / 16.0)
    m = gate(bf16_tensor_to_f32(out_na), want, empty_row_mask(case.slot_idx, case.S))
    print(f"  gate {m}", flush=True)


def test_noalloc_matches_the_workspace_prefill_on_two_calls():
    big = qi.random_case(1401, T=300, S=30000, Hq=16, Hkv=2, W=1100, pad_frac=0.2,
                         interior=True)
    big.slot_idx[[3, 77]] = -1                      # fully masked rows
    small = qi.random_case(1402, T=37, S=5000, Hq=12, Hkv=1, W=130, pad_frac=0.1)
    one_call(big)
    one_call(small)


def test_noalloc_refuses_selections_beyond_its_scratch():
    lib = qsa.load_library()
    cap = qsa.noalloc_scratch_bytes()
    assert cap == 64 << 20
    # 8,000 tokens x 2,100 entries need more than 64 MiB of workspace
    T, W = 8000, 2100
    assert qsa.workspace_bytes(T, W) > cap
    q = torch.zeros((T, 2, 256), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((64, 1, 256), dtype=torch.bfloat16, device=DEV)
    sl = torch.full((T, W), -1, dtype=torch.int32, device=DEV)
    out = torch.empty_like(q)
    with pytest.raises(qsa.QsaError) as err:
        qsa.sparse_prefill_noalloc(q, k, k, sl, out=out)
    assert err.value.status == 7 and "scratch" in str(err.value)
