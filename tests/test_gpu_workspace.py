"""The workspace's extent words on the GPU, through the C ABI.

The compaction records how many cache slots its lists index; an attention
over K/V views of fewer slots must not read through those lists (its gathers
would leave the views).  It writes zero rows instead and qsa_check_status
reports the mismatch; the next compaction (or decode step) clears it.  Also
the gather-only measurement kernel over an empty cache, which has no row a
stand-in slot could read.
"""
import numpy as np
import pytest
import torch

import oracle
import qsa_inputs as qi
import top_sparse_attention_amd as qsa
from qsa_testutil import bf16_tensor_to_f32, empty_row_mask, gate, upload

pytestmark = pytest.mark.gpu

DEV = "cuda"


def test_lists_for_a_larger_cache_are_refused_and_reported():
    case = qi.random_case(1301, T=40, S=2000, Hq=8, Hkv=2, W=300)
    q, k, v, sl = upload(case, DEV)
    ws = qsa.compact_slots(sl, case.S)
    out = torch.full_like(q, 7.0)
    qsa.sparse_attend(q, k[:1000], v[:1000], ws, case.W, out=out)
    torch.cuda.synchronize()
    assert torch.all(out.view(torch.int16) == 0), "refused lists must give +0.0 rows"
    with pytest.raises(qsa.QsaError) as err:
        qsa.check_status(ws, case.T, case.W)
    assert err.value.status == 5                    # QSA_ERR_WORKSPACE
    print(f"refused: {err.value}", flush=True)
    # the same views after a compaction for their own size: normal results
    sel = np.where(case.slot_idx < 1000, case.slot_idx, -1).astype(np.int32)
    sl2 = torch.from_numpy(sel).to(DEV)
    qsa.compact_slots(sl2, 1000, ws)
    out = qsa.sparse_attend(q, k[:1000], v[:1000], ws, case.W)
    torch.cuda.synchronize()
    assert qsa.check_status(ws, case.T, case.W) == 0
    want = oracle.prefill(case.q, case.k_cache, case.v_cache, sel, 1.0 / 16.0)
    m = gate(bf16_tensor_to_f32(out), want, empty_row_mask(sel, 1000))
    print(f"after recompaction: {m}", flush=True)


def test_shard_views_must_cover_the_shard():
    case = qi.random_case(1302, T=24, S=3000, Hq=4, Hkv=1, W=500)
    q, k, v, sl = upload(case, DEV)
    ws = qsa.compact_slot_range(sl, case.S, 1000, 2500)
    parts = qsa.new_partials(1, case.T, case.Hq, DEV)
    qsa.sparse_attend_partial(q, k[1000:2500], v[1000:2500], ws, case.W, 1, 0, 1, parts)
    torch.cuda.synchronize()
    assert qsa.check_status(ws, case.T, case.W) == 0
    qsa.sparse_attend_partial(q, k[1000:2000], v[1000:2000], ws, case.W, 1, 0, 1, parts)
    out = qsa.merge_partials(parts, 1, case.T, case.Hq)
    torch.cuda.synchronize()
    assert torch.all(out.view(torch.int16) == 0), "an empty share merges to +0.0"
    with pytest.raises(qsa.QsaError):
        qsa.check_status(ws, case.T, case.W)


def test_decode_clears_the_flag():
    case = qi.random_case(1303, T=4, S=5000, Hq=16, Hkv=2, W=256)
    q, k, v, sl = upload(case, DEV)
    nbytes = qsa.decode_workspace_bytes(case.T, case.W, case.Hq, case.Hkv)
    dws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    qsa.compact_slots(sl, case.S, dws)
    qsa.sparse_attend(q, k[:100], v[:100], dws, case.W)
    torch.cuda.synchronize()
    with pytest.raises(qsa.QsaError):
        qsa.check_status(dws, case.T, case.W)
    out = qsa.sparse_decode(q, k, v, sl, workspace=dws)
    torch.cuda.synchronize()
    assert qsa.check_status(dws, case.T, case.W) == 0
    want = oracle.prefill(case.q, case.k_cache, case.v_cache, case.slot_idx, 1.0 / 16.0)
    gate(bf16_tensor_to_f32(out), want, empty_row_mask(case.slot_idx, case.S))


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_gather_only_over_an_empty_cache(kv):
    T, Hkv, W = 9, 2, 40
    sel = np.full((T, W), -1, dtype=np.int32)
    sel[::2, :3] = [5, 0, 7]                    # invalid for S = 0: dropped and counted
    sl = torch.from_numpy(sel).to(DEV)
    if kv == "bf16":
        k = torch.empty((0, Hkv, 256), dtype=torch.bfloat16, device=DEV)
        gather = qsa.gather_only
    else:
        k = torch.empty((0, Hkv, 256), dtype=torch.uint8, device=DEV)
        gather = qsa.gather_only_fp8kv
    v = torch.empty_like(k)
    ws = qsa.compact_slots(sl, 0)
    sink = torch.full((T * Hkv,), 12345, dtype=torch.int32, device=DEV)
    gather(k, v, ws, T, W, sink)
    torch.cuda.synchronize()
    assert torch.all(sink == 0)
    with pytest.raises(qsa.QsaError) as err:     # 5 rows x 3 entries outside [0, 0)
        qsa.check_status(ws, T, W)
    assert err.value.status == 6 and "15 selection entries" in str(err.value)
