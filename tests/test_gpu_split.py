"""GPU parity of split attention: qsa_sparse_attend_partial + qsa_merge_partials,
qsa_sparse_decode, and a cache sharded by slot ranges (the context-parallel
layout of the decode work named in section "Where this sits in the Qwen4Exp
serving build-out" of the page "Qwen4-Exp QSA comes to Huawei's Ascend",
rehearsed on one GPU).  Same gate as every floating-point test.
"""
import numpy as np
import pytest
import torch

import oracle
import qsa_inputs as qi
import top_sparse_attention_amd as qsa
from qsa_testutil import bf16_tensor_bits, bf16_tensor_to_f32, empty_row_mask, gate, upload

pytestmark = pytest.mark.gpu

DEV = "cuda"


def oracle_rows(case, rows=None):
    scale = case.scale if case.scale is not None else 1.0 / 16.0
    return oracle.prefill(case.q, case.k_cache, case.v_cache, case.slot_idx, scale, rows=rows)


def check(case, got, rows=None):
    want = oracle_rows(case, rows)
    g = bf16_tensor_to_f32(got if rows is None else got[torch.as_tensor(rows, device=DEV)])
    m = gate(g, want, empty_row_mask(case.slot_idx, case.S, rows))
    print(f"{case.name}: {m}", flush=True)
    return m


def test_decode_batch_workload():
    case = qi.decode_batch()
    q, k, v, sl = upload(case, DEV)
    assert qsa.decode_splits(case.T, case.W, case.Hq, case.Hkv) == 16
    out = qsa.sparse_decode(q, k, v, sl)
    torch.cuda.synchronize()
    check(case, out)


@pytest.mark.parametrize("T,Hq,Hkv,W,pad", [(1, 16, 2, 2048, 0.0), (2, 24, 2, 300, 0.3),
                                           (5, 12, 1, 2051, 0.5), (3, 40, 2, 100, 0.0),
                                           (7, 3, 1, 17, 0.2), (1, 6, 1, 1, 0.0)])
def test_decode_small_batches(T, Hq, Hkv, W, pad):
    case = qi.random_case(800 + T * 7 + W, T=T, S=20000, Hq=Hq, Hkv=Hkv, W=W, pad_frac=pad,
                          interior=True)
    q, k, v, sl = upload(case, DEV)
    out = qsa.sparse_decode(q, k, v, sl, scale=case.scale)
    torch.cuda.synchronize()
    check(case, out)


def test_decode_empty_rows_and_zero_width_are_exact_zero():
    case = qi.random_case(820, T=6, S=999, Hq=8, Hkv=1, W=50)
    case.slot_idx[[1, 4]] = -1
    q, k, v, sl = upload(case, DEV)
    out = qsa.sparse_decode(q, k, v, sl)
    torch.cuda.synchronize()
    check(case, out)
    assert torch.all(out[[1, 4]].view(torch.int16) == 0)
    case0 = qi.random_case(821, T=3, S=64, Hq=4, Hkv=2, W=0)
    q, k, v, sl = upload(case0, DEV)
    out = qsa.sparse_decode(q, k, v, sl)
    torch.cuda.synchronize()
    assert torch.all(out.view(torch.int16) == 0)


def test_decode_single_slot_is_bit_exact():
    case = qi.random_case(822, T=4, S=3000, Hq=24, Hkv=2, W=300, pad_frac=299 / 300,
                          interior=True)
    q, k, v, sl = upload(case, DEV)
    out = qsa.sparse_decode(q, k, v, sl)
    torch.cuda.synchronize()
    bits = bf16_tensor_bits(out)
    for t in range(case.T):
        (s,) = case.slot_idx[t][case.slot_idx[t] != -1]
        for h in range(case.Hq):
            np.testing.assert_array_equal(bits[t, h], case.v_cache[s, h // 12])


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 64, 200])
def test_any_split_count_merges_to_the_same_attention(splits):
    """splits beyond the tile count leave some shares empty."""
    case = qi.random_case(830 + splits, T=9, S=5000, Hq=16, Hkv=2, W=700, pad_frac=0.2,
                          interior=True)
    q, k, v, sl = upload(case, DEV)
    ws = qsa.compact_slots(sl, case.S)
    parts = qsa.new_partials(splits, case.T, case.Hq, DEV)
    qsa.sparse_attend_partial(q, k, v, ws, case.W, splits, 0, splits, parts, scale=case.scale)
    out = qsa.merge_partials(parts, splits, case.T, case.Hq)
    torch.cuda.synchronize()
    check(case, out)


def test_merge_of_all_empty_parts_is_exact_zero():
    T, Hq, n = 5, 6, 3
    parts = qsa.new_partials(n, T, Hq, DEV)
    nbytes = T * Hq * n * 256 * 4
    ml_off = (nbytes + 255) // 256 * 256
    f = parts.view(torch.float32)
    f[: nbytes // 4] = 123.0
    ml = f[ml_off // 4: ml_off // 4 + n * T * Hq * 2].view(n, T, Hq, 2)
    ml[..., 0] = -float("inf")
    ml[..., 1] = 0.0
    out = qsa.merge_partials(parts, n, T, Hq)
    torch.cuda.synchronize()
    assert torch.all(out.view(torch.int16) == 0)


@pytest.mark.parametrize("bounds", [(0.5,), (0.25, 0.3, 0.9), (0.0, 0.999)])
def test_cache_sharded_by_slot_ranges(bounds):
    """Each shard sees only its slot range through a view of the cache that
    starts at its first slot; the merged shares equal the unsharded attention."""
    case = qi.random_case(840 + len(bounds), T=33, S=12000, Hq=16, Hkv=2, W=900,
                          pad_frac=0.1, interior=True)
    q, k, v, sl = upload(case, DEV)
    cuts = [0] + [int(b * case.S) for b in bounds] + [case.S]
    n = len(cuts) - 1
    parts = qsa.new_partials(n, case.T, case.Hq, DEV)
    for i in range(n):
        lo, hi = cuts[i], cuts[i + 1]
        ws = qsa.compact_slot_range(sl, case.S, lo, hi)
        qsa.sparse_attend_partial(q, k[lo:hi], v[lo:hi], ws, case.W, 1, i, n, parts,
                                  scale=case.scale)
    out = qsa.merge_partials(parts, n, case.T, case.Hq)
    torch.cuda.synchronize()
    check(case, out)
    whole = qsa.sparse_prefill(q, k, v, sl, scale=case.scale)
    torch.cuda.synchronize()
    gate(bf16_tensor_to_f32(out), bf16_tensor_to_f32(whole), np.zeros(case.T, dtype=bool))


def _partials_views(parts, n, T, Hq):
    """The O [n, T, Hq, 256] and (m, l) [n, T, Hq, 2] float32 views of a
    partials buffer (the (m, l) block starts at the next 256-byte boundary)."""
    o_bytes = n * T * Hq * 256 * 4
    ml_off = (o_bytes + 255) // 256 * 256
    o = parts[:o_bytes].view(torch.float32).view(n, T, Hq, 256)
    ml = parts[ml_off:ml_off + n * T * Hq * 8].view(torch.float32).view(n, T, Hq, 2)
    return o, ml


@pytest.mark.parametrize("splits", [1, 3, 70, 260])
def test_merge_kernels_agree_bit_for_bit(splits):
    """Merges of 4,096 rows or more run one wave per row; smaller ones a
    four-wave workgroup per row.  Both add the same terms in the same order:
    the 4,096-row merge equals, bit for bit, the merges of its 64-token
    slices (1,024 rows each).  260 parts take more than one round of 64
    weights per part sequence; empty shares (max -inf) occur at every count."""
    case = qi.random_case(870 + splits, T=256, S=8000, Hq=16, Hkv=2, W=1200, pad_frac=0.3,
                          interior=True)
    T, Hq = case.T, case.Hq
    q, k, v, sl = upload(case, DEV)
    ws = qsa.compact_slots(sl, case.S)
    parts = qsa.new_partials(splits, T, Hq, DEV)
    qsa.sparse_attend_partial(q, k, v, ws, case.W, splits, 0, splits, parts, scale=case.scale)
    full = qsa.merge_partials(parts, splits, T, Hq)
    po, pml = _partials_views(parts, splits, T, Hq)
    for t0 in range(0, T, 64):
        cp = qsa.new_partials(splits, 64, Hq, DEV)
        co, cml = _partials_views(cp, splits, 64, Hq)
        co.copy_(po[:, t0:t0 + 64])
        cml.copy_(pml[:, t0:t0 + 64])
        sliced = qsa.merge_partials(cp, splits, 64, Hq)
        torch.cuda.synchronize()
        assert torch.equal(sliced.view(torch.int16), full[t0:t0 + 64].view(torch.int16)), t0
    check(case, full)


def test_shard_compaction_keeps_local_numbering():
    case = qi.random_case(850, T=20, S=3000, Hq=2, Hkv=1, W=200, pad_frac=0.1, interior=True)
    case.slot_idx[3, 5] = 3000          # invalid everywhere
    _, _, _, sl = upload(case, DEV)
    lo, hi = 1000, 2200
    ws = qsa.compact_slot_range(sl, case.S, lo, hi)
    torch.cuda.synchronize()
    lst, cnt, bad = (x.cpu().numpy() for x in qsa.compacted_lists(ws, case.T, case.W))
    for t in range(case.T):
        row = case.slot_idx[t]
        mine = sorted(int(s) - lo for s in row if lo <= s < hi)
        assert cnt[t] == len(mine)
        assert sorted(lst[t, :cnt[t]].tolist()) == mine
        assert bad[t] == (1 if t == 3 else 0)


def test_split_path_on_the_long_prefill_sampled_rows():
    case = qi.long_prefill()
    q, k, v, sl = upload(case, DEV)
    ws = qsa.compact_slots(sl, case.S)
    parts = qsa.new_partials(3, case.T, case.Hq, DEV)
    qsa.sparse_attend_partial(q, k, v, ws, case.W, 3, 0, 3, parts)
    out = qsa.merge_partials(parts, 3, case.T, case.Hq)
    torch.cuda.synchronize()
    rows = qi.sample_rows(case.T, 32)
    check(case, out, rows)
    assert torch.isfinite(out.float()).all()


def test_decode_drops_and_counts_invalid_entries():
    """The decode shares read the selection rows themselves: entries that are
    neither -1 nor in [0, S) are dropped (the result equals the attention over
    the valid entries) and their number reaches qsa_check_status."""
    case = qi.random_case(830, T=8, S=5000, Hq=8, Hkv=1, W=300, pad_frac=0.1, interior=True)
    # Token 0 starts with 40 padding entries: the first tiles of several shares
    # hold no valid row, ahead of tiles that do.
    case.slot_idx[0, :40] = -1
    rng = np.random.Generator(np.random.PCG64(831))
    bad_pos = np.stack([rng.choice(300, size=3, replace=False) for _ in range(case.T)])
    raw = case.slot_idx.copy()
    for t in range(case.T):
        raw[t, bad_pos[t]] = [5000, -7, 1 << 30]
    valid_only = np.where((raw >= 0) & (raw < case.S), raw, -1).astype(np.int32)
    q, k, v, _ = upload(case, DEV)
    sl = torch.from_numpy(raw.astype(np.int32)).to(DEV)
    nbytes = qsa.decode_workspace_bytes(case.T, case.W, case.Hq, case.Hkv)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    out = qsa.sparse_decode(q, k, v, sl, workspace=ws)
    torch.cuda.synchronize()
    want = oracle.prefill(case.q, case.k_cache, case.v_cache, valid_only, 1.0 / 16.0)
    print(gate(bf16_tensor_to_f32(out), want, empty_row_mask(valid_only, case.S)))
    with pytest.raises(qsa.QsaError) as e:
        qsa.check_status(ws, case.T, case.W)
    assert e.value.status == 6 and f"{3 * case.T} selection entries" in str(e.value)


def test_decode_over_an_empty_cache_is_zero_and_counts_entries():
    """S = 0: no entry is valid; the output is exactly +0.0 and every entry
    other than -1 is counted as out of range."""
    T, Hq, Hkv, W = 3, 4, 2, 40
    g = torch.Generator().manual_seed(840)
    q = torch.randn(T, Hq, 256, generator=g).to(torch.bfloat16).to(DEV)
    k = torch.empty(0, Hkv, 256, dtype=torch.bfloat16, device=DEV)
    v = torch.empty(0, Hkv, 256, dtype=torch.bfloat16, device=DEV)
    sl = torch.full((T, W), -1, dtype=torch.int32)
    sl[0, 3] = 0
    sl[2, 10:15] = 7
    sl = sl.to(DEV)
    ws = torch.empty(qsa.decode_workspace_bytes(T, W, Hq, Hkv), dtype=torch.uint8, device=DEV)
    out = qsa.sparse_decode(q, k, v, sl, workspace=ws)
    torch.cuda.synchronize()
    assert torch.all(out.view(torch.int16) == 0)
    with pytest.raises(qsa.QsaError) as e:
        qsa.check_status(ws, T, W)
    assert e.value.status == 6 and "6 selection entries" in str(e.value)


def test_decode_with_one_share_per_item():
    """Enough tokens for one share per item (qsa_decode_splits gives 1): each
    share reads a whole raw row, -1 padding and invalid entries included."""
    case = qi.random_case(850, T=1100, S=5000, Hq=8, Hkv=2, W=70, pad_frac=0.2, interior=True)
    assert qsa.decode_splits(case.T, case.W, case.Hq, case.Hkv) == 1
    raw = case.slot_idx.copy()
    raw[5, 3] = 5000
    raw[700, 69] = -2
    valid_only = np.where((raw >= 0) & (raw < case.S), raw, -1).astype(np.int32)
    q, k, v, _ = upload(case, DEV)
    sl = torch.from_numpy(raw).to(DEV)
    ws = torch.empty(qsa.decode_workspace_bytes(case.T, case.W, case.Hq, case.Hkv),
                     dtype=torch.uint8, device=DEV)
    out = qsa.sparse_decode(q, k, v, sl, workspace=ws)
    torch.cuda.synchronize()
    rows = sorted(set(qi.sample_rows(case.T, 48, seed=851).tolist()) | {5, 700})
    want = oracle.prefill(case.q, case.k_cache, case.v_cache, valid_only, 1.0 / 16.0, rows=rows)
    got = bf16_tensor_to_f32(out[torch.as_tensor(rows, device=DEV)])
    print(gate(got, want, empty_row_mask(valid_only, case.S, rows)))
    with pytest.raises(qsa.QsaError) as e:
        qsa.check_status(ws, case.T, case.W)
    assert "2 selection entries" in str(e.value)
