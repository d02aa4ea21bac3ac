"""GPU parity: the HIP path through the C ABI against the FP32 CPU oracle.

Gate (page "Qwen4-Exp QSA comes to Huawei's Ascend: inside SGLang's opt-in
CANN prefill PR", section "Nine tests that passed, ..."): atol 0.025,
rtol 0.025, relative L2 < 0.008, empty rows exactly zero.  Integer work (the
compaction pass) must match bit for bit.  Cases follow that section's list:
unordered slots at widths 1/63/64/65/2051, default and explicit scales, fully
masked rows, zero width, non-contiguous tensors, causal tails, the two-request
shared prefix, the five local head shapes at 1 and 257 query rows, and the
long prefill (sampled rows, all outputs finite).
"""
import numpy as np
import pytest
import torch

import oracle
import qsa_inputs as qi
import top_sparse_attention_amd as qsa
from qsa_testutil import (bf16_tensor_bits, bf16_tensor_to_f32, empty_row_mask, gate,
                          upload)

pytestmark = pytest.mark.gpu

DEV = "cuda"
SORT_RUN = 2304      # entries the compaction pass sorts together


def run_case(case, rows=None, out=None):
    q, k, v, sl = upload(case, DEV)
    o = qsa.sparse_prefill(q, k, v, sl, scale=case.scale, out=out)
    torch.cuda.synchronize()
    return o, (q, k, v, sl)


def oracle_out(case, rows=None):
    scale = case.scale if case.scale is not None else 1.0 / 16.0
    return oracle.prefill(case.q, case.k_cache, case.v_cache, case.slot_idx, scale, rows=rows)


def check_against_oracle(case, rows=None, out=None):
    o, tensors = run_case(case, out=out)
    got = bf16_tensor_to_f32(o if rows is None else o[torch.as_tensor(rows, device=DEV)])
    want = oracle_out(case, rows)
    m = gate(got, want, empty_row_mask(case.slot_idx, case.S, rows))
    print(f"{case.name}: {m}", flush=True)
    return o, tensors, m


# ------------------------------------------------------------------ compaction

def group_shift(S):
    """r of the header: valid entries are grouped by slot >> r."""
    b = 1
    while b < 31 and (1 << b) < S:
        b += 1
    return max(0, b - 7)


def check_compaction(case):
    _, _, _, sl = upload(case, DEV)
    ws = qsa.compact_slots(sl, case.S)
    torch.cuda.synchronize()
    lst, cnt, bad = (x.cpu().numpy() for x in qsa.compacted_lists(ws, case.T, case.W))
    want_cnt = np.zeros(case.T, dtype=np.int64)
    want_bad = np.zeros(case.T, dtype=np.int64)
    r = group_shift(case.S)
    for t in range(case.T):
        # The oracle filter keeps input order; the library then stably groups
        # each run of SORT_RUN input entries by slot >> r.
        want = []
        for r0 in range(0, case.W, SORT_RUN):
            part = case.slot_idx[t:t + 1, r0:r0 + SORT_RUN]
            kept, k_cnt, k_bad = oracle.compact(np.ascontiguousarray(part), case.S)
            want.extend(sorted(kept[0, :k_cnt[0]].tolist(), key=lambda s_: s_ >> r))
            want_bad[t] += k_bad[0]
        want_cnt[t] = len(want)
        np.testing.assert_array_equal(lst[t, :len(want)], np.array(want, dtype=np.int32))
        pad_end = (len(want) + 31) // 32 * 32
        assert np.all(lst[t, len(want):pad_end] == -1)
    np.testing.assert_array_equal(cnt, want_cnt)
    np.testing.assert_array_equal(bad, want_bad)
    return ws


def test_compaction_tiny_bit_exact():
    check_compaction(qi.tiny())


def test_compaction_edge_mix_bit_exact():
    check_compaction(qi.edge_mix())


def test_compaction_of_rows_longer_than_one_sort_run():
    case = qi.random_case(43, T=6, S=100000, Hq=2, Hkv=1, W=5000, pad_frac=0.1, interior=True)
    check_compaction(case)
    check_against_oracle(case)


def test_compaction_with_duplicates_and_tiny_caches():
    for S in (1, 2, 3, 17):
        rng = np.random.Generator(np.random.PCG64(44 + S))
        case = qi.random_case(45, T=9, S=S, Hq=3, Hkv=1, W=1)
        case.slot_idx = rng.integers(-1, S, size=(9, 70)).astype(np.int32)
        case.bases["slot_idx"] = case.slot_idx
        check_compaction(case)
        check_against_oracle(case)


def test_compaction_counts_invalid_entries_and_drops_them():
    case = qi.random_case(41, T=40, S=500, Hq=2, Hkv=1, W=300, pad_frac=0.2, interior=True)
    sel = case.slot_idx.copy()
    rng = np.random.Generator(np.random.PCG64(42))
    bad_pos = rng.integers(0, 300, size=(40, 3))
    for t in range(40):
        sel[t, bad_pos[t]] = [500, -7, 1 << 30]
    case.slot_idx[:] = sel
    ws = check_compaction(case)
    with pytest.raises(qsa.QsaError) as e:
        qsa.check_status(ws, case.T, case.W)
    assert e.value.status == 6


# ------------------------------------------------------------------ small cases

def test_tiny_workload():
    check_against_oracle(qi.tiny())


def test_edge_mix_workload_strided_views():
    case = qi.edge_mix()
    o, _, _ = check_against_oracle(case)
    empty = empty_row_mask(case.slot_idx, case.S)
    assert empty.sum() >= 40


@pytest.mark.parametrize("Hq,Hkv", [(16, 2), (24, 2), (12, 1), (6, 1), (3, 1)])
@pytest.mark.parametrize("T", [1, 257])
def test_local_head_shapes(Hq, Hkv, T):
    case = qi.random_case(200 + Hq * 10 + Hkv + T, T=T, S=3000, Hq=Hq, Hkv=Hkv, W=300,
                          pad_frac=0.1, interior=True)
    check_against_oracle(case)


@pytest.mark.parametrize("W", [1, 31, 32, 33, 63, 64, 65, 127, 129, 2051])
def test_widths_around_tile_edges(W):
    case = qi.random_case(300 + W, T=19, S=4096, Hq=8, Hkv=1, W=W, scale=0.08)
    check_against_oracle(case)


@pytest.mark.parametrize("Hq,Hkv", [(17, 1), (40, 2), (64, 1), (2, 2)])
def test_head_ratios_beyond_sixteen_and_one(Hq, Hkv):
    case = qi.random_case(400 + Hq, T=9, S=900, Hq=Hq, Hkv=Hkv, W=150, pad_frac=0.05)
    check_against_oracle(case)


@pytest.mark.parametrize("scale", [0.0, 0.0625, 0.2, -0.05, 1.0])
def test_explicit_scales(scale):
    case = qi.random_case(500, T=23, S=2048, Hq=12, Hkv=1, W=200, scale=scale)
    check_against_oracle(case)


def test_zero_width_and_all_masked_rows_are_exact_zero():
    case = qi.random_case(600, T=33, S=256, Hq=6, Hkv=1, W=0)
    o, _, _ = check_against_oracle(case)
    assert torch.all(o.view(torch.int16) == 0)
    case = qi.random_case(601, T=33, S=256, Hq=6, Hkv=1, W=40)
    case.slot_idx[::3] = -1
    o, _, _ = check_against_oracle(case)
    assert torch.all(o[::3].view(torch.int16) == 0)


def test_zero_tokens_is_a_no_op():
    case = qi.random_case(602, T=0, S=64, Hq=4, Hkv=2, W=8)
    o, _ = run_case(case)
    assert o.shape == (0, 4, 256)


def test_non_contiguous_output_view():
    case = qi.random_case(603, T=21, S=700, Hq=12, Hkv=1, W=90)
    big = torch.full((21, 2, 12, 256), 7.0, dtype=torch.bfloat16, device=DEV)
    out = big[:, 1]
    o, _, _ = check_against_oracle(case, out=out)
    assert o.data_ptr() == out.data_ptr()
    assert torch.all(big[:, 0] == 7.0)      # nothing outside the view was written


# ------------------------------------------------------------------ invariants

def test_single_slot_rows_return_the_value_row_bit_exactly():
    case = qi.random_case(700, T=40, S=512, Hq=12, Hkv=2, W=9, pad_frac=8 / 9, interior=True)
    o, _ = run_case(case)
    got = bf16_tensor_bits(o)
    for t in range(case.T):
        (s,) = case.slot_idx[t][case.slot_idx[t] != -1]
        for h in range(case.Hq):
            np.testing.assert_array_equal(got[t, h], case.v_cache[s, h // 6])


def test_identical_value_rows_return_that_row_bit_exactly():
    """Every cache slot holds the same V row (per KV head): the weights sum
    out, out = that row.  The two FP32 sums (the weighted rows and the
    weights) differ by far less than half a BF16 step, so the BF16 output is
    the row bit for bit."""
    case = qi.random_case(710, T=25, S=3000, Hq=16, Hkv=2, W=700, pad_frac=0.2, interior=True)
    case.v_cache[:] = case.v_cache[0]
    case.slot_idx[3] = -1
    o, _ = run_case(case)
    got = bf16_tensor_bits(o)
    G = case.Hq // case.Hkv
    for t in range(case.T):
        if t == 3:
            assert np.all(got[t] == 0)
            continue
        for h in range(case.Hq):
            np.testing.assert_array_equal(got[t, h], case.v_cache[0, h // G])


def test_zero_queries_give_the_mean_of_the_selected_values():
    """All-zero query rows score every selected slot 0: equal weights, so the
    output is the plain mean of the selected V rows (FP64 closed form)."""
    case = qi.random_case(711, T=19, S=2500, Hq=12, Hkv=2, W=300, pad_frac=0.25,
                          interior=True)
    case.q[:] = 0
    o, _ = run_case(case)
    v = qi.bf16_to_f32(case.v_cache).astype(np.float64)
    G = case.Hq // case.Hkv
    want = np.zeros((case.T, case.Hq, 256))
    for t in range(case.T):
        sel = case.slot_idx[t][case.slot_idx[t] != -1]
        for h in range(case.Hq):
            want[t, h] = v[sel, h // G].mean(axis=0)
    m = gate(bf16_tensor_to_f32(o), want.astype(np.float32), empty_row_mask(case.slot_idx, case.S))
    print(f"zero queries: {m}", flush=True)


def test_padding_position_is_bitwise_irrelevant():
    case = qi.random_case(701, T=30, S=3000, Hq=16, Hkv=2, W=400, pad_frac=0.3)
    a, _ = run_case(case)
    # same valid entries in the same order, -1 moved from the tail into the interior
    rng = np.random.Generator(np.random.PCG64(702))
    moved = np.full_like(case.slot_idx, -1)
    for t in range(case.T):
        valid = case.slot_idx[t][case.slot_idx[t] != -1]
        pos = np.sort(rng.choice(case.W, size=valid.size, replace=False))
        moved[t, pos] = valid
    case.slot_idx[:] = moved
    b, _ = run_case(case)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def _relocate(case, new_of_old, S_new):
    """Move cache row s to row new_of_old[s] of a bigger cache and remap the
    selection accordingly; rows not used by the map get fresh values."""
    rng = np.random.Generator(np.random.PCG64(S_new))
    k2 = qi.normal_bf16(rng, (S_new,) + case.k_cache.shape[1:])
    v2 = qi.normal_bf16(rng, (S_new,) + case.v_cache.shape[1:])
    k2[new_of_old] = case.k_cache
    v2[new_of_old] = case.v_cache
    sel = np.where(case.slot_idx >= 0, new_of_old[np.maximum(case.slot_idx, 0)], -1)
    case.k_cache, case.v_cache = k2, v2
    case.slot_idx = sel.astype(np.int32)
    case.bases.update(k=k2, v=v2, slot_idx=case.slot_idx)


def test_any_relocation_stays_within_the_gate():
    case = qi.random_case(705, T=25, S=1500, Hq=24, Hkv=2, W=333)
    a, _ = run_case(case)
    rng = np.random.Generator(np.random.PCG64(706))
    _relocate(case, rng.permutation(case.S), case.S)
    b, _ = check_against_oracle(case)[:2]
    gate(bf16_tensor_to_f32(b), bf16_tensor_to_f32(a), np.zeros(case.T, dtype=bool))


def test_heads_with_identical_queries_give_identical_outputs():
    case = qi.random_case(709, T=17, S=800, Hq=12, Hkv=1, W=100)
    case.q[:] = case.q[:, :1, :]
    o, _ = run_case(case)
    bits = bf16_tensor_bits(o)
    for h in range(1, case.Hq):
        np.testing.assert_array_equal(bits[:, h], bits[:, 0])


def test_repeated_runs_are_bitwise_deterministic():
    case = qi.random_case(706, T=64, S=9000, Hq=16, Hkv=2, W=2051)
    a, tensors = run_case(case)
    q, k, v, sl = tensors
    for _ in range(3):
        b = qsa.sparse_prefill(q, k, v, sl, scale=case.scale)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_slot_order_changes_output_only_within_the_gate():
    case = qi.random_case(707, T=20, S=5000, Hq=8, Hkv=1, W=777, pad_frac=0.2, interior=True)
    a, _ = run_case(case)
    rng = np.random.Generator(np.random.PCG64(708))
    case.slot_idx[:] = rng.permuted(case.slot_idx, axis=1)
    b, _ = check_against_oracle(case)[:2]
    gate(bf16_tensor_to_f32(b), bf16_tensor_to_f32(a), np.zeros(case.T, dtype=bool))


def test_order_of_slot_range_groups_is_bitwise_irrelevant():
    """Rows that differ only in the order of their groups (slot >> r) give
    bitwise identical outputs: the compaction pass orders the groups itself."""
    case = qi.random_case(712, T=12, S=4096, Hq=6, Hkv=1, W=600)
    r = group_shift(case.S)
    a, _ = run_case(case)
    rng = np.random.Generator(np.random.PCG64(713))
    rows = []
    for t in range(case.T):
        groups = {}
        for s_ in case.slot_idx[t].tolist():
            groups.setdefault(s_ >> r, []).append(s_)
        keys = list(groups)
        rng.shuffle(keys)
        rows.append([s_ for k_ in keys for s_ in groups[k_]])
    case.slot_idx[:] = np.array(rows, dtype=np.int32)
    b, _ = run_case(case)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_large_scale_is_finite_and_matches_oracle():
    case = qi.random_case(711, T=16, S=2000, Hq=6, Hkv=1, W=500, scale=3.0)
    o, _, _ = check_against_oracle(case)
    assert torch.isfinite(o.float()).all()


def test_gather_only_reads_exactly_the_selected_rows():
    case = qi.random_case(710, T=37, S=3000, Hq=4, Hkv=2, W=200, pad_frac=0.25, interior=True)
    q, k, v, sl = upload(case, DEV)
    ws = qsa.compact_slots(sl, case.S)
    sink = qsa.gather_only(k, v, ws, case.T, case.W)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    kw = np.ascontiguousarray(case.k_cache).view(np.uint32)   # [S, Hkv, 128] words
    vw = np.ascontiguousarray(case.v_cache).view(np.uint32)
    for t in range(case.T):
        sel = case.slot_idx[t][case.slot_idx[t] != -1]
        for g in range(case.Hkv):
            want = np.bitwise_xor.reduce(np.concatenate([kw[sel, g].ravel(), vw[sel, g].ravel()]))
            assert got[t * case.Hkv + g] == (want if sel.size else 0)


# ------------------------------------------------------------------ full-size workloads

def _full_size(case, n_rows=64):
    rows = qi.sample_rows(case.T, n_rows)
    o, tensors, m = check_against_oracle(case, rows=rows)
    assert torch.isfinite(o.float()).all()
    return o, tensors, m


def test_long_prefill_sampled_rows():
    _full_size(qi.long_prefill())


def test_two_request_shared_prefix_sampled_rows():
    case = qi.two_request()
    o, _, _ = _full_size(case)
    # cache-content reuse: the two requests share their prefix slots
    perm = case.info["perm"]
    prefix = set(perm[:qi.PREFIX].tolist())
    a = set(case.slot_idx[0].tolist()) & prefix
    b = set(case.slot_idx[qi.NEW_PER_REQUEST].tolist()) & prefix
    assert a and b


@pytest.mark.parametrize("heads", [(6, 1), (3, 1)])
def test_max_cache_sampled_rows(heads):
    _full_size(qi.max_cache(heads=heads))
