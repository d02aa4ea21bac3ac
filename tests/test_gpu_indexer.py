"""GPU parity of the QSA indexer and Top-K selection against the oracle.

Readings (page "Qwen4-Exp QSA comes to Huawei's Ascend", section "Why QSA is
the awkward part, in numbers", and the causal tails of section "Nine tests
that passed, ..."): score(t, c) = sum over 4 heads of max(0, iq . ik[c]);
the top `budget` complete causal blocks, ties to the lower block; positions
of those blocks, then the tail, mapped to slots.

The selection is an integer result decided by floating point.  With integer
index values every score is exact in FP32 on both sides, so the selections
must be identical, ties included.  With random values the scores agree to
rounding and the selections may differ only among blocks whose scores lie
within that rounding of the cut.
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


def dev_inputs(case):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    iq = t(case.info["iq"].view(np.int16)).view(torch.bfloat16)
    ik = t(case.info["ik"].view(np.int16)).view(torch.bfloat16)
    return iq, ik, t(case.info["positions"]), t(case.info["slot_of_pos"])


def run_indexer(case):
    iq, ik, pos, sop = dev_inputs(case)
    scores = torch.full((case.T, ik.shape[0]), float("nan"), dtype=torch.float32, device=DEV)
    sel = qsa.indexer_topk(iq, ik, pos, sop, case.info["budget"], scores=scores)
    torch.cuda.synchronize()
    return scores.cpu().numpy(), sel.cpu().numpy()


def limits(case):
    C = case.info["ik"].shape[0]
    return np.minimum((case.info["positions"].astype(np.int64) + 1) // 4, C)


# (20000, 300, 100): rows of a multiple of 4 scores over several key ranges and
# token blocks, the last block partial (the scores pass's unconditional row stores)
@pytest.mark.parametrize("L,T,budget", [(8192, 100, 64), (4099, 37, 300), (777, 50, 8),
                                        (20000, 300, 100)])
def test_integer_scores_and_selection_are_exact(L, T, budget):
    case = qi.indexed_case(1100 + L, L=L, T=T, Hq=8, Hkv=1, budget=budget, integer_keys=True)
    # spread the queries over the whole request, including the first positions
    case.info["positions"][:] = np.sort(np.random.Generator(np.random.PCG64(1101))
                                        .choice(L, size=T, replace=False)).astype(np.int32)
    scores, sel = run_indexer(case)
    want = oracle.indexer_scores(case.info["iq"], case.info["ik"])
    lim = limits(case)
    for t in range(T):
        np.testing.assert_array_equal(scores[t, :lim[t]], want[t, :lim[t]])
    want_sel = oracle.indexer_select(want, case.info["positions"], case.info["slot_of_pos"],
                                     budget)
    np.testing.assert_array_equal(sel, want_sel)


def test_random_scores_match_and_selection_differs_only_at_the_cut():
    case = qi.indexed_case(1110, L=16384, T=64, Hq=8, Hkv=1, budget=256)
    scores, sel = run_indexer(case)
    want = oracle.indexer_scores(case.info["iq"], case.info["ik"])
    lim = limits(case)
    budget = case.info["budget"]
    inv = np.argsort(case.info["slot_of_pos"])
    for t in range(case.T):
        n = lim[t]
        np.testing.assert_allclose(scores[t, :n], want[t, :n], rtol=1e-5, atol=2e-4)
        got_blocks = set((inv[sel[t][:4 * min(n, budget)]] // 4).tolist())
        ref = oracle.indexer_select(want[t:t + 1], case.info["positions"][t:t + 1],
                                    case.info["slot_of_pos"], budget)[0]
        ref_blocks = set((inv[ref[:4 * min(n, budget)]] // 4).tolist())
        assert len(got_blocks) == min(n, budget)
        diff = got_blocks ^ ref_blocks
        if diff:
            cut = np.sort(want[t, :n])[::-1][budget - 1]
            assert all(abs(want[t, c] - cut) <= 4e-4 + 2e-5 * abs(cut) for c in diff)


def test_edge_positions_tails_and_invalid_rows():
    L, budget = 64, 3
    case = qi.indexed_case(1120, L=L, T=12, Hq=4, Hkv=1, budget=budget, integer_keys=True)
    case.info["positions"][:] = [0, 1, 2, 3, 4, 6, 7, 11, 62, 63, -1, 64]
    scores, sel = run_indexer(case)
    want = oracle.indexer_scores(case.info["iq"], case.info["ik"])
    valid = slice(0, 10)
    want_sel = oracle.indexer_select(want[valid], case.info["positions"][valid],
                                     case.info["slot_of_pos"], budget)
    np.testing.assert_array_equal(sel[valid], want_sel)
    assert np.all(sel[10:] == -1)           # positions outside [0, L)


def test_rows_longer_than_the_lds_stage():
    """C > 16384 index keys: the select kernel reads scores from memory."""
    case = qi.indexed_case(1130, L=80000, T=6, Hq=4, Hkv=1, budget=1000, integer_keys=True)
    scores, sel = run_indexer(case)
    want = oracle.indexer_scores(case.info["iq"], case.info["ik"])
    want_sel = oracle.indexer_select(want, case.info["positions"], case.info["slot_of_pos"],
                                     1000)
    np.testing.assert_array_equal(sel, want_sel)


def test_indexer_then_attention_end_to_end():
    """Selection by the indexer feeds the prefill; with exact scores the
    oracle selects the same slots, so its attention is the reference."""
    case = qi.indexed_case(1140, L=6000, T=80, Hq=24, Hkv=2, budget=100, integer_keys=True)
    iq, ik, pos, sop = dev_inputs(case)
    sel = qsa.indexer_topk(iq, ik, pos, sop, 100)
    q, k, v, _ = upload(case, DEV)
    out = qsa.sparse_prefill(q, k, v, sel)
    torch.cuda.synchronize()
    want_sel = oracle.indexer_select(oracle.indexer_scores(case.info["iq"], case.info["ik"]),
                                     case.info["positions"], case.info["slot_of_pos"], 100)
    np.testing.assert_array_equal(sel.cpu().numpy(), want_sel)
    want = oracle.prefill(case.q, case.k_cache, case.v_cache, want_sel, 1.0 / 16.0)
    gate(bf16_tensor_to_f32(out), want, empty_row_mask(want_sel, case.S))


def test_indexed_long_prefill_sampled_rows():
    case = qi.indexed_long_prefill()
    budget = case.info["budget"]
    iq, ik, pos, sop = dev_inputs(case)
    sel = qsa.indexer_topk(iq, ik, pos, sop, budget)
    torch.cuda.synchronize()
    rows = qi.sample_rows(case.T, 32)
    sel_np = sel.cpu().numpy()
    want_scores = oracle.indexer_scores(case.info["iq"][rows], case.info["ik"])
    inv = np.argsort(case.info["slot_of_pos"])
    lim = limits(case)
    for i, t in enumerate(rows):
        n = int(lim[t])
        row = sel_np[t]
        r = (int(case.info["positions"][t]) + 1) % 4
        assert np.all(row[4 * budget + r:] == -1)
        chosen = set((inv[row[:4 * budget]] // 4).tolist())
        assert len(chosen) == budget and max(chosen) < n
        cut = np.sort(want_scores[i, :n])[::-1][budget - 1]
        assert all(want_scores[i, c] >= cut - 1e-3 for c in chosen)
    # The attention at full size on the oracle's own selection for these rows.
    want_sel = oracle.indexer_select(want_scores, case.info["positions"][rows],
                                     case.info["slot_of_pos"], budget)
    q, k, v, _ = upload(case, DEV)
    out = qsa.sparse_prefill(q[torch.as_tensor(rows, device=DEV)].contiguous(), k, v,
                             torch.from_numpy(want_sel).to(DEV))
    torch.cuda.synchronize()
    want = oracle.prefill(np.ascontiguousarray(case.q[rows]), case.k_cache, case.v_cache,
                          want_sel, 1.0 / 16.0)
    gate(bf16_tensor_to_f32(out), want, empty_row_mask(want_sel, case.S))


def select_on(scores_np, positions_np, slot_of_pos_np, budget):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    sel = qsa.indexer_select(t(scores_np), t(positions_np), t(slot_of_pos_np), budget)
    torch.cuda.synchronize()
    return sel.cpu().numpy()


@pytest.mark.parametrize("L,budget", [(80000, 8), (80000, 960), (80000, 961), (80000, 3000),
                                      (20000, 300), (20000, 1500), (9000, 960)])
def test_selection_paths_by_budget_and_row_length(L, budget):
    """Budgets up to 960 take the sampled-threshold kernel, larger ones the
    histogram kernel (rows staged in LDS up to 16,384 blocks, else read from
    memory).  Integer scores with many ties: every path must match the
    oracle exactly."""
    rng = np.random.Generator(np.random.PCG64(1150 + L + budget))
    C = -(-L // 4)
    T = 9
    scores = rng.integers(0, 40, size=(T, C)).astype(np.float32)
    positions = np.sort(rng.choice(L, size=T, replace=False)).astype(np.int32)
    positions[-1] = L - 1
    slot_of_pos = rng.permutation(L).astype(np.int32)
    got = select_on(scores, positions, slot_of_pos, budget)
    want = oracle.indexer_select(scores, positions, slot_of_pos, budget)
    np.testing.assert_array_equal(got, want)


def test_all_equal_scores_keep_the_lowest_blocks():
    """Every score equal: the sampled threshold admits the whole row, more
    than the candidate list holds, so the kernel takes its exact fallback; the
    ties go to the lowest blocks."""
    L, budget, T = 60000, 512, 5
    C = L // 4
    scores = np.zeros((T, C), dtype=np.float32)
    positions = np.array([L - 1, 30000, 20000, 2100, 3], dtype=np.int32)
    slot_of_pos = np.random.Generator(np.random.PCG64(1160)).permutation(L).astype(np.int32)
    got = select_on(scores, positions, slot_of_pos, budget)
    want = oracle.indexer_select(scores, positions, slot_of_pos, budget)
    np.testing.assert_array_equal(got, want)
    assert np.array_equal(got[0][:4 * budget], slot_of_pos[:4 * budget])


def test_fractional_scores_with_one_tied_cut():
    """Random scores with a block of exact ties straddling the cut: the first
    tied blocks in block order are kept."""
    rng = np.random.Generator(np.random.PCG64(1170))
    L, budget, T = 65536, 512, 6
    C = L // 4
    scores = rng.random((T, C), dtype=np.float32)
    for t in range(T):
        cut = np.sort(scores[t])[::-1][budget - 1]
        tied = rng.choice(C, size=300, replace=False)
        scores[t, tied] = cut
    positions = (L - 1 - np.arange(T) * 997).astype(np.int32)
    slot_of_pos = rng.permutation(L).astype(np.int32)
    got = select_on(scores, positions, slot_of_pos, budget)
    want = oracle.indexer_select(scores, positions, slot_of_pos, budget)
    np.testing.assert_array_equal(got, want)


def test_deferred_rows_do_not_disturb_the_others():
    """Budgets up to 512 defer the rows whose sampled threshold admits too
    many candidates to a second, exact launch.  Rows of all-equal scores
    (deferred) interleaved with random rows (selected at once) must each
    match the oracle."""
    rng = np.random.Generator(np.random.PCG64(1180))
    L, budget, T = 40000, 400, 8
    C = L // 4
    scores = rng.random((T, C), dtype=np.float32)
    scores[1::2] = 0.5
    positions = (L - 1 - np.arange(T) * 1201).astype(np.int32)
    slot_of_pos = rng.permutation(L).astype(np.int32)
    got = select_on(scores, positions, slot_of_pos, budget)
    want = oracle.indexer_select(scores, positions, slot_of_pos, budget)
    np.testing.assert_array_equal(got, want)


# ---------------------------------------------------------------- fused Top-K

def fused_topk(case, budget):
    iq, ik, pos, sop = dev_inputs(case)
    sel = qsa.indexer_topk_fused(iq, ik, pos, sop, budget)
    torch.cuda.synchronize()
    return sel.cpu().numpy()


@pytest.mark.parametrize("L,T,budget", [(65536, 300, 512), (20000, 200, 300), (8192, 100, 64),
                                        (4099, 37, 300), (777, 50, 8), (262144, 40, 512)])
def test_fused_topk_is_exact_on_integer_scores(L, T, budget):
    """The fused path (sampled threshold, candidates, exact selection, full
    rows where the threshold missed) selects exactly what the oracle selects,
    ties included, with queries at the end of the request and spread over it."""
    case = qi.indexed_case(1160 + L % 991, L=L, T=T, Hq=8, Hkv=1, budget=budget,
                           integer_keys=True)
    rng = np.random.Generator(np.random.PCG64(1161 + L))
    spread = np.sort(rng.choice(L, size=T // 2, replace=False)).astype(np.int32)
    case.info["positions"][: T // 2] = spread
    sel = fused_topk(case, budget)
    want = oracle.indexer_select(oracle.indexer_scores(case.info["iq"], case.info["ik"]),
                                 case.info["positions"], case.info["slot_of_pos"], budget)
    np.testing.assert_array_equal(sel, want)


@pytest.mark.parametrize("rising", [True, False])
def test_fused_topk_rows_the_estimate_misses(rising):
    """One estimate group of 16 queries with rows of 3,001 and 16,384
    eligible blocks: the sample covers the shorter row's blocks only.  Scores
    that rise with the block index leave the long row far too many
    candidates, scores that fall leave it too few; either way that row takes
    the full scores and the exact selection, and the result equals the
    oracle's, ties to the lower block included."""
    L, T, budget = 65536, 16, 512
    case = qi.indexed_case(1170, L=L, T=T, Hq=8, Hkv=1, budget=budget, integer_keys=True)
    C = case.info["ik"].shape[0]
    level = 1 + (np.arange(C) if rising else (C - 1 - np.arange(C))) // 128   # <= 129: exact in BF16
    ik = np.repeat(level.astype(np.float32)[:, None, None], 128, axis=2)
    case.info["ik"] = qi.bf16_bits(ik)
    case.info["iq"] = qi.bf16_bits(np.ones((T, 4, 128), dtype=np.float32))
    pos = np.full(T, L - 1, dtype=np.int32)
    pos[0] = 4 * 3000 + 3
    pos[5] = 4 * 9000 + 1
    case.info["positions"] = pos
    sel = fused_topk(case, budget)
    want = oracle.indexer_select(oracle.indexer_scores(case.info["iq"], case.info["ik"]),
                                 pos, case.info["slot_of_pos"], budget)
    np.testing.assert_array_equal(sel, want)
