"""Pins for the FP32 CPU oracle (no GPU).

The oracle is pinned here to things other than itself: an FP64 brute-force
dense attention with a slot mask, torch's scaled_dot_product_attention for the
special cases of full and causal selections, and closed forms (single slot,
uniform weights, identical value rows, equal scores, empty rows).  A mistake in
the oracle's head mapping, scale, mask handling or softmax would fail at least
one of them.
"""
import json
import os

import numpy as np
import pytest
import torch

import qsa_inputs as qi

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32(bits):
    return qi.bf16_to_f32(bits)


def dense_masked_attention_fp64(case, scale):
    """Brute force: attend over every cache slot with an explicit membership
    mask, in float64, one query head at a time."""
    q = f32(case.q).astype(np.float64)
    k = f32(case.k_cache).astype(np.float64)
    v = f32(case.v_cache).astype(np.float64)
    T, Hq, D = q.shape
    S, Hkv, _ = k.shape
    G = Hq // Hkv
    member = np.zeros((T, S), dtype=bool)
    for t in range(T):
        row = case.slot_idx[t]
        member[t, row[row != -1]] = True
    out = np.zeros((T, Hq, D))
    for h in range(Hq):
        g = h // G
        logits = scale * (q[:, h, :] @ k[:, g, :].T)
        logits = np.where(member, logits, -np.inf)
        top = logits.max(axis=1, keepdims=True)
        top = np.where(np.isfinite(top), top, 0.0)
        w = np.where(member, np.exp(logits - top), 0.0)
        den = w.sum(axis=1, keepdims=True)
        den = np.where(den > 0, den, 1.0)
        out[:, h, :] = (w / den) @ v[:, g, :]
    return out


def rel_l2(a, b):
    return float(np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300))


@pytest.mark.parametrize("Hq,Hkv", [(2, 1), (4, 2), (3, 1), (12, 1), (6, 2)])
@pytest.mark.parametrize("pad_frac,interior", [(0.0, False), (0.25, False), (0.4, True)])
def test_oracle_matches_dense_bruteforce(oracle_mod, Hq, Hkv, pad_frac, interior):
    seed = 1000 + 10 * Hq + Hkv + int(100 * pad_frac)
    case = qi.random_case(seed, T=6, S=48, Hq=Hq, Hkv=Hkv, W=20, pad_frac=pad_frac,
                          interior=interior)
    scale = 0.0625 if Hq % 2 == 0 else 0.11
    got = oracle_mod.prefill(case.q, case.k_cache, case.v_cache, case.slot_idx, scale)
    want = dense_masked_attention_fp64(case, scale)
    assert rel_l2(got, want) < 1e-5
    np.testing.assert_allclose(got, want, rtol=1e-4, atol=1e-5)


def test_oracle_rows_subset_matches_full(oracle_mod):
    case = qi.random_case(7, T=9, S=40, Hq=4, Hkv=2, W=11, pad_frac=0.2, interior=True)
    full = oracle_mod.prefill(case.q, case.k_cache, case.v_cache, case.slot_idx, 0.07)
    rows = [8, 0, 3]
    part = oracle_mod.prefill(case.q, case.k_cache, case.v_cache, case.slot_idx, 0.07,
                              rows=rows)
    np.testing.assert_array_equal(part, full[rows])


def _sdpa_fp64(q, k, v, scale, causal):
    # q [T,Hq,D], k/v [S,Hkv,D] -> torch layout [1, H, L, D]; KV heads shared
    # by contiguous groups of query heads (enable_gqa).
    qt = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2).unsqueeze(0)
    kt = torch.from_numpy(k.astype(np.float64)).permute(1, 0, 2).unsqueeze(0)
    vt = torch.from_numpy(v.astype(np.float64)).permute(1, 0, 2).unsqueeze(0)
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, is_causal=causal, scale=scale, enable_gqa=True)
    return o.squeeze(0).permute(1, 0, 2).numpy()


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (6, 1), (24, 2)])
def test_full_selection_equals_library_dense_attention(oracle_mod, Hq, Hkv):
    rng = np.random.Generator(np.random.PCG64(31 + Hq))
    T, S = 5, 37
    case = qi.random_case(32 + Hq, T=T, S=S, Hq=Hq, Hkv=Hkv, W=S)
    # every row selects every slot, each row in its own random order
    sel = np.stack([rng.permutation(S) for _ in range(T)]).astype(np.int32)
    got = oracle_mod.prefill(case.q, case.k_cache, case.v_cache, sel, 0.0625)
    want = _sdpa_fp64(f32(case.q), f32(case.k_cache), f32(case.v_cache), 0.0625, False)
    assert rel_l2(got, want) < 1e-5


def test_causal_selection_equals_library_causal_attention(oracle_mod):
    rng = np.random.Generator(np.random.PCG64(77))
    T = S = 24
    case = qi.random_case(78, T=T, S=S, Hq=6, Hkv=2, W=S)
    sel = np.full((T, S), -1, dtype=np.int32)
    for t in range(T):
        sel[t, :t + 1] = np.arange(t + 1)
        sel[t] = rng.permutation(sel[t])      # -1 scattered, slots unordered
    got = oracle_mod.prefill(case.q, case.k_cache, case.v_cache, sel, 0.09)
    want = _sdpa_fp64(f32(case.q), f32(case.k_cache), f32(case.v_cache), 0.09, True)
    assert rel_l2(got, want) < 1e-5


def test_single_slot_returns_value_row_exactly(oracle_mod):
    case = qi.random_case(5, T=8, S=64, Hq=6, Hkv=2, W=7, pad_frac=6 / 7, interior=True)
    got = oracle_mod.prefill(case.q, case.k_cache, case.v_cache, case.slot_idx, 0.3)
    v = f32(case.v_cache)
    for t in range(case.T):
        (s,) = case.slot_idx[t][case.slot_idx[t] != -1]
        for h in range(case.Hq):
            np.testing.assert_array_equal(got[t, h], v[s, h // 3])


def test_zero_scale_and_zero_query_give_mean_of_selected_values(oracle_mod):
    case = qi.random_case(9, T=4, S=64, Hq=4, Hkv=1, W=13, pad_frac=0.3, interior=True)
    v = f32(case.v_cache).astype(np.float64)
    mean = np.stack([v[case.slot_idx[t][case.slot_idx[t] != -1], 0].mean(axis=0)
                     for t in range(case.T)])
    got = oracle_mod.prefill(case.q, case.k_cache, case.v_cache, case.slot_idx, 0.0)
    for h in range(case.Hq):
        np.testing.assert_allclose(got[:, h], mean, rtol=1e-5, atol=1e-6)
    q0 = np.zeros_like(case.q)
    got0 = oracle_mod.prefill(q0, case.k_cache, case.v_cache, case.slot_idx, 0.0625)
    for h in range(case.Hq):
        np.testing.assert_allclose(got0[:, h], mean, rtol=1e-5, atol=1e-6)


def test_identical_value_rows_return_that_row(oracle_mod):
    case = qi.random_case(11, T=5, S=32, Hq=3, Hkv=1, W=9)
    v = case.v_cache.copy()
    v[:] = v[4]
    got = oracle_mod.prefill(case.q, case.k_cache, v, case.slot_idx, 0.2)
    # FP32 sums of W=9 weights: a few ulps of rounding, bounded by W * 2^-24
    np.testing.assert_allclose(got, np.broadcast_to(f32(v[4]), got.shape), rtol=2e-6, atol=0)


def test_equal_scores_average_two_rows_exactly(oracle_mod):
    case = qi.random_case(12, T=3, S=16, Hq=2, Hkv=1, W=2)
    k = case.k_cache.copy()
    sel = np.array([[3, 9], [9, 3], [1, 2]], dtype=np.int32)
    k[9] = k[3]
    k[2] = k[1]
    got = oracle_mod.prefill(case.q, k, case.v_cache, sel, 0.5)
    v = f32(case.v_cache)
    for t, (a, b) in enumerate(sel):
        np.testing.assert_array_equal(got[t, 0], (v[a, 0] + v[b, 0]) / np.float32(2))


def test_empty_rows_are_exact_positive_zero(oracle_mod):
    case = qi.random_case(13, T=6, S=32, Hq=4, Hkv=2, W=5)
    sel = case.slot_idx.copy()
    sel[[1, 4]] = -1
    got = oracle_mod.prefill(case.q, case.k_cache, case.v_cache, sel, 0.0625)
    for t in (1, 4):
        assert np.all(got[t] == 0) and not np.any(np.signbit(got[t]))
    assert np.all(np.any(got[[0, 2, 3, 5]] != 0, axis=-1))
    empty = np.zeros((case.T, 0), dtype=np.int32)
    got0 = oracle_mod.prefill(case.q, case.k_cache, case.v_cache, empty, 0.0625)
    assert np.all(got0 == 0) and not np.any(np.signbit(got0))


def test_slot_order_and_padding_position_invariance(oracle_mod):
    case = qi.random_case(14, T=7, S=200, Hq=4, Hkv=1, W=70, pad_frac=0.3)
    rng = np.random.Generator(np.random.PCG64(15))
    shuffled = rng.permuted(case.slot_idx, axis=1)
    a = oracle_mod.prefill(case.q, case.k_cache, case.v_cache, case.slot_idx, 0.0625)
    b = oracle_mod.prefill(case.q, case.k_cache, case.v_cache, shuffled, 0.0625)
    assert rel_l2(b, a.astype(np.float64)) < 1e-6


def test_large_scale_is_stable_and_picks_the_argmax(oracle_mod):
    case = qi.random_case(16, T=4, S=128, Hq=2, Hkv=1, W=50)
    got = oracle_mod.prefill(case.q, case.k_cache, case.v_cache, case.slot_idx, 100.0)
    assert np.all(np.isfinite(got))
    q, k, v = f32(case.q), f32(case.k_cache), f32(case.v_cache)
    for t in range(case.T):
        sl = case.slot_idx[t]
        for h in range(case.Hq):
            logits = k[sl, 0] @ q[t, h].astype(np.float64)
            best = sl[int(np.argmax(logits))]
            gap = np.sort(logits)[-1] - np.sort(logits)[-2]
            if 100.0 * gap > 30:        # the runner-up weight is below e^-30
                np.testing.assert_allclose(got[t, h], v[best, 0], rtol=1e-6, atol=1e-6)


def test_out_of_range_slot_is_refused(oracle_mod):
    case = qi.random_case(17, T=3, S=16, Hq=2, Hkv=1, W=4)
    for bad in (16, -2, 1 << 30):
        sel = case.slot_idx.copy()
        sel[1, 2] = bad
        with pytest.raises(ValueError):
            oracle_mod.prefill(case.q, case.k_cache, case.v_cache, sel, 0.0625)


def test_strided_views_match_contiguous_copies(oracle_mod):
    case = qi.edge_mix()
    rows = [0, 1, 2, 3, 4, 5, 7, 13, 23, 256]
    a = oracle_mod.prefill(case.q, case.k_cache, case.v_cache, case.slot_idx, case.scale,
                           rows=rows)
    b = oracle_mod.prefill(np.ascontiguousarray(case.q), np.ascontiguousarray(case.k_cache),
                           np.ascontiguousarray(case.v_cache), case.slot_idx, case.scale,
                           rows=rows)
    np.testing.assert_array_equal(a, b)


# ---------------------------------------------------------------- compaction

def test_compaction_golden_cases(oracle_mod):
    with open(os.path.join(GOLDEN, "compaction_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        sel = np.array(c["slot_idx"], dtype=np.int32).reshape(len(c["slot_idx"]), -1)
        lists, counts, n_bad = oracle_mod.compact(sel, c["S"])
        for t, want in enumerate(c["kept"]):
            assert counts[t] == len(want), c["why"]
            assert lists[t, :counts[t]].tolist() == want, c["why"]
        assert n_bad.tolist() == c["n_bad"], c["why"]


def test_compaction_keeps_valid_entries_as_a_subsequence(oracle_mod):
    rng = np.random.Generator(np.random.PCG64(21))
    S = 50
    sel = rng.integers(-3, S + 3, size=(40, 33)).astype(np.int32)
    lists, counts, n_bad = oracle_mod.compact(sel, S)
    for t in range(sel.shape[0]):
        kept = lists[t, :counts[t]]
        assert np.all((kept >= 0) & (kept < S))
        # kept is a subsequence of the row, and nothing valid was skipped
        it = iter(sel[t].tolist())
        assert all(any(x == y for y in it) for x in kept.tolist())
        n_valid = sum(1 for x in sel[t] if 0 <= x < S)
        n_pad = sum(1 for x in sel[t] if x == -1)
        assert counts[t] == n_valid
        assert n_bad[t] == sel.shape[1] - n_valid - n_pad


@pytest.mark.parametrize("where", ["first", "last"])
def test_large_scale_with_the_argmax_at_either_end(oracle_mod, where):
    """The running maximum must see every entry: with logits ~ +-1e3 an entry
    that is missed overflows exp (inf/NaN) instead of dominating."""
    case = qi.random_case(18, T=6, S=96, Hq=1, Hkv=1, W=24)
    q, k, v = f32(case.q), f32(case.k_cache), f32(case.v_cache)
    sel = case.slot_idx.copy()
    for t in range(case.T):
        logits = k[sel[t], 0] @ q[t, 0].astype(np.float64)
        order = np.argsort(logits)            # ascending
        sel[t] = sel[t][order] if where == "last" else sel[t][order[::-1]]
    got = oracle_mod.prefill(case.q, case.k_cache, case.v_cache, sel, 80.0)
    assert np.all(np.isfinite(got))
    for t in range(case.T):
        best = sel[t, -1] if where == "last" else sel[t, 0]
        logits = np.sort(k[sel[t], 0] @ q[t, 0].astype(np.float64))
        if 80.0 * (logits[-1] - logits[-2]) > 30:
            np.testing.assert_allclose(got[t, 0], v[best, 0], rtol=1e-6, atol=1e-6)


# ---------------------------------------------------------------- FP8 KV cache

def test_e4m3_decoding_matches_torch_float8_e4m3fn(oracle_mod):
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    got = np.array([oracle_mod.e4m3_to_float(c) for c in codes], dtype=np.float32)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    np.testing.assert_array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))
    assert oracle_mod.e4m3_to_float(0x7E) == 448.0 and oracle_mod.e4m3_to_float(0x01) == 2.0**-9


def _fp8_as_bf16(codes, kv_scale):
    """Exact BF16 bits of decode(code) * kv_scale for power-of-two scales."""
    real = torch.from_numpy(codes).view(torch.float8_e4m3fn).float() * kv_scale
    bits = real.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(qi.bf16_to_f32(bits), real.numpy())     # exact
    return bits


@pytest.mark.parametrize("k_scale,v_scale", [(1.0, 1.0), (0.0078125, 4.0), (2.0**-10, 2.0**-6)])
def test_fp8_oracle_equals_bf16_oracle_on_exactly_representable_values(oracle_mod, k_scale,
                                                                        v_scale):
    case = qi.random_case(60, T=7, S=90, Hq=6, Hkv=2, W=25, pad_frac=0.2, interior=True)
    rng = np.random.Generator(np.random.PCG64(61))
    k8 = qi.e4m3_codes(rng.standard_normal(case.k_cache.shape).astype(np.float32) * 30, 1.0)
    v8 = qi.e4m3_codes(rng.standard_normal(case.v_cache.shape).astype(np.float32) * 30, 1.0)
    a = oracle_mod.prefill_fp8kv(case.q, k8, v8, k_scale, v_scale, case.slot_idx, 0.07)
    b = oracle_mod.prefill(case.q, _fp8_as_bf16(k8, k_scale), _fp8_as_bf16(v8, v_scale),
                           case.slot_idx, 0.07)
    np.testing.assert_array_equal(a, b)


def test_fp8_oracle_matches_dense_bruteforce_with_arbitrary_scales(oracle_mod):
    case = qi.with_fp8_kv(qi.random_case(62, T=6, S=48, Hq=4, Hkv=2, W=20, pad_frac=0.25,
                                         interior=True))
    k8, v8, ks, vs = (case.info[n] for n in ("k8", "v8", "k_scale", "v_scale"))
    got = oracle_mod.prefill_fp8kv(case.q, k8, v8, ks, vs, case.slot_idx, 0.0625)
    kr = torch.from_numpy(np.ascontiguousarray(k8)).view(torch.float8_e4m3fn).double() * ks
    vr = torch.from_numpy(np.ascontiguousarray(v8)).view(torch.float8_e4m3fn).double() * vs
    # brute force on the dequantized values (float64 throughout)
    q = qi.bf16_to_f32(case.q).astype(np.float64)
    k, v = kr.numpy(), vr.numpy()
    T, Hq, _ = q.shape
    G = Hq // case.Hkv
    want = np.zeros((T, Hq, 256))
    for t in range(T):
        sel = case.slot_idx[t][case.slot_idx[t] != -1]
        for h in range(Hq):
            z = 0.0625 * (k[sel, h // G] @ q[t, h])
            w = np.exp(z - z.max())
            want[t, h] = (w / w.sum()) @ v[sel, h // G]
    assert rel_l2(got, want) < 1e-5


# ---------------------------------------------------------------- micro-blocks

def test_block_expansion_hand_cases(oracle_mod):
    # block b covers slots b*bs .. b*bs + bs - 1; -1 stays "no slot"
    got = oracle_mod.expand_blocks(np.array([[3, -1, 0]], dtype=np.int32), 4)
    assert got.tolist() == [[12, 13, 14, 15, -1, -1, -1, -1, 0, 1, 2, 3]]
    got = oracle_mod.expand_blocks(np.array([[1], [-1], [2]], dtype=np.int32), 2)
    assert got.tolist() == [[2, 3], [-1, -1], [4, 5]]
    same = np.array([[5, 2, -1, 7]], dtype=np.int32)
    assert np.array_equal(oracle_mod.expand_blocks(same, 1), same)
    bad = oracle_mod.expand_blocks(np.array([[-3]], dtype=np.int32), 3)
    assert np.all(bad < -1)                 # stays invalid, not "no slot"


@pytest.mark.parametrize("bs", [2, 4, 8])
def test_block_oracle_matches_dense_bruteforce(oracle_mod, bs):
    S, T = 64, 5
    case = qi.random_case(70 + bs, T=T, S=S, Hq=4, Hkv=2, W=1)
    rng = np.random.Generator(np.random.PCG64(71 + bs))
    blocks = np.full((T, 6), -1, dtype=np.int32)
    for t in range(T):
        k = int(rng.integers(1, 6))
        blocks[t, :k] = rng.choice(S // bs, size=k, replace=False)
        blocks[t] = rng.permutation(blocks[t])
    got = oracle_mod.prefill_blocks(case.q, case.k_cache, case.v_cache, blocks, bs, 0.0625)
    member = np.zeros((T, S), dtype=bool)
    for t in range(T):
        for b in blocks[t][blocks[t] >= 0]:
            member[t, b * bs:(b + 1) * bs] = True
    dense = qi.Case("dense", case.q, case.k_cache, case.v_cache,
                    np.where(member, np.arange(S)[None, :], -1).astype(np.int32), None,
                    case.bases)
    want = dense_masked_attention_fp64(dense, 0.0625)
    assert rel_l2(got, want) < 1e-5


# ---------------------------------------------------------------- indexer + Top-K

def _slot_map(spec):
    kind, *args = spec.split(":")
    n = int(args[0])
    if kind == "identity":
        return np.arange(n, dtype=np.int32)
    a, b = int(args[1]), int(args[2])
    return (a * np.arange(n) + b).astype(np.int32)


def test_indexer_select_golden_cases(oracle_mod):
    with open(os.path.join(GOLDEN, "indexer_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        scores = np.array([c["scores"]], dtype=np.float32)
        row = oracle_mod.indexer_select(scores, np.array([c["p"]]), _slot_map(c["slot_of_pos"]),
                                        c["budget"])
        assert row[0].tolist() == c["row"], c["why"]


def test_indexer_scores_match_float64_einsum(oracle_mod):
    rng = np.random.Generator(np.random.PCG64(80))
    iq = qi.normal_bf16(rng, (9, 4, 128))
    ik = qi.normal_bf16(rng, (37, 128))
    got = oracle_mod.indexer_scores(iq, ik)
    dots = np.einsum("thd,cd->thc", f32(iq).astype(np.float64), f32(ik).astype(np.float64))
    want = np.maximum(dots, 0).sum(axis=1)
    np.testing.assert_allclose(got, want, rtol=2e-5, atol=1e-4)
    # ReLU matters: the plain sum of the dot products differs
    assert not np.allclose(got, dots.sum(axis=1), rtol=1e-3)


def test_indexer_select_properties(oracle_mod):
    rng = np.random.Generator(np.random.PCG64(81))
    T, C, budget = 40, 64, 9
    scores = rng.integers(0, 6, size=(T, C)).astype(np.float32)      # many ties
    positions = rng.integers(0, 4 * C, size=T).astype(np.int32)
    slot_of_pos = rng.permutation(4 * C).astype(np.int32)
    inv = np.argsort(slot_of_pos)
    rows = oracle_mod.indexer_select(scores, positions, slot_of_pos, budget)
    for t in range(T):
        p = int(positions[t])
        eligible = min((p + 1) // 4, C)
        r = (p + 1) % 4
        n = min(eligible, budget)
        row = rows[t]
        assert np.all(row[4 * n + r:] == -1) and np.all(row[:4 * n + r] >= 0)
        pos = inv[row[:4 * n + r]]
        blocks = pos[:4 * n].reshape(n, 4) // 4
        assert np.all(blocks == blocks[:, :1]) and np.all(np.diff(blocks[:, 0]) > 0)
        assert np.all(blocks[:, 0] * 4 + 3 <= p)
        assert pos[4 * n:].tolist() == list(range(p - r + 1, p + 1))
        chosen = set(blocks[:, 0].tolist())
        worst = min(((scores[t, c], -c) for c in chosen), default=None)
        for c in range(eligible):
            if c not in chosen:
                assert (scores[t, c], -c) < worst
