"""Structure of the seeded synthetic workloads (no GPU)."""
import numpy as np
import pytest
import torch

import qsa_inputs as qi


def test_bf16_rounding_matches_torch_round_to_nearest_even():
    rng = np.random.Generator(np.random.PCG64(1))
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0, -0.0, 0.0, 3.0e38, 1e-40, 1.00390625, 1.01171875],
                                 dtype=np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(qi.bf16_bits(x), want)
    np.testing.assert_array_equal(qi.bf16_to_f32(want),
                                  torch.from_numpy(want.view(np.int16)).view(torch.bfloat16)
                                  .float().numpy())


def test_generation_is_deterministic():
    a, b = qi.tiny(), qi.tiny()
    for name in ("q", "k_cache", "v_cache", "slot_idx"):
        np.testing.assert_array_equal(getattr(a, name), getattr(b, name))
    c = qi.tiny(seed=999)
    assert not np.array_equal(a.q, c.q)


def test_distinct_draws_are_distinct_and_in_range():
    rng = np.random.Generator(np.random.PCG64(3))
    high = np.array([10, 50, 2000, 7])
    a = qi.distinct_draws(rng, high, 4, 7)
    for t in range(4):
        assert len(set(a[t].tolist())) == 7
        assert a[t].min() >= 0 and a[t].max() < high[t]


def _assert_distinct_valid_rows(sel, S):
    for t in range(sel.shape[0]):
        row = sel[t][sel[t] != -1]
        assert np.all((row >= 0) & (row < S))
        assert np.unique(row).size == row.size


def test_tiny_workload():
    c = qi.tiny()
    assert (c.T, c.S, c.Hq, c.Hkv, c.D, c.W) == (64, 1024, 16, 2, 256, 64)
    assert c.scale == 1.0 / 16.0
    _assert_distinct_valid_rows(c.slot_idx, c.S)
    assert np.all(c.slot_idx >= 0)
    # unordered: rows are not sorted
    assert not all(np.all(np.diff(r) > 0) for r in c.slot_idx)


def test_edge_mix_workload():
    c = qi.edge_mix()
    assert (c.T, c.S, c.Hq, c.Hkv, c.D, c.W) == (257, 4096, 12, 1, 256, 2051)
    assert c.scale == 0.05
    assert not c.q.flags.c_contiguous and c.q.strides[0] == 2 * 12 * 256 * 2
    assert not c.k_cache.flags.c_contiguous and c.k_cache.strides[0] == 2 * 256 * 2
    assert c.base_of(c.k_cache) is c.base_of(c.v_cache)          # one interleaved buffer
    _assert_distinct_valid_rows(c.slot_idx, c.S)
    n_valid = (c.slot_idx != -1).sum(axis=1)
    interior_seen = False
    for t in range(c.T):
        want = 0 if t % 16 == 7 else qi.EDGE_WIDTHS[t % 6]
        assert n_valid[t] == want
        row = c.slot_idx[t]
        if t % 5 != 3 and want:
            assert np.all(row[:want] != -1) and np.all(row[want:] == -1)
        if t % 5 == 3 and 0 < want < c.W:
            last_valid = np.nonzero(row != -1)[0].max()
            interior_seen |= bool(last_valid >= want)
    assert interior_seen


def test_two_request_workload_structure():
    c = qi.two_request()
    assert (c.T, c.S, c.Hq, c.Hkv, c.W) == (8192, 131072, 24, 2, 2048)
    perm, pos, req = c.info["perm"], c.info["positions"], c.info["request"]
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size)
    rows = np.concatenate([np.arange(0, 40), np.arange(4090, 4100), np.arange(8150, 8192)])
    for t in rows:
        sl = c.slot_idx[t]
        assert np.all(sl >= 0) and np.unique(sl).size == sl.size
        idx = inv[sl]                       # index into the permutation
        base = qi.PREFIX + req[t] * qi.NEW_PER_REQUEST
        in_prefix = idx < qi.PREFIX
        logical = np.where(in_prefix, idx, idx - base + qi.PREFIX)
        # new-token slots belong to this request's own range
        assert np.all((idx[~in_prefix] >= base) & (idx[~in_prefix] < base + qi.NEW_PER_REQUEST))
        # causal: nothing after the query position; the tail r is present
        assert logical.max() <= pos[t]
        r = (pos[t] + 1) % 4
        assert set(range(pos[t] - r + 1, pos[t] + 1)) <= set(logical.tolist())
    # remainders 0..3 all occur
    assert set(c.info["tail"].tolist()) == {0, 1, 2, 3}


@pytest.mark.parametrize("heads", [(6, 1), (3, 1)])
def test_max_cache_workload_shapes(heads):
    c = qi.max_cache(heads=heads)
    assert (c.T, c.S, c.Hq, c.Hkv, c.W) == (16384, 262144, heads[0], heads[1], 2048)
    _assert_distinct_valid_rows(c.slot_idx[:64], c.S)
    assert c.k_cache.nbytes + c.v_cache.nbytes == 262144 * 256 * 2 * 2


def test_sample_rows_includes_ends():
    r = qi.sample_rows(7810, 64)
    assert r[0] == 0 and r[-1] == 7809 and r.size == 64 and np.all(np.diff(r) > 0)
