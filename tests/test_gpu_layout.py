"""The attention's layout choice and its sharing estimate.

Where the sizes leave the cache large against the selection width, a small
kernel samples pairs of neighbouring tokens, counts their common slots and
picks 4 items per CU if the tokens running together share few cache rows,
8 with the keys taken through LDS (BF16) if they share many, else 8 as they
are.  Where the sizes alone bound the sharing high, no estimate runs.
These tests check the choice the estimate writes into the workspace on
selections of known sharing, that every layout gives the oracle's result
within the gate, and that they give the same bits.
"""
import numpy as np
import pytest
import torch

import oracle
import qsa_inputs as qi
import top_sparse_attention_amd as qsa
from qsa_testutil import (bf16_tensor_bits, bf16_tensor_to_f32, empty_row_mask, gate, upload,
                          upload_fp8)

pytestmark = pytest.mark.gpu

DEV = "cuda"
SHARE_PAIRS = 32          # token pairs the estimate samples
# The choice word follows the pairs' (common, length) floats.
CHOICE_BYTE = SHARE_PAIRS * 8


def choice_of(ws: torch.Tensor, T: int, W: int) -> int:
    off = qsa.workspace_layout(T, W)["share_offset"] + CHOICE_BYTE
    return int(ws[off:off + 4].view(torch.int32).item())


def check_rows(out, q_np, k_np, v_np, sl_np, S, rows):
    want = oracle.prefill(np.ascontiguousarray(q_np[rows]), k_np, v_np,
                          np.ascontiguousarray(sl_np[rows]), 1.0 / 16.0)
    got = bf16_tensor_to_f32(out[torch.as_tensor(rows, device=DEV)])
    return gate(got, want, empty_row_mask(sl_np, S, rows))


def prefill_with_choice(q, k, v, sl):
    T, W = sl.shape
    ws = qsa.new_workspace(T, W, DEV)
    # A value the estimate never writes, so a missing write shows.
    off = qsa.workspace_layout(T, W)["share_offset"] + CHOICE_BYTE
    ws[off:off + 4].view(torch.int32).fill_(-7)
    out = qsa.sparse_prefill(q, k, v, sl, workspace=ws)
    torch.cuda.synchronize()
    return out, choice_of(ws, T, W)


def test_large_cache_with_little_sharing_takes_four_per_cu_and_same_bits():
    # 2,048 random slots of 262,144 per token, one KV head: each row is read by
    # about 2 of the 256 tokens an XCD runs at a time.
    case = qi.random_case(1301, T=4096, S=262144, Hq=3, Hkv=1, W=2048)
    q, k, v, sl = upload(case, DEV)
    out, choice = prefill_with_choice(q, k, v, sl)
    assert choice == 1
    rows = qi.sample_rows(case.T, 24, seed=31)
    print(check_rows(out, case.q, case.k_cache, case.v_cache, case.slot_idx, case.S, rows))
    # The same selections padded to width 8,192 with -1: from the sizes
    # alone the sharing is at least 256 * 8192 / 262144 = 8, so the general
    # layout runs without an estimate.  Same valid entries, same bits.
    padded = torch.full((case.T, 8192), -1, dtype=torch.int32, device=DEV)
    padded[:, :case.W] = sl
    out8 = qsa.sparse_prefill(q, k, v, padded)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_tensor_bits(out8), bf16_tensor_bits(out))


def test_two_kv_heads_at_sharing_four_take_four_per_cu():
    case = qi.random_case(1302, T=4096, S=131072, Hq=16, Hkv=2, W=2051)
    q, k, v, sl = upload(case, DEV)
    out, choice = prefill_with_choice(q, k, v, sl)
    assert choice == 1
    rows = qi.sample_rows(case.T, 16, seed=32)
    print(check_rows(out, case.q, case.k_cache, case.v_cache, case.slot_idx, case.S, rows))


def direct_keys_reference(q, k, v, sl, S):
    """The same attention through the split kernel with one share (keys
    gathered straight into the score operands) and the merge: one share's
    O / l, the same bits as the unsplit kernel's."""
    T, W = sl.shape
    ws = qsa.compact_slots(sl, S)
    parts = qsa.new_partials(1, T, q.shape[1], DEV)
    qsa.sparse_attend_partial(q, k, v, ws, W, 1, 0, 1, parts)
    out = qsa.merge_partials(parts, 1, T, q.shape[1])
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("referenced,want_choice", [(40000, 2), (75000, 0)])
def test_large_cache_with_a_small_referenced_part(referenced, want_choice):
    # The tokens select among `referenced` slots scattered over a 262,144-slot
    # cache: the sizes suggest little sharing, the lists show about
    # 256 * 2048 / referenced readers per row: 13 (keys through LDS) or 7
    # (the general layout as it is).
    base = qi.random_case(1303, T=4096, S=referenced, Hq=3, Hkv=1, W=2048)
    q, kb, vb, slb = upload(base, DEV)
    S = 262144
    new_of_old = torch.from_numpy(
        np.random.Generator(np.random.PCG64(1304)).permutation(S)[:base.S].astype(np.int64)
    ).to(DEV)
    k = torch.zeros((S, 1, 256), dtype=torch.bfloat16, device=DEV)
    v = torch.zeros_like(k)
    k[new_of_old] = kb
    v[new_of_old] = vb
    sl = new_of_old[slb.long()].to(torch.int32)
    out, choice = prefill_with_choice(q, k, v, sl)
    assert choice == want_choice
    rows = qi.sample_rows(base.T, 16, seed=33)
    # Relocated rows: the oracle of the original cache gives the same result.
    print(check_rows(out, base.q, base.k_cache, base.v_cache, base.slot_idx, base.S, rows))
    ref = direct_keys_reference(q, k, v, sl, S)
    assert np.array_equal(bf16_tensor_bits(out), bf16_tensor_bits(ref))


def test_sizes_alone_take_keys_through_lds_with_the_same_bits():
    # 2,048 of 16,384 slots per token, (16,2): the sizes bound the sharing at
    # 256 * 2048 / 16384 = 32, so the keys-through-LDS form runs without an
    # estimate (the choice word is not written).
    case = qi.random_case(1309, T=4096, S=16384, Hq=16, Hkv=2, W=2048, pad_frac=0.05,
                          interior=True)
    q, k, v, sl = upload(case, DEV)
    out, choice = prefill_with_choice(q, k, v, sl)
    assert choice == -7
    rows = qi.sample_rows(case.T, 16, seed=37)
    print(check_rows(out, case.q, case.k_cache, case.v_cache, case.slot_idx, case.S, rows))
    ref = direct_keys_reference(q, k, v, sl, case.S)
    assert np.array_equal(bf16_tensor_bits(out), bf16_tensor_bits(ref))


# Sizes bounding the sharing at 9 or more for other head shapes, widths and
# padding: (Hq, Hkv, T, S, W, pad).  G = 20 runs two head blocks per KV head;
# W = 33 leaves a one-slot last tile.
@pytest.mark.parametrize("Hq,Hkv,T,S,W,pad", [(40, 2, 1100, 20000, 1000, 0.1),
                                              (3, 1, 4096, 16000, 777, 0.3),
                                              (16, 2, 4096, 1024, 33, 0.0)])
def test_keys_through_lds_across_shapes(Hq, Hkv, T, S, W, pad):
    case = qi.random_case(1310 + Hq, T=T, S=S, Hq=Hq, Hkv=Hkv, W=W, pad_frac=pad, interior=True)
    q, k, v, sl = upload(case, DEV)
    out, choice = prefill_with_choice(q, k, v, sl)
    assert choice == -7      # no estimate: the sizes decide
    rows = qi.sample_rows(case.T, 12, seed=38)
    print(check_rows(out, case.q, case.k_cache, case.v_cache, case.slot_idx, case.S, rows))
    ref = direct_keys_reference(q, k, v, sl, case.S)
    assert np.array_equal(bf16_tensor_bits(out), bf16_tensor_bits(ref))


def test_keys_through_lds_over_interleaved_cache_views():
    """K and V as views of one [S, 2, Hkv, 256] buffer (slot stride 2 rows)."""
    case = qi.random_case(1320, T=4096, S=12000, Hq=16, Hkv=2, W=1500, pad_frac=0.1,
                          interior=True)
    q, k0, v0, sl = upload(case, DEV)
    kv = torch.empty((case.S, 2, case.Hkv, 256), dtype=torch.bfloat16, device=DEV)
    kv[:, 0] = k0
    kv[:, 1] = v0
    k, v = kv[:, 0], kv[:, 1]
    assert k.stride(0) == 2 * case.Hkv * 256
    out, choice = prefill_with_choice(q, k, v, sl)
    assert choice == -7
    rows = qi.sample_rows(case.T, 12, seed=39)
    print(check_rows(out, case.q, case.k_cache, case.v_cache, case.slot_idx, case.S, rows))
    ref = direct_keys_reference(q, k, v, sl, case.S)
    assert np.array_equal(bf16_tensor_bits(out), bf16_tensor_bits(ref))


def test_fp8_cache_with_more_than_eight_heads_per_kv_head_takes_four_per_cu():
    # FP8 caches with G > 8 run the general layout, so the estimate applies.
    case = qi.with_fp8_kv(qi.random_case(1305, T=4096, S=131072, Hq=12, Hkv=1, W=1024))
    q, _, _, sl = upload(case, DEV)
    k8, v8, ks, vs = upload_fp8(case, DEV)
    ws = qsa.new_workspace(case.T, case.W, DEV)
    off = qsa.workspace_layout(case.T, case.W)["share_offset"] + CHOICE_BYTE
    ws[off:off + 4].view(torch.int32).fill_(-7)
    out = qsa.sparse_prefill_fp8kv(q, k8, v8, ks, vs, sl, workspace=ws)
    torch.cuda.synchronize()
    assert choice_of(ws, case.T, case.W) == 1
    rows = qi.sample_rows(case.T, 16, seed=34)
    want = oracle.prefill_fp8kv(case.q, case.info["k8"], case.info["v8"], ks, vs,
                                case.slot_idx, 1.0 / 16.0, rows=rows)
    got = bf16_tensor_to_f32(out[torch.as_tensor(rows, device=DEV)])
    print(gate(got, want, empty_row_mask(case.slot_idx, case.S, rows)))
    # Padded to width 8,192 the sizes bound the sharing at 16: general layout.
    padded = torch.full((case.T, 8192), -1, dtype=torch.int32, device=DEV)
    padded[:, :case.W] = sl
    out8 = qsa.sparse_prefill_fp8kv(q, k8, v8, ks, vs, padded)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_tensor_bits(out8), bf16_tensor_bits(out))


def test_block_selections_on_a_large_cache_take_the_estimate():
    """Micro-block selections reach the estimate through the block compaction
    (list width 512 blocks x 4 slots against 262,144 slots)."""
    T, S, bs, nblocks = 4096, 262144, 4, 512
    sel = qi.random_case(1306, T=T, S=S // bs, Hq=3, Hkv=1, W=nblocks)
    rng = np.random.Generator(np.random.PCG64(1307))
    k_np = qi.normal_bf16(rng, (S, 1, 256))
    v_np = qi.normal_bf16(rng, (S, 1, 256))
    q = torch.from_numpy(sel.q.view(np.int16)).to(DEV).view(torch.bfloat16)
    k = torch.from_numpy(k_np.view(np.int16)).to(DEV).view(torch.bfloat16)
    v = torch.from_numpy(v_np.view(np.int16)).to(DEV).view(torch.bfloat16)
    bl = torch.from_numpy(sel.slot_idx.astype(np.int32)).to(DEV)
    Wl = nblocks * bs
    ws = qsa.new_workspace(T, Wl, DEV)
    off = qsa.workspace_layout(T, Wl)["share_offset"] + CHOICE_BYTE
    ws[off:off + 4].view(torch.int32).fill_(-7)
    out = qsa.sparse_prefill_blocks(q, k, v, bl, bs, workspace=ws)
    torch.cuda.synchronize()
    assert choice_of(ws, T, Wl) == 1
    rows = qi.sample_rows(T, 12, seed=35)
    slots = oracle.expand_blocks(sel.slot_idx[rows], bs)
    want = oracle.prefill(np.ascontiguousarray(sel.q[rows]), k_np, v_np, slots, 1.0 / 16.0)
    got = bf16_tensor_to_f32(out[torch.as_tensor(rows, device=DEV)])
    print(gate(got, want, empty_row_mask(slots, S)))


def test_mostly_empty_rows_with_the_estimate():
    """Nine rows in ten select nothing: sampled pairs with empty lists count
    nothing, and every output row is right whichever layout is taken (empty
    rows exactly +0.0)."""
    case = qi.random_case(1308, T=4096, S=262144, Hq=6, Hkv=1, W=2048)
    empty = np.arange(case.T) % 10 != 3
    case.slot_idx[empty] = -1
    q, k, v, sl = upload(case, DEV)
    out, choice = prefill_with_choice(q, k, v, sl)
    assert choice in (0, 1, 2)
    rows = np.unique(np.concatenate([qi.sample_rows(case.T, 10, seed=36), [3, 13, 4093]]))
    print(check_rows(out, case.q, case.k_cache, case.v_cache, case.slot_idx, case.S, rows))
    assert torch.count_nonzero(out[torch.as_tensor(np.flatnonzero(empty), device=DEV)]) == 0
