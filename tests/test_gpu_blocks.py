"""GPU parity of micro-block selections (each entry names block_size
consecutive cache slots; page "Qwen4-Exp QSA comes to Huawei's Ascend",
sections "Why QSA is the awkward part, in numbers" and "Nine tests that
passed, ..." for the block4 work).  Same gate as the slot path."""
import numpy as np
import pytest
import torch

import oracle
import qsa_inputs as qi
import top_sparse_attention_amd as qsa
from qsa_testutil import bf16_tensor_to_f32, gate, upload

pytestmark = pytest.mark.gpu

DEV = "cuda"


def block_case(seed, T, S, Hq, Hkv, nblocks, bs, pad_frac=0.0, interior=False):
    case = qi.random_case(seed, T=T, S=S // bs, Hq=Hq, Hkv=Hkv, W=nblocks, pad_frac=pad_frac,
                          interior=interior)
    rng = np.random.Generator(np.random.PCG64(seed + 1))
    k = qi.normal_bf16(rng, (S, Hkv, 256))
    v = qi.normal_bf16(rng, (S, Hkv, 256))
    case.k_cache, case.v_cache = k, v
    case.bases.update(k=k, v=v)
    case.info["block_size"] = bs
    return case


def empty_blocks(case):
    return ~np.any(case.slot_idx >= 0, axis=1)


def check_blocks(case, rows=None):
    bs = case.info["block_size"]
    q, k, v, sl = upload(case, DEV)
    out = qsa.sparse_prefill_blocks(q, k, v, sl, bs, scale=case.scale)
    torch.cuda.synchronize()
    scale = case.scale if case.scale is not None else 1.0 / 16.0
    want = oracle.prefill_blocks(case.q, case.k_cache, case.v_cache, case.slot_idx, bs, scale,
                                 rows=rows)
    got = bf16_tensor_to_f32(out if rows is None else out[torch.as_tensor(rows, device=DEV)])
    empty = empty_blocks(case) if rows is None else empty_blocks(case)[rows]
    m = gate(got, want, empty)
    print(f"{case.name} block{bs}: {m}", flush=True)
    return out, (q, k, v, sl)


@pytest.mark.parametrize("bs", [1, 2, 4, 5, 8, 16, 64])
def test_block_sizes(bs):
    S = 8000 if bs == 5 else 8192          # a multiple of the block size
    check_blocks(block_case(1000 + bs, T=29, S=S, Hq=16, Hkv=2, nblocks=400 // bs + 3, bs=bs,
                            pad_frac=0.2, interior=True))


@pytest.mark.parametrize("Hq,Hkv", [(24, 2), (12, 1), (3, 1), (32, 1)])
def test_block4_head_shapes(Hq, Hkv):
    check_blocks(block_case(1020 + Hq, T=17, S=4096, Hq=Hq, Hkv=Hkv, nblocks=129, bs=4))


def test_block_path_equals_slot_path_on_the_expanded_selection():
    """Blocks are grouped by block id exactly as their slots would be grouped
    by slot id, so both paths sum in the same order: bit-identical outputs."""
    case = block_case(1030, T=23, S=8192, Hq=16, Hkv=2, nblocks=200, bs=4, pad_frac=0.1,
                      interior=True)
    q, k, v, sl = upload(case, DEV)
    plain_ws = qsa.new_workspace(case.T, case.W * 4, DEV)   # no room for aligned lists
    out = qsa.sparse_prefill_blocks(q, k, v, sl, 4, scale=case.scale, workspace=plain_ws)
    slots = torch.from_numpy(oracle.expand_blocks(case.slot_idx, 4)).to(DEV)
    ref = qsa.sparse_prefill(q, k, v, slots)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def _key_bits(n):
    bits = 1
    while bits < 31 and (1 << bits) < n:
        bits += 1
    return bits + 1


def aligned_lists_model(block_idx, S, bs):
    """The aligned lists, written out from their rule: valid block ids grouped
    by the compaction's 128 ranges (stable), super-ranges of at most 2,048
    slots (unions of those ranges); super-range k starts at list position
    max(previous end, min(k * F, room - blocks still to place)), F =
    ceil(1.125 * blocks / ranges), room = 1.5 x the row's width (in blocks)
    rounded up to list pads.  Entries are block ids; the gaps hold -1."""
    T, W = block_idx.shape
    nb = S // bs
    group_shift = max(_key_bits(nb) - 8, 0)
    by_size = 0
    while (bs << (by_size + 1)) <= 2048:
        by_size += 1
    shift = max(group_shift, by_size)
    R = -(-nb // (1 << shift))
    room = -(-((W * 3 + 1) // 2) // 32) * 32
    rows = []
    for r in block_idx.astype(np.int64):
        valid = r[(r >= 0) & (r < nb)]
        valid = valid[np.argsort(valid >> group_shift, kind="stable")]
        n = len(valid)
        F = (33 * n + 32 * R - 1) // (32 * R)
        end, rem, out = 0, n, []
        for kk in range(R):
            seg = valid[(valid >> shift) == kk]
            cs = len(seg)
            start = max(end, min(kk * F, room - rem)) if cs else end
            out += [-1] * (start - end)
            out += seg.tolist()
            end, rem = start + cs, rem - cs
        rows.append(np.array(out, dtype=np.int64))
    return rows, room


@pytest.mark.parametrize("bs,S,nblocks", [(4, 8192, 200), (8, 16384, 120), (16, 4096, 40),
                                          (32, 65536, 70), (64, 65536, 40), (4, 65536, 2300)])
def test_aligned_block_lists_follow_their_rule(bs, S, nblocks):
    """Index work, so bit-exact: the aligned rows (block ids) the prefill
    writes into the workspace equal the rule's, and the output meets the
    gate."""
    case = block_case(1050 + bs, T=19, S=S, Hq=16, Hkv=2, nblocks=nblocks, bs=bs, pad_frac=0.15,
                      interior=True)
    case.slot_idx[3] = -1                                  # an empty row
    q, k, v, sl = upload(case, DEV)
    nbytes = qsa.prefill_blocks_workspace_bytes(case.T, case.W, bs)
    ws = torch.full((nbytes,), 0x7F, dtype=torch.uint8, device=DEV)
    out = qsa.sparse_prefill_blocks(q, k, v, sl, bs, scale=case.scale, workspace=ws)
    torch.cuda.synchronize()
    m = qsa.workspace_layout(case.T, case.W * bs)
    ext = -(-m["total_bytes"] // 256) * 256
    want, room = aligned_lists_model(case.slot_idx, S, bs)
    assert nbytes == ext + -(-(case.T * room * 4) // 256) * 256
    ws32 = ws.view(torch.int32)
    rows = ws32[ext // 4: ext // 4 + case.T * room].view(case.T, room).cpu().numpy()
    count = ws32[m["count_offset"] // 4: m["count_offset"] // 4 + case.T].cpu().numpy()
    gaps = 0
    for t in range(case.T):
        assert count[t] == len(want[t]), t
        assert np.array_equal(rows[t, :count[t]], want[t]), t
        padded = -(-count[t] // 32) * 32
        assert np.all(rows[t, count[t]:padded] == -1), t
        gaps += int((want[t] == -1).sum())
    assert gaps > 0                                         # the rule did insert gaps
    scale = case.scale if case.scale is not None else 1.0 / 16.0
    ref = oracle.prefill_blocks(case.q, case.k_cache, case.v_cache, case.slot_idx, bs, scale)
    print(gate(bf16_tensor_to_f32(out), ref, empty_blocks(case)), "gaps", gaps)


def test_aligned_and_plain_block_paths_agree_within_rounding():
    case = block_case(1060, T=40, S=8192, Hq=24, Hkv=2, nblocks=300, bs=4, pad_frac=0.05)
    q, k, v, sl = upload(case, DEV)
    aligned = qsa.sparse_prefill_blocks(q, k, v, sl, 4)
    plain = qsa.sparse_prefill_blocks(q, k, v, sl, 4,
                                      workspace=qsa.new_workspace(case.T, case.W * 4, DEV))
    torch.cuda.synchronize()
    a, p = bf16_tensor_to_f32(aligned), bf16_tensor_to_f32(plain)
    assert np.all(np.abs(a - p) <= 2.0 ** -7 * np.abs(p) + 1e-4)
    ref = oracle.prefill_blocks(case.q, case.k_cache, case.v_cache, case.slot_idx, 4, 1.0 / 16.0)
    print(gate(a, ref, empty_blocks(case)))


def test_block_compaction_counts_slots_and_invalid_blocks():
    case = block_case(1040, T=12, S=2048, Hq=2, Hkv=1, nblocks=60, bs=4, pad_frac=0.3,
                      interior=True)
    case.slot_idx[2, 0] = 512           # one past the last block
    case.slot_idx[5, 1] = -9
    _, _, _, sl = upload(case, DEV)
    ws = qsa.compact_blocks(sl, 2048, 4)
    torch.cuda.synchronize()
    lst, cnt, bad = (x.cpu().numpy() for x in qsa.compacted_lists(ws, case.T, case.W * 4))
    for t in range(case.T):
        row = case.slot_idx[t]
        good = row[(row >= 0) & (row < 512)]
        assert cnt[t] == 4 * good.size
        assert sorted(lst[t, :cnt[t]].tolist()) == sorted((good[:, None] * 4 + np.arange(4))
                                                          .ravel().tolist())
        assert bad[t] == (1 if t in (2, 5) else 0)
    with pytest.raises(qsa.QsaError):
        qsa.check_status(ws, case.T, case.W * 4)


def test_block_size_must_divide_the_cache():
    case = block_case(1050, T=3, S=64, Hq=2, Hkv=1, nblocks=4, bs=4)
    q, k, v, sl = upload(case, DEV)
    with pytest.raises(qsa.QsaError) as e:
        qsa.sparse_prefill_blocks(q, k[:63], v[:63], sl, 4)
    assert e.value.status == 2


def test_long_prefill_block4_sampled_rows():
    case = qi.long_prefill_blocks()
    rows = qi.sample_rows(case.T, 64)
    out, _ = check_blocks(case, rows)
    assert torch.isfinite(out.float()).all()


def test_aligned_block_prefill_reports_invalid_blocks():
    """The aligned path keeps the standard layout's status words: qsa_check_status
    (width W * block_size) counts the blocks that were neither -1 nor in range."""
    case = block_case(1070, T=30, S=8192, Hq=16, Hkv=2, nblocks=150, bs=4, pad_frac=0.1,
                      interior=True)
    case.slot_idx[4, 7] = 2048            # one past the last block
    case.slot_idx[9, 0] = -3
    case.slot_idx[9, 1] = 1 << 29
    q, k, v, sl = upload(case, DEV)
    ws = torch.empty(qsa.prefill_blocks_workspace_bytes(case.T, case.W, 4), dtype=torch.uint8,
                     device=DEV)
    out = qsa.sparse_prefill_blocks(q, k, v, sl, 4, workspace=ws)
    torch.cuda.synchronize()
    with pytest.raises(qsa.QsaError) as e:
        qsa.check_status(ws, case.T, case.W * 4)
    assert e.value.status == 6 and "3 selection entries" in str(e.value)
    valid = np.where((case.slot_idx >= 0) & (case.slot_idx < 2048), case.slot_idx, -1)
    ref = oracle.prefill_blocks(case.q, case.k_cache, case.v_cache, valid.astype(np.int32), 4,
                                1.0 / 16.0)
    print(gate(bf16_tensor_to_f32(out), ref, ~np.any(valid >= 0, axis=1)))


@pytest.mark.parametrize("bs,S,nblocks", [(4, 65536, 2400), (5, 20000, 300), (2, 8192, 300)])
def test_other_block_rows_take_the_plain_lists(bs, S, nblocks):
    """Rows of more than one sort run (2,304 blocks), block sizes that are not
    powers of two, and blocks of fewer than 4 slots run the plain lists: the
    aligned area stays as it was, and the output meets the gate."""
    case = block_case(1080 + bs, T=21, S=S, Hq=16, Hkv=2, nblocks=nblocks, bs=bs, pad_frac=0.1,
                      interior=True)
    q, k, v, sl = upload(case, DEV)
    nbytes = qsa.prefill_blocks_workspace_bytes(case.T, case.W, bs)
    ws = torch.full((nbytes,), 0x7F, dtype=torch.uint8, device=DEV)
    out = qsa.sparse_prefill_blocks(q, k, v, sl, bs, scale=case.scale, workspace=ws)
    torch.cuda.synchronize()
    m = qsa.workspace_layout(case.T, case.W * bs)
    ext = -(-m["total_bytes"] // 256) * 256
    assert torch.all(ws[ext:] == 0x7F)
    ref = oracle.prefill_blocks(case.q, case.k_cache, case.v_cache, case.slot_idx, bs, 1.0 / 16.0)
    print(gate(bf16_tensor_to_f32(out), ref, empty_blocks(case)))
