"""The prefill (every attention layout), FP8 prefill, micro-block prefill,
decode, FP8 decode and indexer paths captured in a HIP graph.

These paths record no memset and make no synchronous call, so a captured
step replays exactly: every replay is compared bit for bit with the eager
result.  Between replays the output is overwritten with a sentinel and other
eager work and synchronizations run, so a replay that skipped a kernel, or
read a stale buffer, shows.
"""
import numpy as np
import pytest
import torch

import qsa_inputs as qi
import top_sparse_attention_amd as qsa
from qsa_testutil import upload, upload_fp8

pytestmark = pytest.mark.gpu

DEV = "cuda"
REPLAYS = 4


def replay_matches_eager(step, out):
    """Run `step` (which writes `out`) eagerly, capture it, and check every
    replay against the eager bits."""
    step()
    torch.cuda.synchronize()
    eager = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    scratch = torch.randn(512, 512, device=DEV)
    for r in range(REPLAYS):
        if out.dtype == torch.bfloat16:
            out.view(torch.int16).fill_(0x3F3F)        # a sentinel the step never writes
        else:
            out.fill_(0x3F3F3F3F)
        torch.cuda.synchronize()
        graph.replay()
        scratch = scratch @ scratch.T / 512.0      # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out,
                           eager.view(torch.int16) if eager.dtype == torch.bfloat16 else eager), \
            f"replay {r} differs from the eager result"
    assert torch.isfinite(scratch).all()


def test_prefill_graph_replays_exactly():
    case = qi.random_case(1201, T=300, S=20000, Hq=16, Hkv=2, W=700, pad_frac=0.1,
                          interior=True)
    q, k, v, sl = upload(case, DEV)
    out = torch.empty_like(q)
    ws = qsa.new_workspace(case.T, case.W, DEV)
    replay_matches_eager(lambda: qsa.sparse_prefill(q, k, v, sl, out=out, workspace=ws), out)


def test_fp8_prefill_graph_replays_exactly():
    case = qi.with_fp8_kv(qi.random_case(1202, T=200, S=12000, Hq=8, Hkv=1, W=900))
    q, _, _, sl = upload(case, DEV)
    k8, v8, ks, vs = upload_fp8(case, DEV)
    out = torch.empty_like(q)
    ws = qsa.new_workspace(case.T, case.W, DEV)
    replay_matches_eager(
        lambda: qsa.sparse_prefill_fp8kv(q, k8, v8, ks, vs, sl, out=out, workspace=ws), out)


def test_block_prefill_with_aligned_lists_graph_replays_exactly():
    case = qi.random_case(1206, T=150, S=4096, Hq=16, Hkv=2, W=300, pad_frac=0.1,
                          interior=True)                  # block ids in [0, 4096), blocks of 4
    rng = np.random.Generator(np.random.PCG64(1207))
    q, _, _, sl = upload(case, DEV)
    k = torch.from_numpy(qi.normal_bf16(rng, (4 * case.S, case.Hkv, 256)).view(np.int16)).to(DEV)
    v = torch.from_numpy(qi.normal_bf16(rng, (4 * case.S, case.Hkv, 256)).view(np.int16)).to(DEV)
    k, v = k.view(torch.bfloat16), v.view(torch.bfloat16)
    out = torch.empty_like(q)
    ws = torch.empty(qsa.prefill_blocks_workspace_bytes(case.T, case.W, 4), dtype=torch.uint8,
                     device=DEV)
    replay_matches_eager(
        lambda: qsa.sparse_prefill_blocks(q, k, v, sl, 4, out=out, workspace=ws), out)


def test_decode_graph_replays_exactly():
    case = qi.random_case(1203, T=8, S=60000, Hq=24, Hkv=2, W=2048)
    q, k, v, sl = upload(case, DEV)
    out = torch.empty_like(q)
    nbytes = qsa.decode_workspace_bytes(case.T, case.W, case.Hq, case.Hkv)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    replay_matches_eager(lambda: qsa.sparse_decode(q, k, v, sl, out=out, workspace=ws), out)


def test_fp8_decode_graph_replays_exactly():
    case = qi.with_fp8_kv(qi.random_case(1208, T=6, S=30000, Hq=16, Hkv=2, W=1500,
                                         pad_frac=0.1, interior=True))
    q, _, _, sl = upload(case, DEV)
    k8, v8, ks, vs = upload_fp8(case, DEV)
    out = torch.empty_like(q)
    ws = torch.empty(qsa.decode_workspace_bytes(case.T, case.W, case.Hq, case.Hkv),
                     dtype=torch.uint8, device=DEV)
    replay_matches_eager(
        lambda: qsa.sparse_decode_fp8kv(q, k8, v8, ks, vs, sl, out=out, workspace=ws), out)


def test_indexer_topk_graph_replays_exactly():
    case = qi.indexed_case(1204, L=20000, T=64, Hq=8, Hkv=1, budget=256)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    iq = t(case.info["iq"].view(np.int16)).view(torch.bfloat16)
    ik = t(case.info["ik"].view(np.int16)).view(torch.bfloat16)
    pos, sop = t(case.info["positions"]), t(case.info["slot_of_pos"])
    scores = torch.empty((case.T, ik.shape[0]), dtype=torch.float32, device=DEV)
    sel = torch.empty((case.T, 4 * 256 + 3), dtype=torch.int32, device=DEV)
    replay_matches_eager(lambda: qsa.indexer_topk(iq, ik, pos, sop, 256, scores=scores, out=sel),
                         sel)


def test_prefill_with_sharing_estimate_graph_replays_exactly():
    # A large cache against W: the sharing estimate runs, then the gated
    # attention launches.
    case = qi.random_case(1205, T=4096, S=131072, Hq=3, Hkv=1, W=512)
    q, k, v, sl = upload(case, DEV)
    out = torch.empty_like(q)
    ws = qsa.new_workspace(case.T, case.W, DEV)
    replay_matches_eager(lambda: qsa.sparse_prefill(q, k, v, sl, out=out, workspace=ws), out)


def test_prefill_with_keys_through_lds_graph_replays_exactly():
    # High sharing hidden in a large cache: the estimate picks the gated
    # keys-through-LDS launch (choice 2) on every replay.
    base = qi.random_case(1209, T=4096, S=30000, Hq=3, Hkv=1, W=2048)
    q, kb, vb, slb = upload(base, DEV)
    S = 262144
    new_of_old = torch.from_numpy(
        np.random.Generator(np.random.PCG64(1210)).permutation(S)[:base.S].astype(np.int64)
    ).to(DEV)
    k = torch.zeros((S, 1, 256), dtype=torch.bfloat16, device=DEV)
    v = torch.zeros_like(k)
    k[new_of_old] = kb
    v[new_of_old] = vb
    sl = new_of_old[slb.long()].to(torch.int32)
    out = torch.empty_like(q)
    ws = qsa.new_workspace(base.T, base.W, DEV)
    replay_matches_eager(lambda: qsa.sparse_prefill(q, k, v, sl, out=out, workspace=ws), out)
    off = qsa.workspace_layout(base.T, base.W)["share_offset"] + 32 * 8
    assert int(ws[off:off + 4].view(torch.int32).item()) == 2
