"""GPU parity of the FP8 E4M3 KV-cache variant against the FP32 oracle.

Reading (the page names an fp8_e4m3 KV cache in section "Where this sits in
the Qwen4Exp serving build-out" but defines no scaling): one scale per
tensor, element = decode(code) * scale.  Same gate as the BF16 path.
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


def run_fp8(case, out=None):
    q, _, _, sl = upload(case, DEV)
    k8, v8, ks, vs = upload_fp8(case, DEV)
    o = qsa.sparse_prefill_fp8kv(q, k8, v8, ks, vs, sl, scale=case.scale, out=out)
    torch.cuda.synchronize()
    return o


def oracle_fp8(case, rows=None):
    scale = case.scale if case.scale is not None else 1.0 / 16.0
    return oracle.prefill_fp8kv(case.q, case.info["k8"], case.info["v8"], case.info["k_scale"],
                                case.info["v_scale"], case.slot_idx, scale, rows=rows)


def check_fp8(case, rows=None):
    o = run_fp8(case)
    got = bf16_tensor_to_f32(o if rows is None else o[torch.as_tensor(rows, device=DEV)])
    m = gate(got, oracle_fp8(case, rows), empty_row_mask(case.slot_idx, case.S, rows))
    print(f"{case.name} fp8: {m}", flush=True)
    return o


def test_fp8_tiny():
    check_fp8(qi.with_fp8_kv(qi.tiny()))


def test_fp8_edge_mix_strided_views():
    case = qi.with_fp8_kv(qi.edge_mix())
    assert case.info["k8"].strides[0] == 512          # K and V interleaved per slot
    check_fp8(case)


@pytest.mark.parametrize("Hq,Hkv", [(16, 2), (24, 2), (12, 1), (6, 1), (3, 1), (20, 1)])
def test_fp8_head_shapes(Hq, Hkv):
    case = qi.with_fp8_kv(qi.random_case(900 + Hq + Hkv, T=37, S=5000, Hq=Hq, Hkv=Hkv, W=333,
                                         pad_frac=0.15, interior=True))
    check_fp8(case)


@pytest.mark.parametrize("W", [1, 15, 16, 17, 2051])
def test_fp8_widths(W):
    check_fp8(qi.with_fp8_kv(qi.random_case(920 + W, T=11, S=6000, Hq=8, Hkv=1, W=W,
                                            scale=0.09)))


def test_fp8_single_slot_rows_are_bit_exact():
    case = qi.with_fp8_kv(qi.random_case(930, T=20, S=700, Hq=6, Hkv=2, W=5, pad_frac=0.8,
                                         interior=True))
    o = run_fp8(case)
    want = oracle_fp8(case)
    want_bits = torch.from_numpy(want).to(torch.bfloat16).view(torch.int16).numpy()
    np.testing.assert_array_equal(bf16_tensor_bits(o).view(np.int16), want_bits)


@pytest.mark.parametrize("k_scale,v_scale", [(1.0, 1.0), (2.0**-7, 4.0)])
def test_fp8_equals_bf16_path_for_power_of_two_scales(k_scale, v_scale):
    """decode(code) * 2^k is exact in BF16, and folding a power of two into
    the softmax scale or the output commutes with rounding: both GPU paths
    must agree bit for bit."""
    case = qi.random_case(940, T=29, S=4000, Hq=16, Hkv=2, W=700, pad_frac=0.1)
    rng = np.random.Generator(np.random.PCG64(941))
    k8 = qi.e4m3_codes(rng.standard_normal(case.k_cache.shape).astype(np.float32) * 40, 1.0)
    v8 = qi.e4m3_codes(rng.standard_normal(case.v_cache.shape).astype(np.float32) * 40, 1.0)
    q, _, _, sl = upload(case, DEV)
    k8_t, v8_t = torch.from_numpy(k8).to(DEV), torch.from_numpy(v8).to(DEV)
    a = qsa.sparse_prefill_fp8kv(q, k8_t, v8_t, k_scale, v_scale, sl)
    kb = (k8_t.view(torch.float8_e4m3fn).float() * k_scale).to(torch.bfloat16)
    vb = (v8_t.view(torch.float8_e4m3fn).float() * v_scale).to(torch.bfloat16)
    b = qsa.sparse_prefill(q, kb, vb, sl)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_fp8_gather_only_reads_exactly_the_selected_rows():
    case = qi.with_fp8_kv(qi.random_case(950, T=21, S=2500, Hq=4, Hkv=2, W=150, pad_frac=0.3,
                                         interior=True))
    _, _, _, sl = upload(case, DEV)
    k8, v8, _, _ = upload_fp8(case, DEV)
    ws = qsa.compact_slots(sl, case.S)
    sink = qsa.gather_only_fp8kv(k8, v8, ws, case.T, case.W)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    kw = np.ascontiguousarray(case.info["k8"]).view(np.uint32)
    vw = np.ascontiguousarray(case.info["v8"]).view(np.uint32)
    for t in range(case.T):
        sel = case.slot_idx[t][case.slot_idx[t] != -1]
        for g in range(case.Hkv):
            want = np.bitwise_xor.reduce(np.concatenate([kw[sel, g].ravel(), vw[sel, g].ravel()]))
            assert got[t * case.Hkv + g] == (want if sel.size else 0)


def test_fp8_long_prefill_sampled_rows():
    case = qi.with_fp8_kv(qi.long_prefill())
    rows = qi.sample_rows(case.T, 64)
    o = check_fp8(case, rows)
    assert torch.isfinite(o.float()).all()


# ---------------------------------------------------------------- decode

def run_decode_fp8(case, slot_idx=None, workspace=None):
    q, _, _, sl = upload(case, DEV)
    if slot_idx is not None:
        sl = torch.from_numpy(np.ascontiguousarray(slot_idx, dtype=np.int32)).to(DEV)
    k8, v8, ks, vs = upload_fp8(case, DEV)
    o = qsa.sparse_decode_fp8kv(q, k8, v8, ks, vs, sl, scale=case.scale, workspace=workspace)
    torch.cuda.synchronize()
    return o


def test_fp8_decode_batch_workload():
    case = qi.with_fp8_kv(qi.decode_batch())
    o = run_decode_fp8(case)
    m = gate(bf16_tensor_to_f32(o), oracle_fp8(case), empty_row_mask(case.slot_idx, case.S))
    print(f"{case.name} fp8 decode: {m}", flush=True)


# G <= 8 takes the 8-query-row layout, larger groups the 16-row one (two
# head blocks at G = 20).
@pytest.mark.parametrize("T,Hq,Hkv,W,pad", [(1, 16, 2, 2048, 0.0), (2, 24, 2, 300, 0.3),
                                           (5, 12, 1, 2051, 0.5), (3, 40, 2, 100, 0.0),
                                           (7, 3, 1, 17, 0.2), (1, 6, 1, 1, 0.0)])
def test_fp8_decode_small_batches(T, Hq, Hkv, W, pad):
    case = qi.with_fp8_kv(qi.random_case(1800 + T * 7 + W, T=T, S=20000, Hq=Hq, Hkv=Hkv, W=W,
                                         pad_frac=pad, interior=True))
    o = run_decode_fp8(case)
    m = gate(bf16_tensor_to_f32(o), oracle_fp8(case), empty_row_mask(case.slot_idx, case.S))
    print(f"{case.name} fp8 decode: {m}", flush=True)


def test_fp8_decode_edge_mix_strided_views():
    """Stride-2 query tokens, K and V interleaved per slot, interior and tail
    padding, fully masked rows."""
    case = qi.with_fp8_kv(qi.edge_mix())
    assert case.info["k8"].strides[0] == 512
    o = run_decode_fp8(case)
    m = gate(bf16_tensor_to_f32(o), oracle_fp8(case), empty_row_mask(case.slot_idx, case.S))
    print(f"{case.name} fp8 decode: {m}", flush=True)


@pytest.mark.parametrize("Hq,Hkv", [(8, 1), (32, 2)])
def test_fp8_decode_drops_and_counts_invalid_entries(Hq, Hkv):
    """Entries neither -1 nor in [0, S) are dropped (the result is the
    attention over the valid ones) and counted for qsa_check_status."""
    case = qi.with_fp8_kv(qi.random_case(1830 + Hq, T=8, S=5000, Hq=Hq, Hkv=Hkv, W=300,
                                         pad_frac=0.1, interior=True))
    case.slot_idx[0, :40] = -1     # leading tiles with no valid row
    rng = np.random.Generator(np.random.PCG64(1831))
    raw = case.slot_idx.copy()
    for t in range(case.T):
        raw[t, rng.choice(300, size=3, replace=False)] = [5000, -7, 1 << 30]
    valid_only = np.where((raw >= 0) & (raw < case.S), raw, -1).astype(np.int32)
    ws = torch.empty(qsa.decode_workspace_bytes(case.T, case.W, case.Hq, case.Hkv),
                     dtype=torch.uint8, device=DEV)
    o = run_decode_fp8(case, slot_idx=raw, workspace=ws)
    want = oracle.prefill_fp8kv(case.q, case.info["k8"], case.info["v8"], case.info["k_scale"],
                                case.info["v_scale"], valid_only, 1.0 / 16.0)
    print(gate(bf16_tensor_to_f32(o), want, empty_row_mask(valid_only, case.S)), flush=True)
    with pytest.raises(qsa.QsaError) as e:
        qsa.check_status(ws, case.T, case.W)
    assert e.value.status == 6 and f"{3 * case.T} selection entries" in str(e.value)


def test_fp8_decode_empty_rows_zero_width_and_empty_cache_are_exact_zero():
    case = qi.with_fp8_kv(qi.random_case(1840, T=6, S=999, Hq=8, Hkv=1, W=50))
    case.slot_idx[[1, 4]] = -1
    o = run_decode_fp8(case)
    gate(bf16_tensor_to_f32(o), oracle_fp8(case), empty_row_mask(case.slot_idx, case.S))
    assert torch.all(o[[1, 4]].view(torch.int16) == 0)
    o = run_decode_fp8(qi.with_fp8_kv(qi.random_case(1841, T=3, S=64, Hq=4, Hkv=2, W=0)))
    assert torch.all(o.view(torch.int16) == 0)
    T, Hq, Hkv, W = 3, 4, 2, 40
    q = torch.randn(T, Hq, 256, generator=torch.Generator().manual_seed(1842))
    q = q.to(torch.bfloat16).to(DEV)
    k8 = torch.empty(0, Hkv, 256, dtype=torch.uint8, device=DEV)
    sl = torch.full((T, W), -1, dtype=torch.int32)
    sl[0, 3] = 0
    sl[2, 10:15] = 7
    ws = torch.empty(qsa.decode_workspace_bytes(T, W, Hq, Hkv), dtype=torch.uint8, device=DEV)
    o = qsa.sparse_decode_fp8kv(q, k8, k8, 1.0, 1.0, sl.to(DEV), workspace=ws)
    torch.cuda.synchronize()
    assert torch.all(o.view(torch.int16) == 0)
    with pytest.raises(qsa.QsaError) as e:
        qsa.check_status(ws, T, W)
    assert e.value.status == 6 and "6 selection entries" in str(e.value)


def test_fp8_decode_single_slot_rows_are_bit_exact():
    case = qi.with_fp8_kv(qi.random_case(1850, T=4, S=3000, Hq=24, Hkv=2, W=300,
                                         pad_frac=299 / 300, interior=True))
    o = run_decode_fp8(case)
    want_bits = torch.from_numpy(oracle_fp8(case)).to(torch.bfloat16).view(torch.int16).numpy()
    np.testing.assert_array_equal(bf16_tensor_bits(o).view(np.int16), want_bits)


@pytest.mark.parametrize("Hq,Hkv", [(16, 2), (24, 2)])
def test_fp8_decode_equals_bf16_decode_for_power_of_two_scales(Hq, Hkv):
    """As for the prefill: with power-of-two scales the FP8 cache holds
    values BF16 represents exactly, and both decode paths sum in the same
    order over the same shares, so they agree bit for bit (G = 8 runs the
    8-query-row FP8 layout, G = 12 the 16-row one)."""
    case = qi.random_case(1860 + Hq, T=5, S=4000, Hq=Hq, Hkv=Hkv, W=1500, pad_frac=0.1,
                          interior=True)
    rng = np.random.Generator(np.random.PCG64(1861))
    k8 = qi.e4m3_codes(rng.standard_normal(case.k_cache.shape).astype(np.float32) * 40, 1.0)
    v8 = qi.e4m3_codes(rng.standard_normal(case.v_cache.shape).astype(np.float32) * 40, 1.0)
    q, _, _, sl = upload(case, DEV)
    k8_t, v8_t = torch.from_numpy(k8).to(DEV), torch.from_numpy(v8).to(DEV)
    k_scale, v_scale = 2.0**-7, 4.0
    a = qsa.sparse_decode_fp8kv(q, k8_t, v8_t, k_scale, v_scale, sl)
    kb = (k8_t.view(torch.float8_e4m3fn).float() * k_scale).to(torch.bfloat16)
    vb = (v8_t.view(torch.float8_e4m3fn).float() * v_scale).to(torch.bfloat16)
    b = qsa.sparse_decode(q, kb, vb, sl)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
