"""The C-ABI library on a host without a GPU: it loads, exports every entry
point its header declares, and rejects bad arguments on the host before any
HIP call (these calls pass made-up device addresses, which the checks refuse
before anything could read them)."""
import ctypes
import os
import re

import pytest

import top_sparse_attention_amd as qsa

import torch

# These calls hand made-up device addresses to the library and rely on its
# host-side checks to refuse them; never let them reach a real GPU.
host_only = pytest.mark.skipif(torch.cuda.device_count() > 0,
                               reason="passes made-up device addresses: host-only")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsa.h")


def _lib():
    if not os.path.exists(qsa.library_path()):
        from top_sparse_attention_amd import _build
        _build.build()
    return qsa.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qsa_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_entry_point():
    lib = _lib()
    names = declared_functions()
    assert "qsa_sparse_prefill" in names and len(names) >= 10
    for name in names:
        assert hasattr(lib, name), f"{name} declared in qsa.h but not exported"


def test_prefill_blocks_workspace_has_room_for_aligned_lists():
    _lib()
    base = qsa.workspace_bytes(7810, 513 * 4)
    room = -(-((513 * 3 + 1) // 2) // 32) * 32     # 1.5 x the row's blocks, in list pads
    want = -(-base // 256) * 256 + -(-(7810 * room * 4) // 256) * 256
    assert qsa.prefill_blocks_workspace_bytes(7810, 513, 4) == want
    assert qsa.prefill_blocks_workspace_bytes(3, 0, 4) >= qsa.workspace_bytes(3, 0)
    assert qsa.prefill_blocks_workspace_bytes(-1, 5, 4) == 0
    assert qsa.prefill_blocks_workspace_bytes(3, 5, 0) == 0
    assert qsa.prefill_blocks_workspace_bytes(3, 5, 65) == 0


def test_version_and_status_strings():
    lib = _lib()
    assert qsa.version().startswith("libqsa")
    for code, name in qsa.STATUS_NAMES.items():
        assert lib.qsa_status_string(code).decode()
        assert name.startswith("QSA_")


def test_workspace_layout():
    _lib()
    m = qsa.workspace_layout(7810, 2051)
    assert m["row_stride"] == 2080                 # next multiple of 32
    assert m["list_offset"] == 0
    assert m["count_offset"] >= 7810 * 2080 * 4 and m["count_offset"] % 256 == 0
    assert m["bad_offset"] >= m["count_offset"] + 7810 * 4
    assert m["share_offset"] >= m["bad_offset"] + 7810 * 4 and m["share_offset"] % 256 == 0
    assert m["total_bytes"] == m["share_offset"] + 512
    assert m["total_bytes"] == qsa.workspace_bytes(7810, 2051)
    assert qsa.workspace_bytes(0, 0) == 0
    assert qsa.workspace_bytes(-1, 3) == 0
    assert qsa.workspace_layout(5, 0)["row_stride"] == 0


FAKE = 1 << 32        # an aligned address no test ever dereferences


def view(size, stride, data=FAKE):
    return qsa.BF16View(data, (ctypes.c_int64 * 3)(*size), (ctypes.c_int64 * 3)(*stride))


def ivew(size, stride, data=FAKE):
    return qsa.I32View(data, (ctypes.c_int64 * 2)(*size), (ctypes.c_int64 * 2)(*stride))


def good(T=4, Hq=4, S=64, Hkv=2, W=8):
    q = view((T, Hq, 256), (Hq * 256, 256, 1), FAKE)
    k = view((S, Hkv, 256), (Hkv * 256, 256, 1), FAKE + (1 << 24))
    v = view((S, Hkv, 256), (Hkv * 256, 256, 1), FAKE + (2 << 24))
    o = view((T, Hq, 256), (Hq * 256, 256, 1), FAKE + (3 << 24))
    s = ivew((T, W), (W, 1), FAKE + (4 << 24))
    return q, k, v, o, s


def prefill(q, k, v, s, o, scale=0.0625, ws=FAKE + (5 << 24), ws_bytes=1 << 30):
    lib = _lib()
    r = ctypes.byref
    return lib.qsa_sparse_prefill(r(q), r(k), r(v), r(s), scale, r(o), ws, ws_bytes, None)


BAD_CASES = {
    "head dim 128": (lambda q, k, v, o, s: setattr(q, "size", (ctypes.c_int64 * 3)(4, 4, 128)),
                     "QSA_ERR_UNSUPPORTED"),
    "q stride over D": (lambda q, k, v, o, s: q.stride.__setitem__(2, 2), "QSA_ERR_STRIDE"),
    "misaligned k base": (lambda q, k, v, o, s: setattr(k, "data", FAKE + 2), "QSA_ERR_STRIDE"),
    "odd v token stride": (lambda q, k, v, o, s: v.stride.__setitem__(0, 516), "QSA_ERR_STRIDE"),
    "Hq not multiple of Hkv": (lambda q, k, v, o, s: (
        setattr(q, "size", (ctypes.c_int64 * 3)(4, 3, 256)),
        setattr(o, "size", (ctypes.c_int64 * 3)(4, 3, 256))), "QSA_ERR_SHAPE"),
    "out shape differs": (lambda q, k, v, o, s: o.size.__setitem__(0, 5), "QSA_ERR_SHAPE"),
    "v shape differs": (lambda q, k, v, o, s: v.size.__setitem__(0, 63), "QSA_ERR_SHAPE"),
    "slot rows differ": (lambda q, k, v, o, s: s.size.__setitem__(0, 3), "QSA_ERR_SHAPE"),
    "slot stride over W": (lambda q, k, v, o, s: s.stride.__setitem__(1, 2), "QSA_ERR_STRIDE"),
    "null q data": (lambda q, k, v, o, s: setattr(q, "data", None), "QSA_ERR_NULL"),
    "null slot data": (lambda q, k, v, o, s: setattr(s, "data", None), "QSA_ERR_NULL"),
    "negative size": (lambda q, k, v, o, s: k.size.__setitem__(0, -1), "QSA_ERR_SHAPE"),
    "out aliases q": (lambda q, k, v, o, s: setattr(o, "data", q.data), "QSA_ERR_ALIAS"),
    "out overlaps v": (lambda q, k, v, o, s: setattr(o, "data", v.data + 64), "QSA_ERR_ALIAS"),
    # row addresses are formed with a 32-bit slot stride in bytes
    "k slot stride 4 GiB": (lambda q, k, v, o, s: k.stride.__setitem__(0, 1 << 31),
                            "QSA_ERR_UNSUPPORTED"),
}


@host_only
@pytest.mark.parametrize("name", sorted(BAD_CASES))
def test_bad_arguments_are_rejected_on_the_host(name):
    q, k, v, o, s = good()
    mutate, want = BAD_CASES[name]
    mutate(q, k, v, o, s)
    status = prefill(q, k, v, s, o)
    assert qsa.STATUS_NAMES[status] == want, _lib().qsa_last_error()
    assert _lib().qsa_last_error().decode()


@host_only
@pytest.mark.parametrize("scale", [float("nan"), float("inf"), -float("inf")])
def test_non_finite_scale_is_rejected(scale):
    q, k, v, o, s = good()
    assert qsa.STATUS_NAMES[prefill(q, k, v, s, o, scale=scale)] == "QSA_ERR_SCALE"


@host_only
def test_workspace_checks():
    q, k, v, o, s = good()
    need = qsa.workspace_bytes(4, 8)
    assert qsa.STATUS_NAMES[prefill(q, k, v, s, o, ws=None)] == "QSA_ERR_WORKSPACE"
    assert qsa.STATUS_NAMES[prefill(q, k, v, s, o, ws_bytes=need - 1)] == "QSA_ERR_WORKSPACE"
    assert qsa.STATUS_NAMES[prefill(q, k, v, s, o, ws=FAKE + 16)] == "QSA_ERR_WORKSPACE"


@host_only
def test_null_view_pointers():
    lib = _lib()
    q, k, v, o, s = good()
    r = ctypes.byref
    assert lib.qsa_sparse_prefill(None, r(k), r(v), r(s), 0.0625, r(o), FAKE, 1 << 30, None) == 1
    assert lib.qsa_sparse_prefill(r(q), r(k), r(v), None, 0.0625, r(o), FAKE, 1 << 30, None) == 1
    assert lib.qsa_compact_slots(None, 64, FAKE, 1 << 30, None) == 1


def test_python_binding_rejects_wrong_dtypes():
    _lib()
    q = torch.zeros(2, 2, 256, dtype=torch.float32)
    with pytest.raises(TypeError):
        qsa._bf16_view(q, "q")
    with pytest.raises(TypeError):
        qsa._i32_view(torch.zeros(2, 3, dtype=torch.int64), "slot_idx")


def test_partials_and_decode_sizes():
    _lib()
    rows = 3 * 5 * 7
    o_bytes = (rows * 256 * 4 + 255) // 256 * 256
    assert qsa.partials_bytes(3, 5, 7) == o_bytes + (rows * 8 + 255) // 256 * 256
    assert qsa.partials_bytes(-1, 5, 7) == 0
    # about 1,024 workgroups; >= 8 tiles per split unless that leaves fewer
    # than 512 workgroups; >= 4 tiles per split; <= 64 splits
    assert qsa.decode_splits(16, 2048, 24, 2) == 16
    assert qsa.decode_splits(8, 2048, 24, 2) == 32
    assert qsa.decode_splits(32, 2048, 24, 2) == 16
    assert qsa.decode_splits(64, 2048, 24, 2) == 8
    assert qsa.decode_splits(256, 2048, 24, 2) == 2
    assert qsa.decode_splits(1, 2048, 16, 2) == 32
    assert qsa.decode_splits(1, 100000, 16, 2) == 64
    assert qsa.decode_splits(7810, 2051, 16, 2) == 1
    assert qsa.decode_splits(4, 64, 8, 1) == 1
    assert qsa.decode_splits(0, 64, 8, 1) == 1
    ws = qsa.workspace_bytes(16, 2048)
    assert qsa.decode_workspace_bytes(16, 2048, 24, 2) == \
        (ws + 255) // 256 * 256 + qsa.partials_bytes(16, 16, 24)


@host_only
def test_split_entry_points_reject_bad_arguments():
    lib = _lib()
    r = ctypes.byref
    q, k, v, o, s = good()
    ws, part = FAKE + (5 << 24), FAKE + (6 << 24)
    big = 1 << 30

    def partial(splits=2, base=0, n_parts=2, part_bytes=big, parts=part):
        return qsa.STATUS_NAMES[lib.qsa_sparse_attend_partial(
            r(q), r(k), r(v), 8, 0.0625, ws, big, splits, base, n_parts, parts, part_bytes,
            None)]

    assert partial(splits=0) == "QSA_ERR_SHAPE"
    assert partial(base=1) == "QSA_ERR_SHAPE"            # parts [1, 3) beyond n_parts = 2
    assert partial(base=-1) == "QSA_ERR_SHAPE"
    assert partial(part_bytes=qsa.partials_bytes(2, 4, 4) - 1) == "QSA_ERR_WORKSPACE"
    assert partial(parts=None) == "QSA_ERR_WORKSPACE"
    assert partial(parts=FAKE + 8) == "QSA_ERR_WORKSPACE"
    assert partial(parts=q.data) == "QSA_ERR_ALIAS"       # partials on top of q
    assert qsa.STATUS_NAMES[lib.qsa_merge_partials(part, big, 0, 4, 4, r(o), None)] == \
        "QSA_ERR_SHAPE"
    bad_o = view((5, 4, 256), (1024, 256, 1), FAKE + (3 << 24))
    assert qsa.STATUS_NAMES[lib.qsa_merge_partials(part, big, 2, 4, 4, r(bad_o), None)] == \
        "QSA_ERR_SHAPE"
    over = view((4, 4, 256), (1024, 256, 1), part + 256)
    assert qsa.STATUS_NAMES[lib.qsa_merge_partials(part, big, 2, 4, 4, r(over), None)] == \
        "QSA_ERR_ALIAS"
    for lo, hi in ((-1, 10), (10, 5), (0, 65)):
        assert qsa.STATUS_NAMES[lib.qsa_compact_slot_range(r(s), 64, lo, hi, ws, big, None)] == \
            "QSA_ERR_SHAPE"
    assert qsa.STATUS_NAMES[lib.qsa_sparse_decode(
        r(q), r(k), r(v), r(s), 0.0625, r(o), ws, 16, None)] == "QSA_ERR_WORKSPACE"


@host_only
def test_fp8_decode_rejects_bad_arguments():
    lib = _lib()
    r = ctypes.byref
    q, _, _, o, s = good()
    k8 = view((64, 2, 256), (512, 256, 1), FAKE + (1 << 24))
    v8 = view((64, 2, 256), (512, 256, 1), FAKE + (2 << 24))
    ws, big = FAKE + (5 << 24), 1 << 30

    def decode(k_scale=0.5, v_scale=0.25, slot=s, ws=ws, ws_bytes=big, k=k8):
        return qsa.STATUS_NAMES[lib.qsa_sparse_decode_fp8kv(
            r(q), r(k), r(v8), k_scale, v_scale, None if slot is None else r(slot), 0.0625,
            r(o), ws, ws_bytes, None)]

    assert decode(k_scale=float("nan")) == "QSA_ERR_SCALE"
    assert decode(v_scale=float("inf")) == "QSA_ERR_SCALE"
    assert decode(slot=None) == "QSA_ERR_NULL"
    assert decode(ws_bytes=qsa.decode_workspace_bytes(4, 8, 4, 2) - 1) == "QSA_ERR_WORKSPACE"
    assert decode(ws=FAKE + 16) == "QSA_ERR_WORKSPACE"
    assert decode(k=view((64, 2, 256), (512, 256, 1), FAKE + (1 << 24) + 8)) == "QSA_ERR_STRIDE"
    # a BF16-sized token stride over FP8 rows is fine; a 4 GiB one is not
    assert decode(k=view((64, 2, 256), (1 << 32, 256, 1), FAKE + (1 << 24))) == \
        "QSA_ERR_UNSUPPORTED"


@host_only
def test_indexer_entry_points_reject_bad_arguments():
    lib = _lib()
    r = ctypes.byref
    iq = view((8, 4, 128), (512, 128, 1), FAKE)
    ik = view((16, 1, 128), (128, 128, 1), FAKE + (1 << 24))
    out = ivew((8, 4 * 5 + 3), (23, 1), FAKE + (2 << 24))
    pos, sop, sc = FAKE + (3 << 24), FAKE + (4 << 24), FAKE + (5 << 24)
    big = 1 << 30

    def topk(iq_=iq, ik_=ik, L=64, budget=5, out_=out, sc_bytes=big):
        return qsa.STATUS_NAMES[lib.qsa_indexer_topk(r(iq_), r(ik_), pos, sop, L, budget, sc,
                                                     sc_bytes, r(out_), None)]

    assert topk(iq_=view((8, 2, 128), (256, 128, 1), FAKE)) == "QSA_ERR_UNSUPPORTED"
    assert topk(ik_=view((16, 1, 64), (64, 64, 1), FAKE)) == "QSA_ERR_UNSUPPORTED"
    assert topk(L=100) == "QSA_ERR_SHAPE"                    # 16 keys cannot cover 100 positions
    assert topk(budget=0) == "QSA_ERR_SHAPE"
    assert topk(out_=ivew((8, 22), (22, 1), FAKE + (2 << 24))) == "QSA_ERR_SHAPE"
    assert topk(sc_bytes=8 * 16 * 4 - 1) == "QSA_ERR_WORKSPACE"
    assert qsa.indexer_scores.__doc__ and lib.qsa_indexer_scores_bytes(8, 16) == 512
    # fused path: T rows of C floats (C rounded up to even), then the
    # per-range counts and thresholds
    assert lib.qsa_indexer_topk_fused_bytes(8, 16) == 512 + 256 + 256
    up = lambda x: -(-x // 256) * 256
    assert lib.qsa_indexer_topk_fused_bytes(7810, 16384) == \
        up(7810 * 16384 * 4) + up(7810 * 16 * 4) + up(7810 * 4)
    assert lib.qsa_indexer_topk_fused_bytes(9, 1025) == \
        up(9 * 1026 * 4) + up(9 * 2 * 4) + up(9 * 4)

    def fused(budget=5, sc_=sc, sc_bytes=big, ik_=ik, L=64):
        o = ivew((8, 4 * budget + 3), (4 * budget + 3, 1), FAKE + (2 << 24))
        return qsa.STATUS_NAMES[lib.qsa_indexer_topk_fused(r(iq), r(ik_), pos, sop, L, budget,
                                                           sc_, sc_bytes, r(o), None)]

    assert fused(budget=0) == "QSA_ERR_SHAPE"
    assert fused(budget=513) == "QSA_ERR_UNSUPPORTED"         # above the fused path's budget
    assert fused(sc_bytes=lib.qsa_indexer_topk_fused_bytes(8, 16) - 1) == "QSA_ERR_WORKSPACE"
    assert fused(sc_=sc + 4) == "QSA_ERR_WORKSPACE"           # pairs need 8-byte alignment
    many = view((262145, 1, 128), (128, 128, 1), FAKE + (1 << 40))
    assert fused(ik_=many, L=4 * 262145) == "QSA_ERR_UNSUPPORTED"   # more than 256 key ranges


def far_views(T, Hq, S, Hkv, W):
    """Views of made-up addresses 1 TiB apart, so that even huge shapes pass
    the overlap checks and reach the launch-size checks."""
    tib = 1 << 40
    q = view((T, Hq, 256), (Hq * 256, 256, 1), tib)
    k = view((S, Hkv, 256), (Hkv * 256, 256, 1), 2 * tib)
    v = view((S, Hkv, 256), (Hkv * 256, 256, 1), 3 * tib)
    o = view((T, Hq, 256), (Hq * 256, 256, 1), 4 * tib)
    s = ivew((T, W), (W, 1), 5 * tib)
    return q, k, v, o, s, 6 * tib


@host_only
def test_launches_beyond_the_work_item_limit_are_refused():
    """A launch covers at most 2^32 - 1 work-items per grid dimension; larger
    problems are refused as unsupported before anything is enqueued."""
    lib = _lib()
    r = ctypes.byref
    huge = (1 << 62)

    def name(status):
        return qsa.STATUS_NAMES[status]

    # the compaction pass: 256 threads per token, so 2^24 tokens are too many
    q, k, v, o, s, ws = far_views(1 << 24, 1, 64, 1, 1)
    assert name(lib.qsa_sparse_prefill(r(q), r(k), r(v), r(s), 0.0625, r(o), ws, huge,
                                       None)) == "QSA_ERR_UNSUPPORTED"
    assert "work-items" in lib.qsa_last_error().decode()
    assert name(lib.qsa_compact_slots(r(s), 64, ws, huge, None)) == "QSA_ERR_UNSUPPORTED"
    assert name(lib.qsa_compact_blocks(r(s), 64, 4, ws, huge, None)) == "QSA_ERR_UNSUPPORTED"
    # attention: one 64-thread wave per (token, KV head, 16-head block);
    # 2^25 tokens x 2 KV heads = 2^26 waves = 2^32 work-items
    q, k, v, o, s, ws = far_views(1 << 25, 16, 64, 2, 1)
    assert name(lib.qsa_sparse_attend(r(q), r(k), r(v), 1, 0.0625, ws, huge, r(o),
                                      None)) == "QSA_ERR_UNSUPPORTED"
    k8 = view((64, 2, 256), (512, 256, 1), k.data)
    v8 = view((64, 2, 256), (512, 256, 1), v.data)
    assert name(lib.qsa_sparse_attend_fp8kv(r(q), r(k8), r(v8), 1.0, 1.0, 1, 0.0625, ws, huge,
                                            r(o), None)) == "QSA_ERR_UNSUPPORTED"
    # one fewer token fits: the call gets as far as the launch, which fails
    # on a host without a GPU
    q, k, v, o, s, ws = far_views((1 << 25) - 1, 16, 64, 2, 1)
    assert name(lib.qsa_sparse_attend(r(q), r(k), r(v), 1, 0.0625, ws, huge, r(o), None)) == \
        "QSA_ERR_HIP"
    assert "work-items" not in lib.qsa_last_error().decode()
    # split attention multiplies by the splits
    q, k, v, o, s, ws = far_views(1 << 20, 1, 64, 1, 1)
    part = 7 << 40
    assert name(lib.qsa_sparse_attend_partial(r(q), r(k), r(v), 1, 0.0625, ws, huge, 4096, 0,
                                              4096, part, huge, None)) == "QSA_ERR_UNSUPPORTED"
    # the merge: one workgroup of 256 per (token, head)
    mo = view((1 << 24, 16, 256), (16 * 256, 256, 1), 4 << 40)
    assert name(lib.qsa_merge_partials(part, huge, 2, 1 << 24, 16, r(mo), None)) == \
        "QSA_ERR_UNSUPPORTED"
    # the indexer's key ranges of 1,024 along y stop at 65,535
    C = 1 << 27
    iq = view((8, 4, 128), (512, 128, 1), 1 << 40)
    ik = view((C, 1, 128), (128, 128, 1), 2 << 40)
    out = ivew((8, 23), (23, 1), 3 << 40)
    assert name(lib.qsa_indexer_topk(r(iq), r(ik), 4 << 40, 5 << 40, 4 * C, 5, 6 << 40, huge,
                                     r(out), None)) == "QSA_ERR_UNSUPPORTED"


def test_prefill_workspace_alias():
    lib = _lib()
    for T, W in ((7810, 2051), (0, 0), (3, 5), (-1, 2)):
        assert lib.qsa_sparse_prefill_workspace_bytes(T, W) == qsa.workspace_bytes(T, W)
