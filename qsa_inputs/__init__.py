"""Seeded synthetic inputs for QSA sparse main-attention prefill.

This module is shared by the tests, the benchmark and the smoke check.  It
holds no attention arithmetic: it only draws BF16 Q/K/V values and selection
lists with the shapes and structure of the workloads on the page "Qwen4-Exp
QSA comes to Huawei's Ascend: inside SGLang's opt-in CANN prefill PR" (section
"Nine tests that passed, ...": nonzero random BF16 Q/K/V, unordered physical
slots at widths 1/63/64/65/2051, -1 padding, fully masked rows, zero width,
non-contiguous tensors, compression-ratio-4 causal tails, a two-request shared
prefix, the long 7,810 x 65,536 x 2,051 prefill; section "What the pull
request actually adds", "Head shapes" and "Sizing bounds" bullets: head pairs
(16,2) (24,2) (12,1) (6,1) (3,1), D = 256, a 262,144-slot cache cap).

Every array is a numpy array of BF16 bit patterns (``uint16``) or ``int32``
slots.  Values are drawn as float32 N(0, 1) with ``numpy.random.PCG64`` and
rounded to BF16 (round to nearest, ties to even) here on the CPU, so the GPU
and the oracle read identical bits.  Views keep the strides a workload asks for
(a stride-2 token view of Q, K and V interleaved in one buffer, ...).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

D_HEAD = 256


@dataclasses.dataclass
class Case:
    """One synthetic prefill problem.

    ``q`` [T, Hq, D], ``k_cache``/``v_cache`` [S, Hkv, D] are uint16 views
    (BF16 bits) into the arrays of ``bases``; ``slot_idx`` [T, W] int32 uses -1
    for "no slot".  ``scale`` None means the default 1/sqrt(D).
    """
    name: str
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    slot_idx: np.ndarray
    scale: Optional[float]
    bases: Dict[str, np.ndarray]
    info: Dict[str, object] = dataclasses.field(default_factory=dict)

    @property
    def T(self) -> int:
        return self.q.shape[0]

    @property
    def Hq(self) -> int:
        return self.q.shape[1]

    @property
    def D(self) -> int:
        return self.q.shape[2]

    @property
    def S(self) -> int:
        return self.k_cache.shape[0]

    @property
    def Hkv(self) -> int:
        return self.k_cache.shape[1]

    @property
    def W(self) -> int:
        return self.slot_idx.shape[1]

    def base_of(self, view: np.ndarray) -> np.ndarray:
        """The array in ``bases`` whose memory ``view`` lies in."""
        for b in self.bases.values():
            if view is b or view.base is b:
                return b
        for b in self.bases.values():
            if np.shares_memory(view, b):
                return b
        raise KeyError("view is not backed by any base array")


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to BF16 (nearest, ties to even); returns uint16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen BF16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return bf16_bits(rng.standard_normal(size=shape, dtype=np.float32))


def distinct_draws(rng: np.random.Generator, high, T: int, W: int) -> np.ndarray:
    """T rows of W distinct integers; row t is uniform over W-subsets of [0, high[t]).

    Rows come back sorted (callers shuffle).  Draws with replacement and
    redraws duplicates until none are left, which is symmetric in the labels
    and hence uniform over subsets.
    """
    high = np.broadcast_to(np.asarray(high, dtype=np.int64), (T,)).copy()
    if T and W and int(high.min()) < W:
        raise ValueError("a row asks for more distinct values than it has")
    a = rng.integers(0, high[:, None], size=(T, W), dtype=np.int64)
    active = np.arange(T)
    while active.size and W > 1:
        sub = a[active]
        sub.sort(axis=1)
        dup = np.zeros(sub.shape, dtype=bool)
        dup[:, 1:] = sub[:, 1:] == sub[:, :-1]
        has_dup = dup.any(axis=1)
        r, c = np.nonzero(dup)
        if r.size:
            sub[r, c] = rng.integers(0, high[active[r]], dtype=np.int64)
        a[active] = sub
        active = active[has_dup]
    return a


def shuffle_rows(rng: np.random.Generator, a: np.ndarray) -> np.ndarray:
    return rng.permuted(a, axis=1)


def _contiguous_case(name, rng, T, S, Hq, Hkv, slot_idx, scale, info=None) -> Case:
    q = normal_bf16(rng, (T, Hq, D_HEAD))
    k = normal_bf16(rng, (S, Hkv, D_HEAD))
    v = normal_bf16(rng, (S, Hkv, D_HEAD))
    slot_idx = np.ascontiguousarray(slot_idx, dtype=np.int32)
    return Case(name, q, k, v, slot_idx, scale,
                {"q": q, "k": k, "v": v, "slot_idx": slot_idx}, dict(info or {}))


def random_case(seed: int, T: int, S: int, Hq: int, Hkv: int, W: int,
                scale: Optional[float] = None, pad_frac: float = 0.0,
                interior: bool = False, name: str = "random") -> Case:
    """Distinct random slots per token in random order.

    ``pad_frac`` of the W entries of each row become -1 (tail padding, or
    scattered when ``interior``).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    n_valid = W - int(round(pad_frac * W))
    sel = np.full((T, W), -1, dtype=np.int64)
    if n_valid:
        sel[:, :n_valid] = shuffle_rows(rng, distinct_draws(rng, S, T, n_valid))
    if interior:
        sel = shuffle_rows(rng, sel)
    return _contiguous_case(name, rng, T, S, Hq, Hkv, sel, scale,
                            {"seed": seed, "n_valid": n_valid})


# --------------------------------------------------------------------------
# The five workloads.
# --------------------------------------------------------------------------

def tiny(seed: int = 101) -> Case:
    """T=64 tokens, S=1,024 slots, (Hq,Hkv)=(16,2), 64 distinct random slots
    per token in random order, scale 1/16 (the default for D=256)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    T, S, W = 64, 1024, 64
    sel = shuffle_rows(rng, distinct_draws(rng, S, T, W))
    return _contiguous_case("tiny", rng, T, S, 16, 2, sel, 1.0 / 16.0,
                            {"seed": seed})


EDGE_WIDTHS = (0, 1, 63, 64, 65, 2051)


def edge_mix(seed: int = 102) -> Case:
    """The edge-case mix: S=4,096, (12,1), T=257, W=2,051.

    Row t selects EDGE_WIDTHS[t % 6] distinct random slots, then -1 up to W.
    Rows t % 16 == 7 are entirely -1.  Rows t % 5 == 3 have their -1 entries
    scattered through the row.  scale = 0.05.  Q is every second token of a
    [2T, Hq, D] buffer; K and V are the two halves of one [S, 2, Hkv, D]
    buffer, so every tensor is a non-contiguous view.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    T, S, Hq, Hkv, W = 257, 4096, 12, 1, 2051
    sel = np.full((T, W), -1, dtype=np.int64)
    for width in sorted(set(EDGE_WIDTHS) - {0}):
        rows = np.array([t for t in range(T) if EDGE_WIDTHS[t % 6] == width])
        sel[rows, :width] = shuffle_rows(rng, distinct_draws(rng, S, rows.size, width))
    sel[np.arange(T) % 16 == 7] = -1
    scatter = np.nonzero(np.arange(T) % 5 == 3)[0]
    sel[scatter] = shuffle_rows(rng, sel[scatter])
    q_buf = normal_bf16(rng, (2 * T, Hq, D_HEAD))
    kv_buf = normal_bf16(rng, (S, 2, Hkv, D_HEAD))
    slot_idx = np.ascontiguousarray(sel, dtype=np.int32)
    return Case("edge_mix", q_buf[::2], kv_buf[:, 0], kv_buf[:, 1], slot_idx, 0.05,
                {"q": q_buf, "kv": kv_buf, "slot_idx": slot_idx},
                {"seed": seed, "widths": EDGE_WIDTHS})


def long_prefill(seed: int = 103) -> Case:
    """The long prefill: T=7,810, S=65,536, W=2,051 distinct random unordered
    slots per token, (16,2), default scale."""
    rng = np.random.Generator(np.random.PCG64(seed))
    T, S, W = 7810, 65536, 2051
    sel = shuffle_rows(rng, distinct_draws(rng, S, T, W))
    return _contiguous_case("long_prefill", rng, T, S, 16, 2, sel, None,
                            {"seed": seed})


PREFIX = 36096
NEW_PER_REQUEST = 4096
CAUSAL_BUDGET = 2048
COMPRESSION = 4


def two_request(seed: int = 104) -> Case:
    """Two requests sharing a 36,096-token prefix, 4,096 new tokens each.

    Physical slots are a seeded permutation of a 131,072-slot cache.  Logical
    prefix positions 0..36,095 map to perm[0:36,096] for both requests;
    request A's new positions map to perm[36,096:40,192] and request B's to
    perm[40,192:44,288].  A query at absolute position p selects its causal
    tail of r = (p + 1) % 4 positions p-r+1..p (the incomplete block of a
    compression-ratio-4 indexer) plus 2,048 - r distinct positions drawn from
    [0, p - r]; the row is shuffled and mapped logical -> physical.
    (Hq,Hkv)=(24,2), W=2,048, default scale.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    S, Hq, Hkv, W = 131072, 24, 2, CAUSAL_BUDGET
    perm = rng.permutation(S)
    T = 2 * NEW_PER_REQUEST
    req = np.repeat(np.arange(2), NEW_PER_REQUEST)
    pos = PREFIX + np.tile(np.arange(NEW_PER_REQUEST), 2)
    r = (pos + 1) % COMPRESSION
    # Draw W distinct positions from [0, p - r] for every row, shuffle, then
    # overwrite the last r columns with the tail positions (which lie above
    # p - r), leaving W - r draws that are uniform over subsets.
    logical = shuffle_rows(rng, distinct_draws(rng, pos - r + 1, T, W))
    col = np.arange(W)[None, :]
    tail = col >= (W - r)[:, None]
    tail_pos = pos[:, None] - (W - 1 - col)
    logical = np.where(tail, tail_pos, logical)
    new_base = PREFIX + req * NEW_PER_REQUEST
    phys = np.where(logical < PREFIX, perm[np.minimum(logical, S - 1)],
                    perm[np.clip(new_base[:, None] + (logical - PREFIX), 0, S - 1)])
    sel = shuffle_rows(rng, phys)
    return _contiguous_case("two_request", rng, T, S, Hq, Hkv, sel, None,
                            {"seed": seed, "perm": perm, "positions": pos,
                             "request": req, "tail": r})


def max_cache(seed: int = 105, heads=(6, 1)) -> Case:
    """The maximum cache: S=262,144 slots, T=16,384, W=2,048 distinct random
    slots, D=256, at (Hq,Hkv) = (6,1) or (3,1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    T, S, W = 16384, 262144, 2048
    Hq, Hkv = heads
    sel = shuffle_rows(rng, distinct_draws(rng, S, T, W))
    return _contiguous_case(f"max_cache_{Hq}_{Hkv}", rng, T, S, Hq, Hkv, sel, None,
                            {"seed": seed})


E4M3_MAX = 448.0


def e4m3_codes(x: np.ndarray, scale: float) -> np.ndarray:
    """FP8 E4M3 (fn) codes of x / scale, rounded to nearest even by torch's
    float8_e4m3fn conversion; |x / scale| must not exceed 448."""
    import torch
    y = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32) / np.float32(scale))
    return y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def with_fp8_kv(case: Case) -> Case:
    """The same problem with K and V quantized to FP8 E4M3, one scale per
    tensor (amax / 448).  Adds k8, v8, k_scale, v_scale to the case; k8/v8
    keep k_cache/v_cache's layout (strides in bytes = elements)."""
    out = {}
    for name, view in (("k", case.k_cache), ("v", case.v_cache)):
        real = bf16_to_f32(view)
        amax = float(np.abs(real).max()) if real.size else 1.0
        scale = amax / E4M3_MAX if amax > 0 else 1.0
        base = case.base_of(view)
        codes = e4m3_codes(bf16_to_f32(base), scale)
        off = (view.__array_interface__["data"][0] - base.__array_interface__["data"][0]) // 2
        v8 = np.lib.stride_tricks.as_strided(codes.reshape(-1)[off:], shape=view.shape,
                                             strides=[s_ // 2 for s_ in view.strides])
        out[name] = (codes, v8, scale)
    case.info.update(k8=out["k"][1], v8=out["v"][1], k_scale=out["k"][2],
                     v_scale=out["v"][2], k8_base=out["k"][0], v8_base=out["v"][0])
    case.name += "_fp8kv"
    return case


def long_prefill_blocks(seed: int = 107, block_size: int = 4) -> Case:
    """The long prefill with micro-block selections: T=7,810, S=65,536,
    (16,2); every token selects 513 distinct random blocks of 4 consecutive
    slots (2,052 slots) in random order.  ``slot_idx`` holds block ids;
    info["block_size"] says how many slots each covers."""
    rng = np.random.Generator(np.random.PCG64(seed))
    T, S = 7810, 65536
    Wb = -(-2051 // block_size)
    sel = shuffle_rows(rng, distinct_draws(rng, S // block_size, T, Wb))
    return _contiguous_case(f"long_prefill_block{block_size}", rng, T, S, 16, 2, sel, None,
                            {"seed": seed, "block_size": block_size})


INDEX_HEADS = 4
INDEX_DIM = 128


def indexed_case(seed: int, L: int, T: int, Hq: int, Hkv: int, budget: int,
                 integer_keys: bool = False, name: str = "indexed") -> Case:
    """A request of L positions whose last T are being prefilled, with QSA
    indexer inputs: iq [T, 4, 128] and ik [C = ceil(L/4), 1, 128] (one key
    per block of 4 positions), positions [T] = L-T .. L-1, and a seeded
    position -> slot table (page size 1) into an S = L slot cache.  With
    integer_keys the indexer values are small integers, so every score is
    exact in FP32.  slot_idx is left empty (W = 4*budget + 3, all -1): it is
    what the indexer produces."""
    rng = np.random.Generator(np.random.PCG64(seed))
    C = -(-L // 4)
    if integer_keys:
        iq = bf16_bits(rng.integers(-2, 3, size=(T, INDEX_HEADS, INDEX_DIM)).astype(np.float32))
        ik = bf16_bits(rng.integers(-2, 3, size=(C, 1, INDEX_DIM)).astype(np.float32))
    else:
        iq = normal_bf16(rng, (T, INDEX_HEADS, INDEX_DIM))
        ik = normal_bf16(rng, (C, 1, INDEX_DIM))
    positions = (L - T + np.arange(T)).astype(np.int32)
    slot_of_pos = rng.permutation(L).astype(np.int32)
    sel = np.full((T, 4 * budget + 3), -1, dtype=np.int32)
    case = _contiguous_case(name, rng, T, L, Hq, Hkv, sel, None,
                            {"seed": seed, "budget": budget})
    case.info.update(iq=iq, ik=ik, positions=positions, slot_of_pos=slot_of_pos)
    return case


def indexed_long_prefill(seed: int = 108) -> Case:
    """The long prefill with its selection made by the indexer: a 65,536-token
    request whose last 7,810 tokens are prefilled, (16,2), budget 512 blocks
    (2,048 positions + a causal tail of up to 3 = 2,051-wide rows)."""
    return indexed_case(seed, 65536, 7810, 16, 2, 512, name="indexed_long_prefill")


DECODE_REQUESTS = 16


def decode_batch(seed: int = 106) -> Case:
    """A decode step for 16 requests in one 262,144-slot paged cache.

    Request i holds a context of 8,192 + 1,024 i tokens whose logical
    positions map, in order, onto its own range of a seeded permutation of
    the cache slots.  Its one new token sits at the last position p and
    selects, by the causal-tail rule of `two_request`, its last
    r = (p + 1) % 4 positions plus 2,048 - r distinct earlier ones.
    (Hq,Hkv)=(24,2), W=2,048, default scale.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    S, Hq, Hkv, W = 262144, 24, 2, CAUSAL_BUDGET
    T = DECODE_REQUESTS
    lengths = 8192 + 1024 * np.arange(T)
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]])
    perm = rng.permutation(S)
    pos = lengths - 1
    r = (pos + 1) % COMPRESSION
    logical = shuffle_rows(rng, distinct_draws(rng, pos - r + 1, T, W))
    col = np.arange(W)[None, :]
    tail = col >= (W - r)[:, None]
    logical = np.where(tail, pos[:, None] - (W - 1 - col), logical)
    phys = perm[starts[:, None] + logical]
    sel = shuffle_rows(rng, phys)
    return _contiguous_case("decode_batch", rng, T, S, Hq, Hkv, sel, None,
                            {"seed": seed, "perm": perm, "lengths": lengths,
                             "starts": starts, "positions": pos})


WORKLOADS = {
    "tiny": tiny,
    "edge_mix": edge_mix,
    "long_prefill": long_prefill,
    "two_request": two_request,
    "max_cache_6_1": lambda seed=105: max_cache(seed, (6, 1)),
    "max_cache_3_1": lambda seed=105: max_cache(seed, (3, 1)),
    "decode_batch": decode_batch,
    "long_prefill_fp8kv": lambda seed=103: with_fp8_kv(long_prefill(seed)),
    "decode_batch_fp8kv": lambda seed=106: with_fp8_kv(decode_batch(seed)),
    "long_prefill_block4": long_prefill_blocks,
    "indexed_long_prefill": indexed_long_prefill,
}


def sample_rows(T: int, n: int, seed: int = 7) -> np.ndarray:
    """A seeded sorted sample of n token rows that includes the first and last."""
    if n >= T:
        return np.arange(T, dtype=np.int64)
    rng = np.random.Generator(np.random.PCG64(seed))
    mid = rng.choice(np.arange(1, T - 1), size=max(n - 2, 0), replace=False)
    return np.unique(np.concatenate([[0, T - 1], mid]).astype(np.int64))
