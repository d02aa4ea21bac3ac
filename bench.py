"""Benchmark of QSA sparse main-attention prefill on one MI355X.

One step = the whole hot path on one batch of resident synthetic input:
index validation/compaction (qsa_compact_slots) followed by the gather
attention (qsa_sparse_attend), both through the C ABI on torch's current
stream.  Other workloads: `decode_batch` runs qsa_sparse_decode (split
attention over the raw selection rows, then the merge), `long_prefill_fp8kv` the
FP8 E4M3 KV-cache variant (qsa_sparse_attend_fp8kv), `decode_batch_fp8kv` the
decode step over that cache (qsa_sparse_decode_fp8kv) and `long_prefill_block4`
micro-block selections (qsa_sparse_prefill_blocks: compaction into aligned
block lists, then the attention);
`indexed_long_prefill` makes the selection inside the step with the QSA
indexer and Top-K (qsa_indexer_topk) before the same two passes.  The default workload is the long prefill of the page "Qwen4-Exp QSA
comes to Huawei's Ascend: inside SGLang's opt-in CANN prefill PR" (section
"Nine tests that passed, ..."): 7,810 query tokens, a 65,536-slot cache,
2,051 selected slots per token, (Hq, Hkv) = (16, 2), D = 256, BF16.

Prints one JSON line: selected (query-head, slot) pairs per second; the
attention kernel's memory traffic against the HBM roofline (`roofline`: the
bytes it moves beyond the L2s, from rocprofv3 counters recorded for this
version of the kernel, over its live time) and its algorithmic bytes over its
time (`algorithmic_GBps`, which passes the HBM peak because the L2s serve
most of the gathers); the read ceilings of the L2s, the Infinity Cache and
HBM measured in the same run with a plain streaming read; and the FP32 CPU
oracle timed on bounded samples of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
COUNTERS_FILE = os.path.join(ROOT, "profiles", "attend_counters.json")
CSRC = os.path.join(ROOT, "top_sparse_attention_amd", "csrc")
# The sources the attention kernel is compiled from: counters recorded for
# another version of any of them are not used.
KERNEL_SOURCES = [os.path.join(CSRC, n) for n in ("qsa_attend.hip", "qsa_device.h",
                                                   "qsa_kernels.h")]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long_prefill",
                    choices=["tiny", "edge_mix", "long_prefill", "two_request",
                             "max_cache_6_1", "max_cache_3_1", "decode_batch",
                             "long_prefill_fp8kv", "decode_batch_fp8kv", "long_prefill_block4",
                             "indexed_long_prefill"])
    ap.add_argument("--cpu-rows", type=int, default=2048,
                    help="token rows of the workload the CPU oracle is timed on")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a 1 GiB device copy first (for counter calibration)")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache steps, the device-copy reference and the read "
                         "ceilings (they add kernel instances to a profile)")
    ap.add_argument("--graph", action="store_true",
                    help="time the step as replays of one captured HIP graph (the kernels' "
                         "own times still come from the eager loop)")
    return ap.parse_args()


def kernel_sha() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_counters(workload: str):
    """The attention kernel's counters per launch for this workload from the
    committed rocprofv3 summary (calibrated FETCH_SIZE + WRITE_SIZE bytes,
    L2 hits and misses), or None if they were taken on another version of the
    kernel's sources."""
    try:
        with open(COUNTERS_FILE) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != kernel_sha():
        return None
    return rec


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def read_ceilings(qsa, torch, dev, reps=10):
    """Read bandwidth of the L2s, the Infinity Cache and HBM, measured with
    the library's streaming-read kernel (16-byte coalesced loads), in GB/s.

    Workgroups go to the 8 XCDs round robin.  L2: a 16 MiB footprint read
    64 KiB per workgroup, so each XCD reads its own 2 MiB (half its 4 MB L2)
    over and over, 4 GiB in all.  Infinity Cache: 128 MiB read 256 KiB per
    workgroup, 16 MiB per XCD (4x its L2; all of it fits the 256 MB cache),
    each byte 8 times.  HBM: 2 GiB (8x the Infinity Cache) read once per
    launch, 128 KiB per workgroup.  (Grid and slice sizes are the fastest of a
    sweep; slices of 1 MiB let workgroups running together on an XCD read the
    same lines and measure L2 sharing instead.)"""
    buf = torch.empty(1 << 31, dtype=torch.uint8, device=dev)
    buf.fill_(3)
    cases = [("hbm", 1 << 31, 1 << 17, 16384),
             ("infinity_cache", 1 << 27, 1 << 18, 4096),
             ("l2", 1 << 24, 1 << 16, 65536)]
    out = {}
    for name, foot, per_wg, wgs in cases:
        sink = torch.empty(wgs, dtype=torch.int32, device=dev)
        for _ in range(2):
            qsa.stream_read(buf, foot, per_wg, wgs, sink)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            qsa.stream_read(buf, foot, per_wg, wgs, sink)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = {"GBps": per_wg * wgs / (ms * 1e-3) / 1e9, "footprint_MiB": foot >> 20,
                     "read_MiB": (per_wg * wgs) >> 20, "us": ms * 1e3}
    del buf
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import qsa_inputs as qi
    import top_sparse_attention_amd as qsa
    from qsa_testutil import bf16_tensor_to_f32, empty_row_mask, gate, upload, upload_fp8

    qsa.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gen = qi.WORKLOADS[args.workload]
    case = gen() if args.seed is None else gen(args.seed)
    T, S, W, Hq, Hkv = case.T, case.S, case.W, case.Hq, case.Hkv
    q, k, v, sl = upload(case, dev)
    fp8 = "k8" in case.info
    if fp8:
        # The cache in FP8 E4M3 (one scale per tensor); the BF16 copies are freed.
        k, v, k_scale, v_scale = upload_fp8(case, dev)
    out = torch.empty((T, Hq, case.D), dtype=torch.bfloat16, device=dev)
    # Micro-block selections: each entry names `bs` consecutive slots, and the
    # compacted list (the attention's input) is bs times wider.
    bs = int(case.info.get("block_size", 1))
    Wl = W * bs
    ws = qsa.new_workspace(T, Wl, dev)
    # The attention's layout choice word (share area, after the 32 sampled
    # pairs' floats): a value the sharing estimate never writes, so that it
    # stays where no estimate runs.
    choice_off = qsa.workspace_layout(T, Wl)["share_offset"] + 32 * 8
    ws[choice_off:choice_off + 4].view(torch.int32).fill_(-1)
    scale = case.scale if case.scale is not None else 1.0 / np.sqrt(case.D)
    torch.cuda.synchronize()

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        a.fill_(1)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    # Indexed workloads make their selection on the GPU first (QSA indexer
    # scores + Top-K), inside the step.
    indexed = "iq" in case.info
    if indexed:
        to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        iq = to_dev(case.info["iq"].view(np.int16)).view(torch.bfloat16)
        ik = to_dev(case.info["ik"].view(np.int16)).view(torch.bfloat16)
        ipos, isop = to_dev(case.info["positions"]), to_dev(case.info["slot_of_pos"])
        # The [T, C] FP32 scores the indexer writes and the Top-K reads (the
        # faster of the two Top-K paths on MI355X).
        iscores = torch.empty((T, ik.shape[0]), dtype=torch.float32, device=dev)
        budget = case.info["budget"]

    def select():
        if indexed:
            qsa.indexer_topk(iq, ik, ipos, isop, budget, scores=iscores, out=sl)

    # Few-token workloads run qsa_sparse_decode: split attention over the raw
    # selection rows into FP32 partials, then the merge (no compaction pass).
    split = args.workload in ("decode_batch", "decode_batch_fp8kv")
    splits = qsa.decode_splits(T, W, Hq, Hkv) if split else 1
    dws = (torch.empty(qsa.decode_workspace_bytes(T, W, Hq, Hkv), dtype=torch.uint8, device=dev)
           if split else None)

    # Micro-block workloads run qsa_sparse_prefill_blocks (its compaction
    # writes the aligned block lists when the workspace has room for them),
    # so their attend time includes the compaction.
    bws = (torch.empty(qsa.prefill_blocks_workspace_bytes(T, W, bs), dtype=torch.uint8,
                       device=dev) if bs > 1 else None)

    def compact():
        if split or bs > 1:
            return
        qsa.compact_slots(sl, S, ws)

    def attend():
        if split and fp8:
            qsa.sparse_decode_fp8kv(q, k, v, k_scale, v_scale, sl, scale=scale, out=out,
                                    workspace=dws)
        elif split:
            qsa.sparse_decode(q, k, v, sl, scale=scale, out=out, workspace=dws)
        elif bs > 1:
            qsa.sparse_prefill_blocks(q, k, v, sl, bs, scale=scale, out=out, workspace=bws)
        elif fp8:
            qsa.sparse_attend_fp8kv(q, k, v, k_scale, v_scale, ws, W, scale=scale, out=out)
        else:
            qsa.sparse_attend(q, k, v, ws, Wl, scale=scale, out=out)

    def finish():
        pass

    def step():
        select()
        compact()
        attend()
        finish()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(K):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms_total = t0.elapsed_time(t1)
    ms_step = ms_total / K
    ms_step_eager = ms_step
    if args.graph:
        # The whole step captured once (the library records no memset and no
        # synchronous call on these paths) and replayed K times.
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(max(args.warmup, 1)):
            graph.replay()
        torch.cuda.synchronize()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(K):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        ms_step = g0.elapsed_time(g1) / K
    # The passes of the step timed one by one (events between them), in a
    # second run of K steps: the timed loop above has no events inside it.
    a0 = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    a1 = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    s0 = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    s1 = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    for i in range(K):
        s0[i].record()
        select()
        s1[i].record()
        compact()
        a0[i].record()
        attend()
        a1[i].record()
        finish()
    torch.cuda.synchronize()
    attn_ms = [a0[i].elapsed_time(a1[i]) for i in range(K)]
    attn_avg = float(np.mean(attn_ms))
    select_ms = float(np.mean([s0[i].elapsed_time(s1[i]) for i in range(K)])) \
        if indexed else None
    # The compaction pass (a1) alone, where it is a pass of its own; its
    # workspace traffic is implementation traffic, reported apart from the
    # algorithmic bytes: the selection rows read, the lists, counts and
    # invalid counts written.
    compacts = not split and bs == 1
    compact_ms = float(np.mean([s1[i].elapsed_time(a0[i]) for i in range(K)])) \
        if compacts else None
    compact_bytes = (T * W * 4 + T * qsa.workspace_layout(T, W)["row_stride"] * 4 + 8 * T) \
        if compacts else None

    # Gather only: the same rows, loads and launch shape with no arithmetic,
    # the loads issued back to back.
    sink = torch.empty(T * Hkv, dtype=torch.int32, device=dev)
    gather_only = qsa.gather_only_fp8kv if fp8 else qsa.gather_only
    if split:   # the decode step compacts nothing; the reference needs the lists
        qsa.compact_slots(sl, S, ws)
    elif bs > 1:   # plain (unaligned) block lists
        qsa.compact_blocks(sl, S, bs, ws)
    for _ in range(2):
        gather_only(k, v, ws, T, Wl, sink)
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(K):
        gather_only(k, v, ws, T, Wl, sink)
    c1.record()
    torch.cuda.synchronize()
    gather_only_ms = c0.elapsed_time(c1) / K
    peak_mib = torch.cuda.max_memory_allocated(dev) / 2**20

    # Cold steps: before each, a 1 GiB write (untimed) evicts the L2s and the
    # 256 MB Infinity Cache, so the step starts with its inputs in HBM only.
    # Then a device-to-device copy as the streaming reference of this GPU.
    cold, copy_ref = None, None
    if not args.no_cold:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        steps_ms, attend_ms_cold = [], []
        # The step with no events inside it (as in the warm loop; an event
        # between two launches adds a few microseconds to a short step), then
        # separate steps with events around the attention alone.
        for _ in range(min(K, 10)):
            flush.fill_(1)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record()
            step()
            ev[1].record()
            torch.cuda.synchronize()
            steps_ms.append(ev[0].elapsed_time(ev[1]))
        for _ in range(min(K, 10)):
            flush.fill_(1)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            select()
            compact()
            ev[0].record()
            attend()
            ev[1].record()
            finish()
            torch.cuda.synchronize()
            attend_ms_cold.append(ev[0].elapsed_time(ev[1]))
        cold = {"ms_per_step_median": float(np.median(steps_ms)),
                "attend_kernel_ms_median": float(np.median(attend_ms_cold)),
                "steps": len(steps_ms), "flush_bytes": 1 << 30}
        del flush
        src = torch.empty(1 << 31, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        dst.copy_(src)
        x0 = torch.cuda.Event(enable_timing=True)
        x1 = torch.cuda.Event(enable_timing=True)
        x0.record()
        for _ in range(5):
            dst.copy_(src)
        x1.record()
        torch.cuda.synchronize()
        copy_ref = {"GBps": 5 * 2 * src.numel() / (x0.elapsed_time(x1) * 1e-3) / 1e9,
                    "what": "torch device-to-device copy of 2 GiB; read + write bytes / time"}
        del src, dst
    ceilings = None if args.no_cold else read_ceilings(qsa, torch, dev)

    if indexed:
        # 4 positions per kept block (at most `budget` complete causal blocks)
        # plus the causal tail; fixed by the positions alone.
        p_ = case.info["positions"].astype(np.int64)
        n_t = 4 * np.minimum(np.minimum((p_ + 1) // 4, case.info["ik"].shape[0]), budget) \
            + (p_ + 1) % 4
    else:
        valid = (case.slot_idx >= 0) & (case.slot_idx < S // bs)
        n_t = valid.sum(axis=1).astype(np.int64) * bs      # selected slots per token
    pairs = int(n_t.sum()) * Hq
    # Algorithmic bytes of one pass: every selected K and V row of every
    # (token, KV head) once, Q in, O out, and the selection rows (T x W int32).
    kv_bytes = 1 if fp8 else 2
    attn_bytes = (int(n_t.sum()) * Hkv * 2 * case.D * kv_bytes + 2 * T * Hq * case.D * 2
                  + T * W * 4)
    gather_bytes = int(n_t.sum()) * Hkv * 2 * case.D * kv_bytes
    flops = pairs * 4 * case.D
    algorithmic_gbps = attn_bytes / (attn_avg * 1e-3) / 1e9

    # The roofline: bytes the attention kernel moves beyond the L2s (calibrated
    # FETCH_SIZE + WRITE_SIZE counters recorded for this version of its
    # sources; they count Infinity-Cache hits too, so this bounds its HBM
    # traffic from above) over its live time, against the HBM peak.
    counters = recorded_counters(args.workload)
    traffic = counters["fetch_write_bytes_per_launch"] if counters else None
    achieved = traffic / (attn_avg * 1e-3) / 1e9 if traffic else None
    hierarchy = None
    if counters:
        l2_req = counters["l2_requests_per_launch"] * 128
        beyond = counters["l2_misses_per_launch"] * 128
        hierarchy = {
            "l2_request_bytes": l2_req, "l2_request_GBps": l2_req / (attn_avg * 1e-3) / 1e9,
            "l2_hit_rate": 1.0 - counters["l2_misses_per_launch"] /
            counters["l2_requests_per_launch"],
            "beyond_l2_bytes": beyond, "beyond_l2_GBps": beyond / (attn_avg * 1e-3) / 1e9,
            "counters": "rocprofv3 TCC_HIT_sum + TCC_MISS_sum (128-byte requests), "
                        "FETCH_SIZE/WRITE_SIZE; " + os.path.relpath(COUNTERS_FILE, ROOT)}
        if ceilings:
            hierarchy["l2_request_frac_of_l2_ceiling"] = \
                hierarchy["l2_request_GBps"] / ceilings["l2"]["GBps"]
            hierarchy["beyond_l2_frac_of_infinity_cache_ceiling"] = \
                hierarchy["beyond_l2_GBps"] / ceilings["infinity_cache"]["GBps"]
            hierarchy["beyond_l2_frac_of_hbm_ceiling"] = \
                hierarchy["beyond_l2_GBps"] / ceilings["hbm"]["GBps"]

    # The sharing estimate's choice for the prefill attention (0: 8 items per
    # CU, 1: 4 per CU, 2: 8 with the keys through LDS), None where no
    # estimate ran (the sizes decided) or the step has no such attention.
    layout_choice = None
    if not split and bs == 1:
        c_ = int(ws[choice_off:choice_off + 4].view(torch.int32).item())
        layout_choice = c_ if c_ >= 0 else None

    # Parity of this very output on a sample of rows, checked against the oracle.
    import oracle

    def run_oracle(rows_, nthreads=0):
        if bs > 1:
            return oracle.prefill_blocks(case.q, case.k_cache, case.v_cache, case.slot_idx, bs,
                                         scale, rows=rows_, nthreads=nthreads)
        if fp8:
            return oracle.prefill_fp8kv(case.q, case.info["k8"], case.info["v8"], k_scale,
                                        v_scale, case.slot_idx, scale, rows=rows_,
                                        nthreads=nthreads)
        return oracle.prefill(case.q, case.k_cache, case.v_cache, case.slot_idx, scale,
                              rows=rows_, nthreads=nthreads)

    rows = qi.sample_rows(T, 16, seed=11)
    if indexed:
        # The oracle makes its own selection for the sampled rows; rows whose
        # GPU selection is identical are checked against the oracle's
        # attention over that selection (near-tie cuts may differ).
        o_sel = oracle.indexer_select(oracle.indexer_scores(case.info["iq"][rows],
                                                            case.info["ik"]),
                                      case.info["positions"][rows], case.info["slot_of_pos"],
                                      budget)
        same = np.all(sl[torch.as_tensor(rows, device=dev)].cpu().numpy() == o_sel, axis=1)
        rows_same = rows[same]
        want = oracle.prefill(np.ascontiguousarray(case.q[rows_same]), case.k_cache,
                              case.v_cache, np.ascontiguousarray(o_sel[same]), scale)
        got = bf16_tensor_to_f32(out[torch.as_tensor(rows_same, device=dev)])
        parity = gate(got, want, n_t[rows_same] == 0)
        parity["selection_rows_identical"] = f"{int(same.sum())}/{rows.size}"
    else:
        want = run_oracle(rows)
        got = bf16_tensor_to_f32(out[torch.as_tensor(rows, device=dev)])
        parity = gate(got, want, n_t[rows] == 0)

    cpu = None
    if not args.no_cpu_baseline and not indexed:
        cpu_rows = qi.sample_rows(T, min(args.cpu_rows, T), seed=12)
        threads = oracle.default_threads()
        c_t0 = time.perf_counter()
        run_oracle(cpu_rows, threads)
        c_dt = time.perf_counter() - c_t0
        cpu_pairs = int(n_t[cpu_rows].sum()) * Hq
        # The same oracle on one core, over a sixteenth of those rows.
        one_rows = qi.sample_rows(T, max(2, min(args.cpu_rows, T) // 16), seed=13)
        c_t0 = time.perf_counter()
        run_oracle(one_rows, 1)
        one_dt = time.perf_counter() - c_t0
        one_pairs = int(n_t[one_rows].sum()) * Hq
        cpu = {"value": cpu_pairs / c_dt, "unit": "pairs/s", "cores": threads, "kind": "oracle",
               "sample": f"{cpu_rows.size} of {T} token rows (all {Hq} heads, seeded, incl. first "
                         f"and last), {cpu_pairs} pairs in {c_dt:.2f} s",
               "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
               "one_core": {"value": one_pairs / one_dt, "unit": "pairs/s",
                            "sample": f"{one_rows.size} token rows, {one_pairs} pairs in "
                                      f"{one_dt:.2f} s"},
               "full_config_s_extrapolated": pairs / (cpu_pairs / c_dt),
               "gpu_over_cpu": (pairs / (ms_step * 1e-3)) / (cpu_pairs / c_dt),
               "full_config_s_one_core_extrapolated": pairs / (one_pairs / one_dt)}

    record = {
        "metric": "selected (query-head,slot) pairs/sec + achieved gather GB/s & % HBM roofline",
        "value": pairs / (ms_step * 1e-3),
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "ms_per_step_eager": ms_step_eager,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16+fp8kv" if fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": case.name, "T": T, "S": S, "W": W, "Hq": Hq, "Hkv": Hkv,
                   "D": case.D, "scale": scale, "seed": case.info.get("seed"),
                   "splits": splits, "block_size": bs, "parallelism": "none (1 GPU)",
                   "launch": "hip_graph" if args.graph else "eager",
                   "sharing_estimate_choice": layout_choice},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS if achieved else None,
                     "traffic": traffic,
                     "basis": "bytes beyond the L2s per attention launch (calibrated rocprofv3 "
                              "FETCH_SIZE + WRITE_SIZE, an upper bound of its HBM bytes) / "
                              "attend_kernel_ms"},
        "algorithmic_GBps": algorithmic_gbps,
        "hierarchy": hierarchy,
        "read_ceilings": ceilings,
        "cpu_baseline": cpu,
        "attend_kernel_ms": attn_avg,
        "compact_ms": compact_ms,
        "compact_bytes": compact_bytes,
        "indexer_topk_ms": select_ms,
        "attend_kernel_ms_min": float(np.min(attn_ms)),
        "attend_kernel_ms_median": float(np.median(attn_ms)),
        "cold": cold,
        "device_copy": copy_ref,
        "gather_GBps": gather_bytes / (attn_avg * 1e-3) / 1e9,
        "gather_only": {"ms": gather_only_ms,
                        "GBps": gather_bytes / (gather_only_ms * 1e-3) / 1e9},
        "mfma_frac": flops / (attn_avg * 1e-3) / (MFMA_BF16_PEAK_TFLOPS * 1e12),
        "attend_bytes_per_launch": attn_bytes,
        "parity": {"rows": int(rows.size), **{k_: v_ for k_, v_ in parity.items()
                                              if k_ != "rows"}},
        "peak_allocated_MiB": peak_mib,
    }
    print(json.dumps(record), flush=True)


if __name__ == "__main__":
    main()
