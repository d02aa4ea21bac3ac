// Drives every entry point of the C-ABI layer, built for the host only under
// AddressSanitizer and UBSan with the launch stand-ins of host_stubs.cpp:
// valid calls of the workloads' shapes (checking the parameters handed to the
// launchers), refused calls (checking that nothing was launched), launch-size
// limits and the size functions over extreme arguments.  Device pointers are
// made-up addresses that nothing on the host dereferences.  Exit status 0
// when every check holds.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <limits>

#include "host_stubs.h"
#include "qsa.h"

namespace {

int failures = 0;

#define CHECK(cond)                                                                  \
    do {                                                                             \
        if (!(cond)) {                                                               \
            std::fprintf(stderr, "%s:%d: check failed: %s (%s)\n", __FILE__, __LINE__, \
                         #cond, qsa_last_error());                                   \
            ++failures;                                                              \
        }                                                                            \
    } while (0)

void *addr(int64_t tib) { return (void *)(uintptr_t)((uint64_t)tib << 40); }

qsa_bf16_view view3(int64_t tib, int64_t n, int64_t h, int64_t d = 256) {
    qsa_bf16_view v{};
    v.data = addr(tib);
    v.size[0] = n;
    v.size[1] = h;
    v.size[2] = d;
    v.stride[0] = h * d;
    v.stride[1] = d;
    v.stride[2] = 1;
    return v;
}

qsa_i32_view view2(int64_t tib, int64_t t, int64_t w) {
    qsa_i32_view v{};
    v.data = (const int32_t *)addr(tib);
    v.size[0] = t;
    v.size[1] = w;
    v.stride[0] = w;
    v.stride[1] = 1;
    return v;
}

struct Shape {
    int64_t T, S, W, Hq, Hkv;
};

void prefill_shapes() {
    const Shape shapes[] = {{7810, 65536, 2051, 16, 2}, {8192, 131072, 2048, 24, 2},
                            {16384, 262144, 2048, 6, 1}, {16384, 262144, 2048, 3, 1},
                            {64, 1024, 64, 16, 2},      {257, 4096, 2051, 12, 1},
                            {5, 3000, 100, 40, 2},      {1, 7, 0, 64, 1}};
    for (const Shape &s : shapes) {
        qsa_bf16_view q = view3(1, s.T, s.Hq), k = view3(2, s.S, s.Hkv), v = view3(3, s.S, s.Hkv),
                      o = view3(4, s.T, s.Hq);
        qsa_i32_view sl = view2(5, s.T, s.W);
        const size_t ws_bytes = qsa_workspace_bytes(s.T, s.W);
        CHECK(ws_bytes == qsa_sparse_prefill_workspace_bytes(s.T, s.W));
        stub::calls.clear();
        CHECK(qsa_sparse_prefill(&q, &k, &v, &sl, 0.0625f, &o, addr(6), ws_bytes, nullptr) == QSA_OK);
        CHECK(stub::calls.compact.size() == 1 && stub::calls.attend.size() == 1);
        if (stub::calls.compact.size() == 1) {
            const qsa::CompactParams &c = stub::calls.compact[0];
            CHECK(c.T == s.T && c.W == s.W && c.S == s.S && c.lo == 0 && c.hi == s.S);
            CHECK(c.row_stride >= s.W && c.row_stride % 32 == 0 && c.align_shift == -1);
            CHECK((int64_t)1 << (c.key_bits - 1) >= s.S);
        }
        if (stub::calls.attend.size() == 1) {
            const qsa::AttendParams &a = stub::calls.attend[0];
            CHECK(a.G == s.Hq / s.Hkv && a.HB == (a.G + 15) / 16 && a.S_rows == s.S);
            CHECK(std::fabs(a.scale_log2e - 0.0625f * 1.4426950408889634f) < 1e-6f);
            // The long prefill's sizes bound its sharing at 8.1: the general
            // layout without an estimate and with its keys direct.
            if (s.T == 7810) CHECK(!stub::calls.attend_shared[0] && a.keys_lds == 0);
            if (stub::calls.attend_shared[0]) {
                const qsa::SharingParams &sp = stub::calls.share[0];
                CHECK(sp.lds_threshold == qsa::kShareKeysLds && a.keys_lds == 0);
                for (int i = 0; i < sp.pairs; ++i)
                    CHECK(sp.pair_a[i] >= 0 && sp.pair_a[i] < s.T && sp.pair_b[i] >= 0 &&
                          sp.pair_b[i] < s.T && sp.pair_a[i] != sp.pair_b[i]);
            }
        }
        // the same problem as the FP8 and no-workspace-size-check variants
        stub::calls.clear();
        qsa_fp8_view k8{}, v8{};
        k8.data = k.data;
        v8.data = v.data;
        for (int i = 0; i < 3; ++i) {
            k8.size[i] = v8.size[i] = k.size[i];
            k8.stride[i] = v8.stride[i] = k.stride[i];
        }
        CHECK(qsa_sparse_prefill_fp8kv(&q, &k8, &v8, 0.5f, 2.0f, &sl, 0.0625f, &o, addr(6), ws_bytes,
                                       nullptr) == QSA_OK);
        CHECK(stub::calls.attend.size() == 1 && stub::calls.attend_kv[0] == qsa::KvType::kFp8);
        if (stub::calls.attend.size() == 1) {
            // FP8 caches have no keys-through-LDS form
            CHECK(stub::calls.attend[0].keys_lds == 0);
            if (stub::calls.attend_shared[0]) CHECK(stub::calls.share[0].lds_threshold == 0.0f);
        }
    }
    // Sizes that bound the sharing at 32: keys through LDS, no estimate.
    {
        const Shape s{4096, 16384, 2048, 16, 2};
        qsa_bf16_view q = view3(1, s.T, s.Hq), k = view3(2, s.S, s.Hkv), v = view3(3, s.S, s.Hkv),
                      o = view3(4, s.T, s.Hq);
        qsa_i32_view sl = view2(5, s.T, s.W);
        stub::calls.clear();
        CHECK(qsa_sparse_prefill(&q, &k, &v, &sl, 0.0625f, &o, addr(6), qsa_workspace_bytes(s.T, s.W),
                                 nullptr) == QSA_OK);
        CHECK(stub::calls.attend.size() == 1 && !stub::calls.attend_shared[0] &&
              stub::calls.attend[0].keys_lds == 1);
    }
}

void decode_and_split() {
    const int64_t T = 16, S = 262144, W = 2048, Hq = 24, Hkv = 2;
    qsa_bf16_view q = view3(1, T, Hq), k = view3(2, S, Hkv), v = view3(3, S, Hkv), o = view3(4, T, Hq);
    qsa_i32_view sl = view2(5, T, W);
    const size_t bytes = qsa_decode_workspace_bytes(T, W, (int32_t)Hq, (int32_t)Hkv);
    CHECK(qsa_decode_splits(T, W, (int32_t)Hq, (int32_t)Hkv) == 16);
    stub::calls.clear();
    CHECK(qsa_sparse_decode(&q, &k, &v, &sl, 0.0625f, &o, addr(6), bytes, nullptr) == QSA_OK);
    CHECK(stub::calls.compact.empty() && stub::calls.partial.size() == 1 && stub::calls.merge.size() == 1);
    if (stub::calls.partial.size() == 1) {
        const qsa::AttendParams &a = stub::calls.partial[0];
        CHECK(a.raw_rows == 1 && a.splits == 16 && a.W_raw == W && a.bad_part != nullptr);
    }
    if (stub::calls.merge.size() == 1)
        CHECK(stub::calls.merge[0].n_parts == 16 && stub::calls.merge[0].clear_flag != nullptr);
    CHECK(qsa_sparse_decode(&q, &k, &v, &sl, 0.0625f, &o, addr(6), bytes - 1, nullptr) ==
          QSA_ERR_WORKSPACE);
    // the FP8 cache: the same shares, K's scale folded into the softmax scale
    {
        qsa_fp8_view k8{}, v8{};
        k8.data = k.data;
        v8.data = v.data;
        for (int i = 0; i < 3; ++i) {
            k8.size[i] = v8.size[i] = k.size[i];
            k8.stride[i] = v8.stride[i] = k.stride[i];
        }
        stub::calls.clear();
        CHECK(qsa_sparse_decode_fp8kv(&q, &k8, &v8, 0.5f, 2.0f, &sl, 0.0625f, &o, addr(6), bytes,
                                      nullptr) == QSA_OK);
        CHECK(stub::calls.partial.size() == 1 && stub::calls.merge.size() == 1 &&
              stub::calls.attend_kv.size() == 1 && stub::calls.attend_kv[0] == qsa::KvType::kFp8);
        if (stub::calls.partial.size() == 1) {
            const qsa::AttendParams &a = stub::calls.partial[0];
            CHECK(a.raw_rows == 1 && a.splits == 16 && a.v_scale == 2.0f);
            CHECK(std::fabs(a.scale_log2e - 0.03125f * 1.4426950408889634f) < 1e-6f);
        }
        CHECK(qsa_sparse_decode_fp8kv(&q, &k8, &v8, NAN, 2.0f, &sl, 0.0625f, &o, addr(6), bytes,
                                      nullptr) == QSA_ERR_SCALE);
    }
    // an empty cache takes the compaction route
    qsa_bf16_view k0 = view3(2, 0, Hkv), v0 = view3(3, 0, Hkv);
    stub::calls.clear();
    CHECK(qsa_sparse_decode(&q, &k0, &v0, &sl, 0.0625f, &o, addr(6), bytes, nullptr) == QSA_OK);
    CHECK(stub::calls.compact.size() == 1 && stub::calls.partial.size() == 1 &&
          stub::calls.partial[0].raw_rows == 0);
    // shards and the merge
    const size_t ws = qsa_workspace_bytes(T, W);
    stub::calls.clear();
    CHECK(qsa_compact_slot_range(&sl, S, 1000, 5000, addr(6), ws, nullptr) == QSA_OK);
    CHECK(stub::calls.compact.size() == 1 && stub::calls.compact[0].lo == 1000 &&
          stub::calls.compact[0].hi == 5000);
    qsa_bf16_view ks = view3(2, 4000, Hkv), vs = view3(3, 4000, Hkv);
    const size_t pb = qsa_partials_bytes(3, T, Hq);
    CHECK(qsa_sparse_attend_partial(&q, &ks, &vs, W, 0.0625f, addr(6), ws, 2, 1, 3, addr(7), pb,
                                    nullptr) == QSA_OK);
    CHECK(qsa_sparse_attend_partial(&q, &ks, &vs, W, 0.0625f, addr(6), ws, 3, 1, 3, addr(7), pb,
                                    nullptr) == QSA_ERR_SHAPE);
    CHECK(qsa_merge_partials(addr(7), pb, 3, T, Hq, &o, nullptr) == QSA_OK);
}

void blocks() {
    const int64_t T = 7810, S = 65536, W = 513;
    qsa_bf16_view q = view3(1, T, 16), k = view3(2, S, 2), v = view3(3, S, 2), o = view3(4, T, 16);
    qsa_i32_view bl = view2(5, T, W);
    for (int bs : {1, 2, 3, 4, 8, 16, 32, 64}) {
        const int64_t Sb = S / bs * bs;
        qsa_bf16_view kb = view3(2, Sb, 2), vb = view3(3, Sb, 2);
        const size_t bytes = qsa_prefill_blocks_workspace_bytes(T, W, bs);
        CHECK(bytes >= qsa_workspace_bytes(T, W * bs));
        stub::calls.clear();
        CHECK(qsa_sparse_prefill_blocks(&q, &kb, &vb, &bl, bs, 0.0625f, &o, addr(6), bytes,
                                        nullptr) == QSA_OK);
        CHECK(stub::calls.compact.size() == 1 && stub::calls.attend.size() == 1);
        if (stub::calls.compact.size() == 1 && stub::calls.attend.size() == 1) {
            const bool aligned = bs >= 4 && (bs & (bs - 1)) == 0;
            CHECK((stub::calls.compact[0].align_shift >= 0) == aligned);
            CHECK(stub::calls.attend[0].masked == (aligned ? 1 : 0));
            if (aligned) {
                CHECK(stub::calls.compact[0].block_ids == 1);
                CHECK((1 << stub::calls.attend[0].block_shift) == bs);
                CHECK(stub::calls.compact[0].align_cap <= qsa::kAlignRoomMax);
            }
        }
        stub::calls.clear();
        CHECK(qsa_compact_blocks(&bl, Sb, bs, addr(6), qsa_workspace_bytes(T, W * bs), nullptr) == QSA_OK);
        CHECK(stub::calls.compact.size() == 1 && stub::calls.compact[0].block == bs);
    }
    qsa_bf16_view k63 = view3(2, 63, 2), v63 = view3(3, 63, 2);
    CHECK(qsa_sparse_prefill_blocks(&q, &k63, &v63, &bl, 4, 0.0625f, &o, addr(6), 1ull << 40,
                                    nullptr) == QSA_ERR_SHAPE);
    CHECK(qsa_sparse_prefill_blocks(&q, &k, &v, &bl, 65, 0.0625f, &o, addr(6), 1ull << 40,
                                    nullptr) == QSA_ERR_SHAPE);
}

void refused() {
    const int64_t T = 4, S = 64, W = 8;
    struct Case {
        const char *name;
        qsa_status want;
        void (*mutate)(qsa_bf16_view &, qsa_bf16_view &, qsa_bf16_view &, qsa_bf16_view &,
                       qsa_i32_view &, float &);
    };
    const Case cases[] = {
        {"head dim", QSA_ERR_UNSUPPORTED, [](auto &q, auto &, auto &, auto &, auto &, float &) { q.size[2] = 128; }},
        {"inner stride", QSA_ERR_STRIDE, [](auto &q, auto &, auto &, auto &, auto &, float &) { q.stride[2] = 2; }},
        {"misaligned base", QSA_ERR_STRIDE, [](auto &, auto &k, auto &, auto &, auto &, float &) { k.data = (char *)k.data + 2; }},
        {"odd stride", QSA_ERR_STRIDE, [](auto &, auto &, auto &v, auto &, auto &, float &) { v.stride[0] = 516; }},
        {"negative size", QSA_ERR_SHAPE, [](auto &, auto &k, auto &, auto &, auto &, float &) { k.size[0] = -1; }},
        {"negative stride", QSA_ERR_STRIDE, [](auto &q, auto &, auto &, auto &, auto &, float &) { q.stride[0] = -1024; }},
        {"out shape", QSA_ERR_SHAPE, [](auto &, auto &, auto &, auto &o, auto &, float &) { o.size[0] = 5; }},
        {"slot rows", QSA_ERR_SHAPE, [](auto &, auto &, auto &, auto &, auto &s, float &) { s.size[0] = 3; }},
        {"null q", QSA_ERR_NULL, [](auto &q, auto &, auto &, auto &, auto &, float &) { q.data = nullptr; }},
        {"alias", QSA_ERR_ALIAS, [](auto &q, auto &, auto &, auto &o, auto &, float &) { o.data = q.data; }},
        {"nan scale", QSA_ERR_SCALE, [](auto &, auto &, auto &, auto &, auto &, float &sc) { sc = std::nanf(""); }},
        {"inf scale", QSA_ERR_SCALE, [](auto &, auto &, auto &, auto &, auto &, float &sc) { sc = INFINITY; }},
        {"huge heads", QSA_ERR_UNSUPPORTED, [](auto &q, auto &, auto &, auto &o, auto &, float &) { q.size[1] = o.size[1] = (int64_t)1 << 33; }},
        {"Hq % Hkv", QSA_ERR_SHAPE, [](auto &q, auto &, auto &, auto &o, auto &, float &) { q.size[1] = o.size[1] = 3; q.stride[0] = o.stride[0] = 768; }},
    };
    for (const Case &c : cases) {
        qsa_bf16_view q = view3(1, T, 4), k = view3(2, S, 2), v = view3(3, S, 2), o = view3(4, T, 4);
        qsa_i32_view sl = view2(5, T, W);
        float scale = 0.0625f;
        c.mutate(q, k, v, o, sl, scale);
        stub::calls.clear();
        const qsa_status st = qsa_sparse_prefill(&q, &k, &v, &sl, scale, &o, addr(6), 1 << 20, nullptr);
        if (st != c.want) std::fprintf(stderr, "case %s: status %d\n", c.name, (int)st);
        CHECK(st == c.want);
        CHECK(stub::calls.compact.empty() && stub::calls.attend.empty());
        CHECK(qsa_last_error()[0] != 0);
    }
    qsa_bf16_view q = view3(1, T, 4), k = view3(2, S, 2), v = view3(3, S, 2), o = view3(4, T, 4);
    qsa_i32_view sl = view2(5, T, W);
    CHECK(qsa_sparse_prefill(nullptr, &k, &v, &sl, 0.0625f, &o, addr(6), 1 << 20, nullptr) == QSA_ERR_NULL);
    CHECK(qsa_sparse_prefill(&q, &k, &v, nullptr, 0.0625f, &o, addr(6), 1 << 20, nullptr) == QSA_ERR_NULL);
    CHECK(qsa_sparse_prefill(&q, &k, &v, &sl, 0.0625f, &o, nullptr, 1 << 20, nullptr) == QSA_ERR_WORKSPACE);
    CHECK(qsa_sparse_prefill(&q, &k, &v, &sl, 0.0625f, &o, (char *)addr(6) + 16, 1 << 20, nullptr) == QSA_ERR_WORKSPACE);
    CHECK(qsa_sparse_prefill(&q, &k, &v, &sl, 0.0625f, &o, addr(6), 16, nullptr) == QSA_ERR_WORKSPACE);
    CHECK(qsa_compact_slot_range(&sl, S, 10, 5, addr(6), 1 << 20, nullptr) == QSA_ERR_SHAPE);
    CHECK(qsa_gather_only(&k, &v, T, W, addr(6), 1 << 20, nullptr, nullptr) == QSA_ERR_NULL);
    CHECK(qsa_stream_read(addr(1), 100, 16, 4, (uint32_t *)addr(2), nullptr) == QSA_ERR_SHAPE);
    CHECK(qsa_stream_read(addr(1), 1 << 20, 1 << 21, 4, (uint32_t *)addr(2), nullptr) == QSA_ERR_SHAPE);
    stub::calls.clear();
    CHECK(qsa_stream_read(addr(1), 1 << 20, 1 << 16, 4, (uint32_t *)addr(2), nullptr) == QSA_OK);
    CHECK(stub::calls.stream.size() == 1 && stub::calls.stream[0].chunks_per_wg == 4096);
    CHECK(qsa_gather_only(&k, &v, T, W, addr(6), 1 << 20, (uint32_t *)addr(7), nullptr) == QSA_OK);
}

void launch_limits() {
    const size_t huge = (size_t)1 << 62;
    {   // 2^24 tokens: the compaction's 256-thread workgroups exceed 2^32 work-items
        qsa_bf16_view q = view3(1, 1 << 24, 1), k = view3(2, 64, 1), v = view3(3, 64, 1),
                      o = view3(4, 1 << 24, 1);
        qsa_i32_view sl = view2(5, 1 << 24, 1);
        stub::calls.clear();
        CHECK(qsa_sparse_prefill(&q, &k, &v, &sl, 0.0625f, &o, addr(6), huge, nullptr) == QSA_ERR_UNSUPPORTED);
        CHECK(stub::calls.compact.empty() && stub::calls.attend.empty());
    }
    {
        qsa_bf16_view q = view3(1, 1 << 25, 16), k = view3(2, 64, 2), v = view3(3, 64, 2),
                      o = view3(4, 1 << 25, 16);
        CHECK(qsa_sparse_attend(&q, &k, &v, 1, 0.0625f, addr(6), huge, &o, nullptr) == QSA_ERR_UNSUPPORTED);
        qsa_bf16_view q1 = view3(1, (1 << 25) - 1, 16), o1 = view3(4, (1 << 25) - 1, 16);
        CHECK(qsa_sparse_attend(&q1, &k, &v, 1, 0.0625f, addr(6), huge, &o1, nullptr) == QSA_OK);
    }
}

void indexer() {
    const int64_t T = 100, C = 1000, L = 4000;
    const int32_t budget = 512;
    qsa_bf16_view iq = view3(1, T, 4, 128), ik = view3(2, C, 1, 128);
    qsa_i32_view out = view2(3, T, 4 * budget + 3);
    const size_t sb = qsa_indexer_scores_bytes(T, C), fb = qsa_indexer_topk_fused_bytes(T, C);
    CHECK(sb == (size_t)(T * C * 4) && fb > sb);
    stub::calls.clear();
    CHECK(qsa_indexer_topk_fused(&iq, &ik, (const int32_t *)addr(4), (const int32_t *)addr(5), L,
                                 budget, addr(6), fb, &out, nullptr) == QSA_OK);
    // the fused path: estimate, candidates, selection
    CHECK(stub::calls.estimate.size() == 1 && stub::calls.scores.size() == 1 &&
          stub::calls.select.size() == 1);
    if (stub::calls.scores.size() == 1)
        CHECK(stub::calls.scores[0].tau != nullptr && stub::calls.scores[0].R == 1 &&
              stub::calls.scores[0].pair_pitch == C + (C & 1) &&
              stub::calls.select[0].counts != nullptr &&
              stub::calls.select[0].pair_pitch == stub::calls.scores[0].pair_pitch);
    stub::calls.clear();
    CHECK(qsa_indexer_topk_fused(&iq, &ik, (const int32_t *)addr(4), (const int32_t *)addr(5), L,
                                 budget, addr(6), fb - 1, &out, nullptr) == QSA_ERR_WORKSPACE);
    CHECK(stub::calls.estimate.empty() && stub::calls.scores.empty() && stub::calls.select.empty());
    // qsa_indexer_topk, whatever its scratch: scores, then the selection
    for (size_t bytes : {sb, fb}) {
        stub::calls.clear();
        CHECK(qsa_indexer_topk(&iq, &ik, (const int32_t *)addr(4), (const int32_t *)addr(5), L,
                               budget, (float *)addr(6), bytes, &out, nullptr) == QSA_OK);
        CHECK(stub::calls.estimate.empty() && stub::calls.scores.size() == 1 &&
              stub::calls.scores[0].tau == nullptr && stub::calls.select.size() == 1);
    }
    qsa_i32_view out600 = view2(3, T, 4 * 600 + 3);
    stub::calls.clear();
    CHECK(qsa_indexer_topk(&iq, &ik, (const int32_t *)addr(4), (const int32_t *)addr(5), L, 600,
                           (float *)addr(6), sb, &out600, nullptr) == QSA_OK);
    CHECK(stub::calls.estimate.empty() && stub::calls.select.size() == 1);
    CHECK(qsa_indexer_topk_fused(&iq, &ik, (const int32_t *)addr(4), (const int32_t *)addr(5), L,
                                 600, addr(6), fb, &out600, nullptr) == QSA_ERR_UNSUPPORTED);
    CHECK(qsa_indexer_topk(&iq, &ik, (const int32_t *)addr(4), (const int32_t *)addr(5), 100, budget,
                           (float *)addr(6), sb, &out, nullptr) == QSA_ERR_SHAPE);
    CHECK(qsa_indexer_select((const float *)addr(6), (size_t)(T * C * 4) - 4, T, C, (const int32_t *)addr(4),
                             (const int32_t *)addr(5), L, budget, &out, nullptr) == QSA_ERR_WORKSPACE);
}

void sizes() {
    const int64_t big = std::numeric_limits<int64_t>::max();
    const int64_t vals[] = {-1, 0, 1, 31, 32, 33, 2051, 1 << 20, 0x7fffffff, (int64_t)1 << 40, big};
    for (int64_t T : vals)
        for (int64_t W : vals) {
            const size_t b = qsa_workspace_bytes(T, W);
            if (T < 0 || W < 0) CHECK(b == 0);
            qsa_workspace_map m;
            if (qsa_workspace_layout(T, W, &m) == QSA_OK) CHECK((size_t)m.total_bytes == b);
            (void)qsa_partials_bytes(T, W, 24);
            (void)qsa_decode_workspace_bytes(T, W, 24, 2);
            (void)qsa_decode_splits(T, W, 24, 2);
            (void)qsa_indexer_scores_bytes(T, W);
            (void)qsa_indexer_topk_fused_bytes(T, W);
            for (int bs : {1, 4, 64}) (void)qsa_prefill_blocks_workspace_bytes(T, W, bs);
        }
    for (int s = -1; s <= 10; ++s) CHECK(qsa_status_string((qsa_status)s) != nullptr);
    CHECK(qsa_version() != nullptr);
}

}  // namespace

int main() {
    prefill_shapes();
    decode_and_split();
    blocks();
    refused();
    launch_limits();
    indexer();
    sizes();
    if (failures) {
        std::fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    std::printf("all host checks passed\n");
    return 0;
}
