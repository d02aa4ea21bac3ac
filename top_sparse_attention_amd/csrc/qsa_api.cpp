// C ABI of libqsa (declared in include/qsa.h): host-side argument checks,
// workspace layout and kernel launches.  Every check runs on the host before
// any HIP call, so a rejected call enqueues nothing and touches no device.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <numeric>
#include <vector>

#include "qsa.h"
#include "qsa_errors.h"
#include "qsa_indexer.h"
#include "qsa_kernels.h"
#include "qsa_measure.h"

namespace {

thread_local char g_last_error[512] = "";

qsa_status fail(qsa_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return s;
}

}  // namespace

int qsa::set_error(int status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

namespace {

constexpr int64_t kAlign = 256;
constexpr int64_t kMax32 = 0x7fffffff;
// The sharing estimate's words in the workspace: est [kSharePairs][2] floats,
// then the choice.
constexpr int64_t kShareBytes = 512;
// Also in the share area: the compaction's extent words (the number of cache
// slots its lists index, and the flag an attention over a smaller cache view
// sets; see qsa::CompactParams).
constexpr int64_t kExtentOffset = 384;
static_assert(qsa::kSharePairs * 8 + 4 <= kExtentOffset && kExtentOffset + 8 <= kShareBytes &&
                  qsa::kSharePairs <= 64,
              "share-area words");

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// a * b for non-negative operands, saturated at INT64_MAX.
int64_t mul_sat(int64_t a, int64_t b) {
    if (a <= 0 || b <= 0) return 0;
    return a > INT64_MAX / b ? INT64_MAX : a * b;
}

// HIP counts the work-items of a launch along one grid dimension in 32 bits.
constexpr int64_t kMaxWorkItems = 0xffffffffLL;
// Largest grid along y (the indexer's key ranges).
constexpr int64_t kMaxGridY = 65535;

int32_t *extent_words(const void *ws, const qsa_workspace_map &m) {
    return (int32_t *)((char *)ws + m.share_offset + kExtentOffset);
}

// Workspace sizes beyond this many list entries are refused (far beyond any
// device memory; it keeps every byte offset within int64).
constexpr int64_t kMaxListEntries = (int64_t)1 << 56;

bool layout_of(int64_t T, int64_t W, qsa_workspace_map *m) {
    if (T < 0 || W < 0 || T > kMax32 || W > kMax32) return false;
    const int64_t row = round_up(W, qsa::kListPad);
    if (mul_sat(T, row) > kMaxListEntries) return false;
    m->list_offset = 0;
    m->row_stride = row;
    m->count_offset = round_up(T * row * 4, kAlign);
    m->bad_offset = m->count_offset + round_up(T * 4, kAlign);
    m->share_offset = m->bad_offset + round_up(T * 4, kAlign);
    m->total_bytes = m->share_offset + (T > 0 ? kShareBytes : 0);
    return true;
}

// A K/V cache of either element type, seen through the same fields.
struct KvView {
    const qsa_bf16_view *view;   // for FP8, the qsa_fp8_view reinterpreted (same layout)
    int elem_bytes;
};

static_assert(sizeof(qsa_fp8_view) == sizeof(qsa_bf16_view), "view layouts must agree");

const qsa_bf16_view *as_view(const qsa_fp8_view *v) {
    return reinterpret_cast<const qsa_bf16_view *>(v);
}

// Byte span [lo, hi) covered by a strided view (all strides non-negative).
void span_of(const qsa_bf16_view *v, uintptr_t *lo, uintptr_t *hi, int elem_bytes = 2) {
    int64_t last = 0;
    for (int i = 0; i < 3; ++i) last += (v->size[i] - 1) * v->stride[i];
    *lo = (uintptr_t)v->data;
    *hi = (uintptr_t)v->data + (uintptr_t)(last + 1) * elem_bytes;
}

bool any_empty(const qsa_bf16_view *v) {
    return v->size[0] == 0 || v->size[1] == 0 || v->size[2] == 0;
}

// Rows must start on 16-byte boundaries: base aligned, strides a multiple of
// 16 bytes (8 BF16 or 16 FP8 elements), unit innermost stride.
qsa_status check_view(const qsa_bf16_view *v, const char *name, int elem_bytes) {
    if (!v) return fail(QSA_ERR_NULL, "%s: view pointer is NULL", name);
    for (int i = 0; i < 3; ++i) {
        if (v->size[i] < 0) return fail(QSA_ERR_SHAPE, "%s: negative size", name);
        if (v->stride[i] < 0) return fail(QSA_ERR_STRIDE, "%s: negative stride", name);
    }
    if (v->size[2] != qsa::kHeadDim)
        return fail(QSA_ERR_UNSUPPORTED, "%s: head dim %lld, only %d is supported", name,
                    (long long)v->size[2], qsa::kHeadDim);
    if (any_empty(v)) return QSA_OK;
    if (!v->data) return fail(QSA_ERR_NULL, "%s: data is NULL", name);
    if (v->stride[2] != 1) return fail(QSA_ERR_STRIDE, "%s: innermost stride must be 1", name);
    if ((uintptr_t)v->data % 16)
        return fail(QSA_ERR_STRIDE, "%s: base pointer must be 16-byte aligned", name);
    const int64_t per16 = 16 / elem_bytes;
    if (v->stride[0] % per16 || v->stride[1] % per16)
        return fail(QSA_ERR_STRIDE, "%s: strides must be multiples of %lld elements", name,
                    (long long)per16);
    return QSA_OK;
}

qsa_status check_bf16(const qsa_bf16_view *v, const char *name) {
    return check_view(v, name, 2);
}

qsa_status check_workspace(const void *ws, size_t bytes, int64_t T, int64_t W,
                           qsa_workspace_map *m) {
    if (!layout_of(T, W, m)) return fail(QSA_ERR_SHAPE, "T and W must be in [0, 2^31)");
    if (!ws) return fail(QSA_ERR_WORKSPACE, "workspace is NULL");
    if ((uintptr_t)ws % kAlign) return fail(QSA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if ((int64_t)bytes < m->total_bytes)
        return fail(QSA_ERR_WORKSPACE, "workspace holds %zu bytes, %lld needed", bytes,
                    (long long)m->total_bytes);
    return QSA_OK;
}

struct Problem {
    int64_t T, S, W;
    int32_t Hq, Hkv;
};

// The kernels form a cache row's address as base + slot * (slot stride in
// bytes) with one unsigned 32 x 32 -> 64-bit multiply-add, so the slot
// stride of the cache views must stay under 4 GiB.
qsa_status check_slot_strides(const qsa_bf16_view *k, const qsa_bf16_view *v, int kv_bytes) {
    const int64_t lim = (int64_t)UINT32_MAX;
    if (k->stride[0] > lim / kv_bytes || v->stride[0] > lim / kv_bytes)
        return fail(QSA_ERR_UNSUPPORTED, "k_cache/v_cache: slot strides of 4 GiB or more");
    return QSA_OK;
}

// Checks of q, k_cache, v_cache, W and scale shared by every attention entry point.
qsa_status check_inputs(const qsa_bf16_view *q, const qsa_bf16_view *k, const qsa_bf16_view *v,
                        int64_t W, float scale, Problem *pr, int kv_bytes = 2) {
    qsa_status s;
    if ((s = check_bf16(q, "q")) || (s = check_view(k, "k_cache", kv_bytes)) ||
        (s = check_view(v, "v_cache", kv_bytes)))
        return s;
    for (int i = 0; i < 3; ++i)
        if (v->size[i] != k->size[i]) return fail(QSA_ERR_SHAPE, "v_cache must have k_cache's shape");
    if ((s = check_slot_strides(k, v, kv_bytes))) return s;
    pr->T = q->size[0];
    pr->S = k->size[0];
    pr->W = W;
    if (W < 0) return fail(QSA_ERR_SHAPE, "negative W");
    if (q->size[1] > kMax32 || k->size[1] > kMax32)
        return fail(QSA_ERR_UNSUPPORTED, "head counts beyond int32");
    pr->Hq = (int32_t)q->size[1];
    pr->Hkv = (int32_t)k->size[1];
    if (pr->T > 0 && (pr->Hq == 0 || pr->Hkv == 0))
        return fail(QSA_ERR_SHAPE, "Hq and Hkv must be positive");
    if (pr->Hkv > 0 && pr->Hq % pr->Hkv)
        return fail(QSA_ERR_SHAPE, "Hq (%d) must be a multiple of Hkv (%d)", pr->Hq, pr->Hkv);
    if (pr->T > kMax32 || W > kMax32 || pr->S > kMax32)
        return fail(QSA_ERR_UNSUPPORTED, "T, W and S must fit in int32");
    if (!std::isfinite(scale)) return fail(QSA_ERR_SCALE, "scale must be finite");
    return QSA_OK;
}

// A written byte range [lo, hi) must not overlap any of q, k_cache, v_cache.
qsa_status check_no_overlap(uintptr_t lo, uintptr_t hi, const qsa_bf16_view *q,
                            const qsa_bf16_view *k, const qsa_bf16_view *v, const char *what,
                            int kv_bytes = 2) {
    const qsa_bf16_view *ins[3] = {q, k, v};
    for (int i = 0; i < 3; ++i) {
        if (any_empty(ins[i])) continue;
        uintptr_t ilo, ihi;
        span_of(ins[i], &ilo, &ihi, i == 0 ? 2 : kv_bytes);
        if (lo < ihi && ilo < hi) return fail(QSA_ERR_ALIAS, "%s overlaps an input", what);
    }
    return QSA_OK;
}

qsa_status check_attend(const qsa_bf16_view *q, const qsa_bf16_view *k,
                        const qsa_bf16_view *v, const qsa_bf16_view *out, int64_t W,
                        float scale, Problem *pr, int kv_bytes = 2) {
    qsa_status s;
    if ((s = check_bf16(q, "q")) || (s = check_view(k, "k_cache", kv_bytes)) ||
        (s = check_view(v, "v_cache", kv_bytes)) || (s = check_bf16(out, "out")))
        return s;
    for (int i = 0; i < 3; ++i)
        if (out->size[i] != q->size[i]) return fail(QSA_ERR_SHAPE, "out must have q's shape");
    if ((s = check_inputs(q, k, v, W, scale, pr, kv_bytes))) return s;
    if (!any_empty(out)) {
        uintptr_t olo, ohi;
        span_of(out, &olo, &ohi);
        if ((s = check_no_overlap(olo, ohi, q, k, v, "out", kv_bytes))) return s;
    }
    return QSA_OK;
}

qsa_status check_fp8_scales(float k_scale, float v_scale) {
    if (!std::isfinite(k_scale) || !std::isfinite(v_scale))
        return fail(QSA_ERR_SCALE, "k_scale and v_scale must be finite");
    return QSA_OK;
}

qsa_status check_slots(const qsa_i32_view *sl, int64_t T, int64_t *W) {
    if (!sl) return fail(QSA_ERR_NULL, "slot_idx: view pointer is NULL");
    if (sl->size[0] < 0 || sl->size[1] < 0) return fail(QSA_ERR_SHAPE, "slot_idx: negative size");
    if (sl->size[0] != T) return fail(QSA_ERR_SHAPE, "slot_idx must have one row per token");
    *W = sl->size[1];
    if (sl->size[0] == 0 || sl->size[1] == 0) return QSA_OK;
    if (!sl->data) return fail(QSA_ERR_NULL, "slot_idx: data is NULL");
    if (sl->stride[1] != 1) return fail(QSA_ERR_STRIDE, "slot_idx: innermost stride must be 1");
    if (sl->stride[0] < 0) return fail(QSA_ERR_STRIDE, "slot_idx: negative stride");
    if ((uintptr_t)sl->data % 4) return fail(QSA_ERR_STRIDE, "slot_idx: misaligned");
    if (*W > kMax32 || T > kMax32) return fail(QSA_ERR_UNSUPPORTED, "T and W must fit in int32");
    return QSA_OK;
}

qsa_status hip_fail(hipError_t e, const char *what) {
    return fail(QSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// A launch of `blocks` workgroups of `threads` threads must stay within the
// work-items one grid dimension counts; larger problems are refused before
// anything is enqueued (the launch would otherwise fail or cover part of the
// work).
qsa_status check_grid(int64_t blocks, int64_t threads, const char *what) {
    if (mul_sat(blocks, threads) > kMaxWorkItems)
        return fail(QSA_ERR_UNSUPPORTED,
                    "%s: %lld workgroups of %lld threads exceed the 2^32 - 1 work-items of one "
                    "launch; split the call",
                    what, (long long)blocks, (long long)threads);
    return QSA_OK;
}

int64_t ceil_div(int64_t a, int64_t b) { return a / b + (a % b != 0); }

qsa_status check_compact_grid(int64_t T) { return check_grid(T, qsa::kSortThreads, "compaction"); }

// Attention items (token, KV head, block of 16 query heads), times splits.
qsa_status check_attend_grid(int64_t T, int64_t Hq, int64_t Hkv, int64_t splits) {
    if (Hkv <= 0) return QSA_OK;
    const int64_t HB = ceil_div(Hq / Hkv, 16);
    return check_grid(mul_sat(mul_sat(mul_sat(T, Hkv), HB), splits), 64, "attention");
}

// One wave per (token, head) row, four rows per workgroup.
qsa_status check_merge_grid(int64_t T, int64_t Hq) {
    return check_grid(mul_sat(T, Hq), 256, "merge");   // one workgroup per (token, head)
}

// Width of the compaction's sort key for entries in [0, n): the bits of
// n - 1 (at least one) plus the bit that marks invalid entries.
int32_t sort_key_bits(int64_t n) {
    int bits = 1;
    while (bits < 31 && ((int64_t)1 << bits) < n) ++bits;
    return bits + 1;
}

// Aligned block lists (see CompactParams): the super-range shift, their
// number and the row room, or shift -1 for the plain list.
struct AlignSpec {
    int32_t shift = -1, ranges = 0, cap = 0;
    int32_t block_shift = 0;   // log2 of the block size
    int32_t block_ids = 1;     // list entries are block ids (else each block's slots)
    int64_t list_offset = 0;   // of the aligned rows in the workspace
};

qsa_status enqueue_compact(const qsa_i32_view *sl, int64_t T, int64_t W, int64_t S, int64_t lo,
                           int64_t hi, void *ws, const qsa_workspace_map &m, hipStream_t stream,
                           int32_t block = 1, const AlignSpec *align = nullptr) {
    qsa::CompactParams p{};
    p.align_shift = -1;
    p.block = block;
    p.slot_idx = sl->data;
    p.stride_t = sl->stride[0];
    p.T = T;
    p.W = W;
    p.S = S;
    p.lo = lo;
    p.hi = hi;
    p.key_bits = sort_key_bits(hi - lo);
    p.list = (int32_t *)((char *)ws + m.list_offset);
    p.row_stride = m.row_stride;
    if (align != nullptr && align->shift >= 0) {
        p.align_shift = align->shift;
        p.align_ranges = align->ranges;
        p.align_cap = align->cap;
        p.block_ids = align->block_ids;
        p.list = (int32_t *)((char *)ws + align->list_offset);
        p.row_stride = align->cap;
    }
    p.count = (int32_t *)((char *)ws + m.count_offset);
    p.n_bad = (int32_t *)((char *)ws + m.bad_offset);
    p.extent = extent_words(ws, m);
    hipError_t e = qsa::launch_compact(p, stream);
    return e == hipSuccess ? QSA_OK : hip_fail(e, "compaction launch");
}

void fill_attend(qsa::AttendParams &p, const qsa_bf16_view *q, const qsa_bf16_view *k,
                 const qsa_bf16_view *v, const Problem &pr, float scale, const void *ws,
                 const qsa_workspace_map &m);

// KV element type and scales of one call (BF16: scales are 1 and unused).
struct KvKind {
    qsa::KvType type = qsa::KvType::kBf16;
    float k_scale = 1.0f, v_scale = 1.0f;
};

// Below this sharing bound from the sizes alone (rows full, every cache slot
// referenced) the sharing estimate runs; at or above it the estimate could
// only confirm the kItemsPerCU layout (full rows share at least this much).
constexpr double kShareSizeBound = 6.0;

// Parameters of the sharing estimate for an attention launch, or false where
// the kItemsPerCU layout is taken without one: the sizes already bound the
// sharing above kShareSizeBound, or there are fewer than two chip-fulls of
// items for the layout to matter.  Without an estimate, *keys_lds says
// whether the sizes alone bound the sharing at or above kShareKeysLds (BF16:
// the general layout then takes its keys through LDS).
bool sharing_of(const Problem &pr, int32_t HB, void *ws, const qsa_workspace_map &m,
                qsa::SharingParams *sp, bool bf16, bool *keys_lds) {
    *keys_lds = false;
    const int64_t per_t = (int64_t)pr.Hkv * HB;
    const int64_t chip = (int64_t)qsa::kXcds * qsa::kCusPerXcd * qsa::kItemsPerCU;
    if (pr.T < 2 || pr.T > kMax32 || per_t <= 0 || pr.T * per_t < 2 * chip || pr.S <= 0)
        return false;
    // KV heads among the items one XCD runs (items are dealt round robin, so
    // XCD 0 runs items 0, 8, 16, ...: within a token, the item offsets that are
    // multiples of d = gcd(per_t, 8)); KV head g owns offsets [g HB, (g+1) HB).
    const int64_t d = std::gcd(per_t, (int64_t)qsa::kXcds);
    int64_t heads = 0;
    for (int64_t g = 0; g < pr.Hkv; ++g) heads += (g * HB + d - 1) / d * d < (g + 1) * HB;
    const double per_xcd = (double)qsa::kCusPerXcd * qsa::kItemsPerCU / heads;
    const double bound = per_xcd * (double)m.row_stride;   // over S
    if (bound >= kShareSizeBound * (double)pr.S) {
        *keys_lds = bf16 && bound >= (double)qsa::kShareKeysLds * (double)pr.S;
        return false;
    }
    char *base = (char *)ws + m.share_offset;
    sp->list = (const int32_t *)((const char *)ws + m.list_offset);
    sp->row_stride = m.row_stride;
    sp->count = (const int32_t *)((const char *)ws + m.count_offset);
    // Pairs: a spread over [0, T - 2], b at most one chip-full of items later
    // (tokens that run at about the same time).
    const int64_t span = std::max<int64_t>(1, chip / per_t);
    sp->pairs = qsa::kSharePairs;
    for (int i = 0; i < qsa::kSharePairs; ++i) {
        const int64_t a = (int64_t)i * (pr.T - 2) / (qsa::kSharePairs - 1);
        sp->pair_a[i] = (int32_t)a;
        sp->pair_b[i] = (int32_t)std::min<int64_t>(a + 1 + (i * 37) % span, pr.T - 1);
    }
    sp->lambda_scale = (float)per_xcd;
    sp->threshold = m.row_stride >= qsa::kShareLongList ? qsa::kShareThreshold
                                                        : qsa::kShareThresholdShort;
    sp->lds_threshold = bf16 ? qsa::kShareKeysLds : 0.0f;
    sp->est = (float *)base;
    sp->choice = (int32_t *)(base + qsa::kSharePairs * 8);
    return true;
}

qsa_status enqueue_attend(const qsa_bf16_view *q, const qsa_bf16_view *k,
                          const qsa_bf16_view *v, const qsa_bf16_view *out, const Problem &pr,
                          float scale, void *ws, const qsa_workspace_map &m,
                          hipStream_t stream, KvKind kv = KvKind(),
                          const AlignSpec *align = nullptr) {
    if (pr.T == 0 || pr.Hq == 0) return QSA_OK;
    qsa::AttendParams p{};
    fill_attend(p, q, k, v, pr, scale * kv.k_scale, ws, m);
    p.v_scale = kv.v_scale;
    p.out = (uint16_t *)out->data;
    p.o_st = out->stride[0];
    p.o_sh = out->stride[1];
    if (align != nullptr && align->shift >= 0) {
        // Aligned block lists: -1 gaps inside the rows, masked per tile.
        p.list = (const int32_t *)((const char *)ws + align->list_offset);
        p.list_stride = align->cap;
        p.masked = 1;
        p.block_shift = align->block_ids ? align->block_shift : 0;
        p.S_rows = pr.S;
        hipError_t e = qsa::launch_attend(p, kv.type, pr.T, stream, nullptr);
        return e == hipSuccess ? QSA_OK : hip_fail(e, "attention launch");
    }
    qsa::SharingParams sp{};
    bool keys_lds = false;
    const bool share = sharing_of(pr, p.HB, ws, m, &sp, kv.type == qsa::KvType::kBf16, &keys_lds);
    p.keys_lds = keys_lds ? 1 : 0;
    hipError_t e = qsa::launch_attend(p, kv.type, pr.T, stream, share ? &sp : nullptr);
    return e == hipSuccess ? QSA_OK : hip_fail(e, "attention launch");
}

// Aligned rows hold block ids (the attention expands them) rather than each
// block's slots.
constexpr bool kAlignBlockIds = true;

// Room (list entries) of an aligned row for a selection of W blocks.
int64_t align_room(int64_t W, int32_t block_size) {
    const int64_t unit = kAlignBlockIds ? 1 : block_size;
    return round_up((W * unit * qsa::kAlignRoomNum + qsa::kAlignRoomDen - 1) / qsa::kAlignRoomDen,
                    qsa::kListPad);
}

// The standard layout for W * block_size slots, then the aligned rows (at
// *ext_offset).
bool blocks_layout(int64_t T, int64_t W, int32_t block_size, qsa_workspace_map *m,
                   int64_t *ext_offset, int64_t *total) {
    if (!layout_of(T, W * block_size, m)) return false;
    const int64_t entries = mul_sat(T, align_room(W, block_size));
    if (entries > kMaxListEntries) return false;
    *ext_offset = round_up(m->total_bytes, kAlign);
    *total = *ext_offset + round_up(entries * 4, kAlign);
    return true;
}

// Whether a micro-block prefill takes the aligned lists, and their spec:
// power-of-two blocks of kAlignMinBlock to kAlignMaxBlock slots, rows of one
// sort run whose room fits kAlignRoomMax, room in the workspace, and enough
// sharing that the general layout runs without an estimate (the lists only
// help tokens that share the L2).
AlignSpec align_of(const Problem &pr, int64_t W, int32_t block_size, void *ws,
                   size_t ws_bytes, const qsa_workspace_map &m) {
    AlignSpec al;
    const int64_t nb = pr.S / block_size;
    if (block_size < qsa::kAlignMinBlock || block_size > qsa::kAlignMaxBlock ||
        (block_size & (block_size - 1)) || W > qsa::kSortChunk || W <= 0 || nb <= 0 ||
        pr.Hkv <= 0)
        return al;
    qsa_workspace_map mb;
    int64_t ext = 0, total = 0;
    if (!blocks_layout(pr.T, W, block_size, &mb, &ext, &total) || (int64_t)ws_bytes < total)
        return al;
    qsa::SharingParams sp{};
    const int32_t HB = (pr.Hq / pr.Hkv + 15) / 16;
    bool keys_lds = false;   // (aligned lists run the masked form, keys direct)
    if (sharing_of(pr, HB, ws, m, &sp, true, &keys_lds)) return al;
    int32_t shift = std::max(sort_key_bits(nb) - qsa::kSortKeyBits, 0);
    int32_t by_size = 0;   // largest with 2^by_size blocks <= kAlignSlots slots
    while (((int64_t)block_size << (by_size + 1)) <= qsa::kAlignSlots) ++by_size;
    shift = std::max(shift, by_size);
    const int64_t ranges = (nb + ((int64_t)1 << shift) - 1) >> shift;
    if (ranges > qsa::kAlignMaxRanges || align_room(W, block_size) > qsa::kAlignRoomMax) return al;
    al.shift = shift;
    al.ranges = (int32_t)ranges;
    al.cap = (int32_t)align_room(W, block_size);
    al.block_ids = kAlignBlockIds;
    al.list_offset = ext;
    while ((1 << al.block_shift) < block_size) ++al.block_shift;
    return al;
}

// Partials buffer: O [n_parts][T][Hq][256] FP32, then (m, l) [n_parts][T][Hq][2] FP32.
struct PartialsMap {
    int64_t ml_offset, total_bytes;
};

bool partials_of(int64_t n_parts, int64_t T, int64_t Hq, PartialsMap *pm) {
    if (n_parts < 0 || T < 0 || Hq < 0) return false;
    const int64_t rows = mul_sat(mul_sat(n_parts, T), Hq);
    if (rows > kMaxListEntries / qsa::kHeadDim) return false;
    pm->ml_offset = round_up(rows * qsa::kHeadDim * 4, kAlign);
    pm->total_bytes = pm->ml_offset + round_up(rows * 8, kAlign);
    return true;
}

qsa_status check_partials(const void *buf, size_t bytes, int64_t n_parts, int64_t T, int64_t Hq,
                          PartialsMap *pm) {
    if (!partials_of(n_parts, T, Hq, pm)) return fail(QSA_ERR_SHAPE, "negative partials size");
    if (!buf) return fail(QSA_ERR_WORKSPACE, "partials buffer is NULL");
    if ((uintptr_t)buf % kAlign) return fail(QSA_ERR_WORKSPACE, "partials must be 256-byte aligned");
    if ((int64_t)bytes < pm->total_bytes)
        return fail(QSA_ERR_WORKSPACE, "partials buffer holds %zu bytes, %lld needed", bytes,
                    (long long)pm->total_bytes);
    return QSA_OK;
}

// raw (optional): read the selection rows themselves instead of the compacted
// list in ws, and write each share's invalid-entry count to bad_part.
qsa_status enqueue_partial(const qsa_bf16_view *q, const qsa_bf16_view *k,
                           const qsa_bf16_view *v, const Problem &pr, float scale, const void *ws,
                           const qsa_workspace_map &m, int32_t splits, int64_t part_base,
                           void *partials, const PartialsMap &pm, hipStream_t stream,
                           const qsa_i32_view *raw = nullptr, int32_t *bad_part = nullptr,
                           KvKind kv = KvKind()) {
    if (pr.T == 0 || pr.Hq == 0) return QSA_OK;
    qsa::AttendParams p{};
    fill_attend(p, q, k, v, pr, scale * kv.k_scale, ws, m);
    if (raw != nullptr) {
        p.raw_rows = 1;
        p.raw = raw->data;
        p.raw_stride = raw->stride[0];
        p.W_raw = (int32_t)raw->size[1];
        p.S_rows = pr.S;
        p.bad_part = bad_part;
    }
    p.v_scale = kv.v_scale;
    p.splits = splits;
    p.part_base = part_base;
    p.T = pr.T;
    p.Hq = pr.Hq;
    p.part_o = (float *)partials;
    p.part_ml = (float *)((char *)partials + pm.ml_offset);
    hipError_t e = qsa::launch_attend_partial(p, kv.type, pr.T, stream);
    return e == hipSuccess ? QSA_OK : hip_fail(e, "partial attention launch");
}

qsa_status enqueue_merge(const void *partials, const PartialsMap &pm, int64_t n_parts, int64_t T,
                         int32_t Hq, const qsa_bf16_view *out, hipStream_t stream,
                         const int32_t *bad_part = nullptr, int32_t *n_bad = nullptr,
                         int32_t *clear_flag = nullptr) {
    qsa::MergeParams p{};
    p.bad_part = bad_part;
    p.n_bad = n_bad;
    p.clear_flag = clear_flag;
    p.part_o = (const float *)partials;
    p.part_ml = (const float *)((const char *)partials + pm.ml_offset);
    p.n_parts = n_parts;
    p.T = T;
    p.Hq = Hq;
    p.out = (uint16_t *)out->data;
    p.o_st = out->stride[0];
    p.o_sh = out->stride[1];
    hipError_t e = qsa::launch_merge(p, stream);
    return e == hipSuccess ? QSA_OK : hip_fail(e, "merge launch");
}

// Splits per item for qsa_sparse_decode: about kDecodeUnits workgroups;
// at least kDecodeShareTiles tiles per split unless that leaves fewer than
// kDecodeMinUnits workgroups; at least kMinSplitTiles tiles; at most 64.  A
// pure function of the sizes, so results are reproducible.
int32_t decode_splits(int64_t T, int64_t W, int32_t Hq, int32_t Hkv) {
    if (T <= 0 || W <= 0 || Hq <= 0 || Hkv <= 0) return 1;
    const int64_t G = Hq / Hkv;
    const int64_t items = mul_sat(mul_sat(T, Hkv), (G + 15) / 16);
    const int64_t tiles = ceil_div(W, qsa::kTileSlots);
    int64_t s = ceil_div(qsa::kDecodeUnits, items);
    s = std::min<int64_t>(
        s, std::max<int64_t>(tiles / qsa::kDecodeShareTiles, ceil_div(qsa::kDecodeMinUnits, items)));
    s = std::min<int64_t>(s, tiles / qsa::kMinSplitTiles);
    s = std::min<int64_t>(s, 64);
    return (int32_t)std::max<int64_t>(s, 1);
}

void fill_attend(qsa::AttendParams &p, const qsa_bf16_view *q, const qsa_bf16_view *k,
                 const qsa_bf16_view *v, const Problem &pr, float scale, const void *ws,
                 const qsa_workspace_map &m) {
    p.q = (const uint16_t *)q->data;
    p.q_st = q->stride[0];
    p.q_sh = q->stride[1];
    p.k = (const uint16_t *)k->data;
    p.k_ss = k->stride[0];
    p.k_sh = k->stride[1];
    p.v = (const uint16_t *)v->data;
    p.v_ss = v->stride[0];
    p.v_sh = v->stride[1];
    p.list = (const int32_t *)((const char *)ws + m.list_offset);
    p.list_stride = m.row_stride;
    p.count = (const int32_t *)((const char *)ws + m.count_offset);
    p.extent = extent_words(ws, m);
    p.S_rows = pr.S;
    p.Hkv = pr.Hkv;
    p.G = pr.Hq / pr.Hkv;
    p.HB = (p.G + 15) / 16;
    p.scale_log2e = (float)((double)scale * 1.4426950408889634);
    p.splits = 1;
}

// qsa_sparse_decode for a BF16 (kv_bytes 2) or FP8 (kv_bytes 1) cache.
qsa_status decode_any(const qsa_bf16_view *q, const qsa_bf16_view *k_cache,
                      const qsa_bf16_view *v_cache, const qsa_i32_view *slot_idx, float scale,
                      qsa_bf16_view *out, void *workspace, size_t workspace_bytes, void *stream,
                      int kv_bytes, KvKind kv) {
    if (!slot_idx) return fail(QSA_ERR_NULL, "slot_idx: view pointer is NULL");
    Problem pr;
    qsa_status s = check_attend(q, k_cache, v_cache, out, slot_idx->size[1], scale, &pr,
                                kv_bytes);
    if (s) return s;
    if (kv.type == qsa::KvType::kFp8 && (s = check_fp8_scales(kv.k_scale, kv.v_scale))) return s;
    int64_t W = 0;
    if ((s = check_slots(slot_idx, pr.T, &W))) return s;
    const size_t need = qsa_decode_workspace_bytes(pr.T, W, pr.Hq, pr.Hkv);
    if (!workspace) return fail(QSA_ERR_WORKSPACE, "workspace is NULL");
    if ((uintptr_t)workspace % kAlign) return fail(QSA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (workspace_bytes < need)
        return fail(QSA_ERR_WORKSPACE, "workspace holds %zu bytes, %zu needed", workspace_bytes, need);
    if ((s = check_compact_grid(pr.T)) ||
        (s = check_attend_grid(pr.T, pr.Hq, pr.Hkv, decode_splits(pr.T, W, pr.Hq, pr.Hkv))) ||
        (s = check_merge_grid(pr.T, pr.Hq)))
        return s;
    if (pr.T == 0) return QSA_OK;
    qsa_workspace_map m;
    layout_of(pr.T, W, &m);
    const int32_t splits = decode_splits(pr.T, W, pr.Hq, pr.Hkv);
    void *partials = (char *)workspace + round_up(m.total_bytes, kAlign);
    PartialsMap pm;
    partials_of(splits, pr.T, pr.Hq, &pm);
    hipStream_t st = (hipStream_t)stream;
    if (pr.S == 0) {
        // An empty cache: no entry is valid and there is no row for a stand-in
        // slot to read, so the compacted (empty) lists serve instead.
        if ((s = enqueue_compact(slot_idx, pr.T, W, pr.S, 0, pr.S, workspace, m, st))) return s;
        if ((s = enqueue_partial(q, k_cache, v_cache, pr, scale, workspace, m, splits, 0, partials,
                                 pm, st, nullptr, nullptr, kv)))
            return s;
        return enqueue_merge(partials, pm, splits, pr.T, pr.Hq, out, st);
    }
    // No compaction pass: the shares read the selection rows themselves (for
    // a few tokens the grouping by slot range buys nothing) and count their
    // invalid entries in the list area of the workspace; the merge adds them
    // up into n_bad, where qsa_check_status reads them.
    if ((int64_t)splits * pr.T * 4 > m.bad_offset - m.list_offset)
        return fail(QSA_ERR_WORKSPACE, "decode workspace too small for the per-share counts");
    int32_t *bad_part = (int32_t *)((char *)workspace + m.list_offset);
    if ((s = enqueue_partial(q, k_cache, v_cache, pr, scale, workspace, m, splits, 0, partials, pm,
                             st, slot_idx, bad_part, kv)))
        return s;
    return enqueue_merge(partials, pm, splits, pr.T, pr.Hq, out, st, bad_part,
                         (int32_t *)((char *)workspace + m.bad_offset),
                         extent_words(workspace, m) + 1);
}

}  // namespace

extern "C" {

const char *qsa_version(void) { return "libqsa 0.1.0 gfx950"; }

const char *qsa_status_string(qsa_status s) {
    switch (s) {
    case QSA_OK: return "ok";
    case QSA_ERR_NULL: return "null pointer";
    case QSA_ERR_SHAPE: return "bad shape";
    case QSA_ERR_STRIDE: return "bad stride or alignment";
    case QSA_ERR_SCALE: return "scale not finite";
    case QSA_ERR_WORKSPACE: return "bad workspace";
    case QSA_ERR_SLOT_RANGE: return "slot out of range";
    case QSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case QSA_ERR_HIP: return "HIP runtime error";
    case QSA_ERR_ALIAS: return "output aliases an input";
    }
    return "unknown status";
}

const char *qsa_last_error(void) { return g_last_error; }

size_t qsa_workspace_bytes(int64_t T, int64_t W) {
    qsa_workspace_map m;
    return layout_of(T, W, &m) ? (size_t)m.total_bytes : 0;
}

size_t qsa_sparse_prefill_workspace_bytes(int64_t T, int64_t W) { return qsa_workspace_bytes(T, W); }

qsa_status qsa_workspace_layout(int64_t T, int64_t W, qsa_workspace_map *map) {
    if (!map) return fail(QSA_ERR_NULL, "map is NULL");
    if (!layout_of(T, W, map)) return fail(QSA_ERR_SHAPE, "T and W must be in [0, 2^31)");
    return QSA_OK;
}

qsa_status qsa_compact_slot_range(const qsa_i32_view *slot_idx, int64_t S, int64_t lo, int64_t hi,
                                  void *workspace, size_t workspace_bytes, void *stream) {
    if (!slot_idx) return fail(QSA_ERR_NULL, "slot_idx: view pointer is NULL");
    const int64_t T = slot_idx->size[0];
    int64_t W = 0;
    qsa_status s = check_slots(slot_idx, T, &W);
    if (s) return s;
    if (S < 0) return fail(QSA_ERR_SHAPE, "negative S");
    if (S > kMax32) return fail(QSA_ERR_UNSUPPORTED, "S must fit in int32");
    if (lo < 0 || hi < lo || hi > S) return fail(QSA_ERR_SHAPE, "need 0 <= lo <= hi <= S");
    qsa_workspace_map m;
    if ((s = check_workspace(workspace, workspace_bytes, T, W, &m))) return s;
    if ((s = check_compact_grid(T))) return s;
    return enqueue_compact(slot_idx, T, W, S, lo, hi, workspace, m, (hipStream_t)stream);
}

// Micro-block selections: check block_size and S, and give the list width.
qsa_status check_blocks(int32_t block_size, int64_t S, int64_t W, int64_t *slots_wide) {
    if (block_size < 1 || block_size > 64)
        return fail(QSA_ERR_SHAPE, "block_size must be in [1, 64]");
    if (S % block_size)
        return fail(QSA_ERR_SHAPE, "S (%lld) must be a multiple of block_size (%d)", (long long)S,
                    block_size);
    if (W * block_size > kMax32) return fail(QSA_ERR_UNSUPPORTED, "W * block_size beyond int32");
    *slots_wide = W * block_size;
    return QSA_OK;
}

qsa_status qsa_compact_blocks(const qsa_i32_view *block_idx, int64_t S, int32_t block_size,
                              void *workspace, size_t workspace_bytes, void *stream) {
    if (!block_idx) return fail(QSA_ERR_NULL, "block_idx: view pointer is NULL");
    const int64_t T = block_idx->size[0];
    int64_t W = 0, Ws = 0;
    qsa_status s = check_slots(block_idx, T, &W);
    if (s) return s;
    if (S < 0) return fail(QSA_ERR_SHAPE, "negative S");
    if (S > kMax32) return fail(QSA_ERR_UNSUPPORTED, "S must fit in int32");
    if ((s = check_blocks(block_size, S, W, &Ws))) return s;
    qsa_workspace_map m;
    if ((s = check_workspace(workspace, workspace_bytes, T, Ws, &m))) return s;
    if ((s = check_compact_grid(T))) return s;
    const int64_t nb = S / block_size;
    return enqueue_compact(block_idx, T, W, nb, 0, nb, workspace, m, (hipStream_t)stream,
                           block_size);
}

qsa_status qsa_sparse_prefill_blocks(const qsa_bf16_view *q, const qsa_bf16_view *k_cache,
                                     const qsa_bf16_view *v_cache, const qsa_i32_view *block_idx,
                                     int32_t block_size, float scale, qsa_bf16_view *out,
                                     void *workspace, size_t workspace_bytes, void *stream) {
    if (!block_idx) return fail(QSA_ERR_NULL, "block_idx: view pointer is NULL");
    Problem pr;
    qsa_status s = check_attend(q, k_cache, v_cache, out, block_idx->size[1], scale, &pr);
    if (s) return s;
    int64_t W = 0, Ws = 0;
    if ((s = check_slots(block_idx, pr.T, &W))) return s;
    if ((s = check_blocks(block_size, pr.S, W, &Ws))) return s;
    qsa_workspace_map m;
    if ((s = check_workspace(workspace, workspace_bytes, pr.T, Ws, &m))) return s;
    if ((s = check_compact_grid(pr.T)) || (s = check_attend_grid(pr.T, pr.Hq, pr.Hkv, 1)))
        return s;
    if (pr.T == 0) return QSA_OK;
    hipStream_t st = (hipStream_t)stream;
    const int64_t nb = pr.S / block_size;
    const AlignSpec al = align_of(pr, W, block_size, workspace, workspace_bytes, m);
    if ((s = enqueue_compact(block_idx, pr.T, W, nb, 0, nb, workspace, m, st, block_size, &al)))
        return s;
    return enqueue_attend(q, k_cache, v_cache, out, pr, scale, workspace, m, st, KvKind(), &al);
}

size_t qsa_prefill_blocks_workspace_bytes(int64_t T, int64_t W, int32_t block_size) {
    if (T < 0 || W < 0 || block_size < 1 || block_size > 64 || W > kMax32 / block_size) return 0;
    qsa_workspace_map m;
    int64_t ext = 0, total = 0;
    if (!blocks_layout(T, W, block_size, &m, &ext, &total)) return 0;
    return (size_t)total;
}

// ---------------------------------------------------------------- indexer

// iq [T, 4, 128] and ik [C, 1, 128] BF16 views (rows 16-byte aligned).
qsa_status check_index_view(const qsa_bf16_view *v, const char *name, int64_t heads) {
    if (!v) return fail(QSA_ERR_NULL, "%s: view pointer is NULL", name);
    for (int i = 0; i < 3; ++i) {
        if (v->size[i] < 0) return fail(QSA_ERR_SHAPE, "%s: negative size", name);
        if (v->stride[i] < 0) return fail(QSA_ERR_STRIDE, "%s: negative stride", name);
    }
    if (v->size[1] != heads || v->size[2] != qsa::kIndexDim)
        return fail(QSA_ERR_UNSUPPORTED, "%s must be [*, %lld, %d]", name, (long long)heads,
                    qsa::kIndexDim);
    if (any_empty(v)) return QSA_OK;
    if (!v->data) return fail(QSA_ERR_NULL, "%s: data is NULL", name);
    if (v->stride[2] != 1) return fail(QSA_ERR_STRIDE, "%s: innermost stride must be 1", name);
    if ((uintptr_t)v->data % 16 || v->stride[0] % 8 || v->stride[1] % 8)
        return fail(QSA_ERR_STRIDE, "%s: rows must be 16-byte aligned", name);
    if (v->size[0] > kMax32) return fail(QSA_ERR_UNSUPPORTED, "%s: too many rows", name);
    return QSA_OK;
}

// The score kernel: one workgroup of 256 per 128 tokens along x, one per
// 1,024 keys along y.
qsa_status check_scores_grid(int64_t T, int64_t C) {
    qsa_status s = check_grid(ceil_div(T, 128), 256, "indexer scores");
    if (s) return s;
    if (ceil_div(C, 1024) > kMaxGridY)
        return fail(QSA_ERR_UNSUPPORTED, "indexer scores: %lld keys exceed %lld key ranges",
                    (long long)C, (long long)kMaxGridY);
    return QSA_OK;
}

qsa_status check_scores(const void *scores, size_t bytes, int64_t T, int64_t C) {
    if (T > 0 && C > 0 && !scores) return fail(QSA_ERR_WORKSPACE, "scores buffer is NULL");
    if ((uintptr_t)scores % 16) return fail(QSA_ERR_WORKSPACE, "scores must be 16-byte aligned");
    const int64_t need = mul_sat(mul_sat(T, C), 4);
    if ((int64_t)bytes < need)
        return fail(QSA_ERR_WORKSPACE, "scores buffer holds %zu bytes, %lld needed", bytes,
                    (long long)need);
    return QSA_OK;
}

qsa_status enqueue_indexer_scores(const qsa_bf16_view *iq, const qsa_bf16_view *ik,
                                  const int32_t *positions, float *scores, hipStream_t stream) {
    qsa::IndexerScoreParams p{};
    p.iq = (const uint16_t *)iq->data;
    p.q_st = iq->stride[0];
    p.q_sh = iq->stride[1];
    p.ik = (const uint16_t *)ik->data;
    p.k_st = ik->stride[0];
    p.T = iq->size[0];
    p.C = ik->size[0];
    p.positions = positions;
    p.scores = scores;
    hipError_t e = qsa::launch_indexer_scores(p, stream);
    return e == hipSuccess ? QSA_OK : hip_fail(e, "indexer score launch");
}

qsa_status enqueue_indexer_select(const float *scores, int64_t T, int64_t C,
                                  const int32_t *positions, const int32_t *slot_of_pos, int64_t L,
                                  int32_t budget, const qsa_i32_view *out, hipStream_t stream) {
    qsa::IndexerSelectParams p{};
    p.scores = scores;
    p.T = T;
    p.C = C;
    p.positions = positions;
    p.slot_of_pos = slot_of_pos;
    p.L = L;
    p.budget = budget;
    p.out = (int32_t *)out->data;
    p.out_stride = out->stride[0];
    hipError_t e = qsa::launch_indexer_select(p, stream);
    return e == hipSuccess ? QSA_OK : hip_fail(e, "indexer select launch");
}

// Scratch of qsa_indexer_topk: T rows of `pitch` FP32 words (C rounded up
// to even: every score, or, on the fused path, each key range's candidate
// pairs, 8-byte aligned), then the fused path's per-range candidate counts
// [T, R] and thresholds [T], at 256-byte boundaries.
struct TopkScratch {
    int64_t R, pitch, counts_offset, tau_offset, total;
};

bool topk_scratch_of(int64_t T, int64_t C, TopkScratch *ts) {
    if (T < 0 || C < 0 || T > kMax32 || C > kMax32) return false;
    ts->pitch = C + (C & 1);
    const int64_t cells = mul_sat(T, ts->pitch);
    if (cells > kMaxListEntries) return false;
    ts->R = ceil_div(C, qsa::kScoreSplit);
    ts->counts_offset = round_up(cells * 4, kAlign);
    ts->tau_offset = ts->counts_offset + round_up(T * ts->R * 4, kAlign);
    ts->total = ts->tau_offset + round_up(T * 4, kAlign);
    return true;
}

qsa_status enqueue_indexer_topk_fused(const qsa_bf16_view *iq, const qsa_bf16_view *ik,
                                      const int32_t *positions, const int32_t *slot_of_pos,
                                      int64_t L, int32_t budget, float *scratch,
                                      const TopkScratch &ts, const qsa_i32_view *out,
                                      hipStream_t stream) {
    int32_t *counts = (int32_t *)((char *)scratch + ts.counts_offset);
    uint32_t *tau = (uint32_t *)((char *)scratch + ts.tau_offset);
    qsa::IndexerEstimateParams e{};
    e.iq = (const uint16_t *)iq->data;
    e.q_st = iq->stride[0];
    e.q_sh = iq->stride[1];
    e.ik = (const uint16_t *)ik->data;
    e.k_st = ik->stride[0];
    e.T = iq->size[0];
    e.C = ik->size[0];
    e.L = L;
    e.positions = positions;
    e.budget = budget;
    e.tau = tau;
    qsa::IndexerScoreParams sp{};
    sp.iq = e.iq;
    sp.q_st = e.q_st;
    sp.q_sh = e.q_sh;
    sp.ik = e.ik;
    sp.k_st = e.k_st;
    sp.T = e.T;
    sp.C = e.C;
    sp.positions = positions;
    sp.scores = scratch;
    sp.tau = tau;
    sp.counts = counts;
    sp.R = ts.R;
    sp.pair_pitch = ts.pitch;
    qsa::IndexerSelectParams p{};
    p.scores = scratch;
    p.T = e.T;
    p.C = e.C;
    p.positions = positions;
    p.slot_of_pos = slot_of_pos;
    p.L = L;
    p.budget = budget;
    p.out = (int32_t *)out->data;
    p.out_stride = out->stride[0];
    p.counts = counts;
    p.R = ts.R;
    p.pair_pitch = ts.pitch;
    hipError_t err = qsa::launch_indexer_topk_fused(e, sp, p, stream);
    return err == hipSuccess ? QSA_OK : hip_fail(err, "indexer top-k launch");
}

qsa_status check_select_args(int64_t T, int64_t C, const int32_t *positions,
                             const int32_t *slot_of_pos, int64_t L, int32_t budget,
                             const qsa_i32_view *out) {
    if (T < 0 || C < 0 || L < 0) return fail(QSA_ERR_SHAPE, "negative size");
    if (T > kMax32 || C > kMax32 || L > kMax32) return fail(QSA_ERR_UNSUPPORTED, "sizes beyond int32");
    if (budget < 1 || (int64_t)budget * qsa::kIndexBlock + 3 > kMax32)
        return fail(QSA_ERR_SHAPE, "budget must be positive");
    if (C * qsa::kIndexBlock < L - (qsa::kIndexBlock - 1) || C * qsa::kIndexBlock > L + 3)
        return fail(QSA_ERR_SHAPE, "need one index key per complete block: C = L / 4 (rounded)");
    if (!out) return fail(QSA_ERR_NULL, "slot_idx: view pointer is NULL");
    const int64_t width = (int64_t)budget * qsa::kIndexBlock + 3;
    if (out->size[0] != T || out->size[1] != width)
        return fail(QSA_ERR_SHAPE, "slot_idx must be [T, 4 * budget + 3]");
    if (T > 0 && (!out->data || !positions)) return fail(QSA_ERR_NULL, "NULL output or positions");
    if (T > 0 && L > 0 && !slot_of_pos) return fail(QSA_ERR_NULL, "slot_of_pos is NULL");
    if (out->stride[1] != 1 || out->stride[0] < width)
        return fail(QSA_ERR_STRIDE, "slot_idx rows must be contiguous and not overlap");
    return QSA_OK;
}

qsa_status qsa_compact_slots(const qsa_i32_view *slot_idx, int64_t S, void *workspace,
                             size_t workspace_bytes, void *stream) {
    return qsa_compact_slot_range(slot_idx, S, 0, S < 0 ? 0 : S, workspace, workspace_bytes,
                                  stream);
}

qsa_status qsa_sparse_attend(const qsa_bf16_view *q, const qsa_bf16_view *k_cache,
                             const qsa_bf16_view *v_cache, int64_t W, float scale,
                             void *workspace, size_t workspace_bytes,
                             qsa_bf16_view *out, void *stream) {
    Problem pr;
    qsa_status s = check_attend(q, k_cache, v_cache, out, W, scale, &pr);
    if (s) return s;
    qsa_workspace_map m;
    if ((s = check_workspace(workspace, workspace_bytes, pr.T, W, &m))) return s;
    if ((s = check_attend_grid(pr.T, pr.Hq, pr.Hkv, 1))) return s;
    return enqueue_attend(q, k_cache, v_cache, out, pr, scale, workspace, m, (hipStream_t)stream);
}

qsa_status qsa_sparse_prefill(const qsa_bf16_view *q, const qsa_bf16_view *k_cache,
                              const qsa_bf16_view *v_cache, const qsa_i32_view *slot_idx,
                              float scale, qsa_bf16_view *out, void *workspace,
                              size_t workspace_bytes, void *stream) {
    if (!slot_idx) return fail(QSA_ERR_NULL, "slot_idx: view pointer is NULL");
    Problem pr;
    qsa_status s = check_attend(q, k_cache, v_cache, out, slot_idx->size[1], scale, &pr);
    if (s) return s;
    int64_t W = 0;
    if ((s = check_slots(slot_idx, pr.T, &W))) return s;
    qsa_workspace_map m;
    if ((s = check_workspace(workspace, workspace_bytes, pr.T, W, &m))) return s;
    if ((s = check_compact_grid(pr.T)) || (s = check_attend_grid(pr.T, pr.Hq, pr.Hkv, 1)))
        return s;
    if (pr.T == 0) return QSA_OK;
    hipStream_t st = (hipStream_t)stream;
    if ((s = enqueue_compact(slot_idx, pr.T, W, pr.S, 0, pr.S, workspace, m, st))) return s;
    return enqueue_attend(q, k_cache, v_cache, out, pr, scale, workspace, m, st);
}

size_t qsa_partials_bytes(int64_t n_parts, int64_t T, int64_t Hq) {
    PartialsMap pm;
    return partials_of(n_parts, T, Hq, &pm) ? (size_t)pm.total_bytes : 0;
}

qsa_status qsa_sparse_attend_partial(const qsa_bf16_view *q, const qsa_bf16_view *k_cache,
                                     const qsa_bf16_view *v_cache, int64_t W, float scale,
                                     const void *workspace, size_t workspace_bytes,
                                     int32_t splits, int64_t part_base, int64_t n_parts,
                                     void *partials, size_t partials_bytes, void *stream) {
    Problem pr;
    qsa_status s = check_inputs(q, k_cache, v_cache, W, scale, &pr);
    if (s) return s;
    if (splits < 1 || splits > 4096) return fail(QSA_ERR_SHAPE, "splits must be in [1, 4096]");
    if (part_base < 0 || part_base + splits > n_parts)
        return fail(QSA_ERR_SHAPE, "parts [part_base, part_base + splits) must lie in [0, n_parts)");
    qsa_workspace_map m;
    if ((s = check_workspace(workspace, workspace_bytes, pr.T, W, &m))) return s;
    PartialsMap pm;
    if ((s = check_partials(partials, partials_bytes, n_parts, pr.T, pr.Hq, &pm))) return s;
    if ((s = check_no_overlap((uintptr_t)partials, (uintptr_t)partials + (uintptr_t)pm.total_bytes,
                              q, k_cache, v_cache, "partials")))
        return s;
    if ((s = check_attend_grid(pr.T, pr.Hq, pr.Hkv, splits))) return s;
    return enqueue_partial(q, k_cache, v_cache, pr, scale, workspace, m, splits, part_base,
                           partials, pm, (hipStream_t)stream);
}

qsa_status qsa_merge_partials(const void *partials, size_t partials_bytes, int64_t n_parts,
                              int64_t T, int64_t Hq, qsa_bf16_view *out, void *stream) {
    qsa_status s = check_bf16(out, "out");
    if (s) return s;
    if (out->size[0] != T || out->size[1] != Hq)
        return fail(QSA_ERR_SHAPE, "out must be [T, Hq, 256]");
    if (n_parts < 1) return fail(QSA_ERR_SHAPE, "n_parts must be positive");
    if (T > kMax32 || Hq > kMax32) return fail(QSA_ERR_UNSUPPORTED, "sizes beyond int32");
    PartialsMap pm;
    if ((s = check_partials(partials, partials_bytes, n_parts, T, Hq, &pm))) return s;
    uintptr_t olo, ohi;
    if (!any_empty(out)) {
        span_of(out, &olo, &ohi);
        const uintptr_t plo = (uintptr_t)partials, phi = plo + (uintptr_t)pm.total_bytes;
        if (olo < phi && plo < ohi) return fail(QSA_ERR_ALIAS, "out overlaps the partials");
    }
    if ((s = check_merge_grid(T, Hq))) return s;
    if (T == 0 || Hq == 0) return QSA_OK;
    return enqueue_merge(partials, pm, n_parts, T, (int32_t)Hq, out, (hipStream_t)stream);
}

int32_t qsa_decode_splits(int64_t T, int64_t W, int32_t Hq, int32_t Hkv) {
    return decode_splits(T, W, Hq, Hkv);
}

size_t qsa_decode_workspace_bytes(int64_t T, int64_t W, int32_t Hq, int32_t Hkv) {
    qsa_workspace_map m;
    PartialsMap pm;
    if (!layout_of(T, W, &m) || Hq < 0) return 0;
    if (!partials_of(decode_splits(T, W, Hq, Hkv), T, Hq, &pm)) return 0;
    return (size_t)(round_up(m.total_bytes, kAlign) + pm.total_bytes);
}

qsa_status qsa_sparse_decode(const qsa_bf16_view *q, const qsa_bf16_view *k_cache,
                             const qsa_bf16_view *v_cache, const qsa_i32_view *slot_idx,
                             float scale, qsa_bf16_view *out, void *workspace,
                             size_t workspace_bytes, void *stream) {
    return decode_any(q, k_cache, v_cache, slot_idx, scale, out, workspace, workspace_bytes,
                      stream, 2, KvKind());
}

qsa_status qsa_sparse_decode_fp8kv(const qsa_bf16_view *q, const qsa_fp8_view *k8,
                                   const qsa_fp8_view *v8, float k_scale, float v_scale,
                                   const qsa_i32_view *slot_idx, float scale,
                                   qsa_bf16_view *out, void *workspace,
                                   size_t workspace_bytes, void *stream) {
    return decode_any(q, as_view(k8), as_view(v8), slot_idx, scale, out, workspace,
                      workspace_bytes, stream, 1, KvKind{qsa::KvType::kFp8, k_scale, v_scale});
}

qsa_status qsa_check_status(const void *workspace, size_t workspace_bytes, int64_t T,
                            int64_t W, void *stream, int64_t *n_bad) {
    qsa_workspace_map m;
    qsa_status s = check_workspace(workspace, workspace_bytes, T, W, &m);
    if (s) return s;
    if (n_bad) *n_bad = 0;
    if (T == 0) return QSA_OK;
    std::vector<int32_t> bad((size_t)T);
    int32_t extent[2] = {0, 0};
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "stream synchronize");
    e = hipMemcpy(bad.data(), (const char *)workspace + m.bad_offset, (size_t)T * 4,
                  hipMemcpyDeviceToHost);
    if (e == hipSuccess)
        e = hipMemcpy(extent, extent_words(workspace, m), sizeof extent, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "status copy");
    int64_t total = 0;
    for (int32_t b : bad) total += b;
    if (n_bad) *n_bad = total;
    if (extent[1])
        return fail(QSA_ERR_WORKSPACE,
                    "the workspace's lists index %d cache slots, more than the K/V views of the "
                    "attention held; its rows were written as zeros",
                    extent[0]);
    if (total) return fail(QSA_ERR_SLOT_RANGE, "%lld selection entries were neither -1 nor in [0, S)",
                           (long long)total);
    return QSA_OK;
}

}  // extern "C"

namespace {

qsa_status gather_only_any(const qsa_bf16_view *k_cache, const qsa_bf16_view *v_cache,
                           int kv_bytes, qsa::KvType kv, int64_t T, int64_t W,
                           const void *workspace, size_t workspace_bytes, uint32_t *sink,
                           void *stream) {
    qsa_status s;
    if ((s = check_view(k_cache, "k_cache", kv_bytes)) ||
        (s = check_view(v_cache, "v_cache", kv_bytes)))
        return s;
    for (int i = 0; i < 3; ++i)
        if (v_cache->size[i] != k_cache->size[i])
            return fail(QSA_ERR_SHAPE, "v_cache must have k_cache's shape");
    if ((s = check_slot_strides(k_cache, v_cache, kv_bytes))) return s;
    if (T < 0 || W < 0) return fail(QSA_ERR_SHAPE, "negative T or W");
    if (T > kMax32 || k_cache->size[1] > kMax32)
        return fail(QSA_ERR_UNSUPPORTED, "sizes beyond int32");
    qsa_workspace_map m;
    if ((s = check_workspace(workspace, workspace_bytes, T, W, &m))) return s;
    if (T == 0 || k_cache->size[1] == 0) return QSA_OK;
    if (!sink) return fail(QSA_ERR_NULL, "sink is NULL");
    if ((s = check_grid(mul_sat(T, k_cache->size[1]), 64, "gather-only"))) return s;
    qsa::GatherParams p{};
    p.k = k_cache->data;
    p.k_ss = k_cache->stride[0];
    p.k_sh = k_cache->stride[1];
    p.v = v_cache->data;
    p.v_ss = v_cache->stride[0];
    p.v_sh = v_cache->stride[1];
    p.list = (const int32_t *)((const char *)workspace + m.list_offset);
    p.list_stride = m.row_stride;
    p.count = (const int32_t *)((const char *)workspace + m.count_offset);
    p.sink = sink;
    p.Hkv = (int32_t)k_cache->size[1];
    p.S_rows = k_cache->size[0];
    p.extent = extent_words(workspace, m);
    hipError_t e = qsa::launch_gather_only(p, kv, T, (hipStream_t)stream);
    return e == hipSuccess ? QSA_OK : hip_fail(e, "gather-only launch");
}

}  // namespace

extern "C" {

qsa_status qsa_gather_only(const qsa_bf16_view *k_cache, const qsa_bf16_view *v_cache,
                           int64_t T, int64_t W, const void *workspace, size_t workspace_bytes,
                           uint32_t *sink, void *stream) {
    return gather_only_any(k_cache, v_cache, 2, qsa::KvType::kBf16, T, W, workspace,
                           workspace_bytes, sink, stream);
}

qsa_status qsa_stream_read(const void *buf, size_t footprint_bytes, size_t bytes_per_workgroup,
                           int64_t workgroups, uint32_t *sink, void *stream) {
    if (workgroups < 0) return fail(QSA_ERR_SHAPE, "negative workgroup count");
    if (workgroups == 0) return QSA_OK;
    if (!buf || !sink) return fail(QSA_ERR_NULL, "buffer or sink is NULL");
    if ((uintptr_t)buf % 16) return fail(QSA_ERR_STRIDE, "buffer must be 16-byte aligned");
    if (footprint_bytes == 0 || footprint_bytes % 16 || bytes_per_workgroup == 0 ||
        bytes_per_workgroup % 16 || bytes_per_workgroup > footprint_bytes)
        return fail(QSA_ERR_SHAPE,
                    "need 0 < bytes_per_workgroup <= footprint_bytes, both multiples of 16");
    qsa_status s = check_grid(workgroups, 256, "stream read");
    if (s) return s;
    qsa::StreamParams p{};
    p.buf = buf;
    p.footprint_chunks = (int64_t)(footprint_bytes / 16);
    p.chunks_per_wg = (int64_t)(bytes_per_workgroup / 16);
    p.sink = sink;
    hipError_t e = qsa::launch_stream_read(p, workgroups, (hipStream_t)stream);
    return e == hipSuccess ? QSA_OK : hip_fail(e, "stream read launch");
}

qsa_status qsa_gather_only_fp8kv(const qsa_fp8_view *k8, const qsa_fp8_view *v8, int64_t T,
                                 int64_t W, const void *workspace, size_t workspace_bytes,
                                 uint32_t *sink, void *stream) {
    return gather_only_any(as_view(k8), as_view(v8), 1, qsa::KvType::kFp8, T, W, workspace,
                           workspace_bytes, sink, stream);
}

qsa_status qsa_sparse_attend_fp8kv(const qsa_bf16_view *q, const qsa_fp8_view *k8,
                                   const qsa_fp8_view *v8, float k_scale, float v_scale,
                                   int64_t W, float scale, void *workspace,
                                   size_t workspace_bytes, qsa_bf16_view *out, void *stream) {
    Problem pr;
    qsa_status s = check_attend(q, as_view(k8), as_view(v8), out, W, scale, &pr, 1);
    if (s) return s;
    if ((s = check_fp8_scales(k_scale, v_scale))) return s;
    qsa_workspace_map m;
    if ((s = check_workspace(workspace, workspace_bytes, pr.T, W, &m))) return s;
    if ((s = check_attend_grid(pr.T, pr.Hq, pr.Hkv, 1))) return s;
    KvKind kv{qsa::KvType::kFp8, k_scale, v_scale};
    return enqueue_attend(q, as_view(k8), as_view(v8), out, pr, scale, workspace, m,
                          (hipStream_t)stream, kv);
}

qsa_status qsa_sparse_prefill_fp8kv(const qsa_bf16_view *q, const qsa_fp8_view *k8,
                                    const qsa_fp8_view *v8, float k_scale, float v_scale,
                                    const qsa_i32_view *slot_idx, float scale,
                                    qsa_bf16_view *out, void *workspace,
                                    size_t workspace_bytes, void *stream) {
    if (!slot_idx) return fail(QSA_ERR_NULL, "slot_idx: view pointer is NULL");
    Problem pr;
    qsa_status s = check_attend(q, as_view(k8), as_view(v8), out, slot_idx->size[1], scale, &pr, 1);
    if (s) return s;
    if ((s = check_fp8_scales(k_scale, v_scale))) return s;
    int64_t W = 0;
    if ((s = check_slots(slot_idx, pr.T, &W))) return s;
    qsa_workspace_map m;
    if ((s = check_workspace(workspace, workspace_bytes, pr.T, W, &m))) return s;
    if ((s = check_compact_grid(pr.T)) || (s = check_attend_grid(pr.T, pr.Hq, pr.Hkv, 1)))
        return s;
    if (pr.T == 0) return QSA_OK;
    hipStream_t st = (hipStream_t)stream;
    if ((s = enqueue_compact(slot_idx, pr.T, W, pr.S, 0, pr.S, workspace, m, st))) return s;
    KvKind kv{qsa::KvType::kFp8, k_scale, v_scale};
    return enqueue_attend(q, as_view(k8), as_view(v8), out, pr, scale, workspace, m, st, kv);
}

size_t qsa_indexer_scores_bytes(int64_t T, int64_t C) {
    const int64_t need = mul_sat(mul_sat(T, C), 4);
    return (T < 0 || C < 0 || need == INT64_MAX) ? 0 : (size_t)need;
}

size_t qsa_indexer_topk_fused_bytes(int64_t T, int64_t C) {
    TopkScratch ts;
    return topk_scratch_of(T, C, &ts) ? (size_t)ts.total : 0;
}

qsa_status qsa_indexer_scores(const qsa_bf16_view *iq, const qsa_bf16_view *ik,
                              const int32_t *positions, float *scores, size_t scores_bytes,
                              void *stream) {
    qsa_status s;
    if ((s = check_index_view(iq, "iq", qsa::kIndexHeads)) || (s = check_index_view(ik, "ik", 1)))
        return s;
    const int64_t T = iq->size[0], C = ik->size[0];
    if ((s = check_scores(scores, scores_bytes, T, C))) return s;
    if (T > 0 && !positions) return fail(QSA_ERR_NULL, "positions is NULL");
    if ((s = check_scores_grid(T, C))) return s;
    if (T == 0 || C == 0) return QSA_OK;
    return enqueue_indexer_scores(iq, ik, positions, scores, (hipStream_t)stream);
}

qsa_status qsa_indexer_select(const float *scores, size_t scores_bytes, int64_t T, int64_t C,
                              const int32_t *positions, const int32_t *slot_of_pos, int64_t L,
                              int32_t budget, qsa_i32_view *slot_idx, void *stream) {
    qsa_status s = check_select_args(T, C, positions, slot_of_pos, L, budget, slot_idx);
    if (s) return s;
    if ((s = check_scores(scores, scores_bytes, T, C))) return s;
    if ((s = check_grid(T, 256, "indexer select"))) return s;
    if (T == 0) return QSA_OK;
    return enqueue_indexer_select(scores, T, C, positions, slot_of_pos, L, budget, slot_idx,
                                  (hipStream_t)stream);
}

qsa_status qsa_indexer_topk(const qsa_bf16_view *iq, const qsa_bf16_view *ik,
                            const int32_t *positions, const int32_t *slot_of_pos, int64_t L,
                            int32_t budget, float *scores, size_t scores_bytes,
                            qsa_i32_view *slot_idx, void *stream) {
    qsa_status s;
    if ((s = check_index_view(iq, "iq", qsa::kIndexHeads)) || (s = check_index_view(ik, "ik", 1)))
        return s;
    const int64_t T = iq->size[0], C = ik->size[0];
    if ((s = check_select_args(T, C, positions, slot_of_pos, L, budget, slot_idx))) return s;
    if ((s = check_scores(scores, scores_bytes, T, C))) return s;
    if ((s = check_scores_grid(T, C)) || (s = check_grid(T, 256, "indexer select"))) return s;
    if (T == 0) return QSA_OK;
    hipStream_t st = (hipStream_t)stream;
    if (C > 0 && (s = enqueue_indexer_scores(iq, ik, positions, scores, st))) return s;
    return enqueue_indexer_select(scores, T, C, positions, slot_of_pos, L, budget, slot_idx, st);
}

qsa_status qsa_indexer_topk_fused(const qsa_bf16_view *iq, const qsa_bf16_view *ik,
                                  const int32_t *positions, const int32_t *slot_of_pos, int64_t L,
                                  int32_t budget, void *scratch, size_t scratch_bytes,
                                  qsa_i32_view *slot_idx, void *stream) {
    qsa_status s;
    if ((s = check_index_view(iq, "iq", qsa::kIndexHeads)) || (s = check_index_view(ik, "ik", 1)))
        return s;
    const int64_t T = iq->size[0], C = ik->size[0];
    if ((s = check_select_args(T, C, positions, slot_of_pos, L, budget, slot_idx))) return s;
    TopkScratch ts;
    if (!topk_scratch_of(T, C, &ts))
        return fail(QSA_ERR_UNSUPPORTED, "indexer top-k: T %lld x C %lld is too large",
                         (long long)T, (long long)C);
    if (budget > qsa::kFusedBudgetMax || ts.R > qsa::kFusedMaxRanges)
        return fail(QSA_ERR_UNSUPPORTED,
                         "fused top-k takes budgets up to %d and C up to %lld (budget %d, C %lld)",
                         qsa::kFusedBudgetMax, (long long)qsa::kFusedMaxRanges * qsa::kScoreSplit,
                         (int)budget, (long long)C);
    if (T > 0 && C > 0 && (scratch == nullptr || (int64_t)scratch_bytes < ts.total))
        return fail(QSA_ERR_WORKSPACE, "fused top-k scratch: %zu bytes, needs %lld",
                         scratch_bytes, (long long)ts.total);
    if ((uintptr_t)scratch % 8 != 0)
        return fail(QSA_ERR_WORKSPACE, "fused top-k scratch must be 8-byte aligned");
    if ((s = check_scores_grid(T, C)) || (s = check_grid(T, 256, "indexer select"))) return s;
    if (T == 0) return QSA_OK;
    hipStream_t st = (hipStream_t)stream;
    if (C == 0) return enqueue_indexer_select((const float *)scratch, T, C, positions,
                                              slot_of_pos, L, budget, slot_idx, st);
    return enqueue_indexer_topk_fused(iq, ik, positions, slot_of_pos, L, budget, (float *)scratch,
                                      ts, slot_idx, st);
}

}  // extern "C"
