// layout.cpp -- partition layout and bucket plan (host only).
//
// Follows the ZeRO explainer page ("ZeRO: Memory Optimizations Toward
// Training Trillion Parameter Models", azimuth.plus):
//   - model-states paragraph: 2 + 2 + 4 + 4 + 4 bytes of model state per
//     parameter (fp16 parameter, fp16 gradient, fp32 master/momentum/variance);
//   - Stage 1/2/3 paragraphs: optimizer state, then gradients, then fp16
//     parameters are kept as 1/N slices per rank;
//   - constant-size buffers paragraph: gradients stream through one buffer of
//     fixed size B, filled window by window.
// The flattened vector (tensors back to back in list order) is cut into N
// equal shards of S = roundup(ceil(Psi / N), A) elements; the last shards
// carry the padding.  Segments are the pieces of each tensor between
// consecutive shard (and bucket) boundaries.
#include <algorithm>
#include <cstring>
#include <limits>
#include <mutex>
#include <new>
#include <utility>

#include "zp_internal.hpp"

struct zero_layout {
    std::vector<int64_t> numel;
    std::vector<int64_t> offset;
    int32_t n_ranks = 1;
    int32_t stage = 0;
    int64_t align = 1;
    int64_t bucket = 0;
    int64_t psi = 0;
    int64_t shard = 0;
    int64_t n_fills = 0;
    std::vector<zero_segment> seg;

    // device tables of the pack (filled by zero_layout_bind_tensors)
    int device = -1;
    std::vector<int64_t> p_off;   // host copy of the sources' flat offsets, then psi
    zp::PackSrc* d_src = nullptr;
    int32_t* d_first = nullptr;
    int32_t n_src = 0;
    int32_t chunk_shift = 0;

    // device tables of the reduce-to-owner (zero_layout_bind_contributions)
    int r_device = -1;
    int32_t r_ranks = 0;
    int32_t r_nsrc = 0;
    int32_t r_shift = 0;
    int64_t* d_roff = nullptr;
    int64_t* d_rlen = nullptr;
    const uint16_t** d_rptr = nullptr;
    int32_t* d_rfirst = nullptr;
    uint8_t* d_rrec = nullptr;   // per-chunk records (zp::chunk_rec_bytes(R) each)
    // host copy of the contribution tensors' byte ranges, sorted by start,
    // with the running maximum of their ends (overlap queries)
    std::vector<uintptr_t> r_start, r_end_max;
    // host copy of the device flat offsets (r_nsrc + 1 entries, the last psi)
    std::vector<int64_t> r_off;
};

namespace {

constexpr int64_t kMaxSegments = int64_t(1) << 26;
constexpr int64_t kI64Max = std::numeric_limits<int64_t>::max();

bool add_overflows(int64_t a, int64_t b) { return a > kI64Max - b; }

void free_device_tables(zero_layout* l) {
    if (l->d_src) (void)hipFree(l->d_src);
    if (l->d_first) (void)hipFree(l->d_first);
    l->d_src = nullptr;
    l->d_first = nullptr;
    l->device = -1;
    l->n_src = 0;
    l->p_off.clear();
}

void free_reduce_tables(zero_layout* l) {
    void* bufs[5] = {l->d_roff, l->d_rlen, l->d_rptr, l->d_rfirst, l->d_rrec};
    for (void* b : bufs)
        if (b) (void)hipFree(b);
    l->d_roff = nullptr;
    l->d_rlen = nullptr;
    l->d_rptr = nullptr;
    l->d_rfirst = nullptr;
    l->d_rrec = nullptr;
    l->r_device = -1;
    l->r_ranks = 0;
    l->r_nsrc = 0;
    l->r_start.clear();
    l->r_end_max.clear();
    l->r_off.clear();
}

// Chunk index over the flat stream: first[c] = index (among the non-empty
// tensors, whose flat offsets are `offs`, ascending) of the tensor holding
// flat index c << shift; first[n_chunks] = last tensor.  The chunk is at
// least 2048 elements (one wave span) and grows so that the table stays
// <= 2^22 entries.
bool chunk_index(const std::vector<int64_t>& offs, int64_t psi, int* shift_out,
                 std::vector<int32_t>* first) {
    int shift = 11;
    while (((psi + (int64_t(1) << shift) - 1) >> shift) > (int64_t(1) << 22)) ++shift;
    const int64_t n_chunks = (psi + (int64_t(1) << shift) - 1) >> shift;
    try {
        first->assign(size_t(n_chunks) + 1, 0);
    } catch (...) {
        return false;
    }
    size_t s = 0;
    for (int64_t c = 0; c < n_chunks; ++c) {
        const int64_t g = c << shift;
        while (s + 1 < offs.size() && offs[s + 1] <= g) ++s;
        (*first)[size_t(c)] = int32_t(s);
    }
    (*first)[size_t(n_chunks)] = offs.empty() ? 0 : int32_t(offs.size() - 1);
    *shift_out = shift;
    return true;
}

// End of the segment starting at flat index cur inside a tensor ending at
// end: the next shard boundary, the next bucket boundary (bucket > 0) or the
// tensor end, whichever comes first.  Written so that no sum can overflow.
int64_t next_cut(int64_t cur, int64_t end, int64_t shard, int64_t bucket) {
    int64_t cut = end;
    const int64_t to_shard = shard - cur % shard;
    if (to_shard < cut - cur) cut = cur + to_shard;
    if (bucket > 0) {
        const int64_t to_bucket = bucket - cur % bucket;
        if (to_bucket < cut - cur) cut = cur + to_bucket;
    }
    return cut;
}

// Partitioned kinds per stage, in the order param16, grad16, master, m, v.
bool partitioned(int stage, int kind) {
    switch (stage) {
        case 0: return false;
        case 1: return kind >= 2;
        case 2: return kind >= 1;
        default: return true;
    }
}

}  // namespace

extern "C" int zero_partition_layout(const int64_t* numel, int64_t n_tensors, int32_t n_ranks,
                                     int32_t stage, int64_t align_elems, int64_t bucket_elems,
                                     zero_layout** out) {
    zp::clear_error();
    if (!out) return zp::fail(ZERO_ERR_INVALID_ARG, "zero_partition_layout: out is NULL");
    if (n_tensors < 0) return zp::fail(ZERO_ERR_INVALID_ARG, "n_tensors < 0");
    if (n_tensors > 0 && !numel) return zp::fail(ZERO_ERR_INVALID_ARG, "numel is NULL");
    if (n_tensors > std::numeric_limits<int32_t>::max())
        return zp::fail(ZERO_ERR_INVALID_ARG, "more than 2^31-1 tensors");
    if (n_ranks < 1) return zp::fail(ZERO_ERR_INVALID_ARG, "n_ranks < 1");
    if (stage < 0 || stage > 3) return zp::fail(ZERO_ERR_INVALID_ARG, "stage must be 0..3");
    if (align_elems < 1) return zp::fail(ZERO_ERR_INVALID_ARG, "align_elems < 1");
    if (bucket_elems < 0) return zp::fail(ZERO_ERR_INVALID_ARG, "bucket_elems < 0");

    int64_t psi = 0;
    for (int64_t i = 0; i < n_tensors; ++i) {
        if (numel[i] < 0) return zp::fail(ZERO_ERR_INVALID_ARG, "negative tensor size");
        if (add_overflows(psi, numel[i]))
            return zp::fail(ZERO_ERR_INDEX_OVERFLOW, "sum of tensor sizes overflows int64");
        psi += numel[i];
    }
    // S = roundup(ceil(psi / N), A), and 16 bytes for each of N * S elements
    // must stay representable
    const int64_t per = psi / n_ranks + (psi % n_ranks != 0);
    const int64_t rem = per % align_elems;
    if (rem != 0 && add_overflows(per, align_elems - rem))
        return zp::fail(ZERO_ERR_INDEX_OVERFLOW, "shard size overflows int64");
    const int64_t shard = rem ? per + (align_elems - rem) : per;
    if (shard > 0 && shard > kI64Max / 16 / n_ranks)
        return zp::fail(ZERO_ERR_INDEX_OVERFLOW, "16 * n_ranks * shard bytes overflow int64");

    // count the segments before building them
    int64_t n_seg = 0;
    for (int64_t i = 0, off = 0; i < n_tensors; off += numel[i], ++i) {
        int64_t cur = off, end = off + numel[i];
        while (cur < end) {
            cur = next_cut(cur, end, shard, bucket_elems);
            if (++n_seg > kMaxSegments)
                return zp::fail(ZERO_ERR_OUT_OF_MEMORY, "layout would hold more than 2^26 segments");
        }
    }

    zero_layout* l = new (std::nothrow) zero_layout();
    if (!l) return zp::fail(ZERO_ERR_OUT_OF_MEMORY, "layout allocation failed");
    try {
        l->numel.assign(numel, numel + n_tensors);
        l->offset.resize(size_t(n_tensors));
        l->seg.reserve(size_t(n_seg));
    } catch (...) {
        delete l;
        return zp::fail(ZERO_ERR_OUT_OF_MEMORY, "layout allocation failed");
    }
    l->n_ranks = n_ranks;
    l->stage = stage;
    l->align = align_elems;
    l->bucket = bucket_elems;
    l->psi = psi;
    l->shard = shard;
    l->n_fills = bucket_elems > 0 ? psi / bucket_elems + (psi % bucket_elems != 0) : 0;

    int64_t off = 0;
    for (int64_t i = 0; i < n_tensors; ++i) {
        l->offset[size_t(i)] = off;
        const int64_t end = off + numel[i];
        for (int64_t cur = off; cur < end;) {
            zero_segment s;
            s.tensor = int32_t(i);
            s.owner = int32_t(cur / shard);
            const int64_t cut = next_cut(cur, end, shard, bucket_elems);
            if (bucket_elems > 0) {
                s.fill = cur / bucket_elems;
                s.bucket_off = cur - s.fill * bucket_elems;
            } else {
                s.fill = -1;
                s.bucket_off = -1;
            }
            s.tensor_off = cur - off;
            s.flat_off = cur;
            s.len = cut - cur;
            s.shard_off = cur - int64_t(s.owner) * shard;
            l->seg.push_back(s);
            cur = cut;
        }
        off = end;
    }
    *out = l;
    return ZERO_OK;
}

extern "C" int zero_layout_destroy(zero_layout* layout) {
    zp::clear_error();
    if (!layout) return ZERO_OK;
    free_device_tables(layout);
    free_reduce_tables(layout);
    delete layout;
    return ZERO_OK;
}

extern "C" int zero_layout_get_info(const zero_layout* l, zero_layout_info* info) {
    zp::clear_error();
    if (!l || !info) return zp::fail(ZERO_ERR_INVALID_ARG, "zero_layout_get_info: NULL argument");
    zero_layout_info r;
    std::memset(&r, 0, sizeof(r));
    r.psi = l->psi;
    r.shard_elems = l->shard;
    r.padded_elems = int64_t(l->n_ranks) * l->shard;
    r.padding = r.padded_elems - l->psi;
    r.n_tensors = int64_t(l->numel.size());
    r.align_elems = l->align;
    r.bucket_elems = l->bucket;
    r.n_fills = l->n_fills;
    r.n_segments = int64_t(l->seg.size());
    r.n_ranks = l->n_ranks;
    r.stage = l->stage;
    static const int64_t kBytes[5] = {2, 2, 4, 4, 4};
    int64_t* dst[5] = {&r.bytes_param16, &r.bytes_grad16, &r.bytes_master, &r.bytes_momentum,
                       &r.bytes_variance};
    for (int k = 0; k < 5; ++k) {
        *dst[k] = kBytes[k] * (partitioned(l->stage, k) ? l->shard : l->psi);
        r.bytes_total += *dst[k];
    }
    *info = r;
    return ZERO_OK;
}

extern "C" int zero_layout_tensor_offsets(const zero_layout* l, int64_t* out, int64_t cap) {
    zp::clear_error();
    if (!l) return zp::fail(ZERO_ERR_INVALID_ARG, "layout is NULL");
    const int64_t n = int64_t(l->offset.size());
    if (cap < n || (n > 0 && !out))
        return zp::fail(ZERO_ERR_CAPACITY, "tensor offset array too small");
    if (n > 0) std::memcpy(out, l->offset.data(), size_t(n) * sizeof(int64_t));
    return ZERO_OK;
}

extern "C" int zero_layout_rank_range(const zero_layout* l, int32_t rank, int64_t* begin,
                                      int64_t* real_end, int64_t* end) {
    zp::clear_error();
    if (!l || !begin || !real_end || !end)
        return zp::fail(ZERO_ERR_INVALID_ARG, "zero_layout_rank_range: NULL argument");
    if (rank < 0 || rank >= l->n_ranks) return zp::fail(ZERO_ERR_INVALID_ARG, "rank out of range");
    const int64_t b = int64_t(rank) * l->shard;
    const int64_t e = b + l->shard;
    *begin = b;
    *end = e;
    *real_end = std::max(b, std::min(e, l->psi));
    return ZERO_OK;
}

namespace {

int copy_range(const zero_layout* l, size_t lo, size_t hi, zero_segment* out, int64_t cap,
               int64_t* n_out) {
    const int64_t n = int64_t(hi - lo);
    *n_out = n;
    if (cap < n || (n > 0 && !out)) return zp::fail(ZERO_ERR_CAPACITY, "segment array too small");
    if (n > 0) std::memcpy(out, l->seg.data() + lo, size_t(n) * sizeof(zero_segment));
    return ZERO_OK;
}

}  // namespace

extern "C" int zero_layout_segments(const zero_layout* l, zero_segment* out, int64_t cap,
                                    int64_t* n_out) {
    zp::clear_error();
    if (!l || !n_out) return zp::fail(ZERO_ERR_INVALID_ARG, "zero_layout_segments: NULL argument");
    return copy_range(l, 0, l->seg.size(), out, cap, n_out);
}

extern "C" int zero_layout_rank_segments(const zero_layout* l, int32_t rank, zero_segment* out,
                                         int64_t cap, int64_t* n_out) {
    zp::clear_error();
    if (!l || !n_out) return zp::fail(ZERO_ERR_INVALID_ARG, "zero_layout_rank_segments: NULL argument");
    if (rank < 0 || rank >= l->n_ranks) return zp::fail(ZERO_ERR_INVALID_ARG, "rank out of range");
    // segments are sorted by flat offset, so owners never decrease
    auto lo = std::lower_bound(l->seg.begin(), l->seg.end(), rank,
                               [](const zero_segment& s, int32_t r) { return s.owner < r; });
    auto hi = std::lower_bound(lo, l->seg.end(), rank + 1,
                               [](const zero_segment& s, int32_t r) { return s.owner < r; });
    return copy_range(l, size_t(lo - l->seg.begin()), size_t(hi - l->seg.begin()), out, cap, n_out);
}

extern "C" int zero_layout_fill_segments(const zero_layout* l, int64_t fill, zero_segment* out,
                                         int64_t cap, int64_t* n_out) {
    zp::clear_error();
    if (!l || !n_out) return zp::fail(ZERO_ERR_INVALID_ARG, "zero_layout_fill_segments: NULL argument");
    if (l->bucket <= 0) return zp::fail(ZERO_ERR_STATE, "layout has no bucket plan");
    if (fill < 0 || fill >= l->n_fills) return zp::fail(ZERO_ERR_INVALID_ARG, "fill out of range");
    auto lo = std::lower_bound(l->seg.begin(), l->seg.end(), fill,
                               [](const zero_segment& s, int64_t f) { return s.fill < f; });
    auto hi = std::lower_bound(lo, l->seg.end(), fill + 1,
                               [](const zero_segment& s, int64_t f) { return s.fill < f; });
    return copy_range(l, size_t(lo - l->seg.begin()), size_t(hi - l->seg.begin()), out, cap, n_out);
}

// ---------------------------------------------------------------------------
// bucket pack: device tables and launch
// ---------------------------------------------------------------------------

extern "C" int zero_layout_bind_tensors(zero_layout* l, const uint16_t* const* dev_ptrs,
                                        void* stream) {
    zp::clear_error();
    if (!l) return zp::fail(ZERO_ERR_INVALID_ARG, "layout is NULL");
    if (l->bucket <= 0) return zp::fail(ZERO_ERR_STATE, "layout has no bucket plan");
    const size_t nt = l->numel.size();
    if (nt > 0 && !dev_ptrs) return zp::fail(ZERO_ERR_INVALID_ARG, "dev_ptrs is NULL");

    std::vector<zp::PackSrc> src;
    try {
        src.reserve(nt);
    } catch (...) {
        return zp::fail(ZERO_ERR_OUT_OF_MEMORY, "host table allocation failed");
    }
    for (size_t i = 0; i < nt; ++i) {
        if (l->numel[i] == 0) continue;
        if (!dev_ptrs[i]) return zp::fail(ZERO_ERR_INVALID_ARG, "NULL pointer for a non-empty tensor");
        if (reinterpret_cast<uintptr_t>(dev_ptrs[i]) & 1)
            return zp::fail(ZERO_ERR_ALIGNMENT, "tensor pointer not 2-byte aligned");
        src.push_back({dev_ptrs[i], l->offset[i], l->numel[i]});
    }
    if (src.size() > size_t(std::numeric_limits<int32_t>::max()))
        return zp::fail(ZERO_ERR_OUT_OF_MEMORY, "too many tensors");

    std::vector<int64_t> offs;
    std::vector<int32_t> first;
    int shift = 0;
    try {
        offs.reserve(src.size());
        for (const auto& x : src) offs.push_back(x.flat_off);
    } catch (...) {
        return zp::fail(ZERO_ERR_OUT_OF_MEMORY, "host table allocation failed");
    }
    if (!chunk_index(offs, l->psi, &shift, &first))
        return zp::fail(ZERO_ERR_OUT_OF_MEMORY, "host table allocation failed");
    try {
        offs.push_back(l->psi);   // the boundaries of the work order end with psi
    } catch (...) {
        return zp::fail(ZERO_ERR_OUT_OF_MEMORY, "host table allocation failed");
    }

    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return zp::fail_hip(e, "hipGetDevice");
    const int rc = zp::check_stream_device(stream, dev, "zero_layout_bind_tensors");
    if (rc != ZERO_OK) return rc;

    zp::PackSrc* d_src = nullptr;
    int32_t* d_first = nullptr;
    const size_t src_bytes = std::max<size_t>(1, src.size()) * sizeof(zp::PackSrc);
    const size_t first_bytes = first.size() * sizeof(int32_t);
    e = hipMalloc(reinterpret_cast<void**>(&d_src), src_bytes);
    if (e != hipSuccess) return zp::fail_hip(e, "hipMalloc (pack sources)");
    e = hipMalloc(reinterpret_cast<void**>(&d_first), first_bytes);
    if (e != hipSuccess) {
        (void)hipFree(d_src);
        return zp::fail_hip(e, "hipMalloc (pack chunk index)");
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (!src.empty()) e = hipMemcpyAsync(d_src, src.data(), src.size() * sizeof(zp::PackSrc),
                                         hipMemcpyHostToDevice, st);
    if (e == hipSuccess)
        e = hipMemcpyAsync(d_first, first.data(), first_bytes, hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) {
        (void)hipFree(d_src);
        (void)hipFree(d_first);
        return zp::fail_hip(e, "uploading pack tables");
    }
    free_device_tables(l);
    l->d_src = d_src;
    l->d_first = d_first;
    l->n_src = int32_t(src.size());
    l->chunk_shift = shift;
    l->device = dev;
    l->p_off.swap(offs);
    return ZERO_OK;
}

extern "C" int zero_pack_bucket(const zero_layout* l, int64_t fill, uint16_t* bucket, void* stream,
                                int64_t* packed_elems) {
    zp::clear_error();
    if (!l) return zp::fail(ZERO_ERR_INVALID_ARG, "layout is NULL");
    if (l->bucket <= 0) return zp::fail(ZERO_ERR_STATE, "layout has no bucket plan");
    if (l->bucket > ZERO_MAX_SHARD_ELEMS)
        return zp::fail(ZERO_ERR_INVALID_ARG, "bucket_elems above ZERO_MAX_SHARD_ELEMS (one launch's grid)");
    if (l->device < 0) return zp::fail(ZERO_ERR_STATE, "tensors not bound (zero_layout_bind_tensors)");
    if (fill < 0 || fill >= l->n_fills) return zp::fail(ZERO_ERR_INVALID_ARG, "fill out of range");
    if (!bucket) return zp::fail(ZERO_ERR_INVALID_ARG, "bucket is NULL");
    if (reinterpret_cast<uintptr_t>(bucket) & 15)
        return zp::fail(ZERO_ERR_ALIGNMENT, "bucket not 16-byte aligned");
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return zp::fail_hip(e, "hipGetDevice");
    if (dev != l->device) return zp::fail(ZERO_ERR_STATE, "layout was bound on another device");
    const int src = zp::check_stream_device(stream, dev, "zero_pack_bucket");
    if (src != ZERO_OK) return src;

    zp::PackLaunch a;
    a.src = l->d_src;
    a.first = l->d_first;
    a.n_src = l->n_src;
    a.chunk_shift = l->chunk_shift;
    a.psi = l->psi;
    a.fill_base = fill * l->bucket;
    a.bucket_elems = l->bucket;
    a.bucket = bucket;
    a.n_span = (l->bucket + zp::kSpanElems - 1) / zp::kSpanElems;
    const int64_t data = std::min(l->bucket, l->psi - a.fill_base);   // > 0: fill < n_fills
    a.n_data_span = (data + zp::kSpanElems - 1) / zp::kSpanElems;
    a.hard = zp::plan_hard_waves(l->p_off.data(), int64_t(l->p_off.size()), l->chunk_shift, a.fill_base,
                                 a.n_data_span);
    hipStream_t st = static_cast<hipStream_t>(stream);
    zp::KernelEvents ev;
    e = zp::timing_events(&ev);
    if (e != hipSuccess) return zp::fail_hip(e, "timing event");
    e = zp::launch_pack(a, st, ev);
    if (e != hipSuccess) return zp::fail_hip(e, "pack kernel launch");
    zp::timing_done();
    if (packed_elems) *packed_elems = std::min(l->bucket, l->psi - a.fill_base);
    return ZERO_OK;
}

// ---------------------------------------------------------------------------
// bucket reduce-to-owner: device tables and launch
// ---------------------------------------------------------------------------

extern "C" int zero_layout_bind_contributions(zero_layout* l, int32_t R,
                                              const uint16_t* const* dev_ptrs, void* stream) {
    zp::clear_error();
    if (!l) return zp::fail(ZERO_ERR_INVALID_ARG, "layout is NULL");
    if (l->bucket <= 0) return zp::fail(ZERO_ERR_STATE, "layout has no bucket plan");
    if (R < 1 || R > zp::kMaxReduceRanks) return zp::fail(ZERO_ERR_INVALID_ARG, "R must be in 1..16");
    const size_t nt = l->numel.size();
    if (nt > 0 && !dev_ptrs) return zp::fail(ZERO_ERR_INVALID_ARG, "dev_ptrs is NULL");

    std::vector<int64_t> offs, lens;
    std::vector<const uint16_t*> ptrs;
    std::vector<int32_t> first;
    int shift = 0;
    try {
        for (size_t i = 0; i < nt; ++i) {
            if (l->numel[i] == 0) continue;
            offs.push_back(l->offset[i]);
            lens.push_back(l->numel[i]);
        }
        ptrs.reserve(size_t(R) * offs.size());
        for (int32_t r = 0; r < R; ++r) {
            for (size_t i = 0; i < nt; ++i) {
                if (l->numel[i] == 0) continue;
                const uint16_t* p = dev_ptrs[size_t(r) * nt + i];
                if (!p) return zp::fail(ZERO_ERR_INVALID_ARG, "NULL pointer for a non-empty tensor");
                if (reinterpret_cast<uintptr_t>(p) & 1)
                    return zp::fail(ZERO_ERR_ALIGNMENT, "tensor pointer not 2-byte aligned");
                ptrs.push_back(p);
            }
        }
    } catch (...) {
        return zp::fail(ZERO_ERR_OUT_OF_MEMORY, "host table allocation failed");
    }
    if (offs.size() > size_t(std::numeric_limits<int32_t>::max()))
        return zp::fail(ZERO_ERR_OUT_OF_MEMORY, "too many tensors");
    if (!chunk_index(offs, l->psi, &shift, &first))
        return zp::fail(ZERO_ERR_OUT_OF_MEMORY, "host table allocation failed");
    // Per-chunk records: for chunk c, the entries of tensor first[c] (flat
    // offset, length, index, and its R addresses) in one place, so a wave
    // reads everything about the tensor holding its first element with one
    // set of loads from one address.
    const size_t n_chunks = first.size() - 1;
    const size_t rec_bytes = size_t(zp::chunk_rec_bytes(R));
    std::vector<uint8_t> recs;
    try {
        recs.assign(std::max<size_t>(1, n_chunks) * rec_bytes, 0);
    } catch (...) {
        return zp::fail(ZERO_ERR_OUT_OF_MEMORY, "host table allocation failed");
    }
    for (size_t c = 0; c < n_chunks; ++c) {
        const size_t si = size_t(first[c]);
        uint8_t* rec = recs.data() + c * rec_bytes;
        const int64_t off = offs[si], len = lens[si];
        const int32_t idx = first[c];
        std::memcpy(rec + 0, &off, 8);
        std::memcpy(rec + 8, &len, 8);
        std::memcpy(rec + 16, &idx, 4);
        for (int32_t r = 0; r < R; ++r) {
            const uint16_t* p = ptrs[size_t(r) * offs.size() + si];
            std::memcpy(rec + 24 + 8 * size_t(r), &p, 8);
        }
    }
    std::vector<uintptr_t> starts, end_max;
    try {
        std::vector<std::pair<uintptr_t, uintptr_t>> rg;
        rg.reserve(ptrs.size());
        for (size_t k = 0; k < ptrs.size(); ++k) {
            const uintptr_t lo = reinterpret_cast<uintptr_t>(ptrs[k]);
            rg.push_back({lo, lo + uintptr_t(lens[k % lens.size()]) * 2});
        }
        std::sort(rg.begin(), rg.end());
        starts.reserve(rg.size());
        end_max.reserve(rg.size());
        uintptr_t m = 0;
        for (const auto& r : rg) {
            m = std::max(m, r.second);
            starts.push_back(r.first);
            end_max.push_back(m);
        }
    } catch (...) {
        return zp::fail(ZERO_ERR_OUT_OF_MEMORY, "host table allocation failed");
    }

    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return zp::fail_hip(e, "hipGetDevice");
    const int rc = zp::check_stream_device(stream, dev, "zero_layout_bind_contributions");
    if (rc != ZERO_OK) return rc;
    // the offsets end with psi, the end of the last tensor (a sentinel
    // boundary for the kernels' work order)
    try {
        offs.push_back(l->psi);
    } catch (...) {
        return zp::fail(ZERO_ERR_OUT_OF_MEMORY, "host table allocation failed");
    }
    const size_t n = std::max<size_t>(1, lens.size());
    void* d[5] = {nullptr, nullptr, nullptr, nullptr, nullptr};
    const size_t bytes[5] = {offs.size() * sizeof(int64_t), n * sizeof(int64_t),
                             std::max<size_t>(1, ptrs.size()) * sizeof(void*),
                             first.size() * sizeof(int32_t), recs.size()};
    for (int k = 0; k < 5 && e == hipSuccess; ++k) e = hipMalloc(&d[k], bytes[k]);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const void* host[5] = {offs.data(), lens.data(), ptrs.data(), first.data(), recs.data()};
    const size_t used[5] = {offs.size() * sizeof(int64_t), lens.size() * sizeof(int64_t),
                            ptrs.size() * sizeof(void*), first.size() * sizeof(int32_t),
                            n_chunks * rec_bytes};
    for (int k = 0; k < 5 && e == hipSuccess; ++k)
        if (used[k]) e = hipMemcpyAsync(d[k], host[k], used[k], hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) {
        for (void* b : d)
            if (b) (void)hipFree(b);
        return zp::fail_hip(e, "uploading reduce tables");
    }
    free_reduce_tables(l);
    l->d_roff = static_cast<int64_t*>(d[0]);
    l->d_rlen = static_cast<int64_t*>(d[1]);
    l->d_rptr = static_cast<const uint16_t**>(d[2]);
    l->d_rfirst = static_cast<int32_t*>(d[3]);
    l->d_rrec = static_cast<uint8_t*>(d[4]);
    l->r_ranks = R;
    l->r_nsrc = int32_t(lens.size());
    l->r_shift = shift;
    l->r_device = dev;
    l->r_start.swap(starts);
    l->r_end_max.swap(end_max);
    l->r_off.swap(offs);
    return ZERO_OK;
}

namespace zp {

int owner_tables(const zero_layout* l, int32_t rank, ReduceLaunch* out, int* bound_dev) {
    if (l->bucket <= 0) return fail(ZERO_ERR_STATE, "layout has no bucket plan");
    if (l->r_device < 0)
        return fail(ZERO_ERR_STATE, "contributions not bound (zero_layout_bind_contributions)");
    if (rank < 0 || rank >= l->n_ranks) return fail(ZERO_ERR_INVALID_ARG, "rank out of range");
    *bound_dev = l->r_device;
    const int64_t lo = int64_t(rank) * l->shard;
    ReduceLaunch a;
    a.off = l->d_roff;
    a.len = l->d_rlen;
    a.ptr = l->d_rptr;
    a.first = l->d_rfirst;
    a.rec = l->d_rrec;
    a.n_src = l->r_nsrc;
    a.chunk_shift = l->r_shift;
    a.R = l->r_ranks;
    a.base = lo;
    a.g_lo = lo;
    a.g_hi = std::max(lo, std::min(lo + l->shard, l->psi));
    a.shard = nullptr;
    // p, m, v are 16-byte aligned: no misalignment
    plan_reduce_waves(l->r_off.data(), int64_t(l->r_off.size()), l->r_shift, 0, &a);
    *out = a;
    return ZERO_OK;
}

HardWaves plan_hard_waves(const int64_t* off, int64_t n_off, int chunk_shift, int64_t span0, int64_t n_span) {
    HardWaves h;
    h.n_hard = 2;
    h.b_first = 0;
    h.hard_per_b = int32_t((int64_t(1) << chunk_shift) / kSpanElems + 2);
    if (n_span < 3) return h;   // no interior span
    // boundaries that can claim an interior span: cs(F(1) - 7) < b < F(n_span - 1) + 8
    const int64_t lo = ((span0 + kSpanElems - 7) >> chunk_shift) << chunk_shift;
    const int64_t hi = span0 + kSpanElems * (n_span - 1) + 8;
    const int64_t* first = std::upper_bound(off, off + n_off, lo);
    const int64_t* last = std::lower_bound(off, off + n_off, hi);
    const int64_t n_b = last > first ? int64_t(last - first) : 0;
    if (n_b * h.hard_per_b > 8 * n_span + 1024 || 2 + n_b * h.hard_per_b + n_span > kMaxGridWaves) {
        // boundary waves far outnumbering the spans, or a grid past the
        // launch limit: the launch runs in order
        h.n_hard = 0;
        h.hard_per_b = 0;
        return h;
    }
    h.b_first = int64_t(first - off);
    h.n_hard = 2 + n_b * h.hard_per_b;
    return h;
}

void plan_reduce_waves(const int64_t* off, int64_t n_off, int chunk_shift, int mis, ReduceLaunch* a) {
    a->n_span = 0;
    a->hard = plan_hard_waves(off, n_off, chunk_shift, 0, 0);
    if (a->g_hi <= a->g_lo) return;
    const SpanGeometry g = span_geometry(a->base, a->g_lo - a->base, a->g_hi - a->base, mis);
    a->n_span = g.n_span;
    a->hard = plan_hard_waves(off, n_off, chunk_shift, g.span0, g.n_span);
}

bool contributions_overlap(const zero_layout* l, uintptr_t lo, uintptr_t hi) {
    // ranges starting before hi: the first k; one of them meets [lo, hi)
    // exactly when the largest end among them exceeds lo
    const size_t k = size_t(std::lower_bound(l->r_start.begin(), l->r_start.end(), hi) - l->r_start.begin());
    return lo < hi && k > 0 && l->r_end_max[k - 1] > lo;
}

}  // namespace zp

extern "C" int zero_reduce_to_owner(const zero_layout* l, int64_t fill, int32_t rank,
                                    uint16_t* shard, void* stream, int64_t* written) {
    zp::clear_error();
    if (!l) return zp::fail(ZERO_ERR_INVALID_ARG, "layout is NULL");
    if (l->bucket <= 0) return zp::fail(ZERO_ERR_STATE, "layout has no bucket plan");
    if (l->bucket > ZERO_MAX_SHARD_ELEMS)
        return zp::fail(ZERO_ERR_INVALID_ARG, "bucket_elems above ZERO_MAX_SHARD_ELEMS (one launch's grid)");
    if (l->r_device < 0)
        return zp::fail(ZERO_ERR_STATE, "contributions not bound (zero_layout_bind_contributions)");
    if (fill < 0 || fill >= l->n_fills) return zp::fail(ZERO_ERR_INVALID_ARG, "fill out of range");
    if (rank < 0 || rank >= l->n_ranks) return zp::fail(ZERO_ERR_INVALID_ARG, "rank out of range");
    if (!shard) return zp::fail(ZERO_ERR_INVALID_ARG, "shard is NULL");
    if (reinterpret_cast<uintptr_t>(shard) & 1)
        return zp::fail(ZERO_ERR_ALIGNMENT, "shard not 2-byte aligned");
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return zp::fail_hip(e, "hipGetDevice");
    if (dev != l->r_device) return zp::fail(ZERO_ERR_STATE, "contributions were bound on another device");
    const int src = zp::check_stream_device(stream, dev, "zero_reduce_to_owner");
    if (src != ZERO_OK) return src;

    // [fill*B, (fill+1)*B) meets [rank*S, (rank+1)*S) and [0, psi)
    const int64_t fill_lo = fill * l->bucket;                        // < psi
    const int64_t fill_hi = (l->bucket >= l->psi - fill_lo) ? l->psi : fill_lo + l->bucket;
    const int64_t rank_lo = int64_t(rank) * l->shard;
    const int64_t rank_hi = rank_lo + l->shard;
    const int64_t g_lo = std::max(fill_lo, rank_lo);
    const int64_t g_hi = std::min(std::min(fill_hi, rank_hi), l->psi);
    if (written) *written = g_hi > g_lo ? g_hi - g_lo : 0;
    if (g_hi <= g_lo) return ZERO_OK;

    zp::ReduceLaunch a;
    a.off = l->d_roff;
    a.len = l->d_rlen;
    a.ptr = l->d_rptr;
    a.first = l->d_rfirst;
    a.rec = l->d_rrec;
    a.n_src = l->r_nsrc;
    a.chunk_shift = l->r_shift;
    a.R = l->r_ranks;
    a.g_lo = g_lo;
    a.g_hi = g_hi;
    a.base = rank_lo;
    a.shard = shard;
    zp::plan_reduce_waves(l->r_off.data(), int64_t(l->r_off.size()), l->r_shift,
                          int((reinterpret_cast<uintptr_t>(shard) >> 1) & 7), &a);
    hipStream_t st = static_cast<hipStream_t>(stream);
    zp::KernelEvents ev;
    e = zp::timing_events(&ev);
    if (e != hipSuccess) return zp::fail_hip(e, "timing event");
    e = zp::launch_reduce_owner(a, st, ev);
    if (e != hipSuccess) return zp::fail_hip(e, "reduce kernel launch");
    zp::timing_done();
    return ZERO_OK;
}

// ---------------------------------------------------------------------------
// contiguous arena plan
// ---------------------------------------------------------------------------

extern "C" int zero_arena_plan_for(const zero_layout* l, int32_t pingpong, int32_t n_contrib,
                                   int32_t with_bucket, int64_t align_bytes, zero_arena_plan* out) {
    zp::clear_error();
    if (!l || !out) return zp::fail(ZERO_ERR_INVALID_ARG, "zero_arena_plan_for: NULL argument");
    if (n_contrib < 0 || n_contrib > 16) return zp::fail(ZERO_ERR_INVALID_ARG, "n_contrib must be 0..16");
    if (align_bytes == 0) align_bytes = int64_t(1) << 21;
    if (align_bytes < 256 || (align_bytes & (align_bytes - 1)))
        return zp::fail(ZERO_ERR_INVALID_ARG, "align_bytes must be a power of two >= 256");
    if (with_bucket && l->bucket <= 0) return zp::fail(ZERO_ERR_STATE, "layout has no bucket plan");

    const int64_t S = l->shard;
    const int64_t P = int64_t(l->n_ranks) * S;
    const int st = l->stage;
    int64_t elems[ZERO_ARENA_KINDS] = {0};
    int64_t width[ZERO_ARENA_KINDS] = {0};
    bool present[ZERO_ARENA_KINDS] = {false};
    auto want = [&](int kind, int64_t n, int64_t w) {
        elems[kind] = n;
        width[kind] = w;
        present[kind] = true;
    };
    want(ZERO_ARENA_PARAM16, st >= 3 ? S : P, 2);
    want(ZERO_ARENA_GRAD16, st >= 2 ? S : P, 2);
    for (int k = ZERO_ARENA_MASTER; k <= ZERO_ARENA_VARIANCE; ++k) want(k, st >= 1 ? S : P, 4);
    if (pingpong)
        for (int k = ZERO_ARENA_MASTER_ALT; k <= ZERO_ARENA_VARIANCE_ALT; ++k) want(k, st >= 1 ? S : P, 4);
    for (int r = 0; r < n_contrib; ++r) want(ZERO_ARENA_CONTRIB0 + r, S, 2);
    if (with_bucket) want(ZERO_ARENA_BUCKET, l->bucket, 2);

    // fp32 state first, then alternates, gradients, contributions, parameters, bucket
    int order[ZERO_ARENA_KINDS];
    int n_order = 0;
    for (int k = ZERO_ARENA_MASTER; k <= ZERO_ARENA_VARIANCE_ALT; ++k) order[n_order++] = k;
    order[n_order++] = ZERO_ARENA_GRAD16;
    for (int r = 0; r < 16; ++r) order[n_order++] = ZERO_ARENA_CONTRIB0 + r;
    order[n_order++] = ZERO_ARENA_PARAM16;
    order[n_order++] = ZERO_ARENA_BUCKET;

    zero_arena_plan plan;
    plan.align_bytes = align_bytes;
    for (int k = 0; k < ZERO_ARENA_KINDS; ++k) {
        plan.offset[k] = -1;
        plan.bytes[k] = 0;
    }
    constexpr int64_t kMax = std::numeric_limits<int64_t>::max();
    int64_t off = 0;
    for (int j = 0; j < n_order; ++j) {
        const int k = order[j];
        if (!present[k]) continue;
        if (off > kMax - (align_bytes - 1)) return zp::fail(ZERO_ERR_INDEX_OVERFLOW, "arena size overflows int64");
        off = (off + align_bytes - 1) & ~(align_bytes - 1);
        if (elems[k] > (kMax - off) / width[k]) return zp::fail(ZERO_ERR_INDEX_OVERFLOW, "arena size overflows int64");
        plan.offset[k] = off;
        plan.bytes[k] = elems[k] * width[k];
        off += plan.bytes[k];
    }
    plan.total_bytes = off;
    *out = plan;
    return ZERO_OK;
}

