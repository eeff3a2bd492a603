// h3_api.hip -- the C ABI of libh3.so: argument validation, the launch plan
// and the plan report.  Every check runs before anything is enqueued; a
// rejected call leaves no state behind.  See include/h3.h for the contract.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "h3_internal.h"

namespace {

thread_local char g_last_error[512] = "";

h3_status fail(h3_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

h3_status ok() {
    g_last_error[0] = '\0';
    return H3_OK;
}

// Kernel argument blocks travel by value; the kernarg segment holds 4 KB.
static_assert(sizeof(h3::RunCopyArgs) <= 4096, "relayout arguments exceed the kernarg segment");
static_assert(sizeof(h3::AttnArgs) <= 4096, "attention arguments exceed the kernarg segment");
static_assert(sizeof(h3::AttnBwdArgs) <= 4096, "attention backward arguments exceed the kernarg segment");
static_assert(sizeof(h3::AdalnArgs) <= 4096, "AdaLN arguments exceed the kernarg segment");
static_assert(sizeof(h3::RaggedArgs) <= 4096, "ragged collective arguments exceed the kernarg segment");

// ---------------------------------------------------------------------------
// Debug builds (-DH3_DEBUG_BOUNDS) re-check every table a kernel indexes --
// rank slots, run lengths and offsets, the attention work lists, the clipped
// AdaLN table, the ragged row ranges -- right before its launch, against the
// sizes the call validated, and abort with a message on the first violation.
// Release builds compile the checks out.
// ---------------------------------------------------------------------------
#ifdef H3_DEBUG_BOUNDS
[[noreturn]] void debug_bounds_fail(int line, const char *cond, const char *what) {
    std::fprintf(stderr, "h3 debug bounds check failed (h3_api.hip:%d, %s): %s\n", line, what, cond);
    std::fflush(stderr);
    std::abort();
}
#define H3_DEBUG_CHECK(cond, what) \
    do {                            \
        if (!(cond)) debug_bounds_fail(__LINE__, #cond, what); \
    } while (0)
#define H3_DEBUG_ONLY(...) __VA_ARGS__

// Relayout launch: slots 0..nr-1 each copy runs of run_vec vectors that lie
// inside one plane row of plane_vec vectors, with a 32-bit flat index range.
void debug_check_copy(const h3::RunCopyArgs &a, int nr, uint32_t max_run, uint32_t plane_vec) {
    H3_DEBUG_CHECK(nr >= 1 && nr <= h3::kMaxRanks, "relayout rank slots");
    H3_DEBUG_CHECK(a.stride_vec >= plane_vec, "relayout packed stride");
    H3_DEBUG_CHECK(a.n_tokens >= 1, "relayout launch tokens");
    for (int y = 0; y < nr; ++y) {
        H3_DEBUG_CHECK(a.run_vec[y] >= 2 && a.run_vec[y] <= max_run, "relayout run length");
        H3_DEBUG_CHECK(a.div[y].d == a.run_vec[y], "relayout divisor");
        H3_DEBUG_CHECK((uint64_t)a.off_vec[y] + a.run_vec[y] <= plane_vec, "relayout run inside the plane row");
        H3_DEBUG_CHECK((uint64_t)a.n_tokens * a.run_vec[y] < (1ull << 31), "relayout flat index range");
        H3_DEBUG_CHECK(a.src_rank[y] != nullptr || a.dst_rank[y] != nullptr, "relayout rank buffer");
    }
    for (int y = nr; y < h3::kMaxRanks; ++y) H3_DEBUG_CHECK(a.run_vec[y] == 0, "relayout unused slot");
}

// Attention work lists: n entries, each a non-empty segment inside the
// tokens, workgroup prefix = sum of ceil(len / block) * heads, ending at total.
void debug_check_worklist(const int32_t *prefix, const int32_t *begin, const int32_t *len, int n, int64_t n_tokens,
                          int64_t heads, int64_t block, int64_t total, const char *what) {
    H3_DEBUG_CHECK(n >= 1 && n <= h3::kMaxSegments, what);
    H3_DEBUG_CHECK(prefix[0] == 0, what);
    int64_t covered = 0;
    for (int e = 0; e < n; ++e) {
        H3_DEBUG_CHECK(len[e] >= 1 && begin[e] >= 0 && (int64_t)begin[e] + len[e] <= n_tokens, what);
        H3_DEBUG_CHECK((int64_t)prefix[e + 1] - prefix[e] == (len[e] + block - 1) / block * heads, what);
        if (e > 0) H3_DEBUG_CHECK(len[e] <= len[e - 1], what);            // longest first
        covered += len[e];
    }
    H3_DEBUG_CHECK(covered == n_tokens, what);
    H3_DEBUG_CHECK(prefix[n] == total, what);
}

// Clipped AdaLN table: entries start at local row 0, strictly increase, end at
// n_rows, and name increasing global segments below n_segments.
void debug_check_adaln(const h3::AdalnArgs &a, int n_segments) {
    H3_DEBUG_CHECK(a.n_entries >= 1 && a.n_entries <= h3::kMaxSegments, "adaln entries");
    H3_DEBUG_CHECK(a.entry_begin[0] == 0, "adaln first entry");
    for (int e = 0; e < a.n_entries; ++e) {
        H3_DEBUG_CHECK(a.entry_begin[e] < a.entry_begin[e + 1], "adaln entry order");
        H3_DEBUG_CHECK(a.entry_seg[e] >= 0 && a.entry_seg[e] < n_segments, "adaln segment id");
        if (e > 0) H3_DEBUG_CHECK(a.entry_seg[e] > a.entry_seg[e - 1], "adaln segment order");
    }
    H3_DEBUG_CHECK((uint32_t)a.entry_begin[a.n_entries] == a.n_rows, "adaln last entry");
}

// Ragged collectives: every slot's row range lies inside the N x C buffer.
void debug_check_ragged(const h3::RaggedArgs &a, int n_slots, int64_t n_tokens) {
    H3_DEBUG_CHECK(n_slots >= 1 && n_slots <= h3::kMaxRanks, "ragged slots");
    const uint64_t all = (uint64_t)n_tokens * a.nv_row;
    for (int y = 0; y < n_slots; ++y) {
        H3_DEBUG_CHECK(a.n_vec[y] >= 1 && a.n_vec[y] < (1u << 31), "ragged slot length");
        H3_DEBUG_CHECK(a.row_vec0[y] % a.nv_row == 0 && a.n_vec[y] % a.nv_row == 0, "ragged whole rows");
        H3_DEBUG_CHECK(a.row_vec0[y] + a.n_vec[y] <= all, "ragged slot inside the rows");
    }
}
#else
#define H3_DEBUG_ONLY(...)
#endif

// Balanced quotient/remainder split ("Distributed H3 Execution", Partition
// Contract): the first total%parts parts hold one extra item.
void split(int64_t total, int32_t parts, int32_t index, int64_t *begin, int64_t *count) {
    const int64_t q = total / parts, r = total % parts;
    *count = q + (index < r ? 1 : 0);
    *begin = (int64_t)index * q + std::min<int64_t>(index, r);
}

struct Range {
    uintptr_t lo, hi;
    const char *what;
    int index;
};

// Reject any output range that overlaps an input range or another output.
h3_status check_alias(const std::vector<Range> &inputs, const std::vector<Range> &outputs) {
    for (size_t i = 0; i < outputs.size(); ++i) {
        const Range &o = outputs[i];
        if (o.hi <= o.lo) continue;
        for (const Range &in : inputs) {
            if (in.hi > in.lo && o.lo < in.hi && in.lo < o.hi)
                return fail(H3_ERR_ALIAS, "output %s[%d] overlaps input %s[%d]; outputs need storage of "
                            "their own", o.what, o.index, in.what, in.index);
        }
        for (size_t j = i + 1; j < outputs.size(); ++j) {
            const Range &p = outputs[j];
            if (p.hi > p.lo && o.lo < p.hi && p.lo < o.hi)
                return fail(H3_ERR_ALIAS, "outputs %s[%d] and %s[%d] overlap", o.what, o.index, p.what,
                            p.index);
        }
    }
    return H3_OK;
}

Range range_of(const void *p, uint64_t bytes, const char *what, int index) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, lo + bytes, what, index};
}

h3_status check_segments(const int64_t *cu, int32_t n_segments, int64_t n_tokens, bool exact_end) {
    if (!cu) return fail(H3_ERR_ARG, "cu_seqlens is NULL");
    if (n_segments < 1 || n_segments > H3_MAX_SEGMENTS)
        return fail(H3_ERR_SEGMENTS, "n_segments = %d; legal values are 1..%d", n_segments, H3_MAX_SEGMENTS);
    if (cu[0] != 0) return fail(H3_ERR_SEGMENTS, "cu_seqlens[0] = %lld, must be 0", (long long)cu[0]);
    for (int32_t s = 0; s < n_segments; ++s)
        if (cu[s + 1] <= cu[s])
            return fail(H3_ERR_SEGMENTS, "segment %d is empty or reversed (cu[%d] = %lld, cu[%d] = %lld)", s, s,
                        (long long)cu[s], s + 1, (long long)cu[s + 1]);
    if (exact_end ? cu[n_segments] != n_tokens : cu[n_segments] < n_tokens)
        return fail(H3_ERR_SEGMENTS, "cu_seqlens[%d] = %lld does not cover the %lld tokens", n_segments,
                    (long long)cu[n_segments], (long long)n_tokens);
    return H3_OK;
}

// Every kernel moves bf16 data in 16-byte vectors (and fp32 row terms in
// 4-byte words), so a buffer must start on that boundary.  NULL passes: the
// callers check presence separately.
h3_status check_aligned(const void *p, const char *what, int index, unsigned align = 16) {
    if (reinterpret_cast<uintptr_t>(p) % align != 0)
        return fail(H3_ERR_ARG, "%s[%d] = %p is not %u-byte aligned", what, index, p, align);
    return H3_OK;
}

void clear_info(h3_plan_info *info) {
    if (info) std::memset(info, 0, sizeof *info);
}

// Bytes of one plane that a relayout launch moves per token: the heads of
// every selected rank (a valid layout is assumed).
int64_t selected_token_bytes(const h3_layout *L) {
    if (L->rank < 0) return (int64_t)L->n_heads * L->head_dim * 2;
    int64_t hb, hn;
    split(L->n_heads, L->world, L->rank, &hb, &hn);
    return hn * L->head_dim * 2;
}

// Shared validation of a relayout contract.
h3_status check_layout(const h3_layout *L, bool head2seq) {
    if (!L) return fail(H3_ERR_ARG, "layout is NULL");
    if (L->reserved != 0) return fail(H3_ERR_ARG, "layout.reserved must be 0");
    if (L->n_tokens < 1) return fail(H3_ERR_EMPTY_PARTITION, "n_tokens = %lld: no tokens to partition",
                                     (long long)L->n_tokens);
    if (L->n_heads < 1 || L->n_heads > H3_MAX_HEADS)
        return fail(H3_ERR_ARG, "n_heads = %d; legal values are 1..%d", L->n_heads, H3_MAX_HEADS);
    if (L->head_dim != H3_HEAD_DIM)
        return fail(H3_ERR_UNSUPPORTED, "head_dim = %d; only %d is supported", L->head_dim, H3_HEAD_DIM);
    if (head2seq ? L->n_planes != 1 : (L->n_planes < 1 || L->n_planes > 8))
        return fail(H3_ERR_ARG, "n_planes = %d; legal values are %s", L->n_planes, head2seq ? "1" : "1..8");
    const int64_t max_world = std::min<int64_t>(L->n_heads, L->n_tokens);
    if (L->world < 1 || L->world > max_world)
        return fail(H3_ERR_EMPTY_PARTITION,
                    "world = %d would leave a rank without heads or tokens; legal values are 1..%lld",
                    L->world, (long long)max_world);
    if (L->world > h3::kMaxRanks)
        return fail(H3_ERR_UNSUPPORTED, "world = %d; at most %d virtual ranks are supported", L->world,
                    h3::kMaxRanks);
    if (L->rank < -1 || L->rank >= L->world)
        return fail(H3_ERR_ARG, "rank = %d; legal values are -1 (every rank) or 0..%d", L->rank, L->world - 1);
    if (L->max_chunk_bytes < 0)
        return fail(H3_ERR_ARG, "max_chunk_bytes = %lld must be >= 0", (long long)L->max_chunk_bytes);
    const int64_t tok_bytes = selected_token_bytes(L);
    if (L->max_chunk_bytes > 0 && L->max_chunk_bytes < tok_bytes)
        return fail(H3_ERR_ARG, "max_chunk_bytes = %lld is below what one token of one plane moves for the "
                    "selected ranks (%lld bytes)", (long long)L->max_chunk_bytes, (long long)tok_bytes);
    return H3_OK;
}

// Token chunking of one plane.  The cap bounds the source bytes one launch
// reads: a launch moves, per token, the selected ranks' heads of one plane
// (every head for rank = -1, H_j heads for rank j's share), so a chunk holds
// floor(cap / those bytes) tokens.  Then the 32-bit index range of the kernel.
void plan_chunks(const h3_layout *L, uint32_t packed_stride_vec, int64_t *chunk_tokens, int32_t *n_chunks,
                 int64_t *user_chunk) {
    const int64_t tok_bytes = selected_token_bytes(L);
    int64_t c = L->max_chunk_bytes > 0 ? L->max_chunk_bytes / tok_bytes : L->n_tokens;
    c = std::min<int64_t>(c, L->n_tokens);
    *user_chunk = c;
    // keep t*stride + run and tokens*run below 2^31 inside one launch
    const int64_t idx_cap = ((int64_t)1 << 31) / ((int64_t)packed_stride_vec + 1) - 1;
    c = std::max<int64_t>(1, std::min(c, idx_cap));
    *chunk_tokens = c;
    *n_chunks = (int32_t)((L->n_tokens + c - 1) / c);
}

}  // namespace

extern "C" {

const char *h3_status_string(h3_status st) {
    switch (st) {
        case H3_OK: return "H3_OK";
        case H3_ERR_ARG: return "H3_ERR_ARG";
        case H3_ERR_EMPTY_PARTITION: return "H3_ERR_EMPTY_PARTITION";
        case H3_ERR_SEGMENTS: return "H3_ERR_SEGMENTS";
        case H3_ERR_UNSUPPORTED: return "H3_ERR_UNSUPPORTED";
        case H3_ERR_ALIAS: return "H3_ERR_ALIAS";
        case H3_ERR_HIP: return "H3_ERR_HIP";
    }
    return "H3_ERR_UNKNOWN";
}

const char *h3_last_error(void) { return g_last_error; }

const char *h3_version(void) { return "0.1.0"; }

h3_status h3_partition(int64_t total, int32_t parts, int32_t index, int64_t *begin, int64_t *count) {
    if (!begin || !count) return fail(H3_ERR_ARG, "begin/count is NULL");
    if (parts < 1 || parts > total)
        return fail(H3_ERR_EMPTY_PARTITION, "cannot split %lld items over %d ranks without an empty part; "
                    "legal rank counts are 1..%lld", (long long)total, parts, (long long)total);
    if (index < 0 || index >= parts)
        return fail(H3_ERR_ARG, "index = %d; legal values are 0..%d", index, parts - 1);
    split(total, parts, index, begin, count);
    return ok();
}

int32_t h3_clip_segments(const int64_t *cu, int32_t n_segments, int64_t a, int64_t b, int32_t *seg_id,
                         int64_t *local_begin, int64_t *local_end) {
    if (!cu || n_segments < 1 || a < 0 || b <= a) {
        fail(H3_ERR_ARG, "invalid segment table or interval [%lld, %lld)", (long long)a, (long long)b);
        return -1;
    }
    for (int32_t s = 0; s < n_segments; ++s)
        if (cu[s + 1] <= cu[s] || (s == 0 && cu[0] != 0)) {
            fail(H3_ERR_SEGMENTS, "segment table is not strictly increasing from 0");
            return -1;
        }
    if (b > cu[n_segments]) {
        fail(H3_ERR_SEGMENTS, "interval end %lld lies past the last segment (%lld)", (long long)b,
             (long long)cu[n_segments]);
        return -1;
    }
    int32_t n = 0;
    for (int32_t s = 0; s < n_segments; ++s) {
        const int64_t lo = std::max(cu[s], a), hi = std::min(cu[s + 1], b);
        if (lo < hi) {
            if (seg_id) seg_id[n] = s;
            if (local_begin) local_begin[n] = lo - a;
            if (local_end) local_end[n] = hi - a;
            ++n;
        }
    }
    ok();
    return n;
}

h3_status h3_seq2head(const h3_layout *L, const void *src, void *const *dst, void *stream, h3_plan_info *info) {
    clear_info(info);
    h3_status st = check_layout(L, false);
    if (st != H3_OK) return st;
    if (!src) return fail(H3_ERR_ARG, "src is NULL");
    if (!dst) return fail(H3_ERR_ARG, "dst is NULL");
    if ((st = check_aligned(src, "src", 0)) != H3_OK) return st;
    const int P = L->world, K = L->n_planes;
    const int r0 = L->rank < 0 ? 0 : L->rank;
    const int nr = L->rank < 0 ? P : 1;
    const uint64_t row_bytes = (uint64_t)L->n_heads * L->head_dim * 2;
    const uint64_t src_bytes = (uint64_t)L->n_tokens * K * row_bytes;

    std::vector<Range> ins{range_of(src, src_bytes, "src", 0)}, outs;
    int64_t hb[h3::kMaxRanks], hn[h3::kMaxRanks];
    for (int j = 0; j < P; ++j) split(L->n_heads, P, j, &hb[j], &hn[j]);
    for (int j = r0; j < r0 + nr; ++j)
        for (int p = 0; p < K; ++p) {
            if (!dst[j * K + p]) return fail(H3_ERR_ARG, "dst[%d] (rank %d, plane %d) is NULL", j * K + p, j, p);
            if ((st = check_aligned(dst[j * K + p], "dst", j * K + p)) != H3_OK) return st;
            outs.push_back(range_of(dst[j * K + p], (uint64_t)L->n_tokens * hn[j] * L->head_dim * 2, "dst",
                                    j * K + p));
        }
    if ((st = check_alias(ins, outs)) != H3_OK) return st;

    const uint32_t vec_per_head = L->head_dim / 8;
    const uint32_t stride_vec = (uint32_t)K * L->n_heads * vec_per_head;
    int64_t chunk, user_chunk;
    int32_t n_chunks;
    plan_chunks(L, stride_vec, &chunk, &n_chunks, &user_chunk);

    h3::RunCopyArgs a;
    std::memset(&a, 0, sizeof a);
    uint32_t max_run = 0;
    uint64_t rank_bytes = 0;
    for (int y = 0; y < nr; ++y) {
        const int j = r0 + y;
        a.run_vec[y] = (uint32_t)hn[j] * vec_per_head;
        a.off_vec[y] = (uint32_t)hb[j] * vec_per_head;
        a.div[y] = h3::make_fastdiv(a.run_vec[y]);
        max_run = std::max(max_run, a.run_vec[y]);
        rank_bytes += (uint64_t)hn[j] * L->head_dim * 2;
    }
    a.stride_vec = stride_vec;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    int launches = 0, grid_max = 0;
    for (int p = 0; p < K; ++p) {
        for (int c = 0; c < n_chunks; ++c) {
            const int64_t t0 = (int64_t)c * chunk;
            const int64_t nt = std::min<int64_t>(chunk, L->n_tokens - t0);
            a.src_packed = static_cast<const char *>(src) + ((uint64_t)t0 * K + p) * row_bytes;
            for (int y = 0; y < nr; ++y) {
                const int j = r0 + y;
                a.dst_rank[y] = static_cast<char *>(dst[j * K + p]) + (uint64_t)t0 * hn[j] * L->head_dim * 2;
            }
            a.n_tokens = (uint32_t)nt;
            H3_DEBUG_ONLY(debug_check_copy(a, nr, max_run, (uint32_t)L->n_heads * vec_per_head));
            int gx = 0;
            hipError_t e = h3::launch_seq2head(a, nr, max_run, s, &gx);
            if (e != hipSuccess)
                return fail(H3_ERR_HIP, "seq2head launch (plane %d, chunk %d) failed: %s", p, c, hipGetErrorString(e));
            ++launches;
            grid_max = std::max(grid_max, gx);
        }
    }
    if (info) {
        info->launches = launches;
        info->chunks = n_chunks;
        info->grid_x = grid_max;
        info->block_x = h3::kCopyThreads;
        info->chunk_tokens = chunk;
        info->max_launch_src_bytes = (int64_t)(std::min<int64_t>(chunk, L->n_tokens) * rank_bytes);
        info->bytes_read = (int64_t)((uint64_t)L->n_tokens * K * rank_bytes);
        info->bytes_written = info->bytes_read;
    }
    return ok();
}

h3_status h3_head2seq(const h3_layout *L, const void *const *src, void *dst, void *stream, h3_plan_info *info) {
    clear_info(info);
    h3_status st = check_layout(L, true);
    if (st != H3_OK) return st;
    if (!src) return fail(H3_ERR_ARG, "src is NULL");
    if (!dst) return fail(H3_ERR_ARG, "dst is NULL");
    if ((st = check_aligned(dst, "dst", 0)) != H3_OK) return st;
    const int P = L->world;
    const int r0 = L->rank < 0 ? 0 : L->rank;
    const int nr = L->rank < 0 ? P : 1;
    const uint64_t row_bytes = (uint64_t)L->n_heads * L->head_dim * 2;

    int64_t hb[h3::kMaxRanks], hn[h3::kMaxRanks];
    for (int j = 0; j < P; ++j) split(L->n_heads, P, j, &hb[j], &hn[j]);
    std::vector<Range> ins, outs{range_of(dst, (uint64_t)L->n_tokens * row_bytes, "dst", 0)};
    for (int j = r0; j < r0 + nr; ++j) {
        if (!src[j]) return fail(H3_ERR_ARG, "src[%d] is NULL", j);
        if ((st = check_aligned(src[j], "src", j)) != H3_OK) return st;
        ins.push_back(range_of(src[j], (uint64_t)L->n_tokens * hn[j] * L->head_dim * 2, "src", j));
    }
    if ((st = check_alias(ins, outs)) != H3_OK) return st;

    const uint32_t vec_per_head = L->head_dim / 8;
    const uint32_t stride_vec = (uint32_t)L->n_heads * vec_per_head;
    int64_t chunk, user_chunk;
    int32_t n_chunks;
    plan_chunks(L, stride_vec, &chunk, &n_chunks, &user_chunk);

    h3::RunCopyArgs a;
    std::memset(&a, 0, sizeof a);
    uint32_t max_run = 0;
    uint64_t rank_bytes = 0;
    for (int y = 0; y < nr; ++y) {
        const int j = r0 + y;
        a.run_vec[y] = (uint32_t)hn[j] * vec_per_head;
        a.off_vec[y] = (uint32_t)hb[j] * vec_per_head;
        a.div[y] = h3::make_fastdiv(a.run_vec[y]);
        max_run = std::max(max_run, a.run_vec[y]);
        rank_bytes += (uint64_t)hn[j] * L->head_dim * 2;
    }
    a.stride_vec = stride_vec;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    int launches = 0, grid_max = 0;
    for (int c = 0; c < n_chunks; ++c) {
        const int64_t t0 = (int64_t)c * chunk;
        const int64_t nt = std::min<int64_t>(chunk, L->n_tokens - t0);
        a.dst_packed = static_cast<char *>(dst) + (uint64_t)t0 * row_bytes;
        for (int y = 0; y < nr; ++y) {
            const int j = r0 + y;
            a.src_rank[y] = static_cast<const char *>(src[j]) + (uint64_t)t0 * hn[j] * L->head_dim * 2;
        }
        a.n_tokens = (uint32_t)nt;
        H3_DEBUG_ONLY(debug_check_copy(a, nr, max_run, (uint32_t)L->n_heads * vec_per_head));
        int gx = 0;
        hipError_t e = h3::launch_head2seq(a, nr, max_run, s, &gx);
        if (e != hipSuccess) return fail(H3_ERR_HIP, "head2seq launch (chunk %d) failed: %s", c, hipGetErrorString(e));
        ++launches;
        grid_max = std::max(grid_max, gx);
    }
    if (info) {
        info->launches = launches;
        info->chunks = n_chunks;
        info->grid_x = grid_max;
        info->block_x = h3::kCopyThreads;
        info->chunk_tokens = chunk;
        info->max_launch_src_bytes = (int64_t)(std::min<int64_t>(chunk, L->n_tokens) * rank_bytes);
        info->bytes_read = (int64_t)((uint64_t)L->n_tokens * rank_bytes);
        info->bytes_written = info->bytes_read;
    }
    return ok();
}

h3_status h3_seq2head_backward(const h3_layout *L, const void *const *grad_dst, void *grad_src, void *stream,
                               h3_plan_info *info) {
    // Adjoint of h3_seq2head: the rank -> packed copy, with the forward's packed
    // stride (K planes) and the forward's chunk plan.
    clear_info(info);
    h3_status st = check_layout(L, false);
    if (st != H3_OK) return st;
    if (!grad_dst) return fail(H3_ERR_ARG, "grad_dst is NULL");
    if (!grad_src) return fail(H3_ERR_ARG, "grad_src is NULL");
    if ((st = check_aligned(grad_src, "grad_src", 0)) != H3_OK) return st;
    const int P = L->world, K = L->n_planes;
    const int r0 = L->rank < 0 ? 0 : L->rank;
    const int nr = L->rank < 0 ? P : 1;
    const uint64_t row_bytes = (uint64_t)L->n_heads * L->head_dim * 2;

    int64_t hb[h3::kMaxRanks], hn[h3::kMaxRanks];
    for (int j = 0; j < P; ++j) split(L->n_heads, P, j, &hb[j], &hn[j]);
    std::vector<Range> ins, outs{range_of(grad_src, (uint64_t)L->n_tokens * K * row_bytes, "grad_src", 0)};
    for (int j = r0; j < r0 + nr; ++j)
        for (int p = 0; p < K; ++p) {
            if (!grad_dst[j * K + p])
                return fail(H3_ERR_ARG, "grad_dst[%d] (rank %d, plane %d) is NULL", j * K + p, j, p);
            if ((st = check_aligned(grad_dst[j * K + p], "grad_dst", j * K + p)) != H3_OK) return st;
            ins.push_back(range_of(grad_dst[j * K + p], (uint64_t)L->n_tokens * hn[j] * L->head_dim * 2, "grad_dst",
                                   j * K + p));
        }
    if ((st = check_alias(ins, outs)) != H3_OK) return st;

    const uint32_t vec_per_head = L->head_dim / 8;
    const uint32_t stride_vec = (uint32_t)K * L->n_heads * vec_per_head;     // as the forward
    int64_t chunk, user_chunk;
    int32_t n_chunks;
    plan_chunks(L, stride_vec, &chunk, &n_chunks, &user_chunk);

    h3::RunCopyArgs a;
    std::memset(&a, 0, sizeof a);
    uint32_t max_run = 0;
    uint64_t rank_bytes = 0;
    for (int y = 0; y < nr; ++y) {
        const int j = r0 + y;
        a.run_vec[y] = (uint32_t)hn[j] * vec_per_head;
        a.off_vec[y] = (uint32_t)hb[j] * vec_per_head;
        a.div[y] = h3::make_fastdiv(a.run_vec[y]);
        max_run = std::max(max_run, a.run_vec[y]);
        rank_bytes += (uint64_t)hn[j] * L->head_dim * 2;
    }
    a.stride_vec = stride_vec;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    int launches = 0, grid_max = 0;
    for (int p = 0; p < K; ++p) {
        for (int c = 0; c < n_chunks; ++c) {
            const int64_t t0 = (int64_t)c * chunk;
            const int64_t nt = std::min<int64_t>(chunk, L->n_tokens - t0);
            a.dst_packed = static_cast<char *>(grad_src) + ((uint64_t)t0 * K + p) * row_bytes;
            for (int y = 0; y < nr; ++y) {
                const int j = r0 + y;
                a.src_rank[y] = static_cast<const char *>(grad_dst[j * K + p]) + (uint64_t)t0 * hn[j] * L->head_dim * 2;
            }
            a.n_tokens = (uint32_t)nt;
            H3_DEBUG_ONLY(debug_check_copy(a, nr, max_run, (uint32_t)L->n_heads * vec_per_head));
            int gx = 0;
            hipError_t e = h3::launch_head2seq(a, nr, max_run, s, &gx);
            if (e != hipSuccess)
                return fail(H3_ERR_HIP, "seq2head backward launch (plane %d, chunk %d) failed: %s", p, c,
                            hipGetErrorString(e));
            ++launches;
            grid_max = std::max(grid_max, gx);
        }
    }
    if (info) {
        info->launches = launches;
        info->chunks = n_chunks;
        info->grid_x = grid_max;
        info->block_x = h3::kCopyThreads;
        info->chunk_tokens = chunk;
        info->max_launch_src_bytes = (int64_t)(std::min<int64_t>(chunk, L->n_tokens) * rank_bytes);
        info->bytes_read = (int64_t)((uint64_t)L->n_tokens * K * rank_bytes);
        info->bytes_written = info->bytes_read;
    }
    return ok();
}

h3_status h3_head2seq_backward(const h3_layout *L, const void *grad_dst, void *const *grad_src, void *stream,
                               h3_plan_info *info) {
    // Adjoint of h3_head2seq: the packed -> rank copy of one plane, with the
    // forward's chunk plan.
    clear_info(info);
    h3_status st = check_layout(L, true);
    if (st != H3_OK) return st;
    if (!grad_dst) return fail(H3_ERR_ARG, "grad_dst is NULL");
    if (!grad_src) return fail(H3_ERR_ARG, "grad_src is NULL");
    if ((st = check_aligned(grad_dst, "grad_dst", 0)) != H3_OK) return st;
    const int P = L->world;
    const int r0 = L->rank < 0 ? 0 : L->rank;
    const int nr = L->rank < 0 ? P : 1;
    const uint64_t row_bytes = (uint64_t)L->n_heads * L->head_dim * 2;

    int64_t hb[h3::kMaxRanks], hn[h3::kMaxRanks];
    for (int j = 0; j < P; ++j) split(L->n_heads, P, j, &hb[j], &hn[j]);
    std::vector<Range> ins{range_of(grad_dst, (uint64_t)L->n_tokens * row_bytes, "grad_dst", 0)}, outs;
    for (int j = r0; j < r0 + nr; ++j) {
        if (!grad_src[j]) return fail(H3_ERR_ARG, "grad_src[%d] is NULL", j);
        if ((st = check_aligned(grad_src[j], "grad_src", j)) != H3_OK) return st;
        outs.push_back(range_of(grad_src[j], (uint64_t)L->n_tokens * hn[j] * L->head_dim * 2, "grad_src", j));
    }
    if ((st = check_alias(ins, outs)) != H3_OK) return st;

    const uint32_t vec_per_head = L->head_dim / 8;
    const uint32_t stride_vec = (uint32_t)L->n_heads * vec_per_head;           // as the forward
    int64_t chunk, user_chunk;
    int32_t n_chunks;
    plan_chunks(L, stride_vec, &chunk, &n_chunks, &user_chunk);

    h3::RunCopyArgs a;
    std::memset(&a, 0, sizeof a);
    uint32_t max_run = 0;
    uint64_t rank_bytes = 0;
    for (int y = 0; y < nr; ++y) {
        const int j = r0 + y;
        a.run_vec[y] = (uint32_t)hn[j] * vec_per_head;
        a.off_vec[y] = (uint32_t)hb[j] * vec_per_head;
        a.div[y] = h3::make_fastdiv(a.run_vec[y]);
        max_run = std::max(max_run, a.run_vec[y]);
        rank_bytes += (uint64_t)hn[j] * L->head_dim * 2;
    }
    a.stride_vec = stride_vec;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    int launches = 0, grid_max = 0;
    for (int c = 0; c < n_chunks; ++c) {
        const int64_t t0 = (int64_t)c * chunk;
        const int64_t nt = std::min<int64_t>(chunk, L->n_tokens - t0);
        a.src_packed = static_cast<const char *>(grad_dst) + (uint64_t)t0 * row_bytes;
        for (int y = 0; y < nr; ++y) {
            const int j = r0 + y;
            a.dst_rank[y] = static_cast<char *>(grad_src[j]) + (uint64_t)t0 * hn[j] * L->head_dim * 2;
        }
        a.n_tokens = (uint32_t)nt;
        H3_DEBUG_ONLY(debug_check_copy(a, nr, max_run, (uint32_t)L->n_heads * vec_per_head));
        int gx = 0;
        hipError_t e = h3::launch_seq2head(a, nr, max_run, s, &gx);
        if (e != hipSuccess)
            return fail(H3_ERR_HIP, "head2seq backward launch (chunk %d) failed: %s", c, hipGetErrorString(e));
        ++launches;
        grid_max = std::max(grid_max, gx);
    }
    if (info) {
        info->launches = launches;
        info->chunks = n_chunks;
        info->grid_x = grid_max;
        info->block_x = h3::kCopyThreads;
        info->chunk_tokens = chunk;
        info->max_launch_src_bytes = (int64_t)(std::min<int64_t>(chunk, L->n_tokens) * rank_bytes);
        info->bytes_read = (int64_t)((uint64_t)L->n_tokens * rank_bytes);
        info->bytes_written = info->bytes_read;
    }
    return ok();
}

static h3_status packed_attn_impl(const void *q, const void *k, const void *v, const void *g, void *o, float *lse,
                                  int64_t n_tokens, int32_t n_heads, int32_t head_dim, const int64_t *cu,
                                  int32_t n_segments, float scale, void *stream, h3_plan_info *info) {
    clear_info(info);
    if (!q || !k || !v || !o) return fail(H3_ERR_ARG, "q, k, v and o must be non-NULL");
    if (n_tokens < 1) return fail(H3_ERR_EMPTY_PARTITION, "n_tokens = %lld: no tokens", (long long)n_tokens);
    if (n_tokens > INT32_MAX) return fail(H3_ERR_UNSUPPORTED, "n_tokens = %lld exceeds 2^31-1", (long long)n_tokens);
    if (n_heads < 1 || n_heads > H3_MAX_HEADS)
        return fail(H3_ERR_EMPTY_PARTITION, "n_heads = %d; legal values are 1..%d", n_heads, H3_MAX_HEADS);
    if (head_dim != H3_HEAD_DIM)
        return fail(H3_ERR_UNSUPPORTED, "head_dim = %d; only %d is supported", head_dim, H3_HEAD_DIM);
    if (!(scale > 0.f) || scale != scale || scale > 1e30f)
        return fail(H3_ERR_ARG, "scale must be a positive finite number");
    h3_status st = check_segments(cu, n_segments, n_tokens, true);
    if (st != H3_OK) return st;
    {
        const void *vec[] = {q, k, v, g, o};
        const char *names[] = {"q", "k", "v", "g", "o"};
        for (int i = 0; i < 5; ++i)
            if ((st = check_aligned(vec[i], names[i], 0)) != H3_OK) return st;
        if ((st = check_aligned(lse, "lse", 0, 4)) != H3_OK) return st;
    }
    const uint64_t bytes = (uint64_t)n_tokens * n_heads * head_dim * 2;
    std::vector<Range> ins{range_of(q, bytes, "q", 0), range_of(k, bytes, "k", 0), range_of(v, bytes, "v", 0)};
    if (g) ins.push_back(range_of(g, bytes, "g", 0));
    std::vector<Range> outs{range_of(o, bytes, "o", 0)};
    if (lse) outs.push_back(range_of(lse, (uint64_t)n_tokens * n_heads * 4, "lse", 0));
    if ((st = check_alias(ins, outs)) != H3_OK) return st;

    // work list: segments longest first, each expanded to heads x query tiles
    std::vector<int> order(n_segments);
    for (int s = 0; s < n_segments; ++s) order[s] = s;
    std::stable_sort(order.begin(), order.end(),
                     [&](int x, int y) { return cu[x + 1] - cu[x] > cu[y + 1] - cu[y]; });
    h3::AttnArgs a;
    std::memset(&a, 0, sizeof a);
    a.q = q; a.k = k; a.v = v; a.g = g; a.o = o; a.lse = lse;
    a.n_heads = (uint32_t)n_heads;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.n_entries = n_segments;
    int64_t total = 0;
    double flops = 0.0;
    const int64_t block_m = h3::packed_attn_block_m();
    for (int e = 0; e < n_segments; ++e) {
        const int s = order[e];
        const int64_t len = cu[s + 1] - cu[s];
        a.wg_prefix[e] = (int32_t)total;
        a.seg_begin[e] = (int32_t)cu[s];
        a.seg_len[e] = (int32_t)len;
        total += ((len + block_m - 1) / block_m) * n_heads;
        flops += 4.0 * head_dim * n_heads * (double)len * (double)len;
    }
    a.wg_prefix[n_segments] = (int32_t)total;
    if (total > INT32_MAX) return fail(H3_ERR_UNSUPPORTED, "too many work tiles");
    H3_DEBUG_ONLY(debug_check_worklist(a.wg_prefix, a.seg_begin, a.seg_len, a.n_entries, n_tokens, n_heads, block_m,
                                       total, "attention work list"));
    (void)hipGetLastError();
    hipError_t e = h3::launch_packed_attn(a, (int)total, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(H3_ERR_HIP, "packed attention launch failed: %s", hipGetErrorString(e));
    if (info) {
        info->launches = 1;
        info->chunks = 1;
        info->grid_x = (int32_t)total;
        info->block_x = h3::kAttnThreads;
        info->bytes_read = (int64_t)(bytes * (g ? 4 : 3));
        info->bytes_written = (int64_t)bytes;
        info->max_launch_src_bytes = info->bytes_read;
        info->flops = flops;
        info->tiles = total;
    }
    return ok();
}

h3_status h3_packed_attn(const void *q, const void *k, const void *v, const void *g, void *o, int64_t n_tokens,
                         int32_t n_heads, int32_t head_dim, const int64_t *cu, int32_t n_segments, float scale,
                         void *stream, h3_plan_info *info) {
    return packed_attn_impl(q, k, v, g, o, nullptr, n_tokens, n_heads, head_dim, cu, n_segments, scale, stream, info);
}

h3_status h3_packed_attn_lse(const void *q, const void *k, const void *v, const void *g, void *o, float *lse,
                             int64_t n_tokens, int32_t n_heads, int32_t head_dim, const int64_t *cu,
                             int32_t n_segments, float scale, void *stream, h3_plan_info *info) {
    if (!lse) {
        clear_info(info);
        return fail(H3_ERR_ARG, "lse is NULL");
    }
    return packed_attn_impl(q, k, v, g, o, lse, n_tokens, n_heads, head_dim, cu, n_segments, scale, stream, info);
}

static int64_t bwd_delta_bytes(int64_t rows) { return ((rows * 4 + 255) / 256) * 256; }

int64_t h3_packed_attn_backward_workspace(int64_t n_tokens, int32_t n_heads, int32_t gated) {
    if (n_tokens < 1 || n_heads < 1) return 0;
    const int64_t rows = n_tokens * n_heads;
    return bwd_delta_bytes(rows) + (gated ? rows * H3_HEAD_DIM * 2 : 0);
}

}  // extern "C"

// ---- the scratch array of the no-allocation backward ------------------------
// One array per GPU that runs the library, held until the process ends.  Host
// code never uses the name below as an address: each device's address comes
// from hipGetSymbolAddress, taken once with that device current.
static __device__ __align__(256) unsigned char scratch[H3_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxScratchDevices];

// The current device's copy of `scratch` (looked up on the first call there).
h3_status scratch_of_current_device(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(H3_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(H3_ERR_UNSUPPORTED, "device %d: the no-allocation scratch serves devices 0..%d", dev,
                    kMaxScratchDevices - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(H3_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return H3_OK;
}

// The attention backward with a caller workspace, or (use_scratch) with the
// current device's scratch array in its place.  Every argument check runs
// before the scratch address is looked up or anything is enqueued.
h3_status attn_backward_impl(const void *q, const void *k, const void *v, const void *g, const void *o,
                             const void *dout, const float *lse, void *dq, void *dk, void *dv, void *dg,
                             void *workspace, int64_t workspace_bytes, bool use_scratch, int64_t n_tokens,
                             int32_t n_heads, int32_t head_dim, const int64_t *cu, int32_t n_segments, float scale,
                             void *stream, h3_plan_info *info) {
    clear_info(info);
    if (!q || !k || !v || !o || !dout || !lse) return fail(H3_ERR_ARG, "q, k, v, o, dout and lse must be non-NULL");
    if (!dq || !dk || !dv) return fail(H3_ERR_ARG, "dq, dk and dv must be non-NULL");
    if ((g == nullptr) != (dg == nullptr)) return fail(H3_ERR_ARG, "dg must be given exactly when g is");
    if (!use_scratch && !workspace) return fail(H3_ERR_ARG, "workspace is NULL");
    if (n_tokens < 1) return fail(H3_ERR_EMPTY_PARTITION, "n_tokens = %lld: no tokens", (long long)n_tokens);
    if (n_tokens > INT32_MAX) return fail(H3_ERR_UNSUPPORTED, "n_tokens = %lld exceeds 2^31-1", (long long)n_tokens);
    if (n_heads < 1 || n_heads > H3_MAX_HEADS)
        return fail(H3_ERR_EMPTY_PARTITION, "n_heads = %d; legal values are 1..%d", n_heads, H3_MAX_HEADS);
    if (head_dim != H3_HEAD_DIM)
        return fail(H3_ERR_UNSUPPORTED, "head_dim = %d; only %d is supported", head_dim, H3_HEAD_DIM);
    if (!(scale > 0.f) || scale != scale || scale > 1e30f)
        return fail(H3_ERR_ARG, "scale must be a positive finite number");
    h3_status st = check_segments(cu, n_segments, n_tokens, true);
    if (st != H3_OK) return st;
    {
        const void *vec[] = {q, k, v, g, o, dout, dq, dk, dv, dg, workspace};
        const char *names[] = {"q", "k", "v", "g", "o", "dout", "dq", "dk", "dv", "dg", "workspace"};
        for (int i = 0; i < 11; ++i)
            if ((st = check_aligned(vec[i], names[i], 0)) != H3_OK) return st;
        if ((st = check_aligned(lse, "lse", 0, 4)) != H3_OK) return st;
    }
    const int64_t rows = n_tokens * n_heads;
    if ((uint64_t)rows > UINT32_MAX) return fail(H3_ERR_UNSUPPORTED, "n_tokens * n_heads exceeds 2^32-1");
    const int64_t need = h3_packed_attn_backward_workspace(n_tokens, n_heads, g != nullptr);
    if (use_scratch && need > (int64_t)H3_NOALLOC_SCRATCH_BYTES)
        return fail(H3_ERR_UNSUPPORTED, "%lld tokens x %d heads need %lld bytes of scratch; the no-allocation "
                    "variant holds %lld (use h3_packed_attn_backward with a workspace)", (long long)n_tokens,
                    n_heads, (long long)need, (long long)H3_NOALLOC_SCRATCH_BYTES);
    if (!use_scratch && workspace_bytes < need)
        return fail(H3_ERR_ARG, "workspace of %lld bytes is too small: %lld needed", (long long)workspace_bytes,
                    (long long)need);
    const uint64_t bytes = (uint64_t)rows * head_dim * 2;
    std::vector<Range> ins{range_of(q, bytes, "q", 0), range_of(k, bytes, "k", 0), range_of(v, bytes, "v", 0),
                           range_of(o, bytes, "o", 0), range_of(dout, bytes, "dout", 0),
                           range_of(lse, (uint64_t)rows * 4, "lse", 0)};
    if (g) ins.push_back(range_of(g, bytes, "g", 0));
    std::vector<Range> outs{range_of(dq, bytes, "dq", 0), range_of(dk, bytes, "dk", 0), range_of(dv, bytes, "dv", 0)};
    if (!use_scratch) outs.push_back(range_of(workspace, (uint64_t)need, "workspace", 0));
    if (dg) outs.push_back(range_of(dg, bytes, "dg", 0));
    if ((st = check_alias(ins, outs)) != H3_OK) return st;

    std::vector<int> order(n_segments);
    for (int s = 0; s < n_segments; ++s) order[s] = s;
    std::stable_sort(order.begin(), order.end(),
                     [&](int x, int y) { return cu[x + 1] - cu[x] > cu[y + 1] - cu[y]; });
    h3::AttnBwdArgs a;
    std::memset(&a, 0, sizeof a);
    a.q = q; a.k = k; a.v = v; a.g = g; a.o = o; a.dout = dout; a.lse = lse;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg;
    a.n_heads = (uint32_t)n_heads;
    a.n_rows = (uint32_t)rows;
    a.scale = scale;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.n_entries = n_segments;
    h3::AttnBwdArgs akv = a;                          // same arguments, work list over key blocks
    int64_t total_q = 0, total_kv = 0;
    double pairs = 0.0;
    const int64_t kv_block = h3::attn_bwd_key_block();
    for (int e = 0; e < n_segments; ++e) {
        const int s = order[e];
        const int64_t len = cu[s + 1] - cu[s];
        a.wg_prefix[e] = (int32_t)total_q;
        akv.wg_prefix[e] = (int32_t)total_kv;
        a.seg_begin[e] = akv.seg_begin[e] = (int32_t)cu[s];
        a.seg_len[e] = akv.seg_len[e] = (int32_t)len;
        total_q += ((len + h3::kBwdQBlock - 1) / h3::kBwdQBlock) * n_heads;
        total_kv += ((len + kv_block - 1) / kv_block) * n_heads;
        pairs += (double)n_heads * (double)len * (double)len;
    }
    a.wg_prefix[n_segments] = (int32_t)total_q;
    akv.wg_prefix[n_segments] = (int32_t)total_kv;
    if (total_q > INT32_MAX || total_kv > INT32_MAX) return fail(H3_ERR_UNSUPPORTED, "too many work tiles");

    // the scratch: fp32 row terms D first, then (gated) e = dout * sig(g) at a 256-byte boundary
    if (use_scratch && (st = scratch_of_current_device(&workspace)) != H3_OK) return st;
    a.delta = akv.delta = static_cast<float *>(workspace);
    a.e = akv.e = g ? static_cast<void *>(static_cast<char *>(workspace) + bwd_delta_bytes(rows))
                    : const_cast<void *>(dout);

    H3_DEBUG_ONLY(debug_check_worklist(a.wg_prefix, a.seg_begin, a.seg_len, a.n_entries, n_tokens, n_heads,
                                       h3::kBwdQBlock, total_q, "attention backward query work list"));
    H3_DEBUG_ONLY(debug_check_worklist(akv.wg_prefix, akv.seg_begin, akv.seg_len, akv.n_entries, n_tokens, n_heads,
                                       kv_block, total_kv, "attention backward key work list"));
    H3_DEBUG_ONLY(H3_DEBUG_CHECK((int64_t)a.n_rows == rows && akv.n_rows == a.n_rows, "attention backward rows"));
    H3_DEBUG_ONLY(H3_DEBUG_CHECK(a.delta != nullptr && a.e != nullptr && akv.delta == a.delta && akv.e == a.e,
                                 "attention backward scratch"));
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    int gx_pre = 0;
    hipError_t e = h3::launch_attn_bwd_pre(a, s, &gx_pre);
    if (e != hipSuccess) return fail(H3_ERR_HIP, "attention backward row-term launch failed: %s", hipGetErrorString(e));
    e = h3::launch_attn_bwd_dkdv(akv, (int)total_kv, s);
    if (e != hipSuccess) return fail(H3_ERR_HIP, "attention backward dk/dv launch failed: %s", hipGetErrorString(e));
    e = h3::launch_attn_bwd_dq(a, (int)total_q, s);
    if (e != hipSuccess) return fail(H3_ERR_HIP, "attention backward dq launch failed: %s", hipGetErrorString(e));
    if (info) {
        info->launches = 3;
        info->chunks = 1;
        info->grid_x = (int32_t)std::max<int64_t>(std::max<int64_t>(gx_pre, total_kv), total_q);
        info->block_x = h3::kBwdThreads;
        info->tiles = total_q + total_kv;
        // algorithmic work: the five products S, dP, dV, dK, dQ of every same-segment (query, key) pair
        info->flops = 10.0 * head_dim * pairs;
        info->bytes_read = (int64_t)(bytes * (g ? 7 : 6) + (uint64_t)rows * 4);
        info->bytes_written = (int64_t)(bytes * (g ? 4 : 3));
    }
    return ok();
}

}  // namespace

extern "C" {

h3_status h3_packed_attn_backward(const void *q, const void *k, const void *v, const void *g, const void *o,
                                  const void *dout, const float *lse, void *dq, void *dk, void *dv, void *dg,
                                  void *workspace, int64_t workspace_bytes, int64_t n_tokens, int32_t n_heads,
                                  int32_t head_dim, const int64_t *cu, int32_t n_segments, float scale, void *stream,
                                  h3_plan_info *info) {
    return attn_backward_impl(q, k, v, g, o, dout, lse, dq, dk, dv, dg, workspace, workspace_bytes, false, n_tokens,
                              n_heads, head_dim, cu, n_segments, scale, stream, info);
}

h3_status h3_packed_attn_backward_noalloc(const void *q, const void *k, const void *v, const void *g, const void *o,
                                          const void *dout, const float *lse, void *dq, void *dk, void *dv,
                                          void *dg, int64_t n_tokens, int32_t n_heads, int32_t head_dim,
                                          const int64_t *cu, int32_t n_segments, float scale, void *stream,
                                          h3_plan_info *info) {
    return attn_backward_impl(q, k, v, g, o, dout, lse, dq, dk, dv, dg, nullptr, 0, true, n_tokens, n_heads,
                              head_dim, cu, n_segments, scale, stream, info);
}

// Shared checks of the ragged collectives: token split, channels, index range.
static h3_status check_ragged(int64_t n_tokens, int32_t channels, int32_t world) {
    if (n_tokens < 1) return fail(H3_ERR_EMPTY_PARTITION, "n_tokens = %lld: no rows to split", (long long)n_tokens);
    if (world < 1 || world > n_tokens)
        return fail(H3_ERR_EMPTY_PARTITION, "world = %d would leave a rank without rows; legal values are 1..%lld",
                    world, (long long)n_tokens);
    if (world > h3::kMaxRanks)
        return fail(H3_ERR_UNSUPPORTED, "world = %d; at most %d ranks are supported", world, h3::kMaxRanks);
    if (channels < 8 || channels % 8 != 0 || channels > H3_MAX_CHANNELS)
        return fail(H3_ERR_UNSUPPORTED, "channels = %d; must be a multiple of 8 in 8..%d", channels,
                    H3_MAX_CHANNELS);
    int64_t b0, c0;
    split(n_tokens, world, 0, &b0, &c0);              // the largest rank
    if (c0 * (channels / 8) > INT32_MAX)
        return fail(H3_ERR_UNSUPPORTED, "a rank's %lld rows x %d channels exceed 2^31-1 16-byte vectors",
                    (long long)c0, channels);
    return H3_OK;
}

h3_status h3_reduce_scatter(const void *const *partials, const void *bias, void *const *out, int64_t n_tokens,
                            int32_t channels, int32_t world, int32_t rank, void *stream, h3_plan_info *info) {
    clear_info(info);
    h3_status st = check_ragged(n_tokens, channels, world);
    if (st != H3_OK) return st;
    if (!partials || !out) return fail(H3_ERR_ARG, "partials and out must be non-NULL arrays of %d pointers", world);
    if (rank < -1 || rank >= world)
        return fail(H3_ERR_ARG, "rank = %d; legal values are -1 (every rank) or 0..%d", rank, world - 1);
    const uint64_t row_bytes = (uint64_t)channels * 2;
    std::vector<Range> ins, outs;
    for (int j = 0; j < world; ++j) {
        if (!partials[j]) return fail(H3_ERR_ARG, "partials[%d] is NULL", j);
        if ((st = check_aligned(partials[j], "partials", j)) != H3_OK) return st;
        ins.push_back(range_of(partials[j], (uint64_t)n_tokens * row_bytes, "partials", j));
    }
    if (bias) {
        if ((st = check_aligned(bias, "bias", 0)) != H3_OK) return st;
        ins.push_back(range_of(bias, row_bytes, "bias", 0));
    }
    h3::RaggedArgs a;
    std::memset(&a, 0, sizeof a);
    int n_slots = 0;
    uint32_t max_vec = 0;
    int64_t rows_out = 0;
    for (int i = 0; i < world; ++i) {
        if (rank >= 0 && i != rank) continue;
        if (!out[i]) return fail(H3_ERR_ARG, "out[%d] is NULL but rank %d is selected", i, i);
        if ((st = check_aligned(out[i], "out", i)) != H3_OK) return st;
        int64_t begin, count;
        split(n_tokens, world, i, &begin, &count);
        outs.push_back(range_of(out[i], (uint64_t)count * row_bytes, "out", i));
        a.dst[n_slots] = out[i];
        a.row_vec0[n_slots] = (uint64_t)begin * (channels / 8);
        a.n_vec[n_slots] = (uint32_t)(count * (channels / 8));
        max_vec = std::max(max_vec, a.n_vec[n_slots]);
        rows_out += count;
        ++n_slots;
    }
    if ((st = check_alias(ins, outs)) != H3_OK) return st;
    for (int j = 0; j < world; ++j) a.src[j] = partials[j];
    a.bias = bias;
    a.nv_row = (uint32_t)(channels / 8);
    if (a.nv_row >= 2) a.div_row = h3::make_fastdiv(a.nv_row);
    a.world = world;
    H3_DEBUG_ONLY(debug_check_ragged(a, n_slots, n_tokens));
    (void)hipGetLastError();
    int gx = 0;
    hipError_t e = h3::launch_reduce_scatter(a, n_slots, max_vec, static_cast<hipStream_t>(stream), &gx);
    if (e != hipSuccess) return fail(H3_ERR_HIP, "reduce-scatter launch failed: %s", hipGetErrorString(e));
    if (info) {
        info->launches = 1;
        info->chunks = 1;
        info->grid_x = gx;
        info->block_x = h3::kCopyThreads;
        info->bytes_read = (int64_t)((uint64_t)world * rows_out * row_bytes + (bias ? row_bytes : 0));
        info->bytes_written = (int64_t)(rows_out * row_bytes);
        info->max_launch_src_bytes = info->bytes_read;
        info->tiles = n_slots;
    }
    return ok();
}

h3_status h3_gather_rows(const void *const *shards, void *dst, int64_t n_tokens, int32_t channels, int32_t world,
                         void *stream, h3_plan_info *info) {
    clear_info(info);
    h3_status st = check_ragged(n_tokens, channels, world);
    if (st != H3_OK) return st;
    if (!shards || !dst) return fail(H3_ERR_ARG, "shards and dst must be non-NULL");
    if ((st = check_aligned(dst, "dst", 0)) != H3_OK) return st;
    const uint64_t row_bytes = (uint64_t)channels * 2;
    std::vector<Range> ins;
    h3::RaggedArgs a;
    std::memset(&a, 0, sizeof a);
    uint32_t max_vec = 0;
    for (int i = 0; i < world; ++i) {
        if (!shards[i]) return fail(H3_ERR_ARG, "shards[%d] is NULL", i);
        if ((st = check_aligned(shards[i], "shards", i)) != H3_OK) return st;
        int64_t begin, count;
        split(n_tokens, world, i, &begin, &count);
        ins.push_back(range_of(shards[i], (uint64_t)count * row_bytes, "shards", i));
        a.src[i] = shards[i];
        a.row_vec0[i] = (uint64_t)begin * (channels / 8);
        a.n_vec[i] = (uint32_t)(count * (channels / 8));
        max_vec = std::max(max_vec, a.n_vec[i]);
    }
    if ((st = check_alias(ins, {range_of(dst, (uint64_t)n_tokens * row_bytes, "dst", 0)})) != H3_OK) return st;
    a.dst_all = dst;
    a.nv_row = (uint32_t)(channels / 8);
    a.world = world;
    H3_DEBUG_ONLY(debug_check_ragged(a, world, n_tokens));
    (void)hipGetLastError();
    int gx = 0;
    hipError_t e = h3::launch_gather_rows(a, world, max_vec, static_cast<hipStream_t>(stream), &gx);
    if (e != hipSuccess) return fail(H3_ERR_HIP, "row gather launch failed: %s", hipGetErrorString(e));
    if (info) {
        info->launches = 1;
        info->chunks = 1;
        info->grid_x = gx;
        info->block_x = h3::kCopyThreads;
        info->bytes_read = (int64_t)((uint64_t)n_tokens * row_bytes);
        info->bytes_written = info->bytes_read;
        info->max_launch_src_bytes = info->bytes_read;
        info->tiles = world;
    }
    return ok();
}

// The shared body of the AdaLN entry points (mode H3_ADALN_GATE_MODULATE takes
// every parameter row and writes resid as well as y).
static h3_status adaln_impl(int32_t mode, const void *x, const void *branch, const void *shift, const void *scale,
                            const void *gate, void *resid, void *y, int64_t tok_begin, int64_t tok_end,
                            int32_t channels, const int64_t *cu, int32_t n_segments, float eps, void *stream,
                            h3_plan_info *info) {
    clear_info(info);
    const bool modulate = mode != H3_ADALN_GATE_RESIDUAL, gated = mode != H3_ADALN_MODULATE;
    if (!x || !y) return fail(H3_ERR_ARG, "x and y must be non-NULL");
    if (mode == H3_ADALN_GATE_MODULATE && !resid) return fail(H3_ERR_ARG, "resid must be non-NULL");
    if (modulate && (!shift || !scale)) return fail(H3_ERR_ARG, "modulate needs shift and scale");
    if (gated && (!branch || !gate)) return fail(H3_ERR_ARG, "gate residual needs branch and gate");
    if (tok_begin < 0 || tok_end <= tok_begin)
        return fail(H3_ERR_EMPTY_PARTITION, "token interval [%lld, %lld) is empty", (long long)tok_begin,
                    (long long)tok_end);
    if (tok_end - tok_begin > INT32_MAX) return fail(H3_ERR_UNSUPPORTED, "token interval longer than 2^31-1");
    if (channels < 8 || channels % 8 != 0 || channels > H3_MAX_CHANNELS)
        return fail(H3_ERR_UNSUPPORTED, "channels = %d; must be a multiple of 8 in 8..%d", channels,
                    H3_MAX_CHANNELS);
    if (modulate && !(eps >= 0.f && eps < 1e30f)) return fail(H3_ERR_ARG, "eps must be a finite number >= 0");
    h3_status st = check_segments(cu, n_segments, tok_end, false);
    if (st != H3_OK) return st;
    {
        const void *vec[] = {x, branch, shift, scale, gate, resid, y};
        const char *names[] = {"x", "branch", "shift", "scale", "gate", "resid", "y"};
        for (int i = 0; i < 7; ++i)
            if ((st = check_aligned(vec[i], names[i], 0)) != H3_OK) return st;
    }

    const int64_t n_rows = tok_end - tok_begin;
    const uint64_t row_bytes = (uint64_t)channels * 2;
    const uint64_t par_bytes = (uint64_t)n_segments * row_bytes;
    std::vector<Range> ins{range_of(x, n_rows * row_bytes, "x", 0)};
    if (modulate) {
        ins.push_back(range_of(shift, par_bytes, "shift", 0));
        ins.push_back(range_of(scale, par_bytes, "scale", 0));
    }
    if (gated) {
        ins.push_back(range_of(branch, n_rows * row_bytes, "branch", 0));
        ins.push_back(range_of(gate, par_bytes, "gate", 0));
    }
    std::vector<Range> outs{range_of(y, n_rows * row_bytes, "y", 0)};
    if (mode == H3_ADALN_GATE_MODULATE) outs.push_back(range_of(resid, n_rows * row_bytes, "resid", 0));
    if ((st = check_alias(ins, outs)) != H3_OK) return st;

    h3::AdalnArgs a;
    std::memset(&a, 0, sizeof a);
    a.x = x; a.branch = branch; a.shift = shift; a.scale = scale; a.gate = gate; a.y = y;
    a.resid = mode == H3_ADALN_GATE_MODULATE ? resid : nullptr;
    a.n_rows = (uint32_t)n_rows;
    a.channels = (uint32_t)channels;
    a.eps = eps;
    a.mode = mode;
    // clip and rebase the global table to [tok_begin, tok_end)
    int n = 0;
    for (int32_t s = 0; s < n_segments; ++s) {
        const int64_t lo = std::max(cu[s], tok_begin), hi = std::min(cu[s + 1], tok_end);
        if (lo < hi) {
            a.entry_begin[n] = (int32_t)(lo - tok_begin);
            a.entry_seg[n] = s;
            ++n;
        }
    }
    a.entry_begin[n] = (int32_t)n_rows;
    a.n_entries = n;
    H3_DEBUG_ONLY(debug_check_adaln(a, n_segments));
    (void)hipGetLastError();
    int gx = 0;
    hipError_t e = h3::launch_adaln(a, static_cast<hipStream_t>(stream), &gx);
    if (e != hipSuccess) return fail(H3_ERR_HIP, "adaln launch failed: %s", hipGetErrorString(e));
    if (info) {
        info->launches = 1;
        info->chunks = 1;
        info->grid_x = gx;
        info->block_x = h3::kAdalnThreads;
        const uint64_t streams_in = gated ? 2 : 1, params = (modulate ? 2 : 0) + (gated ? 1 : 0);
        const uint64_t streams_out = mode == H3_ADALN_GATE_MODULATE ? 2 : 1;
        info->bytes_read = (int64_t)(streams_in * n_rows * row_bytes + params * (uint64_t)n * row_bytes);
        info->bytes_written = (int64_t)(streams_out * n_rows * row_bytes);
        info->max_launch_src_bytes = info->bytes_read;
        info->tiles = n;
    }
    return ok();
}

h3_status h3_adaln_segment(int32_t mode, const void *x, const void *branch, const void *shift, const void *scale,
                           const void *gate, void *y, int64_t tok_begin, int64_t tok_end, int32_t channels,
                           const int64_t *cu, int32_t n_segments, float eps, void *stream, h3_plan_info *info) {
    if (mode != H3_ADALN_MODULATE && mode != H3_ADALN_GATE_RESIDUAL) {
        clear_info(info);
        return fail(H3_ERR_ARG, "mode = %d; legal values are %d (modulate) and %d (gate residual)", mode,
                    H3_ADALN_MODULATE, H3_ADALN_GATE_RESIDUAL);
    }
    return adaln_impl(mode, x, branch, shift, scale, gate, nullptr, y, tok_begin, tok_end, channels, cu, n_segments,
                      eps, stream, info);
}

h3_status h3_adaln_gate_modulate(const void *x, const void *branch, const void *gate, const void *shift,
                                 const void *scale, void *resid, void *y, int64_t tok_begin, int64_t tok_end,
                                 int32_t channels, const int64_t *cu, int32_t n_segments, float eps, void *stream,
                                 h3_plan_info *info) {
    return adaln_impl(H3_ADALN_GATE_MODULATE, x, branch, shift, scale, gate, resid, y, tok_begin, tok_end, channels,
                      cu, n_segments, eps, stream, info);
}

}  // extern "C"
