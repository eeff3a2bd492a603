// h3_internal.h -- launch descriptors shared between the host contract
// (h3_api.hip) and the kernel translation units.  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "h3.h"

namespace h3 {

constexpr int kMaxRanks = 64;           // P <= min(H, N) and H <= 256, but buffers past 64 are not useful
constexpr int kMaxSegments = H3_MAX_SEGMENTS;

// Unsigned division of n < 2^31 by a runtime-uniform d >= 2 with one
// multiply-high and one correction step (m = ceil(2^32 / d) overestimates
// 1/d by less than 2^-32, so the high word is the quotient or one more).
struct FastDiv {
    uint32_t d;
    uint32_t m;
};

inline FastDiv make_fastdiv(uint32_t d) {
    FastDiv f;
    f.d = d;
    f.m = (uint32_t)(((1ull << 32) + d - 1) / d);
    return f;
}

// ---------------------------------------------------------------------------
// Relayout: copy of contiguous runs between a "packed" side, where rank j's
// run of token t starts at t*stride + off_j (in 16-byte vectors), and a
// "rank" side, where rank j's buffer is dense [tokens][run_j].
// ---------------------------------------------------------------------------
struct RunCopyArgs {
    const void *src_packed;          // seq2head: packed source (plane and chunk offset applied)
    void *dst_packed;                // head2seq: packed destination (chunk offset applied)
    const void *src_rank[kMaxRanks]; // head2seq: per selected rank (chunk offset applied)
    void *dst_rank[kMaxRanks];       // seq2head: per selected rank (chunk offset applied)
    uint32_t run_vec[kMaxRanks];     // H_j * D / 8 vectors per token
    uint32_t off_vec[kMaxRanks];     // hb_j * D / 8
    FastDiv div[kMaxRanks];          // division by run_vec[j]
    uint32_t stride_vec;             // packed-side token stride in vectors (K*H*D/8 or H*D/8)
    uint32_t n_tokens;               // tokens in this launch
    int32_t rank0;                   // rank of grid row y = 0
};

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 8;       // 16-byte vectors in flight per thread

hipError_t launch_seq2head(const RunCopyArgs &a, int n_ranks, uint32_t max_run, hipStream_t s,
                           int *grid_x);
hipError_t launch_head2seq(const RunCopyArgs &a, int n_ranks, uint32_t max_run, hipStream_t s,
                           int *grid_x);

// ---------------------------------------------------------------------------
// Ragged collectives of the token-sharded blocks (reduce-scatter, row gather).
// Grid row y serves rank slot y: its rows are the contiguous vectors
// [row_vec0[y], row_vec0[y] + n_vec[y]) of every [N][C] buffer.
// ---------------------------------------------------------------------------
struct RaggedArgs {
    const void *src[kMaxRanks];      // reduce-scatter: partial of rank j (all N rows); gather: shard of slot y
    void *dst[kMaxRanks];            // reduce-scatter: output rows of slot y
    void *dst_all;                   // gather: the [N][C] result
    const void *bias;                // reduce-scatter: [C] or NULL
    uint64_t row_vec0[kMaxRanks];    // a_i * C / 8 of slot y's rank
    uint32_t n_vec[kMaxRanks];       // N_i * C / 8 of slot y's rank (< 2^31)
    FastDiv div_row;                 // division by nv_row (nv_row >= 2)
    uint32_t nv_row;                 // C / 8
    int32_t world;                   // reduce-scatter: partials summed
};

constexpr int kRsVec = 4;            // reduce-scatter: 16-byte output vectors per thread

hipError_t launch_reduce_scatter(const RaggedArgs &a, int n_slots, uint32_t max_vec, hipStream_t s, int *grid_x);
hipError_t launch_gather_rows(const RaggedArgs &a, int n_slots, uint32_t max_vec, hipStream_t s, int *grid_x);

// ---------------------------------------------------------------------------
// AdaLN on one token interval, with the clipped and rebased segment table.
// ---------------------------------------------------------------------------
struct AdalnArgs {
    const void *x;
    const void *branch;
    const void *shift;
    const void *scale;
    const void *gate;
    void *y;
    void *resid;                             // gated chain: the stored residual x + gate * b
    uint32_t n_rows;
    uint32_t channels;
    float eps;
    int32_t mode;
    int32_t n_entries;
    int32_t entry_begin[kMaxSegments + 1];   // local first row of entry e; [n_entries] = n_rows
    int32_t entry_seg[kMaxSegments];         // global segment id of entry e
};

constexpr int kAdalnThreads = 256;           // 4 waves, one row per wave

hipError_t launch_adaln(const AdalnArgs &a, hipStream_t s, int *grid_x);

// ---------------------------------------------------------------------------
// Segment-masked attention.  The work list is sorted longest segment first;
// workgroup w belongs to the sorted segment e with wg_prefix[e] <= w <
// wg_prefix[e+1], and within it to (head, query tile) with the tile fastest.
// ---------------------------------------------------------------------------
struct AttnArgs {
    const void *q;
    const void *k;
    const void *v;
    const void *g;          // may be null
    void *o;
    float *lse;             // may be null: natural-log log-sum-exp of the scaled logits, [N][n_heads]
    uint32_t n_heads;       // heads in the buffers (row stride = n_heads * 128)
    float scale_log2;       // scale * log2(e)
    int32_t n_entries;
    int32_t wg_prefix[kMaxSegments + 1];
    int32_t seg_begin[kMaxSegments];
    int32_t seg_len[kMaxSegments];     // query tiles of entry e: ceil(seg_len / packed_attn_block_m())
};

constexpr int kAttnThreads = 512;      // 8 waves

// Query rows one attention workgroup covers (the kernel's tile height); the
// host sizes the work list with it.
int packed_attn_block_m();
hipError_t launch_packed_attn(const AttnArgs &a, int n_workgroups, hipStream_t s);

// ---- attention backward ------------------------------------------------------
constexpr int kBwdQBlock = 256;       // queries per workgroup of the dq kernel (8 waves x 32)
constexpr int kBwdThreads = 512;
constexpr int kBwdPreRowsPerWg = 16;  // (token, head) rows per workgroup of the row-term kernel

struct AttnBwdArgs {
    const void *q, *k, *v, *g, *o, *dout;
    const float *lse;       // natural log, [N][H]
    void *dq, *dk, *dv, *dg;
    void *e;                // bf16 [N][H][128]: dout * sig(g) in the workspace, or dout itself when ungated
    float *delta;           // fp32 [N][H] in the workspace
    uint32_t n_heads;
    uint32_t n_rows;        // N * H
    float scale;
    float scale_log2;       // scale * log2(e)
    int32_t n_entries;
    int32_t wg_prefix[kMaxSegments + 1];
    int32_t seg_begin[kMaxSegments];
    int32_t seg_len[kMaxSegments];
};

// Keys one dk/dv workgroup covers; the host sizes that kernel's work list with it.
int attn_bwd_key_block();
hipError_t launch_attn_bwd_pre(const AttnBwdArgs &a, hipStream_t s, int *grid_x);
hipError_t launch_attn_bwd_dkdv(const AttnBwdArgs &a, int n_workgroups, hipStream_t s);
hipError_t launch_attn_bwd_dq(const AttnBwdArgs &a, int n_workgroups, hipStream_t s);

}  // namespace h3
