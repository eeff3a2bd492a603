/*
 * h3.h -- C ABI of the MI355X (gfx950) Ulysses H3 hot-path library, libh3.so.
 *
 * The library implements, for ONE GPU, the data-parallel hot path of a
 * Ulysses sequence-parallel H3 denoiser block: the sequence-to-head relayout
 * of packed QKV/QKVG, segment-masked attention over the natively packed
 * multi-segment sequence, the inverse head-to-sequence relayout, and the
 * per-segment AdaLN modulation / residual gating on segment tables clipped to
 * a token interval.  Beside that forward path it provides the backward of
 * the relayouts and of the attention, the gated AdaLN chain (one sub-block's
 * residual gating fused with the next one's modulation), and the ragged
 * reduce-scatter and row gather of the token-sharded blocks.  The P ranks of
 * the sequence-parallel group are emulated by P "virtual-rank" buffers on the
 * one device; no collective is issued.
 *
 * Sources (by page title and section):
 *   [DIST]  "Distributed H3 Execution" -- introduction, Partition Contract,
 *           Validation.
 *   [PR]    "[perf] Harden Ulysses agreement and tune bounded H3 transfers"
 *           -- Problem and behavior, Implementation.
 *   [SPARK] "MiniMax H3 on NVIDIA DGX Spark (GB10)" -- Choosing the
 *           encoder-node count (only its error style: list the legal values).
 *
 * Conventions common to every entry point
 * ---------------------------------------
 * - Element type: every tensor is bfloat16, row-major, densely packed, except
 *   the attention's row log-sum-exp (fp32) and the backward's workspace
 *   (raw bytes).
 * - Pointers: "device" pointers are HIP device memory owned by the caller;
 *   "host" pointers are ordinary host memory read only during the call.
 *   The library never allocates, frees or synchronises (scratch space, where
 *   a kernel needs it, is a caller-owned workspace); work is enqueued on
 *   `stream` (a hipStream_t passed as void*, NULL = the default stream) and
 *   runs asynchronously.  Buffers must stay alive until that work completes.
 * - Alignment: every device pointer handed to an entry point starts on a
 *   16-byte boundary (the kernels move data in 16-byte vectors), except the
 *   fp32 row log-sum-exp, which needs 4 bytes.  A misaligned pointer is
 *   rejected with H3_ERR_ARG before anything is enqueued.  Whole allocations
 *   of the HIP runtime and of torch always qualify; a view at an element
 *   offset may not.
 * - Independent storage ([PR], Problem and behavior): no output may overlap
 *   an input or another output; overlap is detected on the host from the
 *   address ranges and rejected with H3_ERR_ALIAS.
 * - Validation first: every check runs on the host before anything is
 *   enqueued.  On any error nothing is launched, no state is kept, and the
 *   next valid call behaves as if the failed one never happened (the local
 *   form of [PR], Implementation: a declined call can recover on a later
 *   compatible call).  h3_last_error() returns a message for the calling
 *   thread's last failure.
 * - Empty partitions are rejected ([DIST], introduction): a split that would
 *   leave some rank without heads or tokens returns H3_ERR_EMPTY_PARTITION
 *   and the message lists the legal rank counts ([SPARK] style).
 * - h3_plan_info, when non-NULL, receives what was actually enqueued, so a
 *   caller can assert the execution plan and not just the numbers.
 * - Thread safety: all entry points are stateless and may be called from
 *   several threads; the per-thread error text is thread-local.
 */
#ifndef H3_H
#define H3_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum h3_status {
    H3_OK = 0,
    H3_ERR_ARG = 1,              /* NULL pointer, negative or inconsistent size, bad mode       */
    H3_ERR_EMPTY_PARTITION = 2,  /* P < 1, or P larger than the heads or tokens to split       */
    H3_ERR_SEGMENTS = 3,         /* segment table not 0 = cu[0] < ... < cu[S] = N, or S too big */
    H3_ERR_UNSUPPORTED = 4,      /* head_dim != 128, channels not a multiple of 8 or too large */
    H3_ERR_ALIAS = 5,            /* an output overlaps an input or another output              */
    H3_ERR_HIP = 6               /* the HIP runtime refused a launch                           */
} h3_status;

#define H3_HEAD_DIM 128          /* the only supported head width (56 heads of width 128, [DIST]) */
#define H3_MAX_SEGMENTS 256      /* largest segment table accepted                            */
#define H3_MAX_HEADS 256         /* largest head count accepted                               */
#define H3_MAX_CHANNELS 16384    /* largest AdaLN row width accepted                          */

/* The per-call relayout contract (cf. [PR], Implementation: the call contract
 * carries the chunking and launch size). */
typedef struct h3_layout {
    int64_t n_tokens;        /* N: packed tokens over all segments, >= 1                      */
    int32_t n_heads;         /* H: global heads (56 for H3), 1..H3_MAX_HEADS                  */
    int32_t head_dim;        /* D: must be H3_HEAD_DIM                                        */
    int32_t n_planes;        /* K: planes in the packed operand (3 = QKV, 4 = QKVG); 1 for
                                head2seq                                                      */
    int32_t world;           /* P: virtual ranks, 1 <= P <= min(H, N)                          */
    int32_t rank;            /* -1: every rank; 0..P-1: only that rank's share                */
    int32_t reserved;        /* must be 0                                                     */
    int64_t max_chunk_bytes; /* 0: one launch per plane; > 0: no launch reads more than
                                this many source bytes.  A launch moves, per token of one
                                plane, B = (selected heads)*D*2 bytes (H*D*2 for rank -1,
                                H_j*D*2 for rank j), so it covers floor(max_chunk_bytes / B)
                                tokens.  The 896,000,000-byte window of [PR] gives 62,500
                                tokens of a whole 56-head plane.  Below B: H3_ERR_ARG      */
} h3_layout;

typedef struct h3_plan_info {
    int32_t launches;        /* kernel launches enqueued by the call                          */
    int32_t chunks;          /* token chunks per plane (relayouts), 1 otherwise               */
    int32_t grid_x;          /* workgroups of the largest launch                              */
    int32_t block_x;         /* threads per workgroup                                         */
    int64_t chunk_tokens;    /* tokens per full chunk (relayouts)                             */
    int64_t max_launch_src_bytes; /* most source bytes read by one launch                     */
    int64_t bytes_read;      /* algorithmic bytes read by the whole call                      */
    int64_t bytes_written;   /* algorithmic bytes written by the whole call                   */
    double flops;            /* attention: algorithmic FLOPs (4*D per query-key pair per head) */
    int64_t tiles;           /* attention: query tiles x heads; AdaLN: clipped table entries   */
} h3_plan_info;

/* ------------------------------------------------------------------------
 * h3_seq2head -- sequence-to-head relayout, one plane at a time.
 *
 * [DIST] introduction: Ulysses mode wraps attention in a QKV sequence-to-head
 * all-to-all; [DIST] Partition Contract: rank j owns heads [hb_j, hb_j+H_j)
 * of the balanced quotient/remainder split (10,10,9,9,9,9 for 56 over 6) and
 * tokens [a_j, b_j) of the same split of N; [PR] Problem and behavior: one
 * batch plane at a time, bounded windows, outputs in storage of their own.
 *
 * src: device, [N][K][H][D], the packed operand (token-major, planes Q,K,V[,G]).
 * dst: host array of P*K device pointers; dst[j*K + p] is rank j's buffer of
 *      plane p, [N][H_j][D] (every token of rank j's heads, global token
 *      order -- what the all-to-all leaves on rank j).  When layout->rank = j
 *      only the K entries of rank j are read; the others may be NULL.
 * Effect: dst[j*K+p][t][h][:] = src[t][p][hb_j + h][:], bit for bit.
 * Launches: K * chunks (one per plane and token chunk), in plane order.
 * ------------------------------------------------------------------------ */
h3_status h3_seq2head(const h3_layout *layout, const void *src, void *const *dst,
                      void *stream, h3_plan_info *info);

/* ------------------------------------------------------------------------
 * h3_head2seq -- the inverse, head-to-sequence relayout ([DIST] introduction).
 *
 * src: host array of P device pointers; src[j] is rank j's [N][H_j][D] buffer
 *      (e.g. the attention output of its heads).  With layout->rank = j only
 *      src[j] is read.
 * dst: device, [N][H][D].  Effect: dst[t][hb_j + h][:] = src[j][t][h][:] for
 *      every selected rank j; heads of unselected ranks are left untouched.
 * layout->n_planes must be 1.  Launches: chunks (one per token chunk).
 * ------------------------------------------------------------------------ */
h3_status h3_head2seq(const h3_layout *layout, const void *const *src, void *dst,
                      void *stream, h3_plan_info *info);

/* ------------------------------------------------------------------------
 * h3_seq2head_backward -- the adjoint of h3_seq2head, for the backward pass
 * ([PR] Problem and behavior: backward reuses the plan its forward saved;
 * [PR] Review and validation: the native gate checks exact gradients).
 *
 * The relayout is a permutation, so its adjoint is the inverse copy:
 *   grad_src[t][p][hb_j + h][:] = grad_dst[j*K + p][t][h][:], bit for bit,
 * for every selected rank j and plane p.
 * layout: the forward call's layout, unchanged.  The call derives its chunk
 *      plan from it exactly as the forward does, so `info` reports the same
 *      launches, chunks, chunk_tokens, grid and block as the forward's.
 * grad_dst: host array of P*K device pointers, [N][H_j][D] each (the
 *      gradients of the forward's dst buffers); with layout->rank = j only
 *      the K entries of rank j are read and the others may be NULL.
 * grad_src: device, [N][K][H][D].  Heads of unselected ranks are left
 *      untouched (they belong to other ranks' shares).
 * Launches: K * chunks, in plane order.  Errors as h3_seq2head.
 * ------------------------------------------------------------------------ */
h3_status h3_seq2head_backward(const h3_layout *layout, const void *const *grad_dst, void *grad_src,
                               void *stream, h3_plan_info *info);

/* ------------------------------------------------------------------------
 * h3_head2seq_backward -- the adjoint of h3_head2seq (same passages):
 *   grad_src[j][t][h][:] = grad_dst[t][hb_j + h][:] for every selected rank j.
 * layout: the forward call's layout (n_planes = 1); the chunk plan and the
 *      reported info equal the forward's.
 * grad_dst: device, [N][H][D].  grad_src: host array of P device pointers,
 *      [N][H_j][D] each; with layout->rank = j only grad_src[j] is written.
 * Launches: chunks.  Errors as h3_head2seq.
 * ------------------------------------------------------------------------ */
h3_status h3_head2seq_backward(const h3_layout *layout, const void *grad_dst, void *const *grad_src,
                               void *stream, h3_plan_info *info);

/* ------------------------------------------------------------------------
 * h3_packed_attn -- segment-masked attention over the packed sequence, for
 * the heads one rank holds after seq2head ([DIST] introduction: attention on
 * the whole native packed sequence, no semantic padding).
 *
 * For every head h and token t in segment s = [cu[s], cu[s+1]):
 *   o[t,h,:] = sum_{u in s} softmax_u(scale * <q[t,h,:], k[u,h,:]>) v[u,h,:]
 * and, when g != NULL (QKVG, [PR] Problem and behavior), o[t,h,:] *= 1/(1+exp(-g[t,h,:])).
 * Tokens never attend across a segment boundary; no work is spent on the
 * cross-segment blocks.  bf16 inputs, fp32 accumulation, bf16 output
 * (round to nearest even).
 *
 * q, k, v, g, o: device, [N][n_heads][D] each (g may be NULL).
 * cu_seqlens: host, S+1 int64 offsets, 0 = cu[0] < cu[1] < ... < cu[S] = N,
 *             1 <= S <= H3_MAX_SEGMENTS.
 * scale: logit scale (1/sqrt(128) for H3).  Launches: 1.
 * ------------------------------------------------------------------------ */
h3_status h3_packed_attn(const void *q, const void *k, const void *v, const void *g, void *o,
                         int64_t n_tokens, int32_t n_heads, int32_t head_dim,
                         const int64_t *cu_seqlens, int32_t n_segments, float scale,
                         void *stream, h3_plan_info *info);

/* ------------------------------------------------------------------------
 * h3_packed_attn_lse -- h3_packed_attn that also writes the per-row
 * log-sum-exp the backward pass needs (same passages; training forward).
 *
 * lse: device, fp32 [N][H] (N = n_tokens, H = n_heads), written for every
 *      token and head: lse[t,h] = ln sum_{u in seg(t)} exp(scale * <q[t,h,:], k[u,h,:]>),
 *      the normaliser of the softmax before the gate.  Must not overlap any
 *      other buffer.  NULL is rejected (use h3_packed_attn).
 * Everything else, including o, launches and errors, as h3_packed_attn.
 * ------------------------------------------------------------------------ */
h3_status h3_packed_attn_lse(const void *q, const void *k, const void *v, const void *g, void *o, float *lse,
                             int64_t n_tokens, int32_t n_heads, int32_t head_dim,
                             const int64_t *cu_seqlens, int32_t n_segments, float scale,
                             void *stream, h3_plan_info *info);

/* ------------------------------------------------------------------------
 * h3_packed_attn_backward -- gradients of h3_packed_attn for the backward
 * pass (the forward's passages; the chain rule of softmax attention with the
 * optional sigmoid gate).  With p = softmax over the query's own segment of
 * scale*<q,k>, a = sum p v, o = a * sig(g) and the incoming gradient do:
 *   e   = do * sig(g)                      dg = do * o * (1 - sig(g))
 *   D   = <do, o>  (= <e, a>)              ds = p * (<e, v> - D)
 *   dq  = scale * sum_u ds k_u             dk = scale * sum_t ds q_t
 *   dv  = sum_t p e_t
 * (sig = 1 and no dg when g is NULL).  Cross-segment blocks are skipped as in
 * the forward.
 *
 * q, k, v, g, o, dout: device, bf16 [N][H][128]; o is the forward output.
 * lse: device, fp32 [N][H], from h3_packed_attn_lse of the same inputs.
 * dq, dk, dv: device, bf16 [N][H][128], written for every token.
 * dg: device, bf16 [N][H][128]; required iff g != NULL.
 * workspace: device scratch of at least h3_packed_attn_backward_workspace()
 *      bytes, owned by the caller (the library allocates nothing); its
 *      contents on entry do not matter and on return are unspecified.
 * Outputs must not overlap inputs, the workspace or each other.
 * Launches: 3 (row terms e, D, dg; then dk/dv; then dq).
 * ------------------------------------------------------------------------ */
int64_t h3_packed_attn_backward_workspace(int64_t n_tokens, int32_t n_heads, int32_t gated);

h3_status h3_packed_attn_backward(const void *q, const void *k, const void *v, const void *g,
                                  const void *o, const void *dout, const float *lse,
                                  void *dq, void *dk, void *dv, void *dg,
                                  void *workspace, int64_t workspace_bytes,
                                  int64_t n_tokens, int32_t n_heads, int32_t head_dim,
                                  const int64_t *cu_seqlens, int32_t n_segments, float scale,
                                  void *stream, h3_plan_info *info);

/* ------------------------------------------------------------------------
 * h3_packed_attn_backward_noalloc -- h3_packed_attn_backward for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  It takes no workspace; its
 * scratch (the row terms D and, gated, e = dout * sig(g)) lives in a
 * library-owned device array of H3_NOALLOC_SCRATCH_BYTES bytes, one per GPU
 * the library runs on, created with the code object and held until the
 * process ends.  The call allocates and frees nothing.
 *
 * Arguments, results (bit for bit those of h3_packed_attn_backward on the
 * same inputs), launches and errors as h3_packed_attn_backward, minus the
 * workspace.  Scratch needed, h3_packed_attn_backward_workspace(N, H,
 * g != NULL), above H3_NOALLOC_SCRATCH_BYTES is rejected with
 * H3_ERR_UNSUPPORTED before anything is enqueued (64 MiB: e.g. 8192 tokens
 * x 28 heads gated, or any ungated size up to 16M token-head rows).
 * The array's contents are unspecified on entry and nothing in it has to
 * start at zero.  Every call on one GPU uses that GPU's one array: two
 * calls whose work may overlap in time on the same GPU (different streams,
 * or threads without ordering) race on it and give undefined results;
 * calls ordered on one stream are safe.  The stream must belong to the
 * current device.
 * ------------------------------------------------------------------------ */
#define H3_NOALLOC_SCRATCH_BYTES (64ll << 20)
h3_status h3_packed_attn_backward_noalloc(const void *q, const void *k, const void *v, const void *g,
                                          const void *o, const void *dout, const float *lse,
                                          void *dq, void *dk, void *dv, void *dg,
                                          int64_t n_tokens, int32_t n_heads, int32_t head_dim,
                                          const int64_t *cu_seqlens, int32_t n_segments, float scale,
                                          void *stream, h3_plan_info *info);

/* ------------------------------------------------------------------------
 * h3_adaln_segment -- per-segment AdaLN on one rank's token interval.
 *
 * [DIST] Partition Contract (the segment table of a token-sharded rank):
 * local row i is global token tok_begin + i; every segment [cu[s], cu[s+1])
 * is intersected with [tok_begin, tok_end) and shifted by -tok_begin, and
 * row i takes the parameter row of its GLOBAL segment s.
 *   mode H3_ADALN_MODULATE:      y = (x - mean)/sqrt(var + eps) * (1 + scale[s]) + shift[s]
 *                                 (mean and biased var over the C channels, fp32)
 *   mode H3_ADALN_GATE_RESIDUAL: y = x + gate[s] * branch
 *
 * x, branch, y: device, [tok_end - tok_begin][C].  branch only for GATE.
 * shift, scale (MODULATE) / gate (GATE): device, [S][C].
 * cu_seqlens: host, the GLOBAL table (S+1 offsets, cu[S] >= tok_end).
 * channels: C, a multiple of 8, <= H3_MAX_CHANNELS.  Launches: 1.
 * ------------------------------------------------------------------------ */
#define H3_ADALN_MODULATE 0
#define H3_ADALN_GATE_RESIDUAL 1
h3_status h3_adaln_segment(int32_t mode, const void *x, const void *branch, const void *shift,
                           const void *scale, const void *gate, void *y,
                           int64_t tok_begin, int64_t tok_end, int32_t channels,
                           const int64_t *cu_seqlens, int32_t n_segments, float eps,
                           void *stream, h3_plan_info *info);

/* ------------------------------------------------------------------------
 * h3_adaln_gate_modulate -- one sub-block's gated residual followed by the
 * next sub-block's modulation, in one pass over the rows.
 *
 * [DIST] Partition Contract: the clipped, rebased segment table serves both
 * AdaLN modulation and residual gating; here the two are chained as a DiT
 * block chains them.  For local row i of global segment s, with
 * r = x + gate[s] * branch in fp32:
 *   resid = r rounded to bf16 (stored; the same bits as
 *           h3_adaln_segment(GATE_RESIDUAL))
 *   y     = (r - mean)/sqrt(var + eps) * (1 + scale[s]) + shift[s]
 *           (mean and biased var over the C channels of the fp32 r)
 * x and branch are read once and resid is never read back (4 row streams
 * instead of the unfused 5).  y normalises the unrounded r, so it is one
 * rounding closer to the exact chain than MODULATE applied to the stored
 * resid, and may differ from that in the last bits (it equals it when r is
 * exactly representable, e.g. for a zero gate).
 *
 * x, branch, resid, y: device, [tok_end - tok_begin][C] bf16.
 * gate (this sub-block), shift, scale (the next sub-block): device, [S][C].
 * resid and y must not overlap each other or any input.
 * cu_seqlens, channels, eps, errors: as h3_adaln_segment.  Launches: 1.
 * ------------------------------------------------------------------------ */
#define H3_ADALN_GATE_MODULATE 2
h3_status h3_adaln_gate_modulate(const void *x, const void *branch, const void *gate,
                                 const void *shift, const void *scale, void *resid, void *y,
                                 int64_t tok_begin, int64_t tok_end, int32_t channels,
                                 const int64_t *cu_seqlens, int32_t n_segments, float eps,
                                 void *stream, h3_plan_info *info);

/* ------------------------------------------------------------------------
 * h3_reduce_scatter -- ragged reduce-scatter of per-rank partial outputs with
 * the bias added once, the P ranks held as separate buffers on one device.
 *
 * [DIST] Partition Contract (tensor mode): each rank's partial output covers
 * every token row; the reduce-scatter sums the partials and assigns each
 * rank the rows of its token interval (h3_partition of n_tokens); the
 * projection bias, left out of the partials, is added exactly once after
 * the reduction.  For selected rank i and its rows [a_i, a_i + N_i):
 *   out[i][t - a_i][c] = bf16( (sum over j = 0..P-1 of partials[j][t][c]) + bias[c] )
 * summed in fp32 in rank order, rounded once.
 *
 * partials: host array of P device pointers, each [n_tokens][C] bf16.
 * bias: device [C] bf16, or NULL for none.
 * out: host array of P device pointers; out[i] is [N_i][C] bf16, written
 *      iff rank i is selected (rank == -1: every rank; else only `rank`),
 *      and may be NULL otherwise.  Outputs must not overlap any input or
 *      each other.
 * world: P, 1..min(n_tokens, 64) (an empty part is H3_ERR_EMPTY_PARTITION).
 * channels: C, a multiple of 8, <= H3_MAX_CHANNELS.  Launches: 1.
 * ------------------------------------------------------------------------ */
h3_status h3_reduce_scatter(const void *const *partials, const void *bias, void *const *out,
                            int64_t n_tokens, int32_t channels, int32_t world, int32_t rank,
                            void *stream, h3_plan_info *info);

/* ------------------------------------------------------------------------
 * h3_gather_rows -- ragged row gather with the collective's padding removed.
 *
 * [DIST] introduction: a ragged row gather pads the token shards to one size
 * for the collective, and that temporary padding is removed before any
 * model operation.  Rank i's N_i rows (h3_partition of n_tokens) are placed
 * at their global rows [a_i, a_i + N_i) of dst:
 *   dst[a_i + r][c] = shards[i][r][c],  r < N_i
 * so rows a padded buffer holds past N_i are never read.  For a padded
 * gathered buffer [P][M][C] pass shards[i] = buffer + i*M*C.
 *
 * shards: host array of P device pointers, shards[i] holding >= N_i rows of
 *      C bf16.  dst: device [n_tokens][C] bf16, not overlapping the shards'
 *      first N_i rows.
 * world, channels, alignment and errors as h3_reduce_scatter.  Launches: 1.
 * ------------------------------------------------------------------------ */
h3_status h3_gather_rows(const void *const *shards, void *dst, int64_t n_tokens, int32_t channels,
                         int32_t world, void *stream, h3_plan_info *info);

/* ------------------------------------------------------------------------
 * Host-only helpers (no device work, callable without a GPU).
 * ------------------------------------------------------------------------ */

/* [DIST] Partition Contract: part `index` of `total` items split over
 * `parts` ranks, first (total mod parts) ranks one larger.  Writes its first
 * item and size.  H3_ERR_EMPTY_PARTITION if parts < 1 or parts > total. */
h3_status h3_partition(int64_t total, int32_t parts, int32_t index, int64_t *begin, int64_t *count);

/* [DIST] Partition Contract: clip the global table cu[0..S] to [a, b) and
 * rebase.  Writes up to S entries (global segment id, local begin, local
 * end) of the non-empty pieces, in order.  Returns the entry count, or -1 if
 * the table or the interval is invalid.  Output arrays may be NULL to count. */
int32_t h3_clip_segments(const int64_t *cu, int32_t n_segments, int64_t a, int64_t b,
                         int32_t *seg_id, int64_t *local_begin, int64_t *local_end);

/* Static text for a status code. */
const char *h3_status_string(h3_status status);

/* Message of the calling thread's last failed call ("" if none). */
const char *h3_last_error(void);

/* Library version, "major.minor.patch". */
const char *h3_version(void);

#ifdef __cplusplus
}
#endif

#endif /* H3_H */
