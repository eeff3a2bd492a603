// attn_backward.hip -- gradients of the segment-masked packed attention
// (packed_attn.hip) and of its sigmoid gate, for the backward pass.
//
// The forward's passages ("Distributed H3 Execution", introduction: attention
// over the native packed sequence; "[perf] Harden Ulysses agreement and tune
// bounded H3 transfers", Problem and behavior: QKV/QKVG operands) define the
// function; its gradient is the chain rule of softmax attention.  With
// p_tu = exp(scale*<q_t,k_u> - lse_t) over the keys of t's segment,
// a_t = sum_u p_tu v_u, o_t = a_t * sig(g_t) and the incoming gradient do_t:
//   e_t = do_t * sig(g_t),  dg_t = do_t * o_t * (1 - sig(g_t)),  D_t = <do_t, o_t>,
//   ds_tu = p_tu (<e_t, v_u> - D_t),
//   dq_t = scale sum_u ds_tu k_u,  dk_u = scale sum_t ds_tu q_t,  dv_u = sum_t p_tu e_t.
//
// Three launches:
//   k_attn_bwd_pre   one 16-lane group per (token, head) row: e, dg and D.
//   k_attn_bwd_dkdv  one workgroup per (segment, head, 128-key block).
//                    Waves 0-3 own dK and waves 4-7 own dV of the 32-key
//                    block w%4 (one 64-register accumulator each; the two
//                    waves of a block share a SIMD).  The block's K and V
//                    pass once through LDS into registers (each wave keeps
//                    the operand it multiplies by: K for the dV wave, V for
//                    the dK wave).  64-query tiles of Q and e stream through
//                    LDS (buffer loads to LDS; Q triple, e double buffered),
//                    one barrier per tile.  With the keys as MFMA columns
//                    (lane = key), in tile t the dV wave forms S = Q K^T and
//                    P from it (lse per row from LDS), publishes P in bf16
//                    through LDS and adds e^T P; the dK wave forms
//                    dS = P (dP - D) of tile t-1 from the P published then
//                    and the dP - D it carried over the barrier, adds Q^T dS,
//                    and forms dP - D of tile t (the accumulator seeded with
//                    -D).  The transposing LDS load supplies e^T and Q^T.
//   k_attn_bwd_dq    the forward's structure with the roles of the operands
//                    reassigned: one workgroup per (segment, head, 256-query
//                    tile), lane = query.  Per 64-key tile: S^T = K Q^T and
//                    dP^T = V e^T (Q and e rows in registers), dS^T from them
//                    with the lane's own lse and D, dQ^T += K^T dS^T (K^T
//                    through the transposing LDS load).
// Rows past a segment's end are clamped to its last row on load; keys there
// are masked to -inf (dq kernel), queries there get lse = +inf so their p is 0
// (dk/dv kernel), and no output row past the end is written.
//
// MFMA layouts (v_mfma_f32_32x32x16_bf16) and the transposing read follow
// packed_attn.hip.  The streamed 64-row tiles (K and V in the dq kernel, Q and
// e in the dk/dv kernel) use a padded LDS layout instead of the forward's XOR
// swizzle: it is as free of bank conflicts, and because each chunk of a row
// sits at a constant distance from the row start, one lane base and immediate
// offsets address every read of a tile whichever buffer holds it, so the
// single tile body computes no addresses per tile.
#include "h3_device.h"

namespace h3 {

namespace {

constexpr int kBN = 64;                  // keys per tile (dq) / queries per tile (dk/dv)
constexpr int kWaves = kBwdThreads / 64; // 8
constexpr int kLoadsPerKBlock = kBwdKBlock / (4 * kWaves); // per 128-row key block
constexpr float kLog2e = 1.4426950408889634f;
static_assert(kBwdQBlock == 32 * kWaves, "one 32-query block per wave");
static_assert(kBwdKBlock == 32 * (kWaves / 2), "a dK wave and a dV wave per 32-key block");

__device__ __forceinline__ float sigmoid(float x) { return 1.0f / (1.0f + __builtin_amdgcn_exp2f(-x * kLog2e)); }

__device__ __forceinline__ bf16x8 lds_b128(const uint16_t *p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(p));
}

// Padded LDS layout of a 64-row tile, in 16-byte slots: row r = 4k + a starts
// at slot 77k + 20a and its 16 chunks follow in order.  The slot of (r, c) is
// then f(r) + c mod 16 with f(r) = 4a + 13k mod 16, so 16 rows of an aligned
// group read at one chunk, and the 4 rows x 4 chunks of a transposing read,
// each hit 16 distinct bank groups -- the XOR swizzle's property -- while
// every chunk of a lane's row is its row start plus a constant: all reads of
// a tile are one lane base and immediate offsets, whichever buffer the tile
// is in.  The layout spends 13 padding slots per 4 rows (1232 slots for 64
// rows), filled by 20 direct loads of 64 slots.
constexpr int kPadGroupSlots = 77;                      // 4 rows of 16 slots + 13 padding slots
constexpr int kPadRowSlots = 20;
constexpr int kPadTileLoads = 20;                       // 1 KB direct loads per tile (1280 slots)
constexpr int kPadTileElems = kPadTileLoads * 64 * 8;   // bf16 elements per tile buffer (20 KB)
constexpr int kPad4Rows = kPadGroupSlots * 8;           // elements between rows r and r + 4
static_assert(kBN / 4 * kPadGroupSlots <= kPadTileLoads * 64, "the loads cover the padded tile");

// element offset of (row r, chunk 0) in a padded tile
__device__ __forceinline__ int pad_row(int r) { return 8 * (kPadGroupSlots * (r >> 2) + kPadRowSlots * (r & 3)); }

// the tile row and chunk that slot `lane` of direct load i holds; padding slots
// (and slots past the tile) re-read chunk 15 of their row, or row 63
__device__ __forceinline__ void pad_slot(int i, int lane, int &row, int &chunk) {
    const int p = 64 * i + lane;
    const int k = p / kPadGroupSlots;
    const int q = p - kPadGroupSlots * k;
    const int a = q / kPadRowSlots < 3 ? q / kPadRowSlots : 3;
    const int r = 4 * k + a, c = q - kPadRowSlots * a;
    row = r < kBN - 1 ? r : kBN - 1;
    chunk = c < 15 ? c : 15;
}

// lane bases in a padded tile: the A operand read (row l32, chunk 2ks + half is
// pad_a + 16 ks) and the transposing read (tile row 8 s2 + 4 half + i/4,
// channels 32 db + 16 (grp&1) + 4 (i&3) .. +3 is pad_t + 1232 s2 + 32 db)
__device__ __forceinline__ int pad_a_base(int lane) { return pad_row(lane & 31) + 8 * (lane >> 5); }
__device__ __forceinline__ int pad_t_base(int lane) {
    const int half = lane >> 5, grp = lane >> 4, i = lane & 15;
    return pad_row(4 * half + (i >> 2)) + 16 * (grp & 1) + 4 * (i & 3);
}
// X^T fragment (32 channels x 16 tile rows) from a padded tile; rows points at row 16j's group
__device__ __forceinline__ bf16x8 pad_tr_frag(const uint16_t *rows, int db) {
    const bf16x4 a = lds_read_tr(rows + 32 * db);
    const bf16x4 b = lds_read_tr(rows + 2 * kPad4Rows + 32 * db);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// which (entry, local index) a workgroup id belongs to in a longest-first work list
__device__ __forceinline__ int find_entry(const AttnBwdArgs &a, int w) {
    int lo = 0, hi = a.n_entries - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.wg_prefix[mid] <= w) lo = mid; else hi = mid - 1;
    }
    return lo;
}

}  // namespace

// ---------------------------------------------------------------------------
// row terms: e = do * sig(g), dg = do * o * (1 - sig(g)), D = <do, o>
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_attn_bwd_pre(AttnBwdArgs a) {
    const uint32_t row = blockIdx.x * kBwdPreRowsPerWg + (threadIdx.x >> 4);
    if (row >= a.n_rows) return;
    const uint64_t off = (uint64_t)row * (kD / 8) + (threadIdx.x & 15);
    const u32x4 dov = __builtin_nontemporal_load(static_cast<const u32x4 *>(a.dout) + off);
    const u32x4 ov = __builtin_nontemporal_load(static_cast<const u32x4 *>(a.o) + off);
    float dsum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) dsum += bf16_lo(dov[w]) * bf16_lo(ov[w]) + bf16_hi(dov[w]) * bf16_hi(ov[w]);
    if (a.g) {
        const u32x4 gv = __builtin_nontemporal_load(static_cast<const u32x4 *>(a.g) + off);
        u32x4 ev, dgv;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float s0 = sigmoid(bf16_lo(gv[w])), s1 = sigmoid(bf16_hi(gv[w]));
            ev[w] = pack_bf16x2(bf16_lo(dov[w]) * s0, bf16_hi(dov[w]) * s1);
            dgv[w] = pack_bf16x2(bf16_lo(dov[w]) * bf16_lo(ov[w]) * (1.0f - s0),
                                 bf16_hi(dov[w]) * bf16_hi(ov[w]) * (1.0f - s1));
        }
        static_cast<u32x4 *>(a.e)[off] = ev;
        __builtin_nontemporal_store(dgv, static_cast<u32x4 *>(a.dg) + off);
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) dsum += __shfl_xor(dsum, m, 16);
    if ((threadIdx.x & 15) == 0) a.delta[row] = dsum;
}

// ---------------------------------------------------------------------------
// dk, dv: one workgroup per (segment, head, 128-key block)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBwdThreads, 1) void k_attn_bwd_dkdv(AttnBwdArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t sQ0[kPadTileElems];
    __shared__ __attribute__((aligned(16))) uint16_t sQ1[kPadTileElems];
    __shared__ __attribute__((aligned(16))) uint16_t sQ2[kPadTileElems];
    __shared__ __attribute__((aligned(16))) uint16_t sE0[kPadTileElems];
    __shared__ __attribute__((aligned(16))) uint16_t sE1[kPadTileElems];
    __shared__ __attribute__((aligned(16))) uint32_t sP0[(kBwdKBlock / 32) * 2 * 64 * 8];
    __shared__ __attribute__((aligned(16))) uint32_t sP1[(kBwdKBlock / 32) * 2 * 64 * 8];
    __shared__ __attribute__((aligned(16))) float sL0[kBN];
    __shared__ __attribute__((aligned(16))) float sL1[kBN];
    __shared__ __attribute__((aligned(16))) float sD0[kBN];
    __shared__ __attribute__((aligned(16))) float sD1[kBN];

    const int lo = find_entry(a, blockIdx.x);
    const int seg_len = a.seg_len[lo];
    const int kblocks = (seg_len + kBwdKBlock - 1) / kBwdKBlock;
    const int local = blockIdx.x - a.wg_prefix[lo];
    const int head = local / kblocks;
    const int key0 = (local - head * kblocks) * kBwdKBlock;
    const uint64_t row_stride = (uint64_t)a.n_heads * kD;
    const uint64_t seg_row0 = (uint64_t)a.seg_begin[lo];
    const uint64_t base = seg_row0 * row_stride + (uint64_t)head * kD;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, half = lane >> 5;
    const int kb = wave & 3;
    const bool dv_wave = (wave >> 2) != 0;
    const int row_bytes = (int)(row_stride * 2);

    const uint16_t *qp = static_cast<const uint16_t *>(a.q) + base;
    const uint16_t *kp = static_cast<const uint16_t *>(a.k) + base;
    const uint16_t *vp = static_cast<const uint16_t *>(a.v) + base;
    const uint16_t *ep = static_cast<const uint16_t *>(a.e) + base;

    const int ld_row0 = 4 * wave + (lane >> 4);
    const int ld_chunk = (lane & 15) ^ ((((lane >> 4) & 3) << 2) | (wave & 3));

    // ---- the key block is staged through buffers that are not live yet: K rows 0-63 in sQ1, 64-127 in
    // sQ2, V rows 0-63 in sE1, 64-127 in sP0 (viewed as bf16 rows).  It is read once, so it keeps the
    // compact XOR-swizzled layout of h3_device.h (16 KB per 64 rows) --------------------------------
    uint16_t *const sP0h = reinterpret_cast<uint16_t *>(sP0);
    {
        const uint64_t blk0 = (uint64_t)key0 * row_stride;
        const __amdgpu_buffer_rsrc_t rk =
            __builtin_amdgcn_make_buffer_rsrc((void *)(kp + blk0), 0, kBwdKBlock * row_bytes, kBufferWord3);
        const __amdgpu_buffer_rsrc_t rv =
            __builtin_amdgcn_make_buffer_rsrc((void *)(vp + blk0), 0, kBwdKBlock * row_bytes, kBufferWord3);
        const int last = seg_len - 1 - key0;
#pragma unroll
        for (int i = 0; i < kLoadsPerKBlock; ++i) {
            int key = ld_row0 + 4 * kWaves * i;
            key = key < last ? key : last;
            const int off = key * row_bytes + ld_chunk * 16;
            const int lds_row = 4 * (kWaves * i + wave);             // 0..127; i < 2 -> rows < 64
            uint16_t *kdst = (i < 2 ? sQ1 : sQ2) + (lds_row & 63) * kD;
            uint16_t *vdst = (i < 2 ? sE1 : sP0h) + (lds_row & 63) * kD;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void *)kdst, 16, off, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)vdst, 16, off, 0, 0, 0);
        }
    }
    // Q and e tiles use the padded layout: direct loads i = wave + 8m (three for waves 0-3, two for 4-7)
    constexpr int kLdPerWave = (kPadTileLoads + kWaves - 1) / kWaves;
    const int n_qt = (seg_len + kBN - 1) / kBN;
    int ld_off[kLdPerWave];
#pragma unroll
    for (int m = 0; m < kLdPerWave; ++m) {
        int row, chunk;
        pad_slot(wave + kWaves * m, lane, row, chunk);
        ld_off[m] = row * row_bytes + chunk * 16;
    }
    auto issue_tile = [&](int qt, uint16_t *dq_, uint16_t *de_) {
        const uint64_t tile0 = (uint64_t)qt * kBN * row_stride;
        const __amdgpu_buffer_rsrc_t rq =
            __builtin_amdgcn_make_buffer_rsrc((void *)(qp + tile0), 0, kBN * row_bytes, kBufferWord3);
        const __amdgpu_buffer_rsrc_t re =
            __builtin_amdgcn_make_buffer_rsrc((void *)(ep + tile0), 0, kBN * row_bytes, kBufferWord3);
        const int last = seg_len - 1 - qt * kBN;
#pragma unroll
        for (int m = 0; m < kLdPerWave; ++m) {
            const int i = wave + kWaves * m;                  // wave-uniform
            if (i >= kPadTileLoads) break;
            int off = ld_off[m];
            if ((qt + 1) * kBN > seg_len) {
                int row, chunk;
                pad_slot(i, lane, row, chunk);
                row = row < last ? row : last;
                off = row * row_bytes + chunk * 16;
            }
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void *)(dq_ + i * 512), 16, off, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(re, (lds_void *)(de_ + i * 512), 16, off, 0, 0, 0);
        }
    };
    auto row_value = [&](int qt) -> float {
        const int qrow = qt * kBN + lane;
        if (wave == 0)
            return qrow < seg_len ? a.lse[(seg_row0 + qrow) * a.n_heads + head] * kLog2e : __builtin_inff();
        return qrow < seg_len ? -a.delta[(seg_row0 + qrow) * a.n_heads + head] : 0.0f;
    };

    const int pa = pad_a_base(lane), pt = pad_t_base(lane);
    f32x16 acc[kD / 32];
#pragma unroll
    for (int db = 0; db < kD / 32; ++db) acc[db] = (f32x16){};
    bf16x8 fixed_op[kD / 16];            // K fragments of the wave's keys (dV wave) or their V fragments (dK wave)
    f32x16 dp[2];                        // dK wave: dP - D of the previous tile, carried over the barrier
    const int p_off = (kb * 4 * 64 + lane) * 4;

    // dV wave, tile qt: S, P (published to pw_dst), dV += e^T P
    auto dv_step = [&](const uint16_t *tq, const uint16_t *te, const float *tl, uint32_t *pw_dst) {
        f32x16 sc[2] = {};
#pragma unroll
        for (int ks = 0; ks < kD / 16; ++ks) {
#pragma unroll
            for (int qh = 0; qh < 2; ++qh)
                sc[qh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_b128(tq + pa + 8 * kPad4Rows * qh + 16 * ks),
                                                                 fixed_op[ks], sc[qh], 0, 0, 0);
        }
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) {
            uint32_t pw[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4 lv = *reinterpret_cast<const f32x4 *>(tl + qh * 32 + 8 * i + 4 * half);
                float pr[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    pr[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[qh][4 * i + e], a.scale_log2, -lv[e]));
                pw[2 * i] = pack_bf16x2(pr[0], pr[1]);
                pw[2 * i + 1] = pack_bf16x2(pr[2], pr[3]);
            }
            *reinterpret_cast<u32x4 *>(pw_dst + p_off + qh * 512) = (u32x4){pw[0], pw[1], pw[2], pw[3]};
            *reinterpret_cast<u32x4 *>(pw_dst + p_off + qh * 512 + 256) = (u32x4){pw[4], pw[5], pw[6], pw[7]};
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const bf16x8 b = __builtin_bit_cast(bf16x8, (u32x4){pw[4 * j], pw[4 * j + 1], pw[4 * j + 2], pw[4 * j + 3]});
#pragma unroll
                for (int db = 0; db < kD / 32; ++db)
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        pad_tr_frag(te + pt + kPad4Rows * (8 * qh + 4 * j), db), b, acc[db], 0, 0, 0);
            }
        }
    };
    // dK wave: dS of the previous tile from its P (published last tile) and the carried dP - D, dK += Q^T dS
    auto dk_finish = [&](const uint16_t *tq_prev, const uint32_t *p_src) {
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) {
            const u32x4 p0 = *reinterpret_cast<const u32x4 *>(p_src + p_off + qh * 512);
            const u32x4 p1 = *reinterpret_cast<const u32x4 *>(p_src + p_off + qh * 512 + 256);
            const uint32_t pr[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
            uint32_t w[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                w[2 * i] = pack_bf16x2(bf16_lo(pr[2 * i]) * dp[qh][4 * i], bf16_hi(pr[2 * i]) * dp[qh][4 * i + 1]);
                w[2 * i + 1] = pack_bf16x2(bf16_lo(pr[2 * i + 1]) * dp[qh][4 * i + 2], bf16_hi(pr[2 * i + 1]) * dp[qh][4 * i + 3]);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const bf16x8 b = __builtin_bit_cast(bf16x8, (u32x4){w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]});
#pragma unroll
                for (int db = 0; db < kD / 32; ++db)
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        pad_tr_frag(tq_prev + pt + kPad4Rows * (8 * qh + 4 * j), db), b, acc[db], 0, 0, 0);
            }
        }
    };
    // dK wave, tile qt: dP - D, seeded with -D of each register's query row
    auto dk_start = [&](const uint16_t *te, const float *td) {
#pragma unroll
        for (int qh = 0; qh < 2; ++qh)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4 nd = *reinterpret_cast<const f32x4 *>(td + qh * 32 + 8 * i + 4 * half);
#pragma unroll
                for (int e = 0; e < 4; ++e) dp[qh][4 * i + e] = nd[e];
            }
#pragma unroll
        for (int ks = 0; ks < kD / 16; ++ks) {
#pragma unroll
            for (int qh = 0; qh < 2; ++qh)
                dp[qh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_b128(te + pa + 8 * kPad4Rows * qh + 16 * ks),
                                                                 fixed_op[ks], dp[qh], 0, 0, 0);
        }
    };

    // ---- prologue ----------------------------------------------------------------------------
    issue_tile(0, sQ0, sE0);
    if (wave < 2) (wave == 0 ? sL0 : sD0)[lane] = row_value(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();                                  // key block and tile 0 landed
    {
        const uint16_t *blk = dv_wave ? (kb < 2 ? sQ1 : sQ2) : (kb < 2 ? sE1 : sP0h);
        blk += (kb & 1) * 32 * kD;
#pragma unroll
        for (int ks = 0; ks < kD / 16; ++ks) fixed_op[ks] = lds_b128(blk + swz(l32, 2 * ks + half));
    }
    __syncthreads();                                  // the staging buffers are free again

    // ---- one barrier per tile; the dK wave finishes tile qt-1 in tile qt ---------------------------
    for (int qt = 0; qt <= n_qt; ++qt) {
        if (qt > 0) {
            __builtin_amdgcn_s_waitcnt(0x0F70);
            __syncthreads();
        }
        const int m3 = qt % 3;
        const bool odd = (qt & 1) != 0;
        uint16_t *q_cur = m3 == 0 ? sQ0 : (m3 == 1 ? sQ1 : sQ2);
        uint16_t *q_next = m3 == 0 ? sQ1 : (m3 == 1 ? sQ2 : sQ0);
        uint16_t *q_prev = m3 == 0 ? sQ2 : (m3 == 1 ? sQ0 : sQ1);
        uint16_t *e_cur = odd ? sE1 : sE0, *e_next = odd ? sE0 : sE1;
        uint32_t *p_cur = odd ? sP1 : sP0, *p_prev = odd ? sP0 : sP1;
        const float *l_cur = odd ? sL1 : sL0, *d_cur = odd ? sD1 : sD0;
        float nv = 0.f;
        if (qt + 1 < n_qt) {
            issue_tile(qt + 1, q_next, e_next);
            if (wave < 2) nv = row_value(qt + 1);
        }
        if (dv_wave) {
            if (qt < n_qt) dv_step(q_cur, e_cur, l_cur, p_cur);
        } else {
            if (qt > 0) dk_finish(q_prev, p_prev);
            if (qt < n_qt) dk_start(e_cur, d_cur);
        }
        if (qt + 1 < n_qt && wave < 2) (wave == 0 ? (odd ? sL0 : sL1) : (odd ? sD0 : sD1))[lane] = nv;
    }

    const int key = key0 + kb * 32 + l32;
    if (key >= seg_len) return;
    uint16_t *outp = static_cast<uint16_t *>(dv_wave ? a.dv : a.dk) + base + (uint64_t)key * row_stride;
    const float mul = dv_wave ? 1.0f : a.scale;
#pragma unroll
    for (int db = 0; db < kD / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
            const int d0 = db * 32 + 8 * (r / 4) + 4 * half;
            const u32x2 w = {pack_bf16x2(acc[db][r] * mul, acc[db][r + 1] * mul),
                             pack_bf16x2(acc[db][r + 2] * mul, acc[db][r + 3] * mul)};
            *reinterpret_cast<u32x2 *>(outp + d0) = w;
        }
}

// ---------------------------------------------------------------------------
// dq: one workgroup per (segment, head, 256-query tile), lane = query
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBwdThreads, 1) void k_attn_bwd_dq(AttnBwdArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t sK0[kPadTileElems];
    __shared__ __attribute__((aligned(16))) uint16_t sK1[kPadTileElems];
    __shared__ __attribute__((aligned(16))) uint16_t sV0[kPadTileElems];
    __shared__ __attribute__((aligned(16))) uint16_t sV1[kPadTileElems];

    const int lo = find_entry(a, blockIdx.x);
    const int seg_len = a.seg_len[lo];
    const int tiles = (seg_len + kBwdQBlock - 1) / kBwdQBlock;
    const int local = blockIdx.x - a.wg_prefix[lo];
    const int head = local / tiles;
    const int qtile = local - head * tiles;
    const uint64_t row_stride = (uint64_t)a.n_heads * kD;
    const uint64_t seg_row0 = (uint64_t)a.seg_begin[lo];
    const uint64_t base = seg_row0 * row_stride + (uint64_t)head * kD;

    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, half = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: loads and branches are scalar
    const int q_local = qtile * kBwdQBlock + wave * 32 + l32;
    const bool q_valid = q_local < seg_len;
    const int row_bytes = (int)(row_stride * 2);

    const uint16_t *kp = static_cast<const uint16_t *>(a.k) + base;
    const uint16_t *vp = static_cast<const uint16_t *>(a.v) + base;

    // this lane's q and e rows as B operands (k slots: 8 channels of chunk 2ks+half)
    bf16x8 qreg[kD / 16], ereg[kD / 16];
    {
        const uint64_t r = (uint64_t)(q_valid ? q_local : 0) * row_stride;
        const u32x4 *qs = reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(a.q) + base + r);
        const u32x4 *es = reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(a.e) + base + r);
#pragma unroll
        for (int ks = 0; ks < kD / 16; ++ks) {
            u32x4 x = qs[ks * 2 + half], y = es[ks * 2 + half];
            if (!q_valid) {
                x = (u32x4){0u, 0u, 0u, 0u};
                y = (u32x4){0u, 0u, 0u, 0u};
            }
            qreg[ks] = __builtin_bit_cast(bf16x8, x);
            ereg[ks] = __builtin_bit_cast(bf16x8, y);
        }
    }
    const uint64_t lrow = (seg_row0 + (uint64_t)(q_valid ? q_local : 0)) * a.n_heads + head;
    const float lse2 = a.lse[lrow] * kLog2e;
    // -D of this lane's query in every register: the start value of each dP^T accumulation, so that
    // the accumulator ends as dP^T - D (every register of the C layout belongs to the lane's query)
    f32x16 neg_delta;
#pragma unroll
    for (int r = 0; r < 16; ++r) neg_delta[r] = -a.delta[lrow];

    const int pa = pad_a_base(lane), pt = pad_t_base(lane);

    // direct loads i = wave + 8m of each padded tile (three for waves 0-3, two for 4-7)
    constexpr int kLdPerWave = (kPadTileLoads + kWaves - 1) / kWaves;
    const int n_kt = (seg_len + kBN - 1) / kBN;
    int ld_off[kLdPerWave];
#pragma unroll
    for (int m = 0; m < kLdPerWave; ++m) {
        int row, chunk;
        pad_slot(wave + kWaves * m, lane, row, chunk);
        ld_off[m] = row * row_bytes + chunk * 16;
    }
    auto issue_tile = [&](int kt, uint16_t *dk_, uint16_t *dv_) {
        const uint64_t tile0 = (uint64_t)kt * kBN * row_stride;
        const __amdgpu_buffer_rsrc_t rk =
            __builtin_amdgcn_make_buffer_rsrc((void *)(kp + tile0), 0, kBN * row_bytes, kBufferWord3);
        const __amdgpu_buffer_rsrc_t rv =
            __builtin_amdgcn_make_buffer_rsrc((void *)(vp + tile0), 0, kBN * row_bytes, kBufferWord3);
        const int last = seg_len - 1 - kt * kBN;
#pragma unroll
        for (int m = 0; m < kLdPerWave; ++m) {
            const int i = wave + kWaves * m;                  // wave-uniform
            if (i >= kPadTileLoads) break;
            int off = ld_off[m];
            if ((kt + 1) * kBN > seg_len) {
                int row, chunk;
                pad_slot(i, lane, row, chunk);
                row = row < last ? row : last;
                off = row * row_bytes + chunk * 16;
            }
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void *)(dk_ + i * 512), 16, off, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)(dv_ + i * 512), 16, off, 0, 0, 0);
        }
    };

    f32x16 acc[kD / 32];
#pragma unroll
    for (int db = 0; db < kD / 32; ++db) acc[db] = (f32x16){};

    auto compute_tile = [&](int kt, const uint16_t *tk, const uint16_t *tv) {
        // one 32-key block at a time: S^T = K Q^T and dP^T = V e^T (lane = query), then
        // dS^T = P^T (dP^T - D) packed as the B operand of two 16-key steps, then dQ^T += K^T dS^T
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            f32x16 s = {}, dp = neg_delta;
#pragma unroll
            for (int ks = 0; ks < kD / 16; ++ks) {
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_b128(tk + pa + 8 * kPad4Rows * kb + 16 * ks), qreg[ks], s, 0,
                                                            0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_b128(tv + pa + 8 * kPad4Rows * kb + 16 * ks), ereg[ks], dp,
                                                             0, 0, 0);
            }
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
            for (int i = 0; i < 12; ++i) {
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 4, 0);
            if (__builtin_expect((kt + 1) * kBN > seg_len, 0)) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kt * kBN + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                    if (key >= seg_len) s[r] = -__builtin_inff();
                }
            }
            bf16x8 dsb[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                uint32_t w4[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 8 * j + 2 * e;
                    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], a.scale_log2, -lse2));
                    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r + 1], a.scale_log2, -lse2));
                    w4[e] = pack_bf16x2(p0 * dp[r], p1 * dp[r + 1]);
                }
                dsb[j] = __builtin_bit_cast(bf16x8, (u32x4){w4[0], w4[1], w4[2], w4[3]});
            }
#pragma unroll
            for (int db = 0; db < kD / 32; ++db)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        pad_tr_frag(tk + pt + kPad4Rows * (8 * kb + 4 * j), db), dsb[j], acc[db], 0, 0, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 1);
#pragma unroll
            for (int i = 0; i < 6; ++i) {
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 1);
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 1);
            }
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 1);
        }
    };

    issue_tile(0, sK0, sV0);
    // one instance of the tile body, buffers alternating by tile parity (as in the dk/dv kernel)
    for (int kt = 0; kt < n_kt; ++kt) {
        const bool odd = (kt & 1) != 0;
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        if (kt + 1 < n_kt) issue_tile(kt + 1, odd ? sK0 : sK1, odd ? sV0 : sV1);
        compute_tile(kt, odd ? sK1 : sK0, odd ? sV1 : sV0);
    }

    if (!q_valid) return;
    uint16_t *dqp = static_cast<uint16_t *>(a.dq) + base + (uint64_t)q_local * row_stride;
#pragma unroll
    for (int db = 0; db < kD / 32; ++db)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
            const int d0 = db * 32 + 8 * grp + 4 * half;
            const u32x2 w = {pack_bf16x2(acc[db][grp * 4] * a.scale, acc[db][grp * 4 + 1] * a.scale),
                             pack_bf16x2(acc[db][grp * 4 + 2] * a.scale, acc[db][grp * 4 + 3] * a.scale)};
            *reinterpret_cast<u32x2 *>(dqp + d0) = w;
        }
}

hipError_t launch_attn_bwd_pre(const AttnBwdArgs &a, hipStream_t s, int *grid_x) {
    const uint32_t gx = (uint32_t)(((uint64_t)a.n_rows + kBwdPreRowsPerWg - 1) / kBwdPreRowsPerWg);
    if (grid_x) *grid_x = (int)gx;
    if (gx == 0) return hipSuccess;
    hipLaunchKernelGGL(k_attn_bwd_pre, dim3(gx), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_attn_bwd_dkdv(const AttnBwdArgs &a, int n_workgroups, hipStream_t s) {
    if (n_workgroups <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_attn_bwd_dkdv, dim3(n_workgroups), dim3(kBwdThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_attn_bwd_dq(const AttnBwdArgs &a, int n_workgroups, hipStream_t s) {
    if (n_workgroups <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_attn_bwd_dq, dim3(n_workgroups), dim3(kBwdThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace h3
