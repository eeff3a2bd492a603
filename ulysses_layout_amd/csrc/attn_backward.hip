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
//   k_attn_bwd_dkdv  one workgroup per (segment, head, 192-key block).
//                    Waves w and w+4 share a SIMD and the 48 keys of slice
//                    w: wave w+4 accumulates dV, wave w dK (96 accumulator
//                    registers each, v_mfma_f32_16x16x32_bf16, keys as MFMA
//                    columns).  Each keeps the operand it multiplies by in
//                    registers: K for the dV wave, V for the dK wave.
//                    64-query tiles of Q and e stream through LDS (direct
//                    buffer loads, three buffers), one barrier per tile.  In
//                    tile t the dV wave forms S = Q K^T and P from it (lse
//                    per row from LDS), publishes P in bf16 through LDS and
//                    adds e^T P; the dK wave, one tile behind, forms
//                    dP - D (the accumulator seeded with -D), dS = P (dP - D)
//                    with the published P, and adds Q^T dS.  The transposing
//                    LDS load supplies e^T and Q^T.
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
// MFMA layouts and the transposing read follow packed_attn.hip.  The dk/dv
// kernel streams its Q and e tiles in the forward's 16-row swizzled layout.
// The dq kernel (v_mfma_f32_32x32x16_bf16) streams K and V in a padded LDS
// layout instead: it is as free of bank conflicts, and because each chunk of a
// row sits at a constant distance from the row start, one lane base and
// immediate offsets address every read of a tile whichever buffer holds it,
// so its tile body computes no addresses per tile.
#include "h3_device.h"

namespace h3 {

namespace {

constexpr int kBN = 64;                  // keys per tile (dq) / queries per tile (dk/dv)
constexpr int kWaves = kBwdThreads / 64; // 8
constexpr float kLog2e = 1.4426950408889634f;
static_assert(kBwdQBlock == 32 * kWaves, "one 32-query block per wave");

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
// dk, dv: one workgroup per (segment, head, 192-key block)
// ---------------------------------------------------------------------------
// Waves w and w + 4 share a SIMD and own the same 48 keys (three 16-key
// blocks): wave w + 4 accumulates dV^T, wave w dK^T, 96 registers each, with
// v_mfma_f32_16x16x32_bf16.  The keys are the MFMA columns (lane l%16 = key),
// so every Q, e, Q^T or e^T fragment a wave reads from LDS feeds the MFMAs of
// all three key blocks.  The dV wave holds K^T of its keys and the dK wave
// V^T, as B operands in registers.  64-query tiles of Q and e stream through
// LDS (direct buffer loads, the forward's 16-row swizzle, three buffers), with
// the rows' lse (log2 units) and -D.  In tile t the dV wave forms S = Q K^T and
// P = 2^(c S - lse) per 32-query half, publishes P (bf16) through LDS and adds
// e^T P to dV^T; the dK wave works one tile behind: dP - D = e V^T seeded
// with -D, dS = P (dP - D) with the P published in tile t - 1, and Q^T dS into
// dK^T.  One barrier per tile.  P^T and dS^T as B operands come straight from
// the C layout of S and dP (k slot j of lane group g is query 4g + j or
// 16 + 4g + j - 4 of the half), and the transposing read supplies e^T and Q^T
// in the same query order.
namespace {
constexpr int kKB2 = 3;                                  // 16-key blocks per wave
constexpr int kKeysPerWave = 16 * kKB2;                  // 48
constexpr int kDkdvKeys = kKeysPerWave * (kWaves / 2);   // 192 keys per workgroup
constexpr int kTileE = kBN * kD;                         // elements of one 64-row tile
constexpr int kLdPerTile = kBN / (4 * kWaves);           // direct loads per lane per operand and tile
constexpr int kPVecs = 6;                                // 16-byte P vectors per lane and tile (2 halves x 3)
static_assert(kLdPerTile * 4 * kWaves == kBN, "loads cover the tile");
}  // namespace

__global__ __launch_bounds__(kBwdThreads, 1) void k_attn_bwd_dkdv(AttnBwdArgs a) {
    // Six distinct tile objects (not arrays of buffers), and loops unrolled by three so each
    // names them statically: the compiler can then prove that the direct loads into the next
    // tile's buffers never alias the reads of the current ones, and does not make those reads
    // wait for the loads.
    __shared__ __attribute__((aligned(16))) uint16_t sQ0[kTileE];
    __shared__ __attribute__((aligned(16))) uint16_t sQ1[kTileE];
    __shared__ __attribute__((aligned(16))) uint16_t sQ2[kTileE];
    __shared__ __attribute__((aligned(16))) uint16_t sE0[kTileE];
    __shared__ __attribute__((aligned(16))) uint16_t sE1[kTileE];
    __shared__ __attribute__((aligned(16))) uint16_t sE2[kTileE];
    __shared__ __attribute__((aligned(16))) u32x4 sP[2 * (kWaves / 2) * kPVecs * 64];
    __shared__ __attribute__((aligned(16))) float sL[3 * kBN];
    __shared__ __attribute__((aligned(16))) float sD[3 * kBN];

    const int lo = find_entry(a, blockIdx.x);
    const int seg_len = a.seg_len[lo];
    const int kblocks = (seg_len + kDkdvKeys - 1) / kDkdvKeys;
    const int local = blockIdx.x - a.wg_prefix[lo];
    const int head = local / kblocks;
    const int key0 = (local - head * kblocks) * kDkdvKeys;
    const uint32_t n_heads = a.n_heads;
    const float scale = a.scale, scale_log2 = a.scale_log2;
    const float *const lse_in = a.lse;
    const float *const delta_in = a.delta;
    const uint64_t row_stride = (uint64_t)n_heads * kD;
    const uint64_t seg_row0 = (uint64_t)a.seg_begin[lo];
    const uint64_t base = seg_row0 * row_stride + (uint64_t)head * kD;

    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pair = wave & 3;
    const bool dv_wave = wave >= 4;                          // wave-uniform
    const int kbase = key0 + pair * kKeysPerWave;            // this wave's first key (segment-local)
    const int row_bytes = (int)(row_stride * 2);

    const uint16_t *qp = static_cast<const uint16_t *>(a.q) + base;
    const uint16_t *ep = static_cast<const uint16_t *>(a.e) + base;

    // K^T (dV wave) or V^T (dK wave) of the wave's keys as B operands: key 16kb + l16,
    // MFMA k step ks on the channels of chunk 4 grp + ks (the forward's conflict-free order)
    bf16x8 fixed_op[kKB2][kD / 32];
    {
        const uint16_t *src = static_cast<const uint16_t *>(dv_wave ? a.k : a.v) + base;
#pragma unroll
        for (int kb = 0; kb < kKB2; ++kb) {
            int key = kbase + 16 * kb + l16;
            key = key < seg_len ? key : seg_len - 1;
            const u32x4 *row = reinterpret_cast<const u32x4 *>(src + (uint64_t)key * row_stride);
#pragma unroll
            for (int ks = 0; ks < kD / 32; ++ks) fixed_op[kb][ks] = __builtin_bit_cast(bf16x8, row[4 * grp + ks]);
        }
    }

    // per-lane LDS offsets inside a tile
    int a_off[kD / 32];                  // A operand (16 tile rows x 32 channels): row l16 (+16 i), chunk 4grp + ks
#pragma unroll
    for (int ks = 0; ks < kD / 32; ++ks) a_off[ks] = tile16_off(l16, 4 * grp + ks);
    int t_off[kD / 16];                  // transposing reads: row 4grp + l16/4 (+16, +32h), channels 16cb + 4(l16%4)
#pragma unroll
    for (int cb = 0; cb < kD / 16; ++cb) {
        const int col = 16 * cb + 4 * (l16 & 3);
        t_off[cb] = tile16_off(4 * grp + (l16 >> 2), col >> 3) + (col & 7);
    }

    // direct HBM -> LDS loads of a 64-row Q and e tile: load i of wave w covers rows
    // 4(8i + w) .. +3, lane l row +l/16, LDS slot l; the swizzle is applied on the global side
    const int ld_row0 = 4 * wave + (lane >> 4);
    const int ld_chunk = (lane & 15) ^ tile16_f(ld_row0);
    const int n_qt = (seg_len + kBN - 1) / kBN;
    auto issue_tile = [&](int qt, uint16_t *dst_q, uint16_t *dst_e) __attribute__((always_inline)) {
        const uint64_t tile0 = (uint64_t)qt * kBN * row_stride;
        const __amdgpu_buffer_rsrc_t rq =
            __builtin_amdgcn_make_buffer_rsrc((void *)(qp + tile0), 0, kBN * row_bytes, kBufferWord3);
        const __amdgpu_buffer_rsrc_t re =
            __builtin_amdgcn_make_buffer_rsrc((void *)(ep + tile0), 0, kBN * row_bytes, kBufferWord3);
        const int last = seg_len - 1 - qt * kBN;
#pragma unroll
        for (int i = 0; i < kLdPerTile; ++i) {
            int row = ld_row0 + 4 * kWaves * i;
            row = row < last ? row : last;
            const int off = row * row_bytes + ld_chunk * 16;
            const int lds_row = 4 * (kWaves * i + wave);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void *)(dst_q + lds_row * kD), 16, off, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(re, (lds_void *)(dst_e + lds_row * kD), 16, off, 0, 0, 0);
        }
    };
    // waves 0 and 1 bring the tile's lse (log2 units; +inf past the end) and -D (0 past the end):
    // the raw entry of the lane's row (clamped) is loaded unconditionally when a trip starts and
    // turned into the row term when it ends, so that no wait for the load (which would also
    // wait for the tile loads issued before it) falls inside the trip's products
    auto row_load = [&](int qt) __attribute__((always_inline)) -> float {
        const int q = qt * kBN + lane;
        const uint64_t r = (seg_row0 + (uint64_t)(q < seg_len ? q : seg_len - 1)) * n_heads + head;
        return (wave == 0 ? lse_in : delta_in)[r];
    };
    auto row_term = [&](int qt, float raw) __attribute__((always_inline)) -> float {
        const bool in = qt * kBN + lane < seg_len;
        if (wave == 0) return in ? raw * kLog2e : __builtin_inff();
        return in ? -raw : 0.0f;
    };

    f32x4 acc[kD / 16][kKB2];            // dV^T or dK^T: channels 16cb + 4grp + r of key 16kb + l16
#pragma unroll
    for (int cb = 0; cb < kD / 16; ++cb)
#pragma unroll
        for (int kb = 0; kb < kKB2; ++kb) acc[cb][kb] = (f32x4){};

    // A fragment (16 rows x 32 channels) and transposed A fragment (16 channels x the
    // half's 32 rows in MFMA k-slot order) of a tile
    auto frag = [&](const uint16_t *t, int row0, int ks) __attribute__((always_inline)) {
        return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(t + row0 * kD + a_off[ks]));
    };
    auto tfrag = [&](const uint16_t *t, int h, int cb) __attribute__((always_inline)) {
        const bf16x4 x0 = lds_read_tr(t + (32 * h) * kD + t_off[cb]);
        const bf16x4 x1 = lds_read_tr(t + (32 * h + 16) * kD + t_off[cb]);
        return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    u32x4 *const p_pair = sP + pair * (kPVecs * 64) + lane;       // + buffer * (kWaves/2)*kPVecs*64 + vec * 64

    // dV wave, tile (tq, te) with row lse tl: S, P, publish P in buffer pb, dV^T += e^T P
    auto dv_tile = [&](const uint16_t *tq, const uint16_t *te, const float *tl, int pb) __attribute__((always_inline)) {
        u32x4 *pout = p_pair + pb * ((kWaves / 2) * kPVecs * 64);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            f32x4 sc[2][kKB2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int kb = 0; kb < kKB2; ++kb) sc[i][kb] = (f32x4){};
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int ks = 0; ks < kD / 32; ++ks) {
                    const bf16x8 qf = frag(tq, 32 * h + 16 * i, ks);
#pragma unroll
                    for (int kb = 0; kb < kKB2; ++kb)
                        sc[i][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf, fixed_op[kb][ks], sc[i][kb], 0, 0, 0);
                }
            // P = 2^(c S - lse) of queries 32h + 16i + 4grp + r
            uint32_t w[2][kKB2][2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const f32x4 lv = *reinterpret_cast<const f32x4 *>(tl + 32 * h + 16 * i + 4 * grp);
#pragma unroll
                for (int kb = 0; kb < kKB2; ++kb)
#pragma unroll
                    for (int x = 0; x < 2; ++x) {
                        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i][kb][2 * x], scale_log2, -lv[2 * x]));
                        const float p1 =
                            __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i][kb][2 * x + 1], scale_log2, -lv[2 * x + 1]));
                        w[i][kb][x] = pack_bf16x2(p0, p1);
                    }
            }
            // P^T of key block kb as a B operand, published as is for the dK wave (vector 3h + kb)
            bf16x8 pbv[kKB2];
#pragma unroll
            for (int kb = 0; kb < kKB2; ++kb) {
                const u32x4 pv = {w[0][kb][0], w[0][kb][1], w[1][kb][0], w[1][kb][1]};
                pout[(3 * h + kb) * 64] = pv;
                pbv[kb] = __builtin_bit_cast(bf16x8, pv);
            }
#pragma unroll
            for (int cb = 0; cb < kD / 16; ++cb) {
                const bf16x8 ef = tfrag(te, h, cb);
#pragma unroll
                for (int kb = 0; kb < kKB2; ++kb)
                    acc[cb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ef, pbv[kb], acc[cb][kb], 0, 0, 0);
            }
        }
    };
    // dK wave, tile (tq, te) with row terms -D in td (published P in buffer pb): dP - D, dS,
    // dK^T += Q^T dS
    auto dk_tile = [&](const uint16_t *tq, const uint16_t *te, const float *td, int pb) __attribute__((always_inline)) {
        const u32x4 *pin = p_pair + pb * ((kWaves / 2) * kPVecs * 64);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            f32x4 dp[2][kKB2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const f32x4 nd = *reinterpret_cast<const f32x4 *>(td + 32 * h + 16 * i + 4 * grp);
#pragma unroll
                for (int kb = 0; kb < kKB2; ++kb) dp[i][kb] = nd;
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int ks = 0; ks < kD / 32; ++ks) {
                    const bf16x8 ef = frag(te, 32 * h + 16 * i, ks);
#pragma unroll
                    for (int kb = 0; kb < kKB2; ++kb)
                        dp[i][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ef, fixed_op[kb][ks], dp[i][kb], 0, 0, 0);
                }
            // dS = P (dP - D), in the k-slot order of the B operand (word 2i + x of P^T)
            bf16x8 dsb[kKB2];
#pragma unroll
            for (int kb = 0; kb < kKB2; ++kb) {
                const u32x4 pv = pin[(3 * h + kb) * 64];
                uint32_t ww[4];
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int x = 0; x < 2; ++x)
                        ww[2 * i + x] = pack_bf16x2(bf16_lo(pv[2 * i + x]) * dp[i][kb][2 * x],
                                                    bf16_hi(pv[2 * i + x]) * dp[i][kb][2 * x + 1]);
                dsb[kb] = __builtin_bit_cast(bf16x8, (u32x4){ww[0], ww[1], ww[2], ww[3]});
            }
#pragma unroll
            for (int cb = 0; cb < kD / 16; ++cb) {
                const bf16x8 qf = tfrag(tq, h, cb);
#pragma unroll
                for (int kb = 0; kb < kKB2; ++kb)
                    acc[cb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf, dsb[kb], acc[cb][kb], 0, 0, 0);
            }
        }
    };

    // ---- prologue: tile 0 and its row terms -----------------------------------------------------
    issue_tile(0, sQ0, sE0);
    if (wave < 2) (wave == 0 ? sL : sD)[lane] = row_term(0, row_load(0));

    // ---- one barrier per tile; the dK wave finishes tile t - 1 in tile t ---------------------------
    // The two kinds of wave run loops of their own (one register allocation each) that meet at
    // the same n_qt + 1 barriers.  Tile t sits in buffer t % 3; trip t loads tile t + 1 into the
    // next buffer while the dV wave reads buffer t % 3 and the dK wave buffer (t - 1) % 3.
    auto tile_begin = [&](int t, uint16_t *nq, uint16_t *ne, float &nv) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0x0F70);          // vmcnt(0): this lane's loads of tile t landed
        __syncthreads();                             // ... and everyone's; P of tile t - 1 is published
        if (t + 1 < n_qt) {
            issue_tile(t + 1, nq, ne);
            if (wave < 2) nv = row_load(t + 1);
        }
    };
    auto tile_end = [&](int t, int b_next, float nv) __attribute__((always_inline)) {
        if (t + 1 < n_qt && wave < 2) (wave == 0 ? sL : sD)[b_next * kBN + lane] = row_term(t + 1, nv);
    };
    if (dv_wave) {
        auto trip = [&](int t, const uint16_t *cq, const uint16_t *ce, uint16_t *nq, uint16_t *ne, int b)
            __attribute__((always_inline)) {
            float nv = 0.f;
            tile_begin(t, nq, ne, nv);
            if (t < n_qt) dv_tile(cq, ce, sL + b * kBN, t & 1);
            tile_end(t, b == 2 ? 0 : b + 1, nv);
        };
        for (int t = 0;; t += 3) {
            trip(t, sQ0, sE0, sQ1, sE1, 0);
            if (t == n_qt) break;
            trip(t + 1, sQ1, sE1, sQ2, sE2, 1);
            if (t + 1 == n_qt) break;
            trip(t + 2, sQ2, sE2, sQ0, sE0, 2);
            if (t + 2 == n_qt) break;
        }
    } else {
        auto trip = [&](int t, const uint16_t *pq, const uint16_t *pe, uint16_t *nq, uint16_t *ne, int b)
            __attribute__((always_inline)) {
            float nv = 0.f;
            tile_begin(t, nq, ne, nv);
            if (t > 0) dk_tile(pq, pe, sD + (b == 0 ? 2 : b - 1) * kBN, (t - 1) & 1);
            tile_end(t, b == 2 ? 0 : b + 1, nv);
        };
        for (int t = 0;; t += 3) {
            trip(t, sQ2, sE2, sQ1, sE1, 0);
            if (t == n_qt) break;
            trip(t + 1, sQ0, sE0, sQ2, sE2, 1);
            if (t + 1 == n_qt) break;
            trip(t + 2, sQ1, sE1, sQ0, sE0, 2);
            if (t + 2 == n_qt) break;
        }
    }

    // ---- epilogue: stage the wave's output rows in LDS 16 at a time, store whole rows --------------
    __syncthreads();                                 // every wave is done with the tiles
    uint16_t *stage = (wave < 4 ? sQ0 : sE0) + (wave & 3) * (16 * kD);
    const float mul = dv_wave ? 1.0f : scale;
    uint16_t *outp = static_cast<uint16_t *>(dv_wave ? a.dv : a.dk) + base;
    const int io_chunk = lane & 15;
#pragma unroll
    for (int kb = 0; kb < kKB2; ++kb) {
#pragma unroll
        for (int cb = 0; cb < kD / 16; ++cb) {
            uint16_t *slot = stage + l16 * kD + (((2 * cb + (grp >> 1)) ^ l16) << 3) + 4 * (grp & 1);
            *reinterpret_cast<u32x2 *>(slot) = (u32x2){pack_bf16x2(acc[cb][kb][0] * mul, acc[cb][kb][1] * mul),
                                                        pack_bf16x2(acc[cb][kb][2] * mul, acc[cb][kb][3] * mul)};
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = (lane >> 4) + 4 * i;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(stage + r * kD + ((io_chunk ^ r) << 3));
            const int key = kbase + 16 * kb + r;
            if (key < seg_len) *reinterpret_cast<u32x4 *>(outp + (uint64_t)key * row_stride + io_chunk * 8) = v;
        }
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
    // one instance of the tile body, buffers alternating by tile parity
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

int attn_bwd_key_block() { return kDkdvKeys; }

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
