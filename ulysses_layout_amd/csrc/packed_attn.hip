// packed_attn.hip -- segment-masked attention over the natively packed
// multi-segment sequence, for the heads one virtual rank holds after the
// sequence-to-head relayout ("Distributed H3 Execution", introduction: the
// packed H3 sequence is kept as is, no semantic padding), with the optional
// sigmoid gate of the QKVG form ("[perf] Harden Ulysses agreement and tune
// bounded H3 transfers", Problem and behavior: packed QKV/QKVG operands).
//
// Work decomposition: one workgroup of 8 waves = (segment, head, 256-query
// tile); it walks only the 64-key tiles of its own segment, so cross-segment
// blocks are never visited and only the last key tile of a segment needs a
// mask.  Segments are issued longest first.  Within a head the query tiles
// are consecutive workgroup ids, so the workgroups in flight stream the same
// K/V tiles and share them in L2 and the Infinity Cache; 256 queries per
// workgroup halve the K/V traffic per FLOP against 128.
//
// Per wave (64 lanes, 32 query rows), per 64-key tile, with CDNA4's
// v_mfma_f32_32x32x16_bf16 (A: 32 rows x 16 k, B: 16 k x 32 cols, lane l%32
// owns row/col l%32, lane half l/32 owns k slots 8*(l/32)..+7; C: lane l%32
// owns column l%32, register r holds row 8*(r/4) + 4*(l/32) + r%4):
//   S^T = K Q^T      A = K rows from LDS, B = this wave's Q (registers), so
//                    each lane holds ONE query and 32 of the tile's keys: the
//                    softmax row reductions are lane-local plus one exchange
//                    with lane l^32;
//   online softmax   base 2, log2(e) folded into the scale; the running max
//                    is only raised when a row's new maximum exceeds it by
//                    more than 2^8 (probabilities stay <= 256, exact in the
//                    final normalisation), so the O rescale is rare; the tile
//                    max itself is only computed when a lane's partial row
//                    sum shows a probability of 2^7 or more;
//   O^T += V^T P^T   B = P^T straight from the S^T registers (the MFMA k
//                    slots are assigned to keys in exactly the order the C
//                    layout left them in), A = V^T read with the gfx950
//                    transposing LDS load ds_read_b64_tr_b16 from the
//                    row-major V tile (per 16-lane group it turns a 4-key x
//                    16-channel block into one channel x 4 keys per lane).
// The O^T accumulator keeps each lane on its own query, so the rescale is a
// per-lane scalar and the row sum of P comes from v_dot2 on the rounded bf16
// P the MFMA consumes.
//
// K/V tiles move from HBM straight into LDS with the 128-bit buffer load to
// LDS (no VGPR staging): wave w's i-th load fills LDS bytes
// [1 KB*(8i + w), +1 KB), i.e. rows 4(8i+w)..+3, lane l at 16-byte slot l.
// The buffer resource is rebased to each tile's first key, so the per-lane
// offsets stay below 64 rows.  The buffer form rather than the global one is
// deliberate: the compiler treats an outstanding global load to LDS like a
// flat access that may also count on the LDS counter, and then drains every
// LDS read completely before its first use; with the buffer form it keeps
// exact per-read waits, so K fragments stream into the QK MFMAs.
// LDS holds K and V tiles [64][128] bf16, double buffered (one barrier per
// tile, the loop unrolled by two so buffer addresses are constants).  16-byte
// chunk c of row r sits at chunk c ^ f(r), f(r) = 4*(r%4) + (r/4)%4: 16
// consecutive rows read at one logical chunk, and the 4 rows x 4 chunks a
// 32-lane half reads through the transposing load, both hit 16 distinct
// chunk positions.  Because the LDS side of a direct load is fixed per lane,
// the swizzle is applied on the global side: lane l of a load fetches logical
// chunk (l%16) ^ f(row).  Rows past the end of the segment are clamped to
// its last row (finite data, masked out or weighted by 0).
#include "h3_device.h"

namespace h3 {

constexpr int kBN = 64;                  // keys per tile
constexpr int kTileElems = kBN * kD;     // one K or V tile
constexpr int kWaves = kAttnThreads / 64;
constexpr int kLoadsPerTile = kBN / (4 * kWaves);   // 16-byte direct loads per lane per operand
constexpr float kLazyRescale = 8.0f;     // log2 of the largest tolerated probability
constexpr float kMaxCheck = 128.0f;      // partial row sum that triggers the exact max (2^7 < 2^8)
static_assert(kAttnBlockM == 32 * kWaves, "one 32-query block per wave");
static_assert(kLoadsPerTile * 4 * kWaves == kBN, "loads cover the tile");

__global__ __launch_bounds__(kAttnThreads, 1) void k_packed_attn(AttnArgs a) {
    // Four distinct LDS objects (not one array of buffers) so the compiler can
    // prove that the direct loads into one buffer never alias the reads of the
    // other and does not serialise them with extra counter waits.
    __shared__ __attribute__((aligned(16))) uint16_t sK0[kTileElems];
    __shared__ __attribute__((aligned(16))) uint16_t sK1[kTileElems];
    __shared__ __attribute__((aligned(16))) uint16_t sV0[kTileElems];
    __shared__ __attribute__((aligned(16))) uint16_t sV1[kTileElems];

    // ---- which (segment, head, query tile) this workgroup owns ----------------
    const int w = blockIdx.x;
    int lo = 0, hi = a.n_entries - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.wg_prefix[mid] <= w) lo = mid; else hi = mid - 1;
    }
    const int seg_len = a.seg_len[lo];
    const int tiles = (seg_len + kAttnBlockM - 1) / kAttnBlockM;
    const int local = w - a.wg_prefix[lo];
    const int head = local / tiles;
    const int qtile = local - head * tiles;
    const uint64_t row_stride = (uint64_t)a.n_heads * kD;                    // elements per token
    const uint64_t base = (uint64_t)a.seg_begin[lo] * row_stride + (uint64_t)head * kD;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: load addresses are scalar
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int half = lane >> 5;
    const int q_local = qtile * kAttnBlockM + wave * 32 + l32;            // query of this lane
    const bool q_valid = q_local < seg_len;

    const uint16_t *qp = static_cast<const uint16_t *>(a.q) + base;
    const uint16_t *kp = static_cast<const uint16_t *>(a.k) + base;
    const uint16_t *vp = static_cast<const uint16_t *>(a.v) + base;

    // ---- this lane's query row as the B operand of S^T = K Q^T ----------------
    bf16x8 qreg[kD / 16];
    {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(qp + (uint64_t)(q_valid ? q_local : 0) * row_stride);
#pragma unroll
        for (int ks = 0; ks < kD / 16; ++ks) {
            u32x4 v = src[ks * 2 + half];
            if (!q_valid) v = (u32x4){0u, 0u, 0u, 0u};
            qreg[ks] = __builtin_bit_cast(bf16x8, v);
        }
    }

    // ---- per-lane LDS offsets (independent of the tile and of kb / j) ---------
    int k_off[kD / 16];                        // A operand of S^T: row l32 (+32 kb), chunk 2ks+half
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) k_off[ks] = swz(l32, 2 * ks + half);
    int v_off[kD / 32][2];                     // transposing reads: keys 16j + 8 s2 + 4 half + i/4
    {
        const int grp = lane >> 4, i = lane & 15;
#pragma unroll
        for (int db = 0; db < kD / 32; ++db)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const int r = 8 * s2 + 4 * half + (i >> 2);
                const int col = db * 32 + 16 * (grp & 1) + 4 * (i & 3);
                v_off[db][s2] = swz(r, col >> 3) + (col & 7);
            }
    }

    // ---- direct HBM -> LDS tile loads ------------------------------------------
    // load i of wave `wave` covers tile rows 4*(kWaves*i + wave) .. +3, lane l row +l/16;
    // f(row) does not depend on i because rows step by 4*kWaves (a multiple of 16).
    const int ld_row0 = 4 * wave + (lane >> 4);
    const int ld_chunk = (lane & 15) ^ ((((lane >> 4) & 3) << 2) | (wave & 3));
    const int n_kt = (seg_len + kBN - 1) / kBN;
    const int row_bytes = (int)(row_stride * 2);       // <= 256 heads * 256 B
    int ld_off[kLoadsPerTile];                          // byte offsets inside a full tile
#pragma unroll
    for (int i = 0; i < kLoadsPerTile; ++i) ld_off[i] = (ld_row0 + 4 * kWaves * i) * row_bytes + ld_chunk * 16;
    auto issue_tile = [&](int kt, uint16_t *dk, uint16_t *dv) {
        const uint64_t tile0 = (uint64_t)kt * kBN * row_stride;
        const __amdgpu_buffer_rsrc_t rk =
            __builtin_amdgcn_make_buffer_rsrc((void *)(kp + tile0), 0, kBN * row_bytes, kBufferWord3);
        const __amdgpu_buffer_rsrc_t rv =
            __builtin_amdgcn_make_buffer_rsrc((void *)(vp + tile0), 0, kBN * row_bytes, kBufferWord3);
        if ((kt + 1) * kBN <= seg_len) {
#pragma unroll
            for (int i = 0; i < kLoadsPerTile; ++i) {
                const int lds_row = 4 * (kWaves * i + wave);            // wave-uniform
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void *)(dk + lds_row * kD), 16, ld_off[i], 0, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)(dv + lds_row * kD), 16, ld_off[i], 0, 0, 0);
            }
        } else {
            // last tile of the segment: rows past its end re-read the last row
            const int last = seg_len - 1 - kt * kBN;
#pragma unroll
            for (int i = 0; i < kLoadsPerTile; ++i) {
                int key = ld_row0 + 4 * kWaves * i;
                key = key < last ? key : last;
                const int off = key * row_bytes + ld_chunk * 16;
                const int lds_row = 4 * (kWaves * i + wave);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void *)(dk + lds_row * kD), 16, off, 0, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)(dv + lds_row * kD), 16, off, 0, 0, 0);
            }
        }
    };

    f32x16 acc[kD / 32];
#pragma unroll
    for (int db = 0; db < kD / 32; ++db) acc[db] = (f32x16){};
    float m_run = -__builtin_inff();    // running max, already in log2 units
    float l_run = 0.f;                  // this lane's share of the running denominator
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

    auto compute_tile = [&](int kt, const uint16_t *tk, const uint16_t *tv) {
        // S^T = K Q^T for the two 32-key blocks of the tile: fragment i is block i%2,
        // k step i/2, so the two accumulation chains alternate.  The reads run four
        // ahead of the MFMAs that consume them.
        f32x16 s[2];
        s[0] = (f32x16){};
        s[1] = (f32x16){};
        bf16x8 kf[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
            kf[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(tk + (i & 1) * 32 * kD + k_off[i >> 1]));
#pragma unroll
        for (int i = 0; i < 16; ++i)
            s[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qreg[i >> 1], s[i & 1], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
        for (int i = 0; i < 12; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 4, 0);
        // V^T fragments for the PV step, read now so they land during the softmax;
        // fragment (db, j) covers channels 32db.. and keys 16j..16j+15
        bf16x8 vf[kD / 32][4];
#pragma unroll
        for (int db = 0; db < kD / 32; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bf16x4 v0 = lds_read_tr(tv + 16 * j * kD + v_off[db][0]);
                const bf16x4 v1 = lds_read_tr(tv + 16 * j * kD + v_off[db][1]);
                vf[db][j] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
            }
        // keys past the end of the segment (last tile only)
        if ((kt + 1) * kBN > seg_len) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kt * kBN + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                    if (key >= seg_len) s[kb][r] = -__builtin_inff();
                }
        }
        // online softmax (base 2) with lazy rescaling.  The probabilities are first
        // formed against the running max.  A probability of 2^7 or more, or the
        // NaN/inf of the first tile (running max still -inf), makes that lane's
        // partial row sum reach 2^7 or fail the comparison; only then is the tile
        // max computed, and only if it exceeds the running max by more than 2^8 are
        // the accumulators rescaled and the probabilities formed again.
        float psum;
        bf16x8 pb[4];
        auto form_p = [&]() {
            psum = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int kb = j >> 1, r0 = (j & 1) * 8;
                uint32_t wds[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r0 + 2 * e], a.scale_log2, -m_run));
                    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r0 + 2 * e + 1], a.scale_log2, -m_run));
                    wds[e] = pack_bf16x2(p0, p1);
                    psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wds[e]), ones, psum, false);
                }
                pb[j] = __builtin_bit_cast(bf16x8, (u32x4){wds[0], wds[1], wds[2], wds[3]});
            }
        };
        form_p();
        if (__builtin_amdgcn_ballot_w64(!(psum < kMaxCheck)) != 0) {
            float mx = s[0][0];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[kb][r]);
            mx = half_max(mx) * a.scale_log2;
            if (__builtin_amdgcn_ballot_w64(mx > m_run + kLazyRescale) != 0) {
                const float m_new = __builtin_fmaxf(m_run, mx);
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < kD / 32; ++db) acc[db] *= alpha;
                m_run = m_new;
                form_p();
            }
        }
        l_run += psum;

        // O^T += V^T P^T; MFMA k slot (half, jj) of step j is key 16j + 8*(jj/4) + 4*half + jj%4
#pragma unroll
        for (int db = 0; db < kD / 32; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db][j], pb[j], acc[db], 0, 0, 0);
    };

    // ---- main loop: two tiles per trip so each buffer index is an immediate ---
    issue_tile(0, sK0, sV0);
    for (int kt = 0; kt < n_kt; kt += 2) {
        __builtin_amdgcn_s_waitcnt(0x0F70);           // vmcnt(0): this lane's loads of tile kt landed
        __syncthreads();                              // ... and everyone's; buffer 1 is free
        if (kt + 1 < n_kt) issue_tile(kt + 1, sK1, sV1);
        compute_tile(kt, sK0, sV0);
        if (kt + 1 >= n_kt) break;
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        if (kt + 2 < n_kt) issue_tile(kt + 2, sK0, sV0);
        compute_tile(kt + 1, sK1, sV1);
    }

    // ---- epilogue: normalise, gate, round, store ------------------------------
    const float l_tot = half_sum(l_run);
    const float inv = 1.0f / l_tot;
    if (!q_valid) return;
    if (a.lse && half == 0) {
        // log-sum-exp of the scaled logits (natural log): the probabilities are
        // 2^(c*s - m_run) / l_tot, so lse * log2(e) = m_run + log2(l_tot)
        const float lse2 = m_run + __builtin_amdgcn_logf(l_tot);
        a.lse[((uint64_t)a.seg_begin[lo] + (uint64_t)q_local) * a.n_heads + head] = lse2 * 0.6931471805599453f;
    }
    uint16_t *op = static_cast<uint16_t *>(a.o) + base + (uint64_t)q_local * row_stride;
    const uint16_t *gp = a.g ? static_cast<const uint16_t *>(a.g) + base + (uint64_t)q_local * row_stride
                             : nullptr;
#pragma unroll
    for (int db = 0; db < kD / 32; ++db) {
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
            const int d0 = db * 32 + 8 * grp + 4 * half;      // 4 consecutive channels
            float y[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = acc[db][grp * 4 + e] * inv;
            if (gp) {
                const u32x2 gw = *reinterpret_cast<const u32x2 *>(gp + d0);
                const float gv[4] = {bf16_lo(gw[0]), bf16_hi(gw[0]), bf16_lo(gw[1]), bf16_hi(gw[1])};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    // sigmoid(g) = 1 / (1 + 2^(-g * log2 e))
                    const float den = 1.0f + __builtin_amdgcn_exp2f(-gv[e] * 1.4426950408889634f);
                    y[e] = y[e] / den;
                }
            }
            const u32x2 out = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
            *reinterpret_cast<u32x2 *>(op + d0) = out;
        }
    }
}

hipError_t launch_packed_attn(const AttnArgs &a, int n_workgroups, hipStream_t s) {
    if (n_workgroups <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_packed_attn, dim3(n_workgroups), dim3(kAttnThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace h3
