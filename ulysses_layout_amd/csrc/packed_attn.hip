// packed_attn.hip -- segment-masked attention over the natively packed
// multi-segment sequence, for the heads one virtual rank holds after the
// sequence-to-head relayout ("Distributed H3 Execution", introduction: the
// packed H3 sequence is kept as is, no semantic padding), with the optional
// sigmoid gate of the QKVG form ("[perf] Harden Ulysses agreement and tune
// bounded H3 transfers", Problem and behavior: packed QKV/QKVG operands).
//
// Work decomposition: one workgroup of 8 waves = (segment, head, 384-query
// tile); it walks only the 64-key tiles of its own segment, so cross-segment
// blocks are never visited and only the last key tile of a segment needs a
// mask.  Segments are issued longest first.  Within a head the query tiles
// are consecutive workgroup ids, so the workgroups in flight stream the same
// K/V tiles and share them in L2 and the Infinity Cache.
//
// Per wave: 48 query rows as three 16-row blocks.  CDNA4's
// v_mfma_f32_16x16x32_bf16 takes A (16 rows x 32 k: lane l%16 owns row l%16,
// lane group l/16 owns 8 k slots), B (32 k x 16 columns, the same way) and
// leaves C with lane l%16 on column l%16 and rows 4*(l/16)..+3 in its four
// registers.  Every fragment a wave reads from LDS feeds the MFMAs of all
// three query blocks, so LDS bytes per MFMA FLOP are a third below a
// one-block-per-fragment tiling, at a register budget (O 96, Q 48, S 24)
// that still leaves two waves per SIMD.  Per 32-key step:
//   S^T = K Q^T      A = 16 keys x 32 channels of K (LDS), B = Q (registers):
//                    lane l holds query l%16 of each block against keys
//                    4*(l/16)..+3 of each 16-key half;
//   online softmax   base 2, log2(e) folded into the scale; the running max is
//                    raised only when a row's maximum exceeds it by more than
//                    2^8 (probabilities <= 256, exact in the normalisation),
//                    and the row maximum is only computed when a lane's
//                    partial row sum shows a probability of 2^7 or more;
//   O^T += V^T P^T   B = P^T straight from the S^T registers: MFMA k slot j of
//                    lane group g is key 4g+j (j < 4) or 16+4g+j-4, the order
//                    the C layout left them in; A = V^T (16 channels x those
//                    keys) from two gfx950 transposing LDS loads
//                    ds_read_b64_tr_b16 of a row-major V tile.
// The row sum of P comes from v_dot2 on the rounded bf16 P the MFMA consumes;
// each lane sums its own keys and the four lane groups of a query are added
// once at the end.
//
// K/V tiles move from HBM straight into LDS with the 128-bit buffer load to
// LDS (no VGPR staging), double buffered, one barrier per tile, the loop
// unrolled by two so buffer addresses are constants.  Wave w's i-th load
// fills tile rows 4(8i + w)..+3, lane l at 16-byte slot l.  16-byte chunk c
// of row r sits at chunk c ^ f(r), f(r) = 2*(r%8) + (r/8)%2.  Then the 16
// rows a 16-lane group reads at one logical chunk (K fragments), and the 8
// rows x 2 chunks a 32-lane half reads through the transposing load (V
// fragments), both hit 16 distinct 16-byte bank groups.  The swizzle is
// applied on the global side, because a direct load's LDS slot is fixed per
// lane.  Rows past the end of the segment are clamped to its last row
// (finite data, masked out or weighted by 0).
//
// Epilogue: each wave stages its output rows through LDS, 16 rows at a
// time, so that O is stored (and the gate G read) as whole 256-byte rows by
// 16 lanes each, instead of 8-byte pieces spread over 16 rows.
#include "h3_device.h"

namespace h3 {

namespace {

constexpr int kBN = 64;                            // keys per LDS tile
constexpr int kQB = 3;                             // 16-query blocks per wave
constexpr int kWaves = kAttnThreads / 64;          // 8
constexpr int kBlockM = 16 * kQB * kWaves;         // 384 queries per workgroup
constexpr int kTileElems = kBN * kD;               // one K or V tile
constexpr int kLoadsPerTile = kBN / (4 * kWaves);  // 16-byte direct loads per lane per operand
constexpr int kCB = kD / 16;                       // 16-channel blocks of the output
constexpr float kLazyRescale = 8.0f;               // log2 of the largest tolerated probability
constexpr float kMaxCheck = 128.0f;                // partial row sum that triggers the exact max (2^7 < 2^8)
static_assert(kLoadsPerTile * 4 * kWaves == kBN, "loads cover the tile");

__device__ __forceinline__ float xor_max(float v, int mask) {
    return __builtin_fmaxf(v, __shfl_xor(v, mask, 64));
}

}  // namespace

__global__ __launch_bounds__(kAttnThreads, 1) void k_packed_attn(AttnArgs a) {
    // Four distinct LDS objects (not one array of buffers) so the compiler can
    // prove that the direct loads into one buffer never alias the reads of the
    // other and does not serialise them with extra counter waits.
    __shared__ __attribute__((aligned(16))) uint16_t sK0[kTileElems];
    __shared__ __attribute__((aligned(16))) uint16_t sK1[kTileElems];
    __shared__ __attribute__((aligned(16))) uint16_t sV0[kTileElems];
    __shared__ __attribute__((aligned(16))) uint16_t sV1[kTileElems];
    __shared__ __attribute__((aligned(16))) uint16_t sO[kWaves * 16 * kD];   // epilogue staging, 4 KB per wave

    // ---- which (segment, head, query tile) this workgroup owns ----------------
    const int w = blockIdx.x;
    int lo = 0, hi = a.n_entries - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.wg_prefix[mid] <= w) lo = mid; else hi = mid - 1;
    }
    // Everything the kernel needs from the argument block, as scalars: the
    // lambdas below then never take the block's address (which would make the
    // compiler copy all of it to private memory).
    const int seg_len = a.seg_len[lo];
    const int seg_begin = a.seg_begin[lo];
    const int tiles = (seg_len + kBlockM - 1) / kBlockM;
    const int local = w - a.wg_prefix[lo];
    const int head = local / tiles;
    const int qtile = local - head * tiles;
    const uint32_t n_heads = a.n_heads;
    const float scale_log2 = a.scale_log2;
    float *const lse_out = a.lse;
    const uint64_t row_stride = (uint64_t)n_heads * kD;                      // elements per token
    const uint64_t base = (uint64_t)seg_begin * row_stride + (uint64_t)head * kD;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: load addresses are scalar
    const int lane = tid & 63;
    const int l16 = lane & 15;
    const int grp = lane >> 4;
    const int q0 = qtile * kBlockM + wave * (16 * kQB);       // first query row of this wave (segment-local)

    const uint16_t *qp = static_cast<const uint16_t *>(a.q) + base;
    const uint16_t *kp = static_cast<const uint16_t *>(a.k) + base;
    const uint16_t *vp = static_cast<const uint16_t *>(a.v) + base;

    // ---- the wave's query rows as the B operand of S^T = K Q^T -----------------
    // qreg[qb][ks] = Q[q0 + 16 qb + l16][16-byte chunk 4 grp + ks]: MFMA k step ks
    // gives lane group g the channels of chunk 4g + ks (any assignment shared by
    // K and Q is the same dot product; this one keeps the K reads free of LDS
    // bank conflicts, which chunk 4 ks + g is not)
    bf16x8 qreg[kQB][kD / 32];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        const int q = q0 + 16 * qb + l16;
        const bool valid = q < seg_len;
        const u32x4 *src = reinterpret_cast<const u32x4 *>(qp + (uint64_t)(valid ? q : 0) * row_stride);
#pragma unroll
        for (int ks = 0; ks < kD / 32; ++ks) {
            u32x4 v = src[4 * grp + ks];
            if (!valid) v = (u32x4){0u, 0u, 0u, 0u};
            qreg[qb][ks] = __builtin_bit_cast(bf16x8, v);
        }
    }

    // ---- per-lane LDS offsets (independent of the tile and of the key step) ---
    int k_off[kD / 32];                  // A operand of S^T: tile row l16 (+16 per key half), chunk 4grp + ks
#pragma unroll
    for (int ks = 0; ks < kD / 32; ++ks) k_off[ks] = tile16_off(l16, 4 * grp + ks);
    int v_off[kCB];                      // transposing reads: row 4 grp + l16/4 (+16), channels 16cb + 4(l16%4)
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
        const int r = 4 * grp + (l16 >> 2);
        const int col = 16 * cb + 4 * (l16 & 3);
        v_off[cb] = tile16_off(r, col >> 3) + (col & 7);
    }

    // ---- direct HBM -> LDS tile loads ------------------------------------------
    // load i of wave `wave` covers tile rows 4*(kWaves*i + wave) .. +3, lane l row +l/16;
    // f(row) does not depend on i because rows step by 4*kWaves (a multiple of 16).
    const int ld_row0 = 4 * wave + (lane >> 4);
    const int ld_chunk = (lane & 15) ^ tile16_f(ld_row0);
    const int n_kt = (seg_len + kBN - 1) / kBN;
    const int row_bytes = (int)(row_stride * 2);       // <= 256 heads * 256 B
    int ld_off[kLoadsPerTile];                          // byte offsets inside a full tile
#pragma unroll
    for (int i = 0; i < kLoadsPerTile; ++i) ld_off[i] = (ld_row0 + 4 * kWaves * i) * row_bytes + ld_chunk * 16;
    auto issue_tile = [&](int kt, uint16_t *dk, uint16_t *dv) __attribute__((always_inline)) {
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

    f32x4 acc[kCB][kQB];                 // O^T: channels 16cb + 4grp + r of query l16 of block qb
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) acc[cb][qb] = (f32x4){};
    float m_run[kQB], l_run[kQB];        // running max (log2 units) and this lane's share of the denominator
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        m_run[qb] = -__builtin_inff();
        l_run[qb] = 0.f;
    }
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

    // one 32-key step: keys 32*ks2 .. +31 of the tile in (tk, tv)
    auto key_step = [&](int kt, int ks2, const uint16_t *tk, const uint16_t *tv) __attribute__((always_inline)) {
        f32x4 s[2][kQB];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb) s[kb][qb] = (f32x4){};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int ks = 0; ks < kD / 32; ++ks) {
                const bf16x8 kf = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4 *>(tk + (32 * ks2 + 16 * kb) * kD + k_off[ks]));
#pragma unroll
                for (int qb = 0; qb < kQB; ++qb)
                    s[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qreg[qb][ks], s[kb][qb], 0, 0, 0);
            }
        // V^T fragments of the step: the first half now, so that it lands during
        // the softmax, the second half just before its MFMAs
        auto read_vf = [&](int cb) __attribute__((always_inline)) {
            const bf16x4 v0 = lds_read_tr(tv + (32 * ks2) * kD + v_off[cb]);
            const bf16x4 v1 = lds_read_tr(tv + (32 * ks2 + 16) * kD + v_off[cb]);
            return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        };
        bf16x8 vf[kCB];
#pragma unroll
        for (int cb = 0; cb < kCB / 2; ++cb) vf[cb] = read_vf(cb);
        // keys past the end of the segment (last tile only)
        if ((kt + 1) * kBN > seg_len) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int key = kt * kBN + 32 * ks2 + 16 * kb + 4 * grp + r;
                        if (key >= seg_len) s[kb][qb][r] = -__builtin_inff();
                    }
        }
        // online softmax (base 2) with lazy rescaling.  The probabilities are first
        // formed against the running max.  A probability of 2^7 or more, or the
        // NaN/inf of the first step (running max still -inf), makes a lane's
        // partial row sum reach 2^7 or fail the comparison; only then are the row
        // maxima computed, and only if one exceeds its running max by more than
        // 2^8 are the accumulators rescaled and the probabilities formed again.
        float psum[kQB];
        bf16x8 pb[kQB];
        auto form_p = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb) {
                uint32_t wds[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int kb = e >> 1, r = 2 * (e & 1);
                    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][r], scale_log2, -m_run[qb]));
                    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][r + 1], scale_log2, -m_run[qb]));
                    wds[e] = pack_bf16x2(p0, p1);
                }
                float ps = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wds[e]), ones, ps, false);
                psum[qb] = ps;
                pb[qb] = __builtin_bit_cast(bf16x8, (u32x4){wds[0], wds[1], wds[2], wds[3]});
            }
        };
        form_p();
        bool small = true;
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) small = small && (psum[qb] < kMaxCheck);
        if (__builtin_amdgcn_ballot_w64(!small) != 0) {
            float mx[kQB];
            bool raise = false;
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb) {
                float m = __builtin_fmaxf(__builtin_fmaxf(s[0][qb][0], s[0][qb][1]), __builtin_fmaxf(s[0][qb][2], s[0][qb][3]));
                m = __builtin_fmaxf(m, __builtin_fmaxf(__builtin_fmaxf(s[1][qb][0], s[1][qb][1]),
                                                       __builtin_fmaxf(s[1][qb][2], s[1][qb][3])));
                m = xor_max(xor_max(m, 16), 32);        // the four lane groups of the query
                mx[qb] = m * scale_log2;
                raise = raise || (mx[qb] > m_run[qb] + kLazyRescale);
            }
            if (__builtin_amdgcn_ballot_w64(raise) != 0) {
#pragma unroll
                for (int qb = 0; qb < kQB; ++qb) {
                    const float m_new = __builtin_fmaxf(m_run[qb], mx[qb]);
                    const float alpha = m_new == m_run[qb] ? 1.0f : __builtin_amdgcn_exp2f(m_run[qb] - m_new);
                    l_run[qb] *= alpha;
#pragma unroll
                    for (int cb = 0; cb < kCB; ++cb) acc[cb][qb] *= alpha;
                    m_run[qb] = m_new;
                }
                form_p();
            }
        }
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) l_run[qb] += psum[qb];

        // O^T += V^T P^T
#pragma unroll
        for (int cb = kCB / 2; cb < kCB; ++cb) vf[cb] = read_vf(cb);
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb)
                acc[cb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[cb], pb[qb], acc[cb][qb], 0, 0, 0);
    };
    auto compute_tile = [&](int kt, const uint16_t *tk, const uint16_t *tv) __attribute__((always_inline)) {
        key_step(kt, 0, tk, tv);
        key_step(kt, 1, tk, tv);
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
    // the four lane groups of a query hold disjoint keys: add their partial sums
    float inv[kQB];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 16, 64);
        l_tot += __shfl_xor(l_tot, 32, 64);
        inv[qb] = 1.0f / l_tot;
        const int q = q0 + 16 * qb + l16;
        if (lse_out && grp == 0 && q < seg_len) {
            // log-sum-exp of the scaled logits (natural log): the probabilities are
            // 2^(c*s - m_run) / l_tot, so lse * log2(e) = m_run + log2(l_tot)
            const float lse2 = m_run[qb] + __builtin_amdgcn_logf(l_tot);
            lse_out[((uint64_t)seg_begin + (uint64_t)q) * n_heads + head] = lse2 * 0.6931471805599453f;
        }
    }
    // Per 16-row block: the wave's staging area holds 16 rows of 256 bytes, chunk
    // c of row r at chunk c ^ r.  Lane l's outputs are channels 16cb + 4grp .. +3
    // of row l16, i.e. 8 bytes at chunk 2cb + grp/2, half grp%2: the 32 lanes of a
    // half-wave touch 16 rows at one chunk, all in distinct bank groups.  Rows go
    // to and from HBM whole: 16 lanes per 256-byte row, chunk l%16.
    uint16_t *stage = sO + wave * 16 * kD;
    uint16_t *op = static_cast<uint16_t *>(a.o) + base;
    const uint16_t *gp = a.g ? static_cast<const uint16_t *>(a.g) + base : nullptr;
    const int io_row = lane >> 4;                 // + 4 i: rows of the whole-row transfers
    const int io_chunk = lane & 15;
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        const int row0 = q0 + 16 * qb;            // segment-local query of staging row 0
        if (gp) {
            u32x4 gv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = io_row + 4 * i;
                const int q = row0 + r < seg_len ? row0 + r : seg_len - 1;
                gv[i] = *reinterpret_cast<const u32x4 *>(gp + (uint64_t)q * row_stride + io_chunk * 8);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = io_row + 4 * i;
                *reinterpret_cast<u32x4 *>(stage + r * kD + ((io_chunk ^ r) << 3)) = gv[i];
            }
        }
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb) {
            uint16_t *slot = stage + l16 * kD + (((2 * cb + (grp >> 1)) ^ l16) << 3) + 4 * (grp & 1);
            float y[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = acc[cb][qb][e] * inv[qb];
            if (gp) {
                const u32x2 gw = *reinterpret_cast<const u32x2 *>(slot);
                const float gf[4] = {bf16_lo(gw[0]), bf16_hi(gw[0]), bf16_lo(gw[1]), bf16_hi(gw[1])};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    // sigmoid(g) = 1 / (1 + 2^(-g * log2 e))
                    const float den = 1.0f + __builtin_amdgcn_exp2f(-gf[e] * 1.4426950408889634f);
                    y[e] = y[e] / den;
                }
            }
            *reinterpret_cast<u32x2 *>(slot) = (u32x2){pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = io_row + 4 * i;
            const u32x4 ov = *reinterpret_cast<const u32x4 *>(stage + r * kD + ((io_chunk ^ r) << 3));
            if (row0 + r < seg_len)
                *reinterpret_cast<u32x4 *>(op + (uint64_t)(row0 + r) * row_stride + io_chunk * 8) = ov;
        }
    }
}

int packed_attn_block_m() { return kBlockM; }

hipError_t launch_packed_attn(const AttnArgs &a, int n_workgroups, hipStream_t s) {
    if (n_workgroups <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_packed_attn, dim3(n_workgroups), dim3(kAttnThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace h3
