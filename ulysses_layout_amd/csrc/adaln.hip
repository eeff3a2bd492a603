// adaln.hip -- per-segment AdaLN modulation and residual gating on one token
// interval ("Distributed H3 Execution", Partition Contract: local row i is
// global token a + i, each segment intersected with [a, b) and shifted by
// -a), and the two chained: one sub-block's gated residual, modulated at once
// by the next sub-block's parameters, so x and the branch are read once and
// the residual never has to be read back (the modulation takes the fp32
// residual from registers; only the stored copy is rounded to bf16).
//
// One wave64 owns one row of C channels.  When C is a multiple of 512 (H3:
// 7168 = 14 x 512) every lane owns exactly C/512 16-byte vectors of the row:
// the wave issues all its 128-bit non-temporal loads of x (and of the branch
// for gating) together with the loads of the segment's parameter rows (small,
// [S][C], L2-resident), reduces the mean and then the centred second moment
// with in-wave butterflies (no LDS, no second HBM pass over x), and writes the
// row once.  Other multiples of 8 take a generic path that re-reads the row.
// The segment of a row comes from the clipped table in the kernel arguments
// by a wave-uniform binary search.
#include "h3_device.h"

namespace h3 {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// Wave-uniform row of this wave and the global segment of that row.
__device__ __forceinline__ bool row_and_segment(const AdalnArgs &a, uint32_t *row, uint32_t *seg) {
    const uint32_t r = __builtin_amdgcn_readfirstlane(blockIdx.x * (kAdalnThreads / 64) + (threadIdx.x >> 6));
    if (r >= a.n_rows) return false;
    int lo = 0, hi = a.n_entries - 1;          // last entry e with entry_begin[e] <= r
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((uint32_t)a.entry_begin[mid] <= r) lo = mid; else hi = mid - 1;
    }
    *row = r;
    *seg = (uint32_t)a.entry_seg[lo];
    return true;
}

// x + gate * b for the 8 channels of one 16-byte vector, rounded to bf16.
__device__ __forceinline__ u32x4 gate_vec(u32x4 x, u32x4 g, u32x4 b) {
    u32x4 out;
#pragma unroll
    for (int w = 0; w < 4; ++w)
        out[w] = pack_bf16x2(bf16_lo(x[w]) + bf16_lo(g[w]) * bf16_lo(b[w]),
                             bf16_hi(x[w]) + bf16_hi(g[w]) * bf16_hi(b[w]));
    return out;
}

// LayerNorm of the row this wave holds in xv (lane owns vectors lane + 64 i),
// statistics in fp32, then * (1 + scale) + shift, stored to y.  The plain
// modulation and the gated chain both run this, so they give the same bits.
template <int kVpl>
__device__ __forceinline__ void modulate_store(const u32x4 (&xv)[kVpl], const u32x4 *shift, const u32x4 *scale,
                                               u32x4 *y, uint32_t channels, float eps) {
    u32x4 sh[kVpl], sc[kVpl];
#pragma unroll
    for (int i = 0; i < kVpl; ++i) {
        sc[i] = scale[i * 64];
        sh[i] = shift[i * 64];
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kVpl; ++i)
#pragma unroll
        for (int w = 0; w < 4; ++w) s += bf16_lo(xv[i][w]) + bf16_hi(xv[i][w]);
    const float inv_c = 1.0f / (float)channels;
    const float mean = wave_sum(s) * inv_c;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < kVpl; ++i)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float d0 = bf16_lo(xv[i][w]) - mean, d1 = bf16_hi(xv[i][w]) - mean;
            q += d0 * d0 + d1 * d1;
        }
    const float rstd = __builtin_amdgcn_rsqf(wave_sum(q) * inv_c + eps);
#pragma unroll
    for (int i = 0; i < kVpl; ++i) {
        u32x4 out;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float y0 = (bf16_lo(xv[i][w]) - mean) * rstd * (1.0f + bf16_lo(sc[i][w])) + bf16_lo(sh[i][w]);
            const float y1 = (bf16_hi(xv[i][w]) - mean) * rstd * (1.0f + bf16_hi(sc[i][w])) + bf16_hi(sh[i][w]);
            out[w] = pack_bf16x2(y0, y1);
        }
        __builtin_nontemporal_store(out, y + i * 64);
    }
}

template <int kVpl>   // exactly kVpl 16-byte vectors per lane: C = 512 * kVpl
__global__ __launch_bounds__(kAdalnThreads) void k_adaln_modulate(AdalnArgs a) {
    uint32_t row, seg;
    if (!row_and_segment(a, &row, &seg)) return;
    const int lane = threadIdx.x & 63;
    const uint32_t nv = a.channels >> 3;
    const u32x4 *x = static_cast<const u32x4 *>(a.x) + (uint64_t)row * nv + lane;
    u32x4 xv[kVpl];
#pragma unroll
    for (int i = 0; i < kVpl; ++i) xv[i] = __builtin_nontemporal_load(x + i * 64);
    modulate_store<kVpl>(xv, static_cast<const u32x4 *>(a.shift) + (uint64_t)seg * nv + lane,
                         static_cast<const u32x4 *>(a.scale) + (uint64_t)seg * nv + lane,
                         static_cast<u32x4 *>(a.y) + (uint64_t)row * nv + lane, a.channels, a.eps);
}

// The gated residual r = x + gate[s] * b (stored rounded to bf16) and the
// modulation of r, taken in fp32 from registers, with the next sub-block's
// shift[s] / scale[s].  The statistics and the output take the order of
// modulate_store, so a residual that is exactly x (zero gate) gives the bits
// of the plain modulation.
template <int kVpl>
__global__ __launch_bounds__(kAdalnThreads) void k_adaln_gate_modulate(AdalnArgs a) {
    uint32_t row, seg;
    if (!row_and_segment(a, &row, &seg)) return;
    const int lane = threadIdx.x & 63;
    const uint32_t nv = a.channels >> 3;
    const uint64_t ro = (uint64_t)row * nv + lane, so = (uint64_t)seg * nv + lane;
    const u32x4 *x = static_cast<const u32x4 *>(a.x) + ro;
    const u32x4 *b = static_cast<const u32x4 *>(a.branch) + ro;
    const u32x4 *gate = static_cast<const u32x4 *>(a.gate) + so;
    const u32x4 *shift = static_cast<const u32x4 *>(a.shift) + so;
    const u32x4 *scale = static_cast<const u32x4 *>(a.scale) + so;
    u32x4 *resid = static_cast<u32x4 *>(a.resid) + ro;
    u32x4 *y = static_cast<u32x4 *>(a.y) + ro;
    float r[kVpl][8];
    float s = 0.f;
    {
        u32x4 xv[kVpl], bv[kVpl], gv[kVpl];
#pragma unroll
        for (int i = 0; i < kVpl; ++i) {
            xv[i] = __builtin_nontemporal_load(x + i * 64);
            bv[i] = __builtin_nontemporal_load(b + i * 64);
            gv[i] = gate[i * 64];
        }
#pragma unroll
        for (int i = 0; i < kVpl; ++i) {
            u32x4 out;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                r[i][2 * w] = bf16_lo(xv[i][w]) + bf16_lo(gv[i][w]) * bf16_lo(bv[i][w]);
                r[i][2 * w + 1] = bf16_hi(xv[i][w]) + bf16_hi(gv[i][w]) * bf16_hi(bv[i][w]);
                out[w] = pack_bf16x2(r[i][2 * w], r[i][2 * w + 1]);
                s += r[i][2 * w] + r[i][2 * w + 1];
            }
            __builtin_nontemporal_store(out, resid + i * 64);
        }
    }
    const float inv_c = 1.0f / (float)a.channels;
    const float mean = wave_sum(s) * inv_c;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < kVpl; ++i)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float d0 = r[i][2 * w] - mean, d1 = r[i][2 * w + 1] - mean;
            q += d0 * d0 + d1 * d1;
        }
    const float rstd = __builtin_amdgcn_rsqf(wave_sum(q) * inv_c + a.eps);
#pragma unroll
    for (int i = 0; i < kVpl; ++i) {
        const u32x4 sc = scale[i * 64], sh = shift[i * 64];
        u32x4 out;
#pragma unroll
        for (int w = 0; w < 4; ++w)
            out[w] = pack_bf16x2((r[i][2 * w] - mean) * rstd * (1.0f + bf16_lo(sc[w])) + bf16_lo(sh[w]),
                                 (r[i][2 * w + 1] - mean) * rstd * (1.0f + bf16_hi(sc[w])) + bf16_hi(sh[w]));
        __builtin_nontemporal_store(out, y + i * 64);
    }
}

template <int kVpl>
__global__ __launch_bounds__(kAdalnThreads) void k_adaln_gate(AdalnArgs a) {
    uint32_t row, seg;
    if (!row_and_segment(a, &row, &seg)) return;
    const int lane = threadIdx.x & 63;
    const uint32_t nv = a.channels >> 3;
    const u32x4 *x = static_cast<const u32x4 *>(a.x) + (uint64_t)row * nv + lane;
    const u32x4 *b = static_cast<const u32x4 *>(a.branch) + (uint64_t)row * nv + lane;
    const u32x4 *gate = static_cast<const u32x4 *>(a.gate) + (uint64_t)seg * nv + lane;
    u32x4 *y = static_cast<u32x4 *>(a.y) + (uint64_t)row * nv + lane;
    u32x4 xv[kVpl], bv[kVpl], gv[kVpl];
#pragma unroll
    for (int i = 0; i < kVpl; ++i) {
        xv[i] = __builtin_nontemporal_load(x + i * 64);
        bv[i] = __builtin_nontemporal_load(b + i * 64);
        gv[i] = gate[i * 64];
    }
#pragma unroll
    for (int i = 0; i < kVpl; ++i) __builtin_nontemporal_store(gate_vec(xv[i], gv[i], bv[i]), y + i * 64);
}

// Any multiple of 8 channels: strided loop over the row.  Modulation reads
// its input three times (mean pass, variance pass, output pass); in the chain
// that input is the fp32 gated residual, recomputed from x, b and gate on
// each pass (the same values every time), and stored rounded in the first.
__global__ __launch_bounds__(kAdalnThreads) void k_adaln_generic(AdalnArgs a) {
    uint32_t row, seg;
    if (!row_and_segment(a, &row, &seg)) return;
    const int lane = threadIdx.x & 63;
    const uint32_t nv = a.channels >> 3;
    const u32x4 *x = static_cast<const u32x4 *>(a.x) + (uint64_t)row * nv;
    u32x4 *y = static_cast<u32x4 *>(a.y) + (uint64_t)row * nv;
    const bool gated = a.mode != H3_ADALN_MODULATE;
    const u32x4 *b = gated ? static_cast<const u32x4 *>(a.branch) + (uint64_t)row * nv : nullptr;
    const u32x4 *gate = gated ? static_cast<const u32x4 *>(a.gate) + (uint64_t)seg * nv : nullptr;
    if (a.mode == H3_ADALN_GATE_RESIDUAL) {
        for (uint32_t c = lane; c < nv; c += 64) y[c] = gate_vec(x[c], gate[c], b[c]);
        return;
    }
    const bool chain = a.mode == H3_ADALN_GATE_MODULATE;
    u32x4 *resid = chain ? static_cast<u32x4 *>(a.resid) + (uint64_t)row * nv : nullptr;
    // the 8 fp32 input values of vector c
    auto in = [&](uint32_t c, float (&v)[8]) {
        const u32x4 xv = x[c];
        if (chain) {
            const u32x4 bv = b[c], gv = gate[c];
            for (int w = 0; w < 4; ++w) {
                v[2 * w] = bf16_lo(xv[w]) + bf16_lo(gv[w]) * bf16_lo(bv[w]);
                v[2 * w + 1] = bf16_hi(xv[w]) + bf16_hi(gv[w]) * bf16_hi(bv[w]);
            }
        } else {
            for (int w = 0; w < 4; ++w) {
                v[2 * w] = bf16_lo(xv[w]);
                v[2 * w + 1] = bf16_hi(xv[w]);
            }
        }
    };
    const u32x4 *shift = static_cast<const u32x4 *>(a.shift) + (uint64_t)seg * nv;
    const u32x4 *scale = static_cast<const u32x4 *>(a.scale) + (uint64_t)seg * nv;
    const float inv_c = 1.0f / (float)a.channels;
    float s = 0.f;
    for (uint32_t c = lane; c < nv; c += 64) {
        float v[8];
        in(c, v);
        if (chain) {
            u32x4 out;
            for (int w = 0; w < 4; ++w) out[w] = pack_bf16x2(v[2 * w], v[2 * w + 1]);
            resid[c] = out;
        }
        for (int k = 0; k < 8; k += 2) s += v[k] + v[k + 1];
    }
    const float mean = wave_sum(s) * inv_c;
    float q = 0.f;
    for (uint32_t c = lane; c < nv; c += 64) {
        float v[8];
        in(c, v);
        for (int k = 0; k < 8; k += 2) {
            const float d0 = v[k] - mean, d1 = v[k + 1] - mean;
            q += d0 * d0 + d1 * d1;
        }
    }
    const float rstd = __builtin_amdgcn_rsqf(wave_sum(q) * inv_c + a.eps);
    for (uint32_t c = lane; c < nv; c += 64) {
        float v[8];
        in(c, v);
        const u32x4 sc = scale[c], sh = shift[c];
        u32x4 out;
        for (int w = 0; w < 4; ++w)
            out[w] = pack_bf16x2((v[2 * w] - mean) * rstd * (1.0f + bf16_lo(sc[w])) + bf16_lo(sh[w]),
                                 (v[2 * w + 1] - mean) * rstd * (1.0f + bf16_hi(sc[w])) + bf16_hi(sh[w]));
        y[c] = out;
    }
}

template <int kVpl>
static void launch_exact(const AdalnArgs &a, dim3 grid, hipStream_t s) {
    if (a.mode == H3_ADALN_MODULATE)
        hipLaunchKernelGGL(k_adaln_modulate<kVpl>, grid, dim3(kAdalnThreads), 0, s, a);
    else if (a.mode == H3_ADALN_GATE_RESIDUAL)
        hipLaunchKernelGGL(k_adaln_gate<kVpl>, grid, dim3(kAdalnThreads), 0, s, a);
    else
        hipLaunchKernelGGL(k_adaln_gate_modulate<kVpl>, grid, dim3(kAdalnThreads), 0, s, a);
}

hipError_t launch_adaln(const AdalnArgs &a, hipStream_t s, int *grid_x) {
    const uint32_t rows_per_wg = kAdalnThreads / 64;
    const uint32_t gx = (a.n_rows + rows_per_wg - 1) / rows_per_wg;
    if (grid_x) *grid_x = (int)gx;
    if (gx == 0) return hipSuccess;
    const dim3 grid(gx);
    const uint32_t nv = a.channels >> 3;
    const uint32_t vpl = (nv % 64 == 0) ? nv / 64 : 0;
    switch (vpl) {
        case 1: launch_exact<1>(a, grid, s); break;
        case 2: launch_exact<2>(a, grid, s); break;
        case 4: launch_exact<4>(a, grid, s); break;
        case 6: launch_exact<6>(a, grid, s); break;
        case 8: launch_exact<8>(a, grid, s); break;
        case 12: launch_exact<12>(a, grid, s); break;
        case 14: launch_exact<14>(a, grid, s); break;
        case 16: launch_exact<16>(a, grid, s); break;
        default: hipLaunchKernelGGL(k_adaln_generic, grid, dim3(kAdalnThreads), 0, s, a); break;
    }
    return hipGetLastError();
}

}  // namespace h3
