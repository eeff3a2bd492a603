// adaln.hip -- per-segment AdaLN modulation and residual gating on one token
// interval ("Distributed H3 Execution", Partition Contract: the segment table
// is clipped to the rank's token interval and rebased before these ops).
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
#include "h3_internal.h"

namespace h3 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round two floats to bf16 (nearest even) and pack them, element 0 in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 f = {lo, hi};
    bf16x2 b = __builtin_convertvector(f, bf16x2);
    return __builtin_bit_cast(uint32_t, b);
}

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

template <int kVpl>   // exactly kVpl 16-byte vectors per lane: C = 512 * kVpl
__global__ __launch_bounds__(kAdalnThreads) void k_adaln_modulate(AdalnArgs a) {
    uint32_t row, seg;
    if (!row_and_segment(a, &row, &seg)) return;
    const int lane = threadIdx.x & 63;
    const uint32_t nv = a.channels >> 3;
    const u32x4 *x = static_cast<const u32x4 *>(a.x) + (uint64_t)row * nv + lane;
    const u32x4 *shift = static_cast<const u32x4 *>(a.shift) + (uint64_t)seg * nv + lane;
    const u32x4 *scale = static_cast<const u32x4 *>(a.scale) + (uint64_t)seg * nv + lane;
    u32x4 *y = static_cast<u32x4 *>(a.y) + (uint64_t)row * nv + lane;

    u32x4 xv[kVpl], sh[kVpl], sc[kVpl];
#pragma unroll
    for (int i = 0; i < kVpl; ++i) xv[i] = __builtin_nontemporal_load(x + i * 64);
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
    const float inv_c = 1.0f / (float)a.channels;
    const float mean = wave_sum(s) * inv_c;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < kVpl; ++i)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float d0 = bf16_lo(xv[i][w]) - mean, d1 = bf16_hi(xv[i][w]) - mean;
            q += d0 * d0 + d1 * d1;
        }
    const float rstd = __builtin_amdgcn_rsqf(wave_sum(q) * inv_c + a.eps);
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
    for (int i = 0; i < kVpl; ++i) {
        u32x4 out;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float y0 = bf16_lo(xv[i][w]) + bf16_lo(gv[i][w]) * bf16_lo(bv[i][w]);
            const float y1 = bf16_hi(xv[i][w]) + bf16_hi(gv[i][w]) * bf16_hi(bv[i][w]);
            out[w] = pack_bf16x2(y0, y1);
        }
        __builtin_nontemporal_store(out, y + i * 64);
    }
}

// Any multiple of 8 channels: strided loop over the row, x read twice for
// modulation (mean pass, variance pass) and once more for the output.
__global__ __launch_bounds__(kAdalnThreads) void k_adaln_generic(AdalnArgs a) {
    uint32_t row, seg;
    if (!row_and_segment(a, &row, &seg)) return;
    const int lane = threadIdx.x & 63;
    const uint32_t nv = a.channels >> 3;
    const u32x4 *x = static_cast<const u32x4 *>(a.x) + (uint64_t)row * nv;
    u32x4 *y = static_cast<u32x4 *>(a.y) + (uint64_t)row * nv;
    if (a.mode == H3_ADALN_MODULATE) {
        const u32x4 *shift = static_cast<const u32x4 *>(a.shift) + (uint64_t)seg * nv;
        const u32x4 *scale = static_cast<const u32x4 *>(a.scale) + (uint64_t)seg * nv;
        const float inv_c = 1.0f / (float)a.channels;
        float s = 0.f;
        for (uint32_t c = lane; c < nv; c += 64) {
            const u32x4 v = x[c];
            for (int w = 0; w < 4; ++w) s += bf16_lo(v[w]) + bf16_hi(v[w]);
        }
        const float mean = wave_sum(s) * inv_c;
        float q = 0.f;
        for (uint32_t c = lane; c < nv; c += 64) {
            const u32x4 v = x[c];
            for (int w = 0; w < 4; ++w) {
                const float d0 = bf16_lo(v[w]) - mean, d1 = bf16_hi(v[w]) - mean;
                q += d0 * d0 + d1 * d1;
            }
        }
        const float rstd = __builtin_amdgcn_rsqf(wave_sum(q) * inv_c + a.eps);
        for (uint32_t c = lane; c < nv; c += 64) {
            const u32x4 v = x[c], sc = scale[c], sh = shift[c];
            u32x4 out;
            for (int w = 0; w < 4; ++w)
                out[w] = pack_bf16x2((bf16_lo(v[w]) - mean) * rstd * (1.0f + bf16_lo(sc[w])) + bf16_lo(sh[w]),
                                     (bf16_hi(v[w]) - mean) * rstd * (1.0f + bf16_hi(sc[w])) + bf16_hi(sh[w]));
            y[c] = out;
        }
    } else {
        const u32x4 *b = static_cast<const u32x4 *>(a.branch) + (uint64_t)row * nv;
        const u32x4 *gate = static_cast<const u32x4 *>(a.gate) + (uint64_t)seg * nv;
        for (uint32_t c = lane; c < nv; c += 64) {
            const u32x4 v = x[c], bv = b[c], gv = gate[c];
            u32x4 out;
            for (int w = 0; w < 4; ++w)
                out[w] = pack_bf16x2(bf16_lo(v[w]) + bf16_lo(gv[w]) * bf16_lo(bv[w]),
                                     bf16_hi(v[w]) + bf16_hi(gv[w]) * bf16_hi(bv[w]));
            y[c] = out;
        }
    }
}

template <int kVpl>
static void launch_exact(const AdalnArgs &a, dim3 grid, hipStream_t s) {
    if (a.mode == H3_ADALN_MODULATE)
        hipLaunchKernelGGL(k_adaln_modulate<kVpl>, grid, dim3(kAdalnThreads), 0, s, a);
    else
        hipLaunchKernelGGL(k_adaln_gate<kVpl>, grid, dim3(kAdalnThreads), 0, s, a);
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
