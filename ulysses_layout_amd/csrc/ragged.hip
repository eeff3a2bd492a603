// ragged.hip -- the ragged collectives of the token-sharded blocks, on one
// device with the P ranks as separate buffers ("Distributed H3 Execution",
// Partition Contract: tensor mode's ragged reduce-scatter, which sums the
// ranks' partial outputs, assigns token rows by the quotient/remainder split
// and adds the projection bias once after the reduction; introduction: the
// temporary padding of a ragged row gather is removed before model ops).
//
// Both are streams of 16-byte vectors over row-contiguous ranges: rank i's
// rows [a_i, b_i) are one contiguous run of (b_i - a_i) * C / 8 vectors in
// every [N][C] buffer.  Grid row y serves one rank; consecutive lanes touch
// consecutive vectors, with non-temporal hints because every byte is used
// once.
//   k_reduce_scatter  out_i[f] = bf16(sum_j partial_j[a_i C/8 + f] + bias[c(f)]),
//                     fp32 sum in rank order j = 0..P-1, one rounding.  Each
//                     lane keeps kRsVec vectors of accumulators and the rank
//                     loop is unrolled so that several ranks' loads are in
//                     flight together.
//   k_gather_rows     dst[a_i C/8 + f] = shard_i[f]: the rank's rows land at
//                     their global position, so any padding after a shard's
//                     N_i rows is never read.
#include "h3_device.h"

namespace h3 {

namespace {

// f mod nv for f < 2^31 (nv == 1 needs no division)
__device__ __forceinline__ uint32_t vec_channel(uint32_t f, const RaggedArgs &a) {
    if (a.nv_row == 1) return 0;
    uint32_t q = __umulhi(f, a.div_row.m);
    if (q * a.nv_row > f) --q;
    return f - q * a.nv_row;
}

__device__ __forceinline__ void add_vec(float (&acc)[8], u32x4 v) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        acc[2 * w] += bf16_lo(v[w]);
        acc[2 * w + 1] += bf16_hi(v[w]);
    }
}

__device__ __forceinline__ u32x4 finish_vec(const float (&acc)[8], const u32x4 *bias, uint32_t f,
                                            const RaggedArgs &a) {
    u32x4 out;
    if (bias) {
        const u32x4 bv = bias[vec_channel(f, a)];
#pragma unroll
        for (int w = 0; w < 4; ++w) out[w] = pack_bf16x2(acc[2 * w] + bf16_lo(bv[w]), acc[2 * w + 1] + bf16_hi(bv[w]));
    } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) out[w] = pack_bf16x2(acc[2 * w], acc[2 * w + 1]);
    }
    return out;
}

}  // namespace

__global__ __launch_bounds__(kCopyThreads) void k_reduce_scatter(RaggedArgs a) {
    const int y = blockIdx.y;
    const uint32_t total = a.n_vec[y];                // host guarantees < 2^31
    const uint32_t first = blockIdx.x * (uint32_t)(kCopyThreads * kRsVec);
    if (first >= total) return;                       // smaller ranks need fewer workgroups
    const uint64_t base = a.row_vec0[y];
    const u32x4 *bias = static_cast<const u32x4 *>(a.bias);
    u32x4 *out = static_cast<u32x4 *>(a.dst[y]);
    const uint32_t f0 = first + threadIdx.x;
    float acc[kRsVec][8];
#pragma unroll
    for (int u = 0; u < kRsVec; ++u)
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[u][k] = 0.f;

    if (first + (uint32_t)(kCopyThreads * kRsVec) <= total) {
        // whole workgroup in range
#pragma unroll 2
        for (int j = 0; j < a.world; ++j) {
            const u32x4 *p = static_cast<const u32x4 *>(a.src[j]) + base;
            u32x4 v[kRsVec];
#pragma unroll
            for (int u = 0; u < kRsVec; ++u) v[u] = __builtin_nontemporal_load(p + f0 + u * kCopyThreads);
#pragma unroll
            for (int u = 0; u < kRsVec; ++u) add_vec(acc[u], v[u]);
        }
#pragma unroll
        for (int u = 0; u < kRsVec; ++u) {
            const uint32_t f = f0 + u * kCopyThreads;
            __builtin_nontemporal_store(finish_vec(acc[u], bias, f, a), out + f);
        }
    } else {
        // ragged tail of the rank's range
        for (int u = 0; u < kRsVec; ++u) {
            const uint32_t f = f0 + u * kCopyThreads;
            if (f >= total) break;
            for (int j = 0; j < a.world; ++j)
                add_vec(acc[u], __builtin_nontemporal_load(static_cast<const u32x4 *>(a.src[j]) + base + f));
            __builtin_nontemporal_store(finish_vec(acc[u], bias, f, a), out + f);
        }
    }
}

__global__ __launch_bounds__(kCopyThreads) void k_gather_rows(RaggedArgs a) {
    const int y = blockIdx.y;
    const uint32_t total = a.n_vec[y];
    const uint32_t first = blockIdx.x * (uint32_t)(kCopyThreads * kCopyUnroll);
    if (first >= total) return;
    const u32x4 *src = static_cast<const u32x4 *>(a.src[y]);
    u32x4 *dst = static_cast<u32x4 *>(a.dst_all) + a.row_vec0[y];
    const uint32_t f0 = first + threadIdx.x;
    if (first + (uint32_t)(kCopyThreads * kCopyUnroll) <= total) {
        u32x4 buf[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) buf[u] = __builtin_nontemporal_load(src + f0 + u * kCopyThreads);
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) __builtin_nontemporal_store(buf[u], dst + f0 + u * kCopyThreads);
    } else {
        for (uint32_t f = f0; f < total; f += kCopyThreads)
            __builtin_nontemporal_store(__builtin_nontemporal_load(src + f), dst + f);
    }
}

hipError_t launch_reduce_scatter(const RaggedArgs &a, int n_slots, uint32_t max_vec, hipStream_t s, int *grid_x) {
    const uint64_t per_wg = (uint64_t)kCopyThreads * kRsVec;
    const uint32_t gx = (uint32_t)((max_vec + per_wg - 1) / per_wg);
    if (grid_x) *grid_x = (int)gx * n_slots;
    if (gx == 0) return hipSuccess;
    hipLaunchKernelGGL(k_reduce_scatter, dim3(gx, n_slots), dim3(kCopyThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_gather_rows(const RaggedArgs &a, int n_slots, uint32_t max_vec, hipStream_t s, int *grid_x) {
    const uint64_t per_wg = (uint64_t)kCopyThreads * kCopyUnroll;
    const uint32_t gx = (uint32_t)((max_vec + per_wg - 1) / per_wg);
    if (grid_x) *grid_x = (int)gx * n_slots;
    if (gx == 0) return hipSuccess;
    hipLaunchKernelGGL(k_gather_rows, dim3(gx, n_slots), dim3(kCopyThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace h3
