// relayout.hip -- the sequence-to-head and head-to-sequence relayouts of the
// Ulysses layout on one GPU ("Distributed H3 Execution", introduction: QKV
// sequence-to-head all-to-all before attention, the inverse after it).
//
// With P virtual ranks on one device the all-to-all is a permutation of
// 256-byte (token, head) rows.  For a fixed rank j and token t the rows of
// rank j's heads are one contiguous run of H_j*256 bytes on BOTH sides (the
// packed [N][K][H][D] row of plane p, and rank j's dense [N][H_j][D] buffer),
// so the kernel copies runs: each grid row y serves one rank, the rank side is
// a dense stream of 16-byte vectors, the packed side is runs at a fixed stride.
// Consecutive lanes touch consecutive 16-byte vectors on both sides (fully
// coalesced 128-bit accesses), every lane keeps kCopyUnroll loads in flight
// before its stores.  Every byte is read once and written once, so the loads
// and the rank-side stores carry non-temporal hints; the packed-side stores do
// not (see store_vec).  No LDS staging is needed: the smallest
// contiguous piece is a 256-byte row, four times the 64-byte HBM access unit.
#include "h3_device.h"

namespace h3 {

__device__ __forceinline__ uint32_t fast_udiv(uint32_t n, FastDiv f) {
    uint32_t q = __umulhi(n, f.m);
    return (q * f.d > n) ? q - 1 : q;
}

// Address of vector f of the selected rank's run sequence on the packed side.
__device__ __forceinline__ uint64_t packed_index(uint32_t f, FastDiv dv, uint32_t run, uint64_t stride,
                                                 uint32_t off) {
    const uint32_t t = fast_udiv(f, dv);
    return t * stride + off + (f - t * run);
}

// One 16-byte store.  The dense rank side streams with a non-temporal hint;
// the packed side (runs of H_j*256 bytes at the token stride) takes a plain
// store, which leaves the runs to the L2's write-back: head2seq measured 72%
// of the HBM peak with non-temporal stores there and 81% with plain ones,
// while plain stores on the rank side or plain loads of the packed side were
// slower.
template <bool kToRank>
__device__ __forceinline__ void store_vec(u32x4 *dst, uint64_t idx, u32x4 v) {
    if constexpr (kToRank) __builtin_nontemporal_store(v, dst + idx);
    else dst[idx] = v;
}

// kToRank = true : seq2head, packed side is the source.
// kToRank = false: head2seq, packed side is the destination.
template <bool kToRank>
__global__ __launch_bounds__(kCopyThreads) void k_relayout(RunCopyArgs a) {
    const int y = blockIdx.y;                         // grid row = selected rank slot
    const uint32_t run = a.run_vec[y];
    const uint32_t total = a.n_tokens * run;          // host guarantees < 2^31
    const uint32_t first = blockIdx.x * (uint32_t)(kCopyThreads * kCopyUnroll);
    if (first >= total) return;                       // shorter runs need fewer workgroups
    const FastDiv dv = a.div[y];
    const uint32_t off = a.off_vec[y];
    const uint64_t stride = a.stride_vec;
    const u32x4 *src = kToRank ? static_cast<const u32x4 *>(a.src_packed)
                               : static_cast<const u32x4 *>(a.src_rank[y]);
    u32x4 *dst = kToRank ? static_cast<u32x4 *>(a.dst_rank[y]) : static_cast<u32x4 *>(a.dst_packed);
    const uint32_t f0 = first + threadIdx.x;

    if (first + (uint32_t)(kCopyThreads * kCopyUnroll) <= total) {
        // whole workgroup in range: all loads in flight, then all stores
        u32x4 buf[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const uint32_t f = f0 + u * kCopyThreads;
            buf[u] = __builtin_nontemporal_load(src + (kToRank ? packed_index(f, dv, run, stride, off) : f));
        }
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const uint32_t f = f0 + u * kCopyThreads;
            store_vec<kToRank>(dst, kToRank ? f : packed_index(f, dv, run, stride, off), buf[u]);
        }
    } else {
        // ragged tail of the index range
        for (uint32_t f = f0; f < total; f += kCopyThreads) {
            const u32x4 v = __builtin_nontemporal_load(src + (kToRank ? packed_index(f, dv, run, stride, off) : f));
            store_vec<kToRank>(dst, kToRank ? f : packed_index(f, dv, run, stride, off), v);
        }
    }
}

static hipError_t launch_relayout(bool to_rank, const RunCopyArgs &a, int n_ranks, uint32_t max_run,
                                  hipStream_t s, int *grid_x) {
    const uint64_t total = (uint64_t)a.n_tokens * max_run;
    const uint64_t per_wg = (uint64_t)kCopyThreads * kCopyUnroll;
    const uint32_t gx = (uint32_t)((total + per_wg - 1) / per_wg);
    if (grid_x) *grid_x = (int)gx * n_ranks;
    if (gx == 0) return hipSuccess;
    if (to_rank)
        hipLaunchKernelGGL(k_relayout<true>, dim3(gx, n_ranks), dim3(kCopyThreads), 0, s, a);
    else
        hipLaunchKernelGGL(k_relayout<false>, dim3(gx, n_ranks), dim3(kCopyThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_seq2head(const RunCopyArgs &a, int n_ranks, uint32_t max_run, hipStream_t s,
                           int *grid_x) {
    return launch_relayout(true, a, n_ranks, max_run, s, grid_x);
}

hipError_t launch_head2seq(const RunCopyArgs &a, int n_ranks, uint32_t max_run, hipStream_t s,
                           int *grid_x) {
    return launch_relayout(false, a, n_ranks, max_run, s, grid_x);
}

}  // namespace h3
