// Streaming device copy: the library's own measure of the HBM rate a plain
// read-once / write-once kernel reaches on this GPU (the reference beside the
// published peak that the kernels' bandwidth fractions are compared with).
//
// One workgroup per 16 KiB tile (grid-stride only beyond 2^20 tiles): each
// thread issues its four 16-byte non-temporal loads, each wave's load covering
// 1 KiB contiguous, before its four stores. Measured on MI355X over 1 GiB:
// one tile per workgroup 6.36 TB/s (read + written), against 4.4-5.8 TB/s for
// persistent grid-stride forms and 5.2 TB/s for the runtime's device copy.
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

constexpr int kCopyUnroll = 4;
constexpr int64_t kCopyTile = 256 * kCopyUnroll;     // 16-byte pieces per workgroup tile

__global__ __launch_bounds__(256) void stream_copy_kernel(const i32x4 *__restrict__ src,
                                                          i32x4 *__restrict__ dst, int64_t n16)
{
    for (int64_t t0 = (int64_t)blockIdx.x * kCopyTile; t0 < n16; t0 += (int64_t)gridDim.x * kCopyTile) {
        if (t0 + kCopyTile <= n16) {
            i32x4 x[kCopyUnroll];
#pragma unroll
            for (int u = 0; u < kCopyUnroll; ++u)
                x[u] = __builtin_nontemporal_load(src + t0 + 256 * u + threadIdx.x);
#pragma unroll
            for (int u = 0; u < kCopyUnroll; ++u)
                __builtin_nontemporal_store(x[u], dst + t0 + 256 * u + threadIdx.x);
        } else {
            for (int64_t i = t0 + threadIdx.x; i < n16; i += 256) dst[i] = src[i];
        }
    }
}

hipError_t launch_stream_copy(const void *src, void *dst, size_t bytes, hipStream_t stream) {
    const int64_t n16 = (int64_t)(bytes / 16);
    if (n16 == 0) return hipSuccess;
    int64_t blocks = (n16 + kCopyTile - 1) / kCopyTile;
    if (blocks > ((int64_t)1 << 20)) blocks = (int64_t)1 << 20;
    stream_copy_kernel<<<(unsigned)blocks, 256, 0, stream>>>((const i32x4 *)src, (i32x4 *)dst, n16);
    return hipGetLastError();
}

}  // namespace kda
