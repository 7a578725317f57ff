// Block-max pooled pre-selection, first step ("The Secret GPU Kernel Behind
// DeepSeek V4.1 Flash", transcript 7:22-7:46): the layer that scores the
// whole context also groups positions into blocks, scores each block by its
// best position, and keeps the newest blocks unconditionally.
//
// One work item per block of a row.  It reduces the block's valid scores
// with the same order-preserving keys the selection uses (IEEE total order,
// -0.0 below +0.0), writes the block's best score to the block-maxima row,
// and, when the block is one of the row's newest `pinned`, also writes it
// straight to its output slot (newest first).  Work items past a short row's
// blocks fill its unused pinned slots with (-inf, -1).  The selection kernel
// then picks the best older blocks from the block-maxima rows and writes
// them behind the pinned slots.
//
// Traffic: each score is read once (coalesced: neighbouring work items read
// neighbouring blocks), each block writes one 4-byte maximum.
#include <hip/hip_runtime.h>

#include "common.h"
#include "internal.h"

namespace topk {
namespace {

constexpr int kPoolThreads = 256;

template <bool VEC>
__global__ __launch_bounds__(kPoolThreads) void block_max_kernel(PoolArgs a) {
    const int64_t r = (int64_t)a.row0 + blockIdx.y;
    const int64_t t = (int64_t)blockIdx.x * kPoolThreads + threadIdx.x;
    if (t >= a.span) return;
    int64_t L = a.n;
    if (a.lengths) {
        const int64_t l = a.lengths[r];
        L = l < 0 ? 0 : (l > a.n ? a.n : l);
    }
    const int64_t g = a.group;
    const int64_t nb = (L + g - 1) / g;
    const int64_t P = a.pinned < nb ? a.pinned : nb;
    float *ov = a.out_vals + r * (int64_t)a.keep;
    int32_t *oi = a.out_idx + r * (int64_t)a.keep;
    if (t == 0) a.older[r] = (int32_t)(nb - P);
    if (t >= P && t < a.pinned) {
        ov[t] = -__builtin_inff();
        oi[t] = -1;
    }
    if (t >= nb) return;

    const float *row = a.scores + r * a.n;
    const int64_t lo = t * g;
    const int64_t hi = lo + g < L ? lo + g : L;
    uint32_t best = 0u;  // below every non-NaN key; the block holds at least one position
    if constexpr (VEC) {
        // group % 4 == 0 and the row is 16-byte aligned: whole float4s, the
        // last one masked at L (it stays inside the row since n % 4 == 0).
        const float4 *p = reinterpret_cast<const float4 *>(row + lo);
        for (int64_t j = 0; lo + 4 * j < hi; ++j) {
            const float4 v = p[j];
            const int64_t q = lo + 4 * j;
            const uint32_t k0 = order_key(__float_as_uint(v.x));
            const uint32_t k1 = q + 1 < hi ? order_key(__float_as_uint(v.y)) : 0u;
            const uint32_t k2 = q + 2 < hi ? order_key(__float_as_uint(v.z)) : 0u;
            const uint32_t k3 = q + 3 < hi ? order_key(__float_as_uint(v.w)) : 0u;
            best = max(best, max(max(k0, k1), max(k2, k3)));
        }
    } else {
        for (int64_t q = lo; q < hi; ++q) best = max(best, order_key(__float_as_uint(row[q])));
    }
    const float bv = __uint_as_float(key_bits(best));
    a.bm[r * a.bm_ld + t] = bv;
    if (t >= nb - P) {
        const int64_t s = nb - 1 - t;
        ov[s] = bv;
        oi[s] = (int32_t)t;
    }
}

}  // namespace

hipError_t launch_block_max(const PoolArgs &a, hipStream_t stream) {
    if (a.rows <= 0 || a.span <= 0) return hipSuccess;
    const bool vec = a.group % 4 == 0 && a.n % 4 == 0 &&
                     reinterpret_cast<uintptr_t>(a.scores) % 16 == 0;
    const dim3 grid((unsigned)((a.span + kPoolThreads - 1) / kPoolThreads), (unsigned)a.rows);
    if (vec) {
        hipLaunchKernelGGL(block_max_kernel<true>, grid, dim3(kPoolThreads), 0, stream, a);
    } else {
        hipLaunchKernelGGL(block_max_kernel<false>, grid, dim3(kPoolThreads), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace topk
