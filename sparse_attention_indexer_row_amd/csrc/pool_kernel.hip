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

// Selection inside a block pool ("The Secret GPU Kernel Behind DeepSeek V4.1
// Flash", transcript 7:46-8:00): the layers above score only the pooled
// positions.  The selection kernel gives equal values to the earlier element
// of its row, so the pool is first laid out in ascending position order:
// one workgroup per row sorts the (block, slot) pairs by block with a
// bitonic network in LDS (empty slots last), records the sorted blocks, and
// copies each block's scores into that order.  Since the blocks are
// distinct and ascending, the positions along the gathered row increase
// strictly, so the scores below the row length form a prefix whose length
// is the selection's row length.  After the selection, a map turns gathered
// offsets back into context positions.
constexpr int kOrderThreads = 256;

__global__ __launch_bounds__(kOrderThreads) void pool_order_kernel(PooledArgs a, int p2) {
    extern __shared__ uint64_t sorted[];  // p2 words: block << 32 | slot
    __shared__ int32_t count;
    const int64_t r = (int64_t)a.row0 + blockIdx.x;
    const int tid = threadIdx.x;
    const int32_t *pi = a.pool_idx + r * (int64_t)a.keep;
    for (int i = tid; i < p2; i += kOrderThreads) {
        uint64_t w = ~0ull;
        if (i < a.keep) {
            const int32_t b = pi[i];
            w = ((uint64_t)(b < 0 ? 0xFFFFFFFFu : (uint32_t)b) << 32) | (uint32_t)i;
        }
        sorted[i] = w;
    }
    if (tid == 0) count = 0;
    __syncthreads();
    for (int size = 2; size <= p2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int t = tid; t < (p2 >> 1); t += kOrderThreads) {
                const int lo = ((t & ~(stride - 1)) << 1) | (t & (stride - 1));
                const int hi = lo + stride;
                const uint64_t x = sorted[lo], y = sorted[hi];
                const bool up = (lo & size) == 0;
                if ((x > y) == up) {
                    sorted[lo] = y;
                    sorted[hi] = x;
                }
            }
            __syncthreads();
        }
    }
    int64_t L = a.n;
    if (a.lengths) {
        const int64_t l = a.lengths[r];
        L = l < 0 ? 0 : (l > a.n ? a.n : l);
    }
    const int64_t g = a.group;
    int32_t *blk = a.blocks + r * (int64_t)a.keep;
    for (int i = tid; i < a.keep; i += kOrderThreads) {
        const uint32_t b = (uint32_t)(sorted[i] >> 32);
        blk[i] = b == 0xFFFFFFFFu ? -1 : (int32_t)b;
    }
    const float *ps = a.pool_scores + r * (int64_t)a.keep * g;
    float *out = a.gathered + r * a.ld;
    // keep * group < 2^31 (checked on the host): 32-bit offsets, and the
    // (slot, lane) pair of offset c advances by a fixed step per iteration,
    // so the loop divides nothing.
    const uint32_t total = (uint32_t)a.keep * (uint32_t)a.group;
    const uint32_t ug = (uint32_t)a.group;
    const uint32_t di = (uint32_t)kOrderThreads / ug, dj = (uint32_t)kOrderThreads % ug;
    uint32_t i = (uint32_t)tid / ug, j = (uint32_t)tid % ug;
    int mine = 0;
    for (uint32_t c = (uint32_t)tid; c < total; c += kOrderThreads) {
        const uint64_t w = sorted[i];
        const uint32_t b = (uint32_t)(w >> 32);
        if (b != 0xFFFFFFFFu && (int64_t)b * g + j < L) {
            out[c] = ps[(size_t)(uint32_t)w * ug + j];
            ++mine;
        }
        i += di;
        j += dj;
        if (j >= ug) {
            j -= ug;
            ++i;
        }
    }
    if (mine) atomicAdd(&count, mine);
    __syncthreads();
    if (tid == 0) a.valid[r] = count;
}

__global__ __launch_bounds__(256) void pool_positions_kernel(PooledArgs a) {
    const int64_t r = (int64_t)a.row0 + blockIdx.y;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= a.k) return;
    int32_t *idx = a.out_idx + r * (int64_t)a.k;
    const int32_t c = idx[t];
    if (c < 0) return;
    const uint32_t g = (uint32_t)a.group;
    const uint32_t i = (uint32_t)c / g;
    idx[t] = (int32_t)((uint32_t)a.blocks[r * (int64_t)a.keep + i] * g + ((uint32_t)c - i * g));
}

}  // namespace

hipError_t launch_pool_order(const PooledArgs &a, hipStream_t stream) {
    if (a.rows <= 0) return hipSuccess;
    int p2 = 1;
    while (p2 < a.keep) p2 <<= 1;
    if (p2 < 2) p2 = 2;
    hipLaunchKernelGGL(pool_order_kernel, dim3((unsigned)a.rows), dim3(kOrderThreads),
                       (size_t)p2 * 8, stream, a, p2);
    return hipGetLastError();
}

hipError_t launch_pool_positions(const PooledArgs &a, hipStream_t stream) {
    if (a.rows <= 0) return hipSuccess;
    const dim3 grid((unsigned)((a.k + 255) / 256), (unsigned)a.rows);
    hipLaunchKernelGGL(pool_positions_kernel, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

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
