// Kernels of the block-max pool, of the per-row radix selection, and of
// selection inside a pool.
//
// Block maxima ("The Secret GPU Kernel Behind DeepSeek V4.1 Flash",
// transcript 7:22-7:46: the layer that scores the whole context also groups
// positions into blocks, scores each block by its best position, and keeps
// the newest blocks unconditionally).  One work item per block of a row (or,
// for blocks of 8 on aligned rows, one float4 per lane with lane pairs
// combining): the block's valid scores are reduced with the library's
// order-preserving keys (IEEE total order, -0.0 below +0.0), the best is
// written to the block-maxima row and, for the row's newest `pinned` blocks,
// straight to its output slot (newest first); unused pinned slots of short
// rows get (-inf, -1).  Traffic: each score read once, one 4-byte maximum
// written per block.
//
// Radix selection: the exact best k of each row by the 64-bit (key,
// position) words, one workgroup per row (a sampled estimate, one admission
// pass into LDS, an 11-bit-digit search in LDS, and a sort of the winners
// in register runs).  It picks the pool's best older blocks from the
// block-maxima rows, serves topk_select_radix, and, with words that carry
// context positions, selection inside a pool ("The Secret GPU Kernel Behind
// DeepSeek V4.1 Flash", transcript 7:46-8:00).
#include <hip/hip_runtime.h>

#include "common.h"
#include "internal.h"
#include "wave_sort.h"

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

// Blocks of 8 on 16-byte aligned rows (n % 4 == 0): every lane reads one
// float4, so a wave's load instruction covers 1 KiB of the row, with two
// nontemporal loads per thread (the scores are read once); a workgroup
// covers 8 KiB and the chip keeps many small workgroups in flight.  On 128
// rows of 1M scores the block-max pass plus selection took 147.9 us with
// eight loads per thread, 143.9 with four, 139.8 with two and 152.9 with
// one: fewer loads outstanding per compute unit read faster, down to the
// point where the workgroups' fixed costs take over.  The two lanes holding
// a block's halves combine their maxima with one shuffle, and the even lane
// writes.  Work item f is the row's f-th float4; block b = f / 2.
constexpr int kPool8Unroll = 2;

__global__ __launch_bounds__(kPoolThreads) void block_max8_kernel(PoolArgs a) {
    const int64_t r = (int64_t)a.row0 + blockIdx.y;
    int64_t L = a.n;
    if (a.lengths) {
        const int64_t l = a.lengths[r];
        L = l < 0 ? 0 : (l > a.n ? a.n : l);
    }
    const int64_t nb = (L + 7) / 8;
    const int64_t P = a.pinned < nb ? a.pinned : nb;
    float *ov = a.out_vals + r * (int64_t)a.keep;
    int32_t *oi = a.out_idx + r * (int64_t)a.keep;
    const float4 *row4 = reinterpret_cast<const float4 *>(a.scores + r * a.n);
    const int64_t base = (int64_t)blockIdx.x * (kPoolThreads * kPool8Unroll) + threadIdx.x;
    if (base == 0) a.older[r] = (int32_t)(nb - P);
    float4 v[kPool8Unroll];
#pragma unroll
    for (int u = 0; u < kPool8Unroll; ++u) {
        const int64_t f = base + (int64_t)u * kPoolThreads;
        v[u] = 4 * f < L ? load_stream4(reinterpret_cast<const float *>(row4 + f))
                         : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < kPool8Unroll; ++u) {
        const int64_t f = base + (int64_t)u * kPoolThreads;
        const int64_t q = 4 * f;
        uint32_t m = 0u;  // below every non-NaN key
        if (q < L) m = order_key(__float_as_uint(v[u].x));
        if (q + 1 < L) m = max(m, order_key(__float_as_uint(v[u].y)));
        if (q + 2 < L) m = max(m, order_key(__float_as_uint(v[u].z)));
        if (q + 3 < L) m = max(m, order_key(__float_as_uint(v[u].w)));
        m = max(m, (uint32_t)__shfl_xor((int)m, 1));
        const int64_t b = f >> 1;
        if ((f & 1) == 0) {
            if (b < nb) {
                const float bv = __uint_as_float(key_bits(m));
                a.bm[r * a.bm_ld + b] = bv;
                if (b >= nb - P) {
                    ov[nb - 1 - b] = bv;
                    oi[nb - 1 - b] = (int32_t)b;
                }
            }
            if (b >= P && b < a.pinned) {
                ov[b] = -__builtin_inff();
                oi[b] = -1;
            }
        }
    }
}

// Bitonic sort of p2 (a power of two, >= 2) words in LDS by all THREADS
// threads of the workgroup, ascending or descending.  A stage with stride
// at most 64 pairs elements inside the 128-element segment of one wave
// (thread t handles lo = 2t - t mod stride, and the wave's threads cover one
// segment per round), so consecutive such stages need only the wave's own
// LDS ordering; a workgroup barrier is needed around the wider stages.
// The caller syncs before; the function ends with a barrier.
template <int THREADS, bool DESC>
__device__ __forceinline__ void lds_bitonic(uint64_t *x, uint32_t p2) {
    const uint32_t tid = threadIdx.x;
    for (uint32_t size = 2; size <= p2; size <<= 1) {
        for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
            for (uint32_t t = tid; t < (p2 >> 1); t += THREADS) {
                const uint32_t lo = ((t & ~(stride - 1)) << 1) | (t & (stride - 1));
                const uint32_t hi = lo + stride;
                const uint64_t a = x[lo], b = x[hi];
                const bool first_big = ((lo & size) == 0) == DESC;
                if (first_big ? a < b : a > b) {
                    x[lo] = b;
                    x[hi] = a;
                }
            }
            const uint32_t next = stride > 1 ? stride >> 1 : size;
            if (stride > (uint32_t)kWave || next > (uint32_t)kWave) {
                __syncthreads();
            } else {
                __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront", "local");
                __builtin_amdgcn_wave_barrier();
            }
        }
    }
    __syncthreads();
}

// Best k of a row of block maxima by radix selection.  The row is short
// (one value per block of positions) and fully written before the selection
// starts, so instead of streaming it through trays, one workgroup per row
// finds the k-th largest 64-bit word (order key above the complemented
// position, as everywhere in the library) digit by digit, most significant
// first: each step histograms one digit of the words that match the digits
// fixed so far and keeps the bin that holds the k-th word.  While that bin
// is larger than the LDS candidate buffer, the steps re-read the row; once
// it fits, one pass collects the words above the bin (certain winners) and
// the bin itself, and the remaining steps run in LDS.  The winners (exactly
// min(k, count) words, all distinct) are sorted by a bitonic network in LDS
// and written out.  Words are unique, so the result does not depend on the
// order of any step.
constexpr int kRadixThreads = 1024;
constexpr int kRadixBins = 2048;
constexpr int kRadixLevels = 6;

// LDS capacities: SEL winners (>= k) and CAND candidates.  Lists up to
// 2,048 take 72 KiB; lists up to 8,192 take 158 KiB, the most one
// workgroup may have.  (The smaller size's LDS would admit two workgroups
// per compute unit, but the kernel's register count admits one.)
template <int SEL, int CAND>
struct RadixCap {
    static constexpr int kSel = SEL;
    static constexpr int kCand = CAND;
    static constexpr size_t kLds = (size_t)kRadixBins * 4 + (size_t)(SEL + CAND) * 8;
};
using RadixSmall = RadixCap<2048, 6144>;
using RadixLarge = RadixCap<8192, 11008>;

__device__ __forceinline__ int radix_shift(int level) {
    // digits of 11, 11, 10 bits over the key, then over the position half
    return level == 0 ? 53 : level == 1 ? 42 : level == 2 ? 32 : level == 3 ? 21 : level == 4 ? 10 : 0;
}

__device__ __forceinline__ uint64_t radix_word(float v, uint32_t i) {
    return pack_word(order_key(__float_as_uint(v)), i);
}

// The 64-bit word of element i (value v) of a row: the order key above the
// complemented index.
struct PlainWords {
    __device__ __forceinline__ uint64_t operator()(float v, uint32_t i) const {
        return radix_word(v, i);
    }
};

// Rows of pooled scores: element i is context position
// pool[i / group] * group + i % group, so the word carries that position and
// equal values go to the lower position.  Elements of empty slots or past
// the context length get key 0 (below every score; written out as filler)
// and stay distinct through their element index.
struct PooledWords {
    const int32_t *pool;  // this row's pool slots (an LDS copy)
    uint32_t group;
    int32_t gshift;       // log2(group) when group is a power of two, else -1
    int64_t len;          // this row's context length
    __device__ __forceinline__ uint64_t operator()(float v, uint32_t i) const {
        const uint32_t s = gshift >= 0 ? i >> gshift : i / group;
        const uint32_t j = i - s * group;
        const int32_t b = pool[s];
        const int64_t pos = (int64_t)b * group + j;
        if (b < 0 || pos >= len) return (uint64_t)(0xFFFFFFFFu - i);
        return pack_word(order_key(__float_as_uint(v)), (uint32_t)pos);
    }
};

// A row of m floats at any 4-byte alignment: `head` scalars up to the
// first 16-byte boundary, `n4` aligned float4s, then `tail` scalars.
// Nothing past the row is read.
struct RowParts {
    uint32_t head, n4, tail;
    const float4 *body;
};

__device__ __forceinline__ RowParts row_parts(const float *row, uint32_t m) {
    RowParts p;
    const uint32_t mis = (uint32_t)(reinterpret_cast<uintptr_t>(row) & 15u) / 4u;
    p.head = mis ? 4u - mis : 0u;
    if (p.head > m) p.head = m;
    p.n4 = (m - p.head) / 4u;
    p.tail = m - p.head - 4u * p.n4;
    p.body = reinterpret_cast<const float4 *>(row + p.head);
    return p;
}

// Calls fn(word, valid) once per thread for the head and tail scalars
// (thread t takes the t-th of them; valid is false for the rest).
template <class W, class F>
__device__ __forceinline__ void for_each_scalar(const float *row, RowParts p, const W &wm, F &&fn) {
    const uint32_t t = threadIdx.x;
    const uint32_t i = t < p.head ? t : p.head + 4u * p.n4 + (t - p.head);
    const bool valid = t < p.head + p.tail;
    float x = 0.f;
    if (valid) x = row[i];
    fn(wm(x, i), valid);
}

// Calls fn(word, valid) for every element of a row of m floats: eight
// float4 loads in flight per thread, neighbouring threads on neighbouring
// 16 bytes, the unaligned ends one scalar per thread.  Every lane of a wave
// makes the same calls (`valid` is false where there is no element), so fn
// may use wave-wide ballots.
template <class W, class F>
__device__ __forceinline__ void for_each_word(const float *row, uint32_t m, const W &wm, F &&fn) {
    constexpr uint32_t U = 8;
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const RowParts p = row_parts(row, m);
    for (uint32_t base = threadIdx.x; base - lane < p.n4; base += U * kRadixThreads) {
        float4 v[U];
#pragma unroll
        for (uint32_t u = 0; u < U; ++u) {
            const uint32_t q = base + u * kRadixThreads;
            v[u] = q < p.n4 ? p.body[q] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (uint32_t u = 0; u < U; ++u) {
            const uint32_t q = base + u * kRadixThreads;
            const uint32_t i = p.head + 4u * q;
            const bool ok = q < p.n4;
            fn(wm(v[u].x, i), ok);
            fn(wm(v[u].y, i + 1), ok);
            fn(wm(v[u].z, i + 2), ok);
            fn(wm(v[u].w, i + 3), ok);
        }
    }
    for_each_scalar(row, p, wm, fn);
}

// Appends every word of the row with w >= lo to buf: per group of eight
// float4 loads each thread counts its admitted words, one shuffle scan and
// one atomic per wave place them, and the thread writes them at its offset
// (the unaligned ends go through wave_append).  Slots at or past `cap` are
// dropped; *counter still counts every word.
__device__ __forceinline__ void wave_append(uint64_t *buf, uint32_t *counter, uint32_t cap,
                                            uint64_t w, bool take);

// Float4s per thread in one group of the admission pass (two groups are in
// flight): eight on rows above kAdmitShortRow scores, four on shorter ones.
// Rows of 16K-64K scores read faster with fewer loads outstanding (pooled
// rows of 16,000: 27.6 -> 24.5 us per call; 4 x 16K 20.2 -> 18.8), rows of
// 128K and more slower (vocabulary rows: 51.1 -> 52.0).
constexpr uint32_t kAdmitU = 8;
constexpr uint32_t kAdmitUShort = 4;
constexpr uint32_t kAdmitShortRow = 65536;

// Loads group `base` (thread index plus a multiple of U * 1024) of a row's
// aligned body.  Indices past the body read its last float4 again (no
// per-lane branch around a load); the counting masks them.
template <uint32_t U>
__device__ __forceinline__ void admit_load(float4 (&d)[U], const RowParts &p, uint32_t base) {
#pragma unroll
    for (uint32_t u = 0; u < U; ++u) {
        const uint32_t q = base + u * kRadixThreads;
        d[u] = load_stream4(reinterpret_cast<const float *>(p.body + (q < p.n4 ? q : p.n4 - 1u)));
    }
}

// `first` holds the row's first group (admit_load at threadIdx.x), issued
// early by the caller so that its memory latency overlaps other work.
template <uint32_t U, class W>
__device__ __forceinline__ void append_at_least(const float *row, uint32_t m, const W &wm,
                                                uint64_t lo, uint64_t *buf, uint32_t *counter,
                                                uint32_t cap, const float4 (&first)[U]) {
    constexpr uint32_t STEP = U * kRadixThreads;
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const RowParts p = row_parts(row, m);
    // Two register sets: the next group of loads is in flight while the
    // current one is counted and written, so the pass is not one memory
    // round trip per group.
    float4 v[2][U];
    auto load = [&](float4 (&d)[U], uint32_t base) __attribute__((always_inline)) {
        admit_load(d, p, base);
    };
    auto consume = [&](const float4 (&d)[U], uint32_t base) __attribute__((always_inline)) {
        uint32_t mine = 0;
#pragma unroll
        for (uint32_t u = 0; u < U; ++u) {
            const uint32_t q = base + u * kRadixThreads;
            const uint32_t i = p.head + 4u * q;
            if (q < p.n4) {
                mine += wm(d[u].x, i) >= lo;
                mine += wm(d[u].y, i + 1) >= lo;
                mine += wm(d[u].z, i + 2) >= lo;
                mine += wm(d[u].w, i + 3) >= lo;
            }
        }
        // inclusive prefix of `mine` over the wave, and the wave's total
        const uint32_t incl = wave_incl_scan(mine);
        const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1);
        if (total == 0) return;
        uint32_t at = 0;
        if (lane == kWave - 1) at = atomicAdd(counter, total);
        at = (uint32_t)__builtin_amdgcn_readlane((int)at, kWave - 1) + incl - mine;
        if (mine == 0) return;
#pragma unroll
        for (uint32_t u = 0; u < U; ++u) {
            const uint32_t q = base + u * kRadixThreads;
            const uint32_t i = p.head + 4u * q;
            const float e[4] = {d[u].x, d[u].y, d[u].z, d[u].w};
#pragma unroll
            for (uint32_t c = 0; c < 4; ++c) {
                const uint64_t w = wm(e[c], i + c);
                if (q < p.n4 && w >= lo) {
                    if (at < cap) buf[at] = w;
                    ++at;
                }
            }
        }
    };
    uint32_t base = threadIdx.x;
#pragma unroll
    for (uint32_t u = 0; u < U; ++u) v[0][u] = first[u];
    for (; base - lane < p.n4; base += 2u * STEP) {
        const uint32_t b1 = base + STEP;
        const bool more1 = b1 - lane < p.n4;
        if (more1) load(v[1], b1);
        consume(v[0], base);
        if (!more1) break;
        const uint32_t b2 = b1 + STEP;
        if (b2 - lane < p.n4) load(v[0], b2);
        consume(v[1], b1);
    }
    for_each_scalar(row, p, wm, [&](uint64_t w, bool valid) {
        wave_append(buf, counter, cap, w, valid && w >= lo);
    });
}

// Appends w for the lanes where `take` holds: one atomic per wave, slots
// by lane rank.  Slots at or past `cap` are dropped (never reached when the
// counts are exact).  All lanes of the wave must call it together.
__device__ __forceinline__ void wave_append(uint64_t *buf, uint32_t *counter, uint32_t cap,
                                            uint64_t w, bool take) {
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint64_t mask = __ballot(take);
    if (mask == 0ull) return;
    const int leader = __ffsll((unsigned long long)mask) - 1;
    uint32_t base = 0;
    if ((int)lane == leader) base = atomicAdd(counter, (uint32_t)__popcll(mask));
    base = (uint32_t)__builtin_amdgcn_readlane((int)base, leader);
    if (take) {
        const uint32_t at = base + (uint32_t)__popcll(mask & ((1ull << lane) - 1ull));
        if (at < cap) buf[at] = w;
    }
}

// Descending sort of p2 <= 1,024 words (a power of two) in LDS with the
// waves' registers doing most of the work.  Runs of R = 64 E words (one per wave,
// E per lane) are sorted in registers, alternately descending and
// ascending; each further level of the bitonic network then needs LDS only
// for its stages of stride >= R, and finishes every run with a register
// merge.  Between the register phases a run is kept transposed in LDS (its
// word lane*E + e at e*64 + lane), so a wave moves it with conflict-free
// 64-lane accesses; only the first load and the last store use the plain
// layout.  Every run is permuted the same way and the LDS stages (stride >=
// R) pair equal offsets of different runs, with a direction set by a bit
// above the run, so they index the transposed words directly, consecutive
// threads on consecutive words.  They go two strides at a time where they
// can: each
// thread takes the four words {b, b+h, b+2h, b+3h} and does both
// compare-exchange stages (strides 2h and h) in registers, one barrier for
// the pair.  For 4,096 words: 6 barriers for the LDS stages instead of 10
// (and 78 for the plain network).  The caller syncs before; ends with a
// barrier.
template <int E>
__device__ __forceinline__ void run_sort_bitonic(uint64_t *x, uint32_t p2, uint32_t nw) {
    constexpr uint32_t R = 64u * E;
    const uint32_t tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
    const bool active = w < nw;
    // Compare-exchange of the words held for positions lo < hi: the larger
    // first when the pair lies in a descending part (bit `size` clear).
    auto cx = [](uint64_t &u, uint64_t &v, bool first_big) __attribute__((always_inline)) {
        const uint64_t big = u > v ? u : v, small = u > v ? v : u;
        u = first_big ? big : small;
        v = first_big ? small : big;
    };
    uint64_t a[E];
    if (active) {
#pragma unroll
        for (int e = 0; e < E; ++e) a[e] = x[w * R + lane * E + e];
        if ((w & 1u) == 0u) wave_sort<E, false>(a, lane);
        else wave_sort<E, true>(a, lane);
        if (p2 == R) {
#pragma unroll
            for (int e = 0; e < E; ++e) x[w * R + lane * E + e] = a[e];
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) x[w * R + (uint32_t)e * kWave + lane] = a[e];
        }
    }
    __syncthreads();
    for (uint32_t size = 2 * R; size <= p2; size <<= 1) {
        uint32_t stride = size >> 1;
        for (; stride >= 2u * R; stride >>= 2) {
            // strides `stride` and stride/2 together, over groups of four
            const uint32_t h = stride >> 1;
            for (uint32_t t = tid; t < (p2 >> 2); t += kRadixThreads) {
                const uint32_t b = ((t / h) * (stride << 1)) + (t % h);
                const bool first_big = (b & size) == 0u;
                uint64_t v0 = x[b], v1 = x[b + h], v2 = x[b + stride], v3 = x[b + stride + h];
                cx(v0, v2, first_big);
                cx(v1, v3, first_big);
                cx(v0, v1, first_big);
                cx(v2, v3, first_big);
                x[b] = v0;
                x[b + h] = v1;
                x[b + stride] = v2;
                x[b + stride + h] = v3;
            }
            __syncthreads();
        }
        if (stride >= R) {
            for (uint32_t t = tid; t < (p2 >> 1); t += kRadixThreads) {
                const uint32_t lo = ((t & ~(stride - 1)) << 1) | (t & (stride - 1));
                const uint32_t hi = lo + stride;
                uint64_t u = x[lo], v = x[hi];
                cx(u, v, (lo & size) == 0u);
                x[lo] = u;
                x[hi] = v;
            }
            __syncthreads();
        }
        if (active) {
#pragma unroll
            for (int e = 0; e < E; ++e) a[e] = x[w * R + (uint32_t)e * kWave + lane];
            if (((w * R) & size) == 0u) wave_merge<E, false>(a, lane);
            else wave_merge<E, true>(a, lane);
            if (size == p2) {
#pragma unroll
                for (int e = 0; e < E; ++e) x[w * R + lane * E + e] = a[e];
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) x[w * R + (uint32_t)e * kWave + lane] = a[e];
            }
        }
        __syncthreads();
    }
}

// One merge-path level: pairs of descending runs of length L in src become
// descending runs of 2L in dst.  Each thread writes c = p2 / threads
// consecutive outputs (at least one): it finds how many of the first i
// outputs of its pair come from the first run by a binary search along the
// diagonal i, then merges its c outputs one at a time.  Equal words go to the
// first run first, in the search and the merge alike (only the zero padding
// repeats).
__device__ __forceinline__ void merge_level_desc(const uint64_t *src, uint64_t *dst, uint32_t p2,
                                                 uint32_t L) {
    const uint32_t c = p2 > (uint32_t)kRadixThreads ? p2 / (uint32_t)kRadixThreads : 1u;
    for (uint32_t o = threadIdx.x * c; o < p2; o += (uint32_t)kRadixThreads * c) {
        const uint32_t base = o & ~(2u * L - 1u), i = o - base;
        const uint64_t *A = src + base, *B = A + L;
        uint32_t lo = i > L ? i - L : 0u, hi = i < L ? i : L;
        while (lo < hi) {
            const uint32_t m = (lo + hi + 1u) >> 1;
            if (A[m - 1u] >= B[i - m]) lo = m;
            else hi = m - 1u;
        }
        uint32_t a = lo, b = i - lo;
        uint64_t va = a < L ? A[a] : 0ull, vb = b < L ? B[b] : 0ull;
        for (uint32_t j = 0; j < c; ++j) {
            const bool take_a = b >= L || (a < L && va >= vb);
            dst[o + j] = take_a ? va : vb;
            if (take_a) {
                ++a;
                va = a < L ? A[a] : 0ull;
            } else {
                ++b;
                vb = b < L ? B[b] : 0ull;
            }
        }
    }
}

// Descending sort of p2 >= 2,048 words (a power of two) in LDS: runs of
// R = 64 E words (one per wave, E per lane) are sorted in registers by the
// bitonic network, then merged pairwise level by level by merge path,
// between x and the scratch buffer tmp (p2 words).  The bitonic network's
// own merge levels cost several times the VALU work of these merges at that
// size (68 register stages per word for 4,096 words, with four waves sharing
// each SIMD: vocabulary rows at k = 4,096 56.3 -> 51.8 us per call); up to
// 1,024 words they are the faster of the two.  The caller syncs before; ends
// with a barrier.
template <int E>
__device__ __forceinline__ void run_sort_merge(uint64_t *x, uint64_t *tmp, uint32_t p2,
                                               uint32_t nw) {
    constexpr uint32_t R = 64u * E;
    const uint32_t tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
    if (w < nw) {
        uint64_t a[E];
#pragma unroll
        for (int e = 0; e < E; ++e) a[e] = x[w * R + lane * E + e];
        wave_sort<E, false>(a, lane);
#pragma unroll
        for (int e = 0; e < E; ++e) x[w * R + lane * E + e] = a[e];
    }
    __syncthreads();
    uint64_t *src = x, *dst = tmp;
    for (uint32_t L = R; L < p2; L <<= 1) {
        merge_level_desc(src, dst, p2, L);
        __syncthreads();
        uint64_t *t = src;
        src = dst;
        dst = t;
    }
    if (src != x) {
        for (uint32_t i = tid; i < p2; i += (uint32_t)kRadixThreads) x[i] = src[i];
        __syncthreads();
    }
}

// Descending sort of the p2 <= 8,192 winners (tmp: p2 words of scratch):
// runs of 64 E words over up to 16 waves, the plain LDS network below 64
// words.
__device__ __forceinline__ void sort_winners_desc(uint64_t *x, uint64_t *tmp, uint32_t p2) {
    if (p2 < 64u) {
        lds_bitonic<kRadixThreads, true>(x, p2);
    } else if (p2 <= 1024u) {
        run_sort_bitonic<1>(x, p2, p2 / 64u);
    } else if (p2 == 2048u) {
        run_sort_merge<2>(x, tmp, p2, 16u);
    } else if (p2 == 4096u) {
        run_sort_merge<4>(x, tmp, p2, 16u);
    } else {
        run_sort_merge<8>(x, tmp, p2, 16u);
    }
}

// State of one radix search, shared by the workgroup.
struct RadixShared {
    uint32_t wave_sum[kRadixThreads / kWave];
    uint32_t t, above, h, nsel, ncand;
};

// Finds the top-most histogram bin whose suffix count reaches `need`.
// Each thread holds two neighbouring bins; suffix sums run from the top
// bin down: a shuffle scan inside each wave, then the totals of the waves
// above.  The one thread whose bin crosses `need` publishes it; everyone
// reads it after the barrier.  The histogram is left all zero.
__device__ __forceinline__ void radix_pick(uint32_t *hist, uint32_t need, RadixShared &sh) {
    static_assert(kRadixBins == 2 * kRadixThreads, "two bins per thread");
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wv = tid / kWave;
    const uint32_t h0 = hist[2 * tid], h1 = hist[2 * tid + 1];
    // Each thread reads only its own two bins: it clears them for the next
    // count (the barriers below order that before any later increment).
    hist[2 * tid] = 0u;
    hist[2 * tid + 1] = 0u;
    // sum of this lane's bins and every bin above it in the wave: the wave's
    // total less the inclusive prefix below this lane
    const uint32_t own = h0 + h1;
    const uint32_t incl = wave_incl_scan(own);
    uint32_t suf = (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1) - incl + own;
    if (lane == 0) sh.wave_sum[wv] = suf;
    lds_barrier();
    for (int u = wv + 1; u < kRadixThreads / kWave; ++u) suf += sh.wave_sum[u];
    // suf = S(2 tid); S(2 tid + 1) = suf - h0; S(b) counts bins >= b
    const uint32_t s1 = suf - h0;
    if (s1 >= need && s1 - h1 < need) {
        sh.t = (uint32_t)(2 * tid + 1);
        sh.above = s1 - h1;
        sh.h = h1;
    } else if (suf >= need && suf - h0 < need) {
        sh.t = (uint32_t)(2 * tid);
        sh.above = suf - h0;
        sh.h = h0;
    }
    lds_barrier();
}

// Radix search in LDS: for `need` <= n distinct words buf[0, n), returns
// (shift, thr) such that exactly `need` of them satisfy (w >> shift) >= thr.
// With slack > 0 it may stop early, at the first digit whose bin holding the
// need-th word has at most `slack` words: then between need and need +
// slack - 1 of them satisfy it (the bin's lower edge; an estimate needs no
// more).  All threads of the workgroup call it together.  Inlined, with the
// result returned by value, so the kernel makes no calls and keeps nothing
// on the stack.
struct RadixCut {
    int shift;
    uint64_t thr;
};

__device__ __forceinline__ RadixCut lds_radix(const uint64_t *buf, uint32_t n, uint32_t need,
                                              uint32_t *hist, RadixShared &sh,
                                              uint32_t slack = 0u) {
    const int tid = threadIdx.x;
    const uint32_t lane = (uint32_t)tid & (kWave - 1);
    uint64_t pfx = 0;
    // radix_pick leaves the histogram zero for the next level.
    for (int b = tid; b < kRadixBins; b += kRadixThreads) hist[b] = 0u;
    lds_barrier();
    for (int level = 0;; ++level) {
        const int s = radix_shift(level);
        const int ps = level == 0 ? 64 : radix_shift(level - 1);
        const uint32_t dmask = (1u << (ps - s)) - 1u;
        for (uint32_t c = tid; c - lane < n; c += kRadixThreads) {
            const uint64_t w = c < n ? buf[c] : 0ull;
            // Plain LDS atomics: on CDNA4 they beat merging a wave's equal
            // bins first, even where many words share a bin.
            const bool in = c < n && (level == 0 || (w >> ps) == pfx);
            if (in) atomicAdd(&hist[(uint32_t)(w >> s) & dmask], 1u);
        }
        lds_barrier();
        radix_pick(hist, need, sh);
        const uint32_t t = sh.t, above = sh.above, h = sh.h;
        need -= above;
        pfx = level == 0 ? (uint64_t)t : ((pfx << (ps - s)) | t);
        if (h == need || h <= slack || level == kRadixLevels - 1) {
            lds_barrier();  // everyone has read the pick before the caller goes on
            return RadixCut{s, pfx};
        }
        // The next level's pick is written two barriers from here, after
        // every thread has read this one.
    }
}

// Sample size of the threshold estimate: 64 chunks of 64 consecutive
// elements spread evenly over the row.
constexpr uint32_t kSampleChunks = 64;
constexpr uint32_t kSampleWords = kSampleChunks * kWave;
constexpr uint32_t kEstimateMinRow = 2 * kSampleWords;

// Per-row word maker; `slots` is LDS room for a pooled row's slots.
template <class Words>
__device__ __forceinline__ Words row_words(const RadixArgs &a, int64_t r, int32_t *slots);

template <>
__device__ __forceinline__ PlainWords row_words<PlainWords>(const RadixArgs &, int64_t, int32_t *) {
    return PlainWords{};
}

template <>
__device__ __forceinline__ PooledWords row_words<PooledWords>(const RadixArgs &a, int64_t r,
                                                              int32_t *slots) {
    int64_t len = a.n_ctx;
    if (a.ctx_lengths) {
        const int64_t l = a.ctx_lengths[r];
        len = l < 0 ? 0 : (l > a.n_ctx ? a.n_ctx : l);
    }
    const int32_t *pool = a.pool + r * (int64_t)a.pool_keep;
    for (int s = threadIdx.x; s < a.pool_keep; s += kRadixThreads) slots[s] = pool[s];
    __syncthreads();
    const uint32_t g = (uint32_t)a.group;
    const int32_t gshift = (g & (g - 1)) == 0 ? (int32_t)__builtin_ctz(g) : -1;
    return PooledWords{slots, g, gshift, len};
}

// LDS a pooled launch adds for the row's slots.
__host__ __device__ constexpr size_t pooled_slot_bytes(int keep) { return (size_t)keep * 4; }

template <class Cap, class Words>
__global__ __launch_bounds__(kRadixThreads) void radix_select_kernel(RadixArgs a) {
    constexpr int kRadixSel = Cap::kSel;
    constexpr int kRadixCand = Cap::kCand;
    extern __shared__ uint64_t lds[];
    uint64_t *sel = lds;                                  // kRadixSel
    uint64_t *cand = lds + kRadixSel;                     // kRadixCand
    uint32_t *hist = reinterpret_cast<uint32_t *>(lds + kRadixSel + kRadixCand);  // kRadixBins
    __shared__ RadixShared sh;

    const int64_t r = (int64_t)a.row0 + blockIdx.x;
    const int tid = threadIdx.x;
    const uint32_t lane = (uint32_t)tid & (kWave - 1);
    int64_t m64 = a.count ? (int64_t)a.count[r] : a.ld;
    m64 = m64 < 0 ? 0 : (m64 > a.ld ? a.ld : m64);
    const uint32_t m = (uint32_t)m64;
    const uint32_t k = (uint32_t)a.k;
    const float *row = a.vals + r * a.ld;
    const Words wm = row_words<Words>(
        a, r, reinterpret_cast<int32_t *>(hist + kRadixBins));

    if (tid == 0) {
        sh.nsel = 0;
        sh.ncand = 0;
    }
    __syncthreads();
    int thr_shift = 0;
    uint64_t thr = 0;          // winners: (w >> thr_shift) >= thr
    bool done = false;
    if (m <= k) {
        // every word wins (thr = 0 admits all)
        for_each_word(row, m, wm, [&](uint64_t w, bool valid) {
            wave_append(sel, &sh.nsel, kRadixSel, w, valid);
        });
        done = true;
    } else if (m >= kEstimateMinRow) {
        // Estimate: at or a little below the j-th best word of an evenly
        // spread sample, with j about four standard deviations above its
        // expected count, it admits a little more than k words; one pass
        // appends every word at or above it to LDS.  When at least k and at
        // most the buffer's capacity arrive, the winners are found among
        // them exactly.
        const float lam = (float)k * (float)kSampleWords / (float)m;
        const uint32_t j = (uint32_t)ceilf(lam + 4.0f * sqrtf(lam) + 4.0f);
        if (j < kSampleWords) {
            // the sample fills the winner and candidate lists' room (both
            // empty until the admission pass, which then overwrites it)
            static_assert(kRadixSel + kRadixCand >= (int)kSampleWords, "sample room");
            uint64_t *samp = lds;
            for (uint32_t q = tid; q < kSampleWords; q += kRadixThreads) {
                const uint32_t c = q / kWave, o = q % kWave;
                const uint32_t i = (uint32_t)(((uint64_t)c * m) / kSampleChunks) + o;
                samp[q] = wm(row[i], i);
            }
            // The admission pass's first group is issued now, before the
            // sample's selection.
            const RowParts body = row_parts(row, m);
            float4 first[kAdmitU];
            float4 (&first_short)[kAdmitUShort] = *reinterpret_cast<float4 (*)[kAdmitUShort]>(first);
            const bool short_row = m <= kAdmitShortRow;
            if (threadIdx.x - (threadIdx.x & (kWave - 1)) < body.n4) {
                if (short_row) admit_load(first_short, body, threadIdx.x);
                else admit_load(first, body, threadIdx.x);
            }
            // The sample's selection synchronises through LDS only, so the
            // first group stays in flight meanwhile.
            lds_barrier();
            const RadixCut ec = lds_radix(samp, kSampleWords, j, hist, sh, j / 4u + 1u);
            lds_barrier();  // the sample is read before the admission pass overwrites it
            // words >= est: j to j + j/4 of the sample (the search stops at
            // the first digit whose bin is that small)
            const uint64_t est = ec.thr << ec.shift;
            if (short_row) {
                append_at_least<kAdmitUShort>(row, m, wm, est, cand, &sh.ncand, kRadixCand,
                                              first_short);
            } else {
                append_at_least<kAdmitU>(row, m, wm, est, cand, &sh.ncand, kRadixCand, first);
            }
            __syncthreads();
            const uint32_t nc = sh.ncand;
            if (nc >= k && nc <= (uint32_t)kRadixCand) {
                const RadixCut c = lds_radix(cand, nc, k, hist, sh);
                thr_shift = c.shift;
                thr = c.thr;
                for (uint32_t c = tid; c - lane < nc; c += kRadixThreads) {
                    const uint64_t w = c < nc ? cand[c] : 0ull;
                    wave_append(sel, &sh.nsel, kRadixSel, w, c < nc && (w >> thr_shift) >= thr);
                }
                done = true;
            } else {
                __syncthreads();
                if (tid == 0) sh.ncand = 0;
                __syncthreads();
            }
        }
    }
    if (!done) {
        // Digit by digit over the row until the k-th word's bin fits in
        // LDS (or is decided), then in LDS.
        uint32_t need = k;
        uint64_t pfx = 0;
        for (int level = 0;; ++level) {
            const int s = radix_shift(level);
            const int ps = level == 0 ? 64 : radix_shift(level - 1);
            const uint32_t dmask = (1u << (ps - s)) - 1u;
            for (int b = tid; b < kRadixBins; b += kRadixThreads) hist[b] = 0u;
            __syncthreads();
            if (level == 0) {
                for_each_word(row, m, wm, [&](uint64_t w, bool valid) {
                    if (valid) atomicAdd(&hist[(uint32_t)(w >> s) & dmask], 1u);
                });
            } else {
                for_each_word(row, m, wm, [&](uint64_t w, bool valid) {
                    const bool in = valid && (w >> ps) == pfx;
                    if (in) atomicAdd(&hist[(uint32_t)(w >> s) & dmask], 1u);
                });
            }
            __syncthreads();
            radix_pick(hist, need, sh);
            const uint32_t t = sh.t, above = sh.above, h = sh.h;
            __syncthreads();
            need -= above;
            pfx = level == 0 ? (uint64_t)t : ((pfx << (ps - s)) | t);
            if (h == need || level == kRadixLevels - 1) {
                // the whole bin wins: winners are the words at or above it
                // (after the last level the bin is one word)
                for_each_word(row, m, wm, [&](uint64_t w, bool valid) {
                    wave_append(sel, &sh.nsel, kRadixSel, w, valid && (w >> s) >= pfx);
                });
                break;
            }
            if (h <= (uint32_t)kRadixCand) {
                // words above the bin win; the bin goes to LDS
                for_each_word(row, m, wm, [&](uint64_t w, bool valid) {
                    const uint64_t top = w >> s;
                    wave_append(sel, &sh.nsel, kRadixSel, w, valid && top > pfx);
                    wave_append(cand, &sh.ncand, kRadixCand, w, valid && top == pfx);
                });
                __syncthreads();
                const uint32_t nc = sh.ncand;
                const RadixCut c = lds_radix(cand, nc, need, hist, sh);
                thr_shift = c.shift;
                thr = c.thr;
                for (uint32_t c = tid; c - lane < nc; c += kRadixThreads) {
                    const uint64_t w = c < nc ? cand[c] : 0ull;
                    wave_append(sel, &sh.nsel, kRadixSel, w, c < nc && (w >> thr_shift) >= thr);
                }
                break;
            }
        }
    }
    __syncthreads();
    const uint32_t ns = sh.nsel < (uint32_t)kRadixSel ? sh.nsel : (uint32_t)kRadixSel;
    uint32_t p2 = 2;
    while (p2 < ns) p2 <<= 1;
    for (uint32_t c = ns + tid; c < p2; c += kRadixThreads) sel[c] = 0ull;
    __syncthreads();
    static_assert(kRadixCand >= kRadixSel, "the sort's scratch");
    sort_winners_desc(sel, cand, p2);
    float *ov = a.out_vals + r * a.out_ld;
    int32_t *oi = a.out_idx + r * a.out_ld;
    for (uint32_t t = tid; t < k; t += kRadixThreads) {
        const uint64_t w = t < ns ? sel[t] : 0ull;
        // key 0: no element (padding, or an element outside the pool's rows)
        const bool real = (w >> 32) != 0ull;
        ov[t] = real ? __uint_as_float(key_bits((uint32_t)(w >> 32))) : -__builtin_inff();
        oi[t] = real ? (int32_t)word_pos(w) : -1;
    }
}

}  // namespace

template <class Cap, class Words>
hipError_t launch_radix_cap(const RadixArgs &a, hipStream_t stream) {
    // pooled rows also keep the row's slots in LDS, after the histogram
    const size_t lds = Cap::kLds + (a.pool ? pooled_slot_bytes(a.pool_keep) : 0);
    // Set on every launch (as for the selection kernel): the attribute
    // belongs to the current device, and calls may come on several.
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&radix_select_kernel<Cap, Words>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((radix_select_kernel<Cap, Words>), dim3((unsigned)a.rows),
                       dim3(kRadixThreads), lds, stream, a);
    return hipGetLastError();
}

template <class Words>
hipError_t launch_radix_words(const RadixArgs &a, hipStream_t stream) {
    if (a.rows <= 0) return hipSuccess;
    if (a.pool && (a.pool_keep > kMaxPooledSlots || a.k > RadixSmall::kSel))
        return hipErrorInvalidValue;
    if (a.k <= RadixSmall::kSel) return launch_radix_cap<RadixSmall, Words>(a, stream);
    if (a.k <= RadixLarge::kSel) return launch_radix_cap<RadixLarge, Words>(a, stream);
    return hipErrorInvalidValue;
}

size_t radix_lds_bytes(int k, int pool_keep) {
    const size_t slots = pool_keep > 0 ? pooled_slot_bytes(pool_keep) : 0;
    return (k <= RadixSmall::kSel ? RadixSmall::kLds : RadixLarge::kLds) + slots;
}

hipError_t launch_radix_select(const RadixArgs &a, hipStream_t stream) {
    return a.pool ? launch_radix_words<PooledWords>(a, stream)
                  : launch_radix_words<PlainWords>(a, stream);
}

hipError_t launch_block_max(const PoolArgs &a, hipStream_t stream) {
    if (a.rows <= 0 || a.span <= 0) return hipSuccess;
    const bool vec = a.group % 4 == 0 && a.n % 4 == 0 &&
                     reinterpret_cast<uintptr_t>(a.scores) % 16 == 0;
    if (vec && a.group == 8) {
        const int64_t items = 2 * (int64_t)a.span;
        const int64_t per = (int64_t)kPoolThreads * kPool8Unroll;
        const dim3 grid8((unsigned)((items + per - 1) / per), (unsigned)a.rows);
        hipLaunchKernelGGL(block_max8_kernel, grid8, dim3(kPoolThreads), 0, stream, a);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((a.span + kPoolThreads - 1) / kPoolThreads), (unsigned)a.rows);
    if (vec) {
        hipLaunchKernelGGL(block_max_kernel<true>, grid, dim3(kPoolThreads), 0, stream, a);
    } else {
        hipLaunchKernelGGL(block_max_kernel<false>, grid, dim3(kPoolThreads), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace topk
