// Per-row exact top-k selection kernel for gfx950.
//
// Method ("The Secret GPU Kernel Behind DeepSeek V4.1 Flash", transcript
// 3:18-5:33): a threshold that starts at minus infinity and only rises; rows
// cut into 1,024-element blocks visited in a data-independent shuffled
// order; one comparison per score; survivors into a small tray; a sort that
// runs on the tray only when it passes its mark, keeping the best k and
// raising the threshold to the k-th of those; a split-row mode in which
// several compute units each keep a local top-k and a leader merges them.
//
// Mapping to CDNA4:
//   * One workgroup is one selection stream over its share of a row, run by
//     two kinds of waves.  Streamer waves only read, test and compact: each
//     walks its own blocks of the shuffled order with four 1 KiB dwordx4
//     loads per 4 KiB block, several blocks in flight (the order does not
//     depend on the data, so future addresses are known), and appends
//     survivors to a double-buffered tray in LDS.  When a tray passes the
//     watermark the streamer publishes it and keeps streaming into the other
//     buffer.  One sorter wave owns the kept list (the best 64*E words so
//     far) in registers, sorts each published tray with a register bitonic
//     network, merges it into the kept list and raises the shared threshold.
//     Streamers never stop for a sort, and the threshold is the k-th best of
//     everything the workgroup has seen.
//   * The per-score test is one compare against the threshold's value, done
//     on the integer maximum of each lane's 16 score bit patterns of a block;
//     only blocks in which some lane passes take the exact 64-bit word compare
//     and the ballot/mbcnt compaction into the tray.
//   * Split rows: the row's workgroups publish their threshold words with a
//     64-bit atomic max in the workspace and streamers read it back with
//     every block (any stale value is still a lower bound of the row's k-th
//     word, so it is safe).  Each sorter writes its kept list to the
//     workspace and takes an atomic ticket; the last to arrive merges all
//     lists, writes the row and resets the row's ticket and threshold words
//     to zero (an accumulator that is never reset is the failure the
//     kernelbench.com "DeepSeek V4.1 Flash" Kimi-Linear paragraph describes).
#include "common.h"
#include "internal.h"
#include "wave_sort.h"

namespace topk {

namespace {

constexpr int kLoadsPerBlock = kBlock / (kWave * 4);  // dwordx4 loads per lane per block

template <int E>
struct Cfg {
    static constexpr int KP = kWave * E;       // kept-list words
    static constexpr int D = E <= 8 ? 4 : 2;   // blocks in flight per wave
};

__device__ __forceinline__ uint32_t mbcnt64(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// First test of a block, on the raw float bits as signed integers.  For
// non-negative floats the signed-integer order is the value order, and every
// negative float (and -0.0) is below every non-negative bit pattern.  So once
// the threshold's value is >= +0.0, "bits(x) >= bits(threshold value)" is
// implied by word(x) > T for every non-NaN x and is a safe first test.  While
// the threshold is below +0.0 the bound is INT_MIN and every block takes the
// exact test (at that stage most scores pass anyway).
__device__ __forceinline__ int32_t prefilter_bound(uint64_t T) {
    const uint32_t key = (uint32_t)(T >> 32);
    return (key & 0x80000000u) ? (int32_t)(key & 0x7FFFFFFFu) : INT32_MIN;
}

__device__ __forceinline__ uint64_t lds_load_word(uint64_t *p) {
    return uniform64(__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
}

// Kept lists are stored "transposed": list position lane*E + e sits at word
// e*64 + lane, so a wave moves a whole list with coalesced 64-lane accesses.
template <int E>
__device__ __forceinline__ void store_list(uint64_t *dst, const uint64_t (&a)[E], uint32_t lane) {
#pragma unroll
    for (int e = 0; e < E; ++e) dst[e * kWave + lane] = a[e];
}

// Loads a descending transposed list reversed, i.e. ascending, into the
// blocked register layout.
template <int E>
__device__ __forceinline__ void load_list_reversed(uint64_t (&a)[E], const uint64_t *src,
                                                   uint32_t lane) {
#pragma unroll
    for (int e = 0; e < E; ++e) a[e] = src[(E - 1 - e) * kWave + (kWave - 1 - lane)];
}

// Writes one output slot from a packed word (0 = empty slot).
__device__ __forceinline__ void write_slot(float *vals, int32_t *idx, uint32_t i, uint64_t w) {
    if (w != 0) {
        vals[i] = __uint_as_float(key_bits((uint32_t)(w >> 32)));
        idx[i] = (int32_t)word_pos(w);
    } else {
        vals[i] = -__builtin_inff();
        idx[i] = -1;
    }
}

template <int E>
__device__ __forceinline__ void write_row(float *vals, int32_t *idx, uint32_t k,
                                          const uint64_t (&kept)[E], uint32_t lane) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const uint32_t i = lane * E + (uint32_t)e;
        if (i < k) write_slot(vals, idx, i, kept[e]);
    }
}

__device__ __forceinline__ uint32_t lds_load_u32(uint32_t *p) {
    return __builtin_amdgcn_readfirstlane(
        (int)__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
}

__device__ __forceinline__ void lds_store_u32(uint32_t *p, uint32_t v, uint32_t lane) {
    if (lane == 0) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// ---------------------------------------------------------------------------
// Streamer waves: read blocks, test, compact survivors into a tray.

// Exact test and tray compaction of one block already in registers.
__device__ __forceinline__ uint32_t admit_block(uint64_t *tray, uint32_t cnt, uint64_t T,
                                                const float4 (&x)[kLoadsPerBlock], uint32_t vbase,
                                                uint32_t off0, uint32_t vend, bool ragged,
                                                uint32_t lane) {
#pragma unroll
    for (int u = 0; u < kLoadsPerBlock; ++u) {
        const float v4[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t g = vbase + (uint32_t)u * 256u + lane * 4u + (uint32_t)c;
            const bool valid = !ragged || (g >= off0 && g < vend);
            const uint64_t w = pack_word(order_key(__float_as_uint(v4[c])), g - off0);
            const bool pass = valid && (w > T);
            const uint64_t m = __ballot(pass);
            if (m) {
                if (pass) tray[cnt + mbcnt64(m)] = w;
                cnt += (uint32_t)__popcll(m);
            }
        }
    }
    return cnt;
}

// Publishes the tray (its word count) to the sorter.
__device__ __forceinline__ void publish_tray(uint32_t *fill, uint32_t cnt, uint32_t lane) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    lds_store_u32(fill, cnt, lane);
}

// Waits until the sorter has emptied the tray buffer behind `fill`.
__device__ __forceinline__ void wait_tray_free(uint32_t *fill) {
    while (lds_load_u32(fill) != 0u) __builtin_amdgcn_s_sleep(1);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------------------
// Sorter wave: fold published trays into the kept list (in registers).

// Compacts buf[0, c) in place to the words above T; returns the new count.
__device__ __forceinline__ uint32_t compact_above(uint64_t *buf, uint32_t c, uint64_t T,
                                                  uint32_t lane) {
    uint32_t out = 0;
    for (uint32_t base = 0; base < c; base += kWave) {
        const uint32_t i = base + lane;
        const uint64_t v = i < c ? buf[i] : 0ull;
        const bool keep = v > T;
        const uint64_t m = __ballot(keep);
        if (keep) buf[out + mbcnt64(m)] = v;
        out += (uint32_t)__popcll(m);
    }
    return out;
}

struct SorterState {
    uint64_t T;       // k-th best word of the kept list, or any larger bound
    uint32_t sorts;   // sort passes run
};

// Sorts one published tray into `kept` chunk by chunk (tray sort on
// registers, then keep-the-best merge), refiltering the rest of the tray
// against the raised threshold before each chunk.
template <int E, bool SPLIT>
__device__ __forceinline__ void sort_tray(uint64_t (&kept)[E], SorterState &ss, uint64_t *buf,
                                          uint32_t c, uint64_t *sT, uint64_t *gT, uint32_t k,
                                          uint32_t lane) {
    constexpr uint32_t KP = (uint32_t)Cfg<E>::KP;
    for (;;) {
        ss.T = umax64(ss.T, lds_load_word(sT));
        if constexpr (SPLIT) {
            ss.T = umax64(ss.T, uniform64(__hip_atomic_load(gT, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT)));
        }
        c = compact_above(buf, c, ss.T, lane);
        if (c == 0) break;
        const uint32_t take = c < KP ? c : KP;
        const uint32_t start = c - take;
        uint64_t a[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const uint32_t i = (uint32_t)e * kWave + lane;
            a[e] = i < take ? buf[start + i] : 0ull;
        }
        c = start;
        wave_sort<E, true>(a, lane);
        keep_best<E>(kept, a, lane);
        ++ss.sorts;
        const uint64_t nt = list_word_at<E>(kept, k - 1);
        if (nt > ss.T) {
            ss.T = nt;
            if (lane == 0) {
                __hip_atomic_fetch_max(sT, nt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                if constexpr (SPLIT) {
                    __hip_atomic_fetch_max(gT, nt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------

template <int E, bool SPLIT>
__global__ __launch_bounds__(256) void select_kernel(SelectArgs p) {
    constexpr int KP = Cfg<E>::KP;
    constexpr int D = Cfg<E>::D;
    extern __shared__ uint64_t trays[];          // [streamers][2][tray_words]
    __shared__ uint64_t s_T;                      // workgroup threshold word
    __shared__ uint32_t s_fill[kMaxWaves][2];     // published tray word counts
    __shared__ uint32_t s_done;                   // streamers finished

    const uint32_t lane = lane_id();
    const uint32_t w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const uint32_t NW = blockDim.x / kWave;
    const uint32_t NS = NW - 1;                   // streamer waves; wave NS sorts
    const uint32_t S = (uint32_t)p.split;
    const uint32_t s = blockIdx.x % S;
    const uint32_t r = (uint32_t)p.row0 + blockIdx.x / S;
    const uint32_t k = (uint32_t)p.k;
    const uint32_t CW = (uint32_t)p.tray_words;
    uint64_t *gT = SPLIT ? p.ws_ctrl + 2 * (size_t)r : nullptr;
    uint32_t *ticket = SPLIT ? reinterpret_cast<uint32_t *>(gT + 1) : nullptr;

    if (threadIdx.x == 0) {
        s_T = 0ull;
        s_done = 0u;
    }
    if (threadIdx.x < 2 * kMaxWaves) s_fill[threadIdx.x / 2][threadIdx.x % 2] = 0u;
    __syncthreads();

    if (w < NS) {
        // ---- streamer ----
        // Row geometry.  Blocks are aligned to 16 bytes of the row's storage:
        // virtual position g = position + off0, off0 being the row start's
        // misalignment in floats, so interior blocks are whole dwordx4 groups.
        int64_t L = p.n;
        if (p.lengths) {
            L = p.lengths[r];
            L = L < 0 ? 0 : (L > p.n ? p.n : L);
        }
        const float *rowp = p.scores + (int64_t)r * p.n;
        const uint32_t off0 = (uint32_t)(((uintptr_t)rowp >> 2) & 3u);
        const float *abase = rowp - off0;
        const uint32_t vend = (uint32_t)L + off0;
        const uint32_t nb = L > 0 ? (vend + kBlock - 1) / kBlock : 0u;
        const uint32_t last_group = L > 0 ? ((vend - 1u) & ~3u) : 0u;
        const VisitOrder ord = make_visit_order(p.seed, r, nb);
        const uint32_t Q = S * NS;                // streams over this row
        const uint32_t q = s * NS + w;            // this wave's stream
        const uint32_t mine = q < nb ? (nb - 1u - q) / Q + 1u : 0u;
        const uint32_t Wm = (uint32_t)p.watermark;

        uint32_t cur = 0, cnt = 0, entered = 0;
        uint64_t T = 0ull;
        uint64_t *tray = trays + (size_t)(2 * w) * CW;

        if (mine > 0) {
            float4 buf[D][kLoadsPerBlock];
            uint32_t bid[D];
            uint64_t gbuf[D];
            // Every slot issues exactly one set of loads per visit (past the
            // stream's end it re-reads its last block), so the wait before
            // each slot is the same static count every time.
            auto issue = [&](float4 (&dst)[kLoadsPerBlock], uint32_t &b_out, uint64_t &g_out,
                             uint32_t t) __attribute__((always_inline)) {
                const uint32_t tt = t < mine ? t : mine - 1u;
                const uint32_t b = visit_block(ord, q + tt * Q);
                b_out = b;
                if constexpr (SPLIT) {
                    g_out = __hip_atomic_load(gT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                const uint32_t vbase = b * (uint32_t)kBlock;
                const bool ragged = vbase < off0 || vbase + (uint32_t)kBlock > vend;
#pragma unroll
                for (int u = 0; u < kLoadsPerBlock; ++u) {
                    uint32_t g = vbase + (uint32_t)u * 256u + lane * 4u;
                    if (ragged) g = g > last_group ? last_group : g;  // stay on a valid group
                    dst[u] = *reinterpret_cast<const float4 *>(abase + g);
                }
            };
#pragma unroll
            for (int d = 0; d < D; ++d) issue(buf[d], bid[d], gbuf[d], (uint32_t)d);

            for (uint32_t t0 = 0; t0 < mine; t0 += D) {
#pragma unroll
                for (int d = 0; d < D; ++d) {
                    const uint32_t t = t0 + (uint32_t)d;
                    if (t < mine) {
                        if constexpr (SPLIT) T = umax64(T, uniform64(gbuf[d]));
                        const int32_t tb = prefilter_bound(T);
                        const uint32_t vbase = bid[d] * (uint32_t)kBlock;
                        const bool ragged = vbase < off0 || vbase + (uint32_t)kBlock > vend;
                        int32_t mx = INT32_MIN;
#pragma unroll
                        for (int u = 0; u < kLoadsPerBlock; ++u) {
                            const int32_t a0 = __float_as_int(buf[d][u].x);
                            const int32_t a1 = __float_as_int(buf[d][u].y);
                            const int32_t a2 = __float_as_int(buf[d][u].z);
                            const int32_t a3 = __float_as_int(buf[d][u].w);
                            mx = max(max(mx, a0), a1);
                            mx = max(max(mx, a2), a3);
                        }
                        if (__ballot(ragged || mx >= tb) != 0ull) {
                            const uint32_t before = cnt;
                            cnt = admit_block(tray, cnt, T, buf[d], vbase, off0, vend, ragged, lane);
                            entered += cnt - before;
                        }
                    }
                    issue(buf[d], bid[d], gbuf[d], t + (uint32_t)D);
                    T = umax64(T, lds_load_word(&s_T));
                    if (cnt >= Wm) {
                        publish_tray(&s_fill[w][cur], cnt, lane);
                        cur ^= 1u;
                        cnt = 0;
                        tray = trays + (size_t)(2 * w + cur) * CW;
                        wait_tray_free(&s_fill[w][cur]);
                    }
                }
            }
            if (cnt > 0) publish_tray(&s_fill[w][cur], cnt, lane);
        }
        if (p.stats && lane == 0 && entered > 0) {
            atomicAdd(p.stats + 2 * (size_t)r, (unsigned long long)entered);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        if (lane == 0) __hip_atomic_fetch_add(&s_done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        return;
    }

    // ---- sorter (wave NS) ----
    uint64_t kept[E];
#pragma unroll
    for (int e = 0; e < E; ++e) kept[e] = 0ull;
    SorterState ss;
    ss.T = 0ull;
    ss.sorts = 0u;
    for (;;) {
        const uint32_t done = lds_load_u32(&s_done);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
        bool worked = false;
        for (uint32_t v = 0; v < NS; ++v) {
            for (uint32_t b = 0; b < 2; ++b) {
                const uint32_t c = lds_load_u32(&s_fill[v][b]);
                if (c == 0u) continue;
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
                sort_tray<E, SPLIT>(kept, ss, trays + (size_t)(2 * v + b) * CW, c, &s_T, gT, k,
                                    lane);
                publish_tray(&s_fill[v][b], 0u, lane);
                worked = true;
            }
        }
        if (!worked) {
            if (done == NS) break;
            __builtin_amdgcn_s_sleep(2);
        }
    }
    if (p.stats && lane == 0 && ss.sorts > 0) {
        atomicAdd(p.stats + 2 * (size_t)r + 1, (unsigned long long)ss.sorts);
    }

    if constexpr (!SPLIT) {
        write_row<E>(p.out_vals + (size_t)r * k, p.out_idx + (size_t)r * k, k, kept, lane);
    } else {
        // Publish this segment's list, take a ticket; the last of the row's
        // segments to arrive merges every list and writes the row.
        uint64_t *lists = p.ws_lists + (size_t)r * S * KP;
        store_list<E>(lists + (size_t)s * KP, kept, lane);
        __threadfence();
        uint32_t old = 0;
        if (lane == 0) {
            old = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        }
        old = __builtin_amdgcn_readfirstlane((int)old);
        if (old != S - 1u) return;
        __threadfence();
        for (uint32_t j = 0; j < S; ++j) {
            if (j == s) continue;
            uint64_t b[E];
            load_list_reversed<E>(b, lists + (size_t)j * KP, lane);
            keep_best<E>(kept, b, lane);
        }
        write_row<E>(p.out_vals + (size_t)r * k, p.out_idx + (size_t)r * k, k, kept, lane);
        // Leave this row's part of the workspace all zero, so the next call
        // may use the same memory with any shape.
        uint64_t zero[E];
#pragma unroll
        for (int e = 0; e < E; ++e) zero[e] = 0ull;
        for (uint32_t j = 0; j < S; ++j) store_list<E>(lists + (size_t)j * KP, zero, lane);
        if (lane == 0) {
            __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(gT, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

__global__ void fill_zero_kernel(uint4 *p, size_t n16) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
         i += (size_t)gridDim.x * blockDim.x) {
        p[i] = make_uint4(0u, 0u, 0u, 0u);
    }
}

// Streaming read with the selection kernel's access pattern (1 KiB per wave
// per dwordx4 instruction, 4 KiB per wave per block), folded into one word
// per workgroup so the loads cannot be removed.
constexpr int kProbeThreads = 256;
constexpr size_t kProbeBytesPerGroup = (size_t)64 << 10;

__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const float4 *src, size_t n16,
                                                                   uint32_t *sink) {
    const size_t per_group = kProbeBytesPerGroup / 16;
    const size_t begin = (size_t)blockIdx.x * per_group;
    size_t end = begin + per_group;
    end = end < n16 ? end : n16;
    uint32_t acc = 0;
    for (size_t i = begin + threadIdx.x; i < end; i += kProbeThreads) {
        const float4 v = src[i];
        acc ^= __float_as_uint(v.x) ^ __float_as_uint(v.y) ^ __float_as_uint(v.z) ^
               __float_as_uint(v.w);
    }
    __shared__ uint32_t red[kProbeThreads];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int h = kProbeThreads / 2; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h) red[threadIdx.x] ^= red[threadIdx.x + h];
        __syncthreads();
    }
    if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(256) void probe_copy_kernel(const float4 *src, float4 *dst, size_t n16) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
         i += (size_t)gridDim.x * blockDim.x) {
        dst[i] = src[i];
    }
}

template <int E>
hipError_t launch_e(const SelectArgs &a, int waves, size_t lds, hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)a.rows * a.split));
    const dim3 block((unsigned)(waves * kWave));
    if (a.split > 1) {
        hipLaunchKernelGGL((select_kernel<E, true>), grid, block, lds, stream, a);
    } else {
        hipLaunchKernelGGL((select_kernel<E, false>), grid, block, lds, stream, a);
    }
    return hipGetLastError();
}

template <int E>
hipError_t raise_lds_limit(size_t lds) {
    hipError_t e1 = hipFuncSetAttribute(reinterpret_cast<const void *>(&select_kernel<E, true>),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipError_t e2 = hipFuncSetAttribute(reinterpret_cast<const void *>(&select_kernel<E, false>),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    return e1 != hipSuccess ? e1 : e2;
}

}  // namespace

hipError_t launch_select(const SelectArgs &a, int E, int waves, size_t lds, hipStream_t stream) {
    if (lds > 65536) {
        hipError_t e = hipSuccess;
        switch (E) {
            case 1: e = raise_lds_limit<1>(lds); break;
            case 2: e = raise_lds_limit<2>(lds); break;
            case 4: e = raise_lds_limit<4>(lds); break;
            case 8: e = raise_lds_limit<8>(lds); break;
            case 16: e = raise_lds_limit<16>(lds); break;
            case 32: e = raise_lds_limit<32>(lds); break;
            default: return hipErrorInvalidValue;
        }
        if (e != hipSuccess) return e;
    }
    switch (E) {
        case 1: return launch_e<1>(a, waves, lds, stream);
        case 2: return launch_e<2>(a, waves, lds, stream);
        case 4: return launch_e<4>(a, waves, lds, stream);
        case 8: return launch_e<8>(a, waves, lds, stream);
        case 16: return launch_e<16>(a, waves, lds, stream);
        case 32: return launch_e<32>(a, waves, lds, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t stream) {
    const size_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    size_t groups = (n16 + 255) / 256;
    if (groups > 4096) groups = 4096;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)groups), dim3(256), 0, stream,
                       reinterpret_cast<uint4 *>(p), n16);
    return hipGetLastError();
}

size_t probe_read_groups(size_t bytes) {
    return (bytes + kProbeBytesPerGroup - 1) / kProbeBytesPerGroup;
}

hipError_t launch_probe_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream) {
    const size_t groups = probe_read_groups(bytes);
    if (groups == 0) return hipSuccess;
    hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)groups), dim3(kProbeThreads), 0, stream,
                       reinterpret_cast<const float4 *>(src), bytes / 16, sink);
    return hipGetLastError();
}

hipError_t launch_probe_copy(const void *src, void *dst, size_t bytes, hipStream_t stream) {
    const size_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    size_t groups = (n16 + 255) / 256;
    if (groups > 65536) groups = 65536;
    hipLaunchKernelGGL(probe_copy_kernel, dim3((unsigned)groups), dim3(256), 0, stream,
                       reinterpret_cast<const float4 *>(src), reinterpret_cast<float4 *>(dst), n16);
    return hipGetLastError();
}

}  // namespace topk
