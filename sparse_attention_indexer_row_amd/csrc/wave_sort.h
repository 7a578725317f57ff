// Wave-level bitonic sort and merge of 64*E packed words held in registers.
//
// Element i of a list lives in lane i / E, register i % E ("blocked" layout):
// compare-exchange distances below E stay inside a lane's registers, larger
// ones pair lane l with lane l ^ (distance / E) through DPP or permlane-swap
// lane exchanges.  No LDS traffic and no barrier: one wavefront sorts its
// own list with VALU instructions only.
//
// Keep-the-best merge (kernelbench.com "DeepSeek V4.1 Flash",
// bitonic-selection paragraph: the second list is compared in reverse
// where it lies, so the union is bitonic without a reversed copy): with A
// sorted descending and B sorted ascending in the same layout,
// max(A[i], B[i]) holds the best 64*E words of A and B and forms a bitonic
// sequence, which one bitonic merge sorts.
#pragma once

#include "common.h"

namespace topk {

__device__ __forceinline__ uint32_t lane_id() {
    return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t umin64(uint64_t a, uint64_t b) { return a < b ? a : b; }

// Lane permutation inside a row of 16.  Every control used with it names a
// valid source lane for every lane, so no old value is needed (a plain DPP
// move, without the extra register that update_dpp's old operand costs).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}

template <int CTRL, int ROW_MASK, bool BOUND_ZERO>
__device__ __forceinline__ uint32_t dpp_add_src(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, BOUND_ZERO);
}

// Inclusive prefix sum over the wave's lanes with DPP: shifts by 1, 2, 4, 8
// inside each 16-lane row, then row_bcast:15 and row_bcast:31 carry the row
// totals upward.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    v += dpp_add_src<0x111, 0xF, true>(v);
    v += dpp_add_src<0x112, 0xF, true>(v);
    v += dpp_add_src<0x114, 0xF, true>(v);
    v += dpp_add_src<0x118, 0xF, true>(v);
    v += dpp_add_src<0x142, 0xA, false>(v);
    v += dpp_add_src<0x143, 0xC, false>(v);
    return v;
}

// Value of `v` in lane (lane ^ D), with VALU lane exchanges only:
//   D = 1, 2     DPP quad_perm [1,0,3,2] / [2,3,0,1]
//   D = 4        DPP row_half_mirror (l -> 7-l in 8) then quad_perm [3,2,1,0]
//   D = 8        DPP row_ror:8 (rotating a 16-lane row by 8 is l ^ 8)
//   D = 16, 32   v_permlane16_swap / v_permlane32_swap of the value with
//                itself: the first result holds the lower half-group's data
//                in both halves, the second the upper half-group's.
template <int D>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v, uint32_t lane) {
    if constexpr (D == 1) {
        return dpp_mov<0xB1>(v);
    } else if constexpr (D == 2) {
        return dpp_mov<0x4E>(v);
    } else if constexpr (D == 4) {
        return dpp_mov<0x1B>(dpp_mov<0x141>(v));
    } else if constexpr (D == 8) {
        return dpp_mov<0x128>(v);
    } else if constexpr (D == 16) {
        const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (lane & 16u) ? p[0] : p[1];
    } else {
        static_assert(D == 32, "lane distance must be a power of two below 64");
        const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (lane & 32u) ? p[0] : p[1];
    }
}

template <int D>
__device__ __forceinline__ uint64_t xor_lane64(uint64_t v, uint32_t lane) {
    const uint32_t lo = xor_lane<D>((uint32_t)v, lane);
    const uint32_t hi = xor_lane<D>((uint32_t)(v >> 32), lane);
    return ((uint64_t)hi << 32) | lo;
}

// One compare-exchange stage at distance J inside sub-sequences of length
// SIZE.  Sub-sequence direction: ascending when (i & SIZE) == 0 for the
// ascending network (ASC), flipped for the descending one.  When SIZE equals
// the whole list every sub-sequence runs in the final direction.
template <int E, int SIZE, int J, bool ASC>
__device__ __forceinline__ void bitonic_stage(uint64_t (&a)[E], uint32_t lane) {
    constexpr int N = 64 * E;
    if constexpr (J < E) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if ((e & J) != 0) continue;
            const int e2 = e | J;
            bool up;
            if constexpr (SIZE >= N) {
                up = ASC;
            } else if constexpr (SIZE < E) {
                up = (((e & SIZE) == 0) == ASC);
            } else {
                up = ((((lane * E) & SIZE) == 0) == ASC);
            }
            const uint64_t x = a[e], y = a[e2];
            const bool swap = (x > y) == up;
            a[e] = swap ? y : x;
            a[e2] = swap ? x : y;
        }
    } else {
        constexpr int D = J / E;
        const bool lower = (lane & D) == 0;
        bool up;
        if constexpr (SIZE >= N) {
            up = ASC;
        } else {
            up = ((((lane * E) & SIZE) == 0) == ASC);
        }
        const bool take_min = (lower == up);
        // All exchanges first, then all compares, then all selects: the E
        // independent chains overlap instead of each waiting on its own
        // cross-lane move.
        uint64_t y[E];
#pragma unroll
        for (int e = 0; e < E; ++e) y[e] = xor_lane64<D>(a[e], lane);
        bool keep[E];
#pragma unroll
        for (int e = 0; e < E; ++e) keep[e] = (a[e] < y[e]) == take_min;
#pragma unroll
        for (int e = 0; e < E; ++e) a[e] = keep[e] ? a[e] : y[e];
    }
}

template <int E, int SIZE, int J, bool ASC>
__device__ __forceinline__ void bitonic_stages_from(uint64_t (&a)[E], uint32_t lane) {
    bitonic_stage<E, SIZE, J, ASC>(a, lane);
    if constexpr (J > 1) bitonic_stages_from<E, SIZE, J / 2, ASC>(a, lane);
}

template <int E, int SIZE, bool ASC>
__device__ __forceinline__ void bitonic_levels_from(uint64_t (&a)[E], uint32_t lane) {
    bitonic_stages_from<E, SIZE, SIZE / 2, ASC>(a, lane);
    if constexpr (SIZE < 64 * E) bitonic_levels_from<E, SIZE * 2, ASC>(a, lane);
}

// Full sort of the wave's 64*E words (ascending if ASC, else descending).
template <int E, bool ASC>
__device__ __forceinline__ void wave_sort(uint64_t (&a)[E], uint32_t lane) {
    bitonic_levels_from<E, 2, ASC>(a, lane);
}

// Sorts a bitonic sequence of 64*E words.
template <int E, bool ASC>
__device__ __forceinline__ void wave_merge(uint64_t (&a)[E], uint32_t lane) {
    bitonic_stages_from<E, 64 * E, 32 * E, ASC>(a, lane);
}

// acc (descending) := best 64*E words of acc and b (b ascending), descending.
template <int E>
__device__ __forceinline__ void keep_best(uint64_t (&acc)[E], const uint64_t (&b)[E],
                                          uint32_t lane) {
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = umax64(acc[e], b[e]);
    wave_merge<E, false>(acc, lane);
}

// Word at list position `pos` (any lane may ask; all get the same answer).
template <int E>
__device__ __forceinline__ uint64_t list_word_at(const uint64_t (&a)[E], uint32_t pos) {
    const uint32_t e_sel = pos % E;
    uint64_t v = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) v = (e == (int)e_sel) ? a[e] : v;
    const int src = (int)(pos / E);
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, src);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), src);
    return ((uint64_t)hi << 32) | lo;
}

}  // namespace topk
