// Shared device/host helpers: order-preserving keys, packed words, constants.
//
// Every score travels as one 64-bit word: the high half is an unsigned key
// whose order is the IEEE-754 total order of the float (-inf < ... < -0.0 <
// +0.0 < ... < +inf), the low half is 0xFFFFFFFF - position.  A larger word
// is a better element: higher value first, and for equal values the lower
// position.  Unpacking gives the original float bits and position back
// exactly, and two elements never share a word, so indices cannot repeat
// (kernelbench.com "DeepSeek V4.1 Flash", bitonic-selection paragraph; the
// position complement is how this library gives ties to the lower index).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define TOPK_HD __host__ __device__ __forceinline__

namespace topk {

// Elements per block: the unit of the shuffled visit order ("The Secret GPU
// Kernel Behind DeepSeek V4.1 Flash", transcript 3:30).
constexpr int kBlock = 1024;
constexpr int kWave = 64;
constexpr int kMaxWaves = 8;

TOPK_HD uint32_t order_key(uint32_t bits) {
    // negative floats: flip all bits; non-negative: set the sign bit
    return bits ^ ((uint32_t)((int32_t)bits >> 31) | 0x80000000u);
}

TOPK_HD uint32_t key_bits(uint32_t key) {
    return (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
}

TOPK_HD uint64_t pack_word(uint32_t key, uint32_t pos) {
    return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - pos);
}

TOPK_HD uint32_t word_pos(uint64_t w) { return 0xFFFFFFFFu - (uint32_t)w; }

// Four floats as a native vector (the operand type of the buffer-load
// builtins).
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Workgroup barrier that orders LDS accesses only: global loads a wave has in
// flight stay in flight across it (a full __syncthreads() waits for them).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One 16-byte load of scores that are read once, with the nontemporal hint
// (on gfx950 a read-only sweep streams at 6.5-7.0 TB/s with it against
// 5.8-6.1 TB/s without).  `p` is 16-byte aligned.
__device__ __forceinline__ float4 load_stream4(const float *p) {
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}

// Largest key that is not a real number: keys at or below it are negative
// NaN patterns, key 0x007FFFFF is -inf itself.
constexpr uint32_t kKeyNegInf = 0x007FFFFFu;

TOPK_HD uint64_t splitmix64(uint64_t x) {
    x += 0x9E3779B97F4A7C15ull;
    x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
    x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
    return x ^ (x >> 31);
}

TOPK_HD uint32_t mix32(uint32_t x) {
    // MurmurHash3 finalizer
    x ^= x >> 16;
    x *= 0x85EBCA6Bu;
    x ^= x >> 13;
    x *= 0xC2B2AE35u;
    x ^= x >> 16;
    return x;
}

// Block visit order of one row: a keyed Feistel permutation of [0, 2^m)
// (m even, 2^m >= nblocks) walked until it lands in [0, nblocks).  It depends
// only on (seed, row, nblocks), never on the scores, so no input can be
// arranged to make the filter slow ("The Secret GPU Kernel Behind DeepSeek
// V4.1 Flash", transcript 4:55-5:10).
struct VisitOrder {
    uint32_t nblocks;
    uint32_t half;      // bits per Feistel half
    uint32_t mask;      // (1 << half) - 1
    uint32_t key[4];
};

TOPK_HD VisitOrder make_visit_order(uint64_t seed, uint32_t row, uint32_t nblocks) {
    VisitOrder o;
    o.nblocks = nblocks;
    uint32_t m = 2;
    while ((1u << m) < nblocks) m += 2;
    o.half = m / 2;
    o.mask = (1u << o.half) - 1u;
    uint64_t s = splitmix64(seed ^ (0xD1B54A32D192ED03ull * ((uint64_t)row + 1)));
    uint64_t t = splitmix64(s);
    o.key[0] = (uint32_t)s;
    o.key[1] = (uint32_t)(s >> 32);
    o.key[2] = (uint32_t)t;
    o.key[3] = (uint32_t)(t >> 32);
    return o;
}

TOPK_HD uint32_t feistel(const VisitOrder &o, uint32_t x) {
    uint32_t l = x >> o.half, r = x & o.mask;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t f = mix32(r * 0x9E3779B1u ^ o.key[i]) & o.mask;
        uint32_t nl = r;
        r = l ^ f;
        l = nl;
    }
    return (l << o.half) | r;
}

// Block visited at step p (p < nblocks).  A bijection of [0, nblocks).
TOPK_HD uint32_t visit_block(const VisitOrder &o, uint32_t p) {
    uint32_t x = feistel(o, p);
    while (x >= o.nblocks) x = feistel(o, x);
    return x;
}

}  // namespace topk
