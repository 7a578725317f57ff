// Sparse-attention decode over the selected positions: the consumer of the
// top-k indices ("The Secret GPU Kernel Behind DeepSeek V4.1 Flash",
// transcript 1:48-2:13: the indexer picks which positions the expensive
// attention reads; "The Full-Stack Optimization of DeepSeek-V4-Flash on
// Blackwell GPUs", chunk 68.0 summary: a sparse-MLA decode kernel splits the
// top-k dimension across workgroups and merges the parts by log-sum-exp).
//
// Layout (the pages give none): one latent cache kv[n][dqk] in bf16 shared
// by every head, values = its first dv channels; queries q[rows][heads][dqk]
// in bf16; idx[rows][k] from the selection (-1 and out-of-range entries
// select nothing).
//
// decode_partial_kernel: workgroup (split s, 16-head group, row r), four
// waves.  Its share of the row's selected positions is walked in tiles of
// 32: the tile's cache rows are gathered into LDS (16-byte loads), the
// scores S = Q K^T (16 heads x 32 positions) come from gfx950's bf16 MFMA
// 16x16x32 (16-byte operands, 32 of the dqk dimension per issue) with the
// dqk dimension spread over the four waves and summed through LDS,
// an online softmax updates each head's running maximum and sum, and
// O += P V runs on the same MFMA, one issue per 16 value columns for the
// tile's 32 positions, with each wave owning a quarter of the dv columns
// (P rounded to bf16, and the running sum adds the rounded weights, so the
// weights stay normalised).  The split writes (O, max, sum) per head.
// decode_combine_kernel merges the splits by their log-sum-exp.
#include <hip/hip_runtime.h>

#include "common.h"
#include "internal.h"

namespace topk {
namespace {

typedef short bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// bf16 MFMA 16x16x32 (gfx950): lane l holds A[l % 16][8 (l / 16) + i] and
// B[8 (l / 16) + i][l % 16] for i < 8, and D[4 (l / 16) + e][l % 16].
__device__ __forceinline__ f32x4_t mfma32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef short bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

// gfx950's transposing LDS read (ds_read_b64_tr_b16): inside each group of
// 16 lanes, lane j receives element j % 4 of the 8-byte pieces read by lanes
// j / 4 + 4 e, e = 0..3.  When lane L of a group reads the four columns
// c + 4 (L % 4) .. c + 4 (L % 4) + 3 of row r0 + L / 4 of a row-major bf16
// matrix, lane j receives rows r0 .. r0 + 3 of column c + j: a column slice,
// which is how the MFMA's B operand wants the value rows.
__device__ __forceinline__ bf16x4_t lds_read_tr16(const uint16_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bf16x4_t *)(p));
}

constexpr int kDecThreads = 256;
constexpr int kDecTile = 32;       // selected positions per tile
constexpr int kDecHeads = 16;      // heads per workgroup (MFMA rows)
// Register arrays are sized per instantiation: MS 32-wide dqk steps and MV
// 16-column value tiles per wave.  The compact one covers dqk <= 576 and
// dv <= 512 (the MLA shape); the general one the limits.
constexpr int kDecStepsSmall = (576 / 32 + 3) / 4, kDecVTilesSmall = 512 / 64;
constexpr int kDecStepsMax = kMaxDecodeDqk / 32 / 4, kDecVTilesMax = kMaxDecodeDv / 64;
// 16-byte pieces per thread prefetched for the next tile (the rest load at
// commit): all nine of a dqk = 576 tile in the compact instantiation.
constexpr int kDecChunksSmall = kDecTile * 576 / 8 / kDecThreads, kDecChunksMax = 8;

__device__ __forceinline__ uint16_t to_bf16(float x) {
    // round to nearest even (weights are finite and non-negative)
    const uint32_t b = __float_as_uint(x);
    return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float from_bf16(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

template <int kDecMaxSteps, int kDecMaxVTiles, int kDecChunks, int kExactDqk = 0, int kExactDv = 0>
__global__ __launch_bounds__(kDecThreads) void decode_partial_kernel(DecodeArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int ldk = a.dqk + 8;  // padded row (16-byte multiple) against bank conflicts
    uint16_t *kt = reinterpret_cast<uint16_t *>(smem);                        // [32][ldk]
    float *sred = reinterpret_cast<float *>(smem + (size_t)kDecTile * ldk * 2);  // [4][16][32]
    uint16_t *pw = reinterpret_cast<uint16_t *>(sred + 4 * kDecHeads * kDecTile);  // [16][32]
    float *alpha = reinterpret_cast<float *>(pw + kDecHeads * kDecTile);       // [16]
    float *mrun = alpha + kDecHeads;
    float *lrun = mrun + kDecHeads;
    __shared__ int32_t pos[kDecTile];       // the current tile's positions (-1: none)
    __shared__ int32_t pos_next[kDecTile];  // the prefetched tile's

    const int s = blockIdx.x;
    const int h0 = blockIdx.y * kDecHeads;
    const int64_t r = (int64_t)a.row0 + blockIdx.z;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
    const int col16 = lane & 15, grp = lane >> 4;
    const int t0 = s * a.per_split;
    const int t1 = min(a.k, t0 + a.per_split);
    // exact-shape instantiations know these at compile time, so the guards
    // in the unrolled loops fold away and operand loads can be issued early
    // 32-wide dqk steps; when dqk is an odd multiple of 16 the last step's
    // upper half (lanes with grp >= 2) is zero on both operands
    const int dqk = kExactDqk ? kExactDqk : a.dqk;
    const int nks = (dqk + 31) / 32;
    const int nvt = kExactDv ? kExactDv / 64 : a.dv / 64;

    // This wave's query operands: k-steps ks = wv, wv + 4, ... (A layout:
    // lane holds row col16, k = 8 grp .. 8 grp + 7 of the step).
    bf16x8_t qa[kDecMaxSteps];
    const uint16_t *qrow = a.q + ((size_t)r * a.heads + h0 + col16) * a.dqk;
#pragma unroll
    for (int i = 0; i < kDecMaxSteps; ++i) {
        const int ks = wv + 4 * i;
        bf16x8_t v = {0, 0, 0, 0, 0, 0, 0, 0};
        if (ks < nks && ks * 32 + grp * 8 < dqk)
            v = *reinterpret_cast<const bf16x8_t *>(qrow + ks * 32 + grp * 8);
        qa[i] = v;
    }
    f32x4_t acc[kDecMaxVTiles];
#pragma unroll
    for (int i = 0; i < kDecMaxVTiles; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (tid < kDecHeads) {
        mrun[tid] = -__builtin_inff();
        lrun[tid] = 0.f;
    }

    // The next tile's cache rows are loaded into registers while the
    // current tile computes, then stored to LDS once the current tile is
    // done with it.  A tile is 32 rows x dqk/8 16-byte pieces over 256
    // threads; each thread prefetches up to kDecChunks of them (all of them
    // for dqk <= 512) and loads any rest when it stores.
    const int cpr = kExactDqk ? kExactDqk / 8 : a.dqk / 8;
    uint4 pre[kDecChunks];
    int32_t pre_pos = -1;  // threads 0..31: the position of their tile row
    auto fetch = [&](int tb) __attribute__((always_inline)) {
        if (tid < kDecTile) {
            const int t = tb + tid;
            int32_t j = -1;
            if (t < t1) {
                j = a.idx[(size_t)r * a.k + t];
                if (j < 0 || (int64_t)j >= a.n_kv) j = -1;
            }
            pre_pos = j;
            pos_next[tid] = j;
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kDecChunks; ++u) {
            const int c = tid + u * kDecThreads;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (c < kDecTile * cpr) {
                const int row = c / cpr, cc = c - row * cpr;
                const int32_t j = pos_next[row];
                if (j >= 0) v = *reinterpret_cast<const uint4 *>(a.kv + (size_t)j * a.dqk + cc * 8);
            }
            pre[u] = v;
        }
    };
    auto commit = [&]() __attribute__((always_inline)) {
        if (tid < kDecTile) pos[tid] = pre_pos;
#pragma unroll
        for (int u = 0; u < kDecChunks; ++u) {
            const int c = tid + u * kDecThreads;
            if (c < kDecTile * cpr) {
                const int row = c / cpr, cc = c - row * cpr;
                *reinterpret_cast<uint4 *>(kt + row * ldk + cc * 8) = pre[u];
            }
        }
        for (int c = tid + kDecChunks * kDecThreads; c < kDecTile * cpr; c += kDecThreads) {
            const int row = c / cpr, cc = c - row * cpr;
            const int32_t j = pos_next[row];
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (j >= 0) v = *reinterpret_cast<const uint4 *>(a.kv + (size_t)j * a.dqk + cc * 8);
            *reinterpret_cast<uint4 *>(kt + row * ldk + cc * 8) = v;
        }
    };
    if (t0 < t1) {
        fetch(t0);
        commit();
    }
    __syncthreads();

    for (int tb = t0; tb < t1; tb += kDecTile) {
        const bool more = tb + kDecTile < t1;
        if (more) fetch(tb + kDecTile);   // loads in flight during this tile
        // partial scores over this wave's k-steps (B layout: lane holds
        // column col16 of the n-tile, k = 8 grp .. 8 grp + 7: one 16-byte
        // LDS read)
        f32x4_t sacc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int i = 0; i < kDecMaxSteps; ++i) {
            const int ks = wv + 4 * i;
            if (ks < nks) {
                const bool in = ks * 32 + grp * 8 < dqk;
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    bf16x8_t b = {0, 0, 0, 0, 0, 0, 0, 0};
                    if (in) {
                        b = *reinterpret_cast<const bf16x8_t *>(kt + (nt * 16 + col16) * ldk +
                                                                ks * 32 + grp * 8);
                    }
                    sacc[nt] = mfma32(qa[i], b, sacc[nt]);
                }
            }
        }
        // D layout: lane holds rows 4 grp + e, column col16
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sred[(wv * kDecHeads + grp * 4 + e) * kDecTile + nt * 16 + col16] = sacc[nt][e];
            }
        }
        __syncthreads();
        // online softmax: 16 threads per head (one 16-lane group), two
        // positions each
        {
            const int hh = tid >> 4, c0 = (tid & 15) * 2;
            float sv[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int c = c0 + e;
                float x = 0.f;
#pragma unroll
                for (int w = 0; w < 4; ++w) x += sred[(w * kDecHeads + hh) * kDecTile + c];
                sv[e] = pos[c] >= 0 ? x * a.scale : -__builtin_inff();
            }
            float mx = fmaxf(sv[0], sv[1]);
#pragma unroll
            for (int off = 8; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
            const float mold = mrun[hh];
            const float mnew = fmaxf(mold, mx);
            float al = 1.f, p[2] = {0.f, 0.f};
            if (mnew != -__builtin_inff()) {
                al = expf(mold - mnew);
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    if (sv[e] != -__builtin_inff()) p[e] = from_bf16(to_bf16(expf(sv[e] - mnew)));
                }
            }
            float ps = p[0] + p[1];
#pragma unroll
            for (int off = 8; off > 0; off >>= 1) ps += __shfl_xor(ps, off);
            pw[hh * kDecTile + c0] = to_bf16(p[0]);
            pw[hh * kDecTile + c0 + 1] = to_bf16(p[1]);
            if ((tid & 15) == 0) {
                mrun[hh] = mnew;
                lrun[hh] = lrun[hh] * al + ps;
                alpha[hh] = al;
            }
        }
        __syncthreads();
        // O = alpha O + P V over this wave's column tiles
        float al[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) al[e] = alpha[grp * 4 + e];
#pragma unroll
        for (int nt = 0; nt < kDecMaxVTiles; ++nt) {
            if (nt < nvt) {
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[nt][e] *= al[e];
            }
        }
        // the tile's 32 positions are one k-step: A = P (lane holds head
        // col16, positions 8 grp .. 8 grp + 7), B = V (lane holds value
        // column col16 of those positions, two transposing LDS reads)
        {
            const bf16x8_t pa = *reinterpret_cast<const bf16x8_t *>(pw + col16 * kDecTile + grp * 8);
            const int dv4 = kExactDv ? kExactDv / 4 : a.dv / 4;
            const uint16_t *vrow = kt + (grp * 8 + (col16 >> 2)) * ldk + 4 * (col16 & 3);
#pragma unroll
            for (int nt = 0; nt < kDecMaxVTiles; ++nt) {
                if (nt < nvt) {
                    const int cb = wv * dv4 + nt * 16;
                    const bf16x4_t lo = lds_read_tr16(vrow + cb);
                    const bf16x4_t hi = lds_read_tr16(vrow + 4 * ldk + cb);
                    const bf16x8_t b = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    acc[nt] = mfma32(pa, b, acc[nt]);
                }
            }
        }
        __syncthreads();
        if (more) {
            commit();
            __syncthreads();
        }
    }
    // this split's (O, max, sum) per head
#pragma unroll
    for (int nt = 0; nt < kDecMaxVTiles; ++nt) {
        if (nt < nvt) {
            const int col = wv * (a.dv / 4) + nt * 16 + col16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int head = h0 + grp * 4 + e;
                a.part_o[(((size_t)r * a.heads + head) * a.splits + s) * a.dv + col] = acc[nt][e];
            }
        }
    }
    if (tid < kDecHeads) {
        float *ml = a.part_ml + (((size_t)r * a.heads + h0 + tid) * a.splits + s) * 2;
        ml[0] = mrun[tid];
        ml[1] = lrun[tid];
    }
}

// One workgroup per (row, head): out = sum_s e^(m_s - M) O_s / sum_s
// e^(m_s - M) l_s.  Wave 0 reduces the splits' maxima and sums once and
// leaves one weight per split in LDS; every thread then sums its columns
// over the splits with independent loads.
constexpr int kMaxCombineSplits = kRadixMaxK / kDecTile;   // splits of >= 32 positions

__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
    __shared__ float wgt[kMaxCombineSplits];
    __shared__ float s_scale;
    const int64_t rh = blockIdx.x;   // r * heads + h
    const int tid = threadIdx.x;
    const float *ml = a.part_ml + (size_t)rh * a.splits * 2;
    if (tid < kWave) {
        float M = -__builtin_inff();
        for (int q = tid; q < a.splits; q += kWave) M = fmaxf(M, ml[2 * q]);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
        float L = 0.f;
        for (int q = tid; q < a.splits; q += kWave) {
            const float w = M == -__builtin_inff() ? 0.f : expf(ml[2 * q] - M);
            wgt[q] = w;
            L += w * ml[2 * q + 1];
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off);
        if (tid == 0) s_scale = L > 0.f ? 1.f / L : 0.f;
    }
    __syncthreads();
    const float scale = s_scale;
    const float *po = a.part_o + (size_t)rh * a.splits * a.dv;
    float *out = a.out + (size_t)rh * a.dv;
    for (int c = tid; c < a.dv; c += blockDim.x) {
        float o = 0.f;
        for (int q = 0; q < a.splits; ++q) o += wgt[q] * po[(size_t)q * a.dv + c];
        out[c] = o * scale;
    }
}

}  // namespace

size_t decode_lds_bytes(int dqk) {
    return (size_t)kDecTile * (dqk + 8) * 2 + (size_t)4 * kDecHeads * kDecTile * 4 +
           (size_t)kDecHeads * kDecTile * 2 + 3 * kDecHeads * 4;
}

template <int MS, int MV, int PC, int XQ = 0, int XV = 0>
hipError_t launch_partial(const DecodeArgs &a, hipStream_t stream) {
    // Set on every launch (as for the selection kernel): the attribute
    // belongs to the current device, and calls may come on several.
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&decode_partial_kernel<MS, MV, PC, XQ, XV>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)decode_lds_bytes(a.dqk));
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)a.splits, (unsigned)(a.heads / kDecHeads), (unsigned)a.rows);
    hipLaunchKernelGGL((decode_partial_kernel<MS, MV, PC, XQ, XV>), grid, dim3(kDecThreads),
                       decode_lds_bytes(a.dqk), stream, a);
    return hipGetLastError();
}

hipError_t launch_decode_partial(const DecodeArgs &a, hipStream_t stream) {
    if (a.rows <= 0) return hipSuccess;
    if (a.dqk == 576 && a.dv == 512)   // the MLA shape, exactly
        return launch_partial<kDecStepsSmall, kDecVTilesSmall, kDecChunksSmall, 576, 512>(a, stream);
    if (a.dqk <= 16 * 4 * kDecStepsSmall && a.dv <= 64 * kDecVTilesSmall)
        return launch_partial<kDecStepsSmall, kDecVTilesSmall, kDecChunksSmall>(a, stream);
    return launch_partial<kDecStepsMax, kDecVTilesMax, kDecChunksMax>(a, stream);
}

// Combines every row of the call (a.rows is the total; row0 unused).
hipError_t launch_decode_combine(const DecodeArgs &a, hipStream_t stream) {
    if (a.rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)((int64_t)a.rows * a.heads)), dim3(256),
                       0, stream, a);
    return hipGetLastError();
}

}  // namespace topk
