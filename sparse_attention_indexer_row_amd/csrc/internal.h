// Host <-> kernel interface inside the library (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "select_args.h"

namespace topk {

// Block-max pooled pre-selection, first step: block maxima and pinned slots.
struct PoolArgs {
    const float *scores;       // [rows][n]
    const int32_t *lengths;    // [rows] or null
    int64_t n;
    int64_t bm_ld;             // row stride of bm (>= ceil(n / group))
    int32_t rows;              // rows handled by this launch
    int32_t row0;
    int32_t group;             // positions per block
    int32_t pinned;            // newest blocks kept whatever their scores
    int32_t keep;              // output slots per row
    int32_t span;              // work items per row: max(ceil(n / group), pinned)
    float *bm;                 // [rows][bm_ld] block maxima (blocks < nb_r written)
    int32_t *older;            // [rows] nb_r - min(pinned, nb_r)
    float *out_vals;           // [rows][keep]: slots [0, pinned) written
    int32_t *out_idx;
};

hipError_t launch_block_max(const PoolArgs &a, hipStream_t stream);

// Best `k` of each row: an exact radix selection over the rows' 64-bit
// (key, position) words, one workgroup per row.
constexpr int kRadixMaxK = 8192;
constexpr int kMaxPooledSlots = 8192;

struct RadixArgs {
    const float *vals;         // [rows][ld], any 4-byte alignment
    const int32_t *count;      // [rows] valid elements per row (clamped to [0, ld]) or null (ld)
    int64_t ld;
    int32_t rows;              // rows handled by this launch
    int32_t row0;
    int32_t k;                 // 1..kRadixMaxK
    float *out_vals;           // [rows][out_ld], first k slots of each row written
    int32_t *out_idx;
    int64_t out_ld;
    // Pooled rows (pool non-null): element i of row r is context position
    // pool[r][i / group] * group + i % group; empty slots and positions at or
    // past the row's context length are not candidates.
    const int32_t *pool;       // [rows][pool_keep] or null
    int32_t pool_keep;         // <= kMaxPooledSlots; pooled rows take k <= 2048
    int32_t group;
    int64_t n_ctx;
    const int32_t *ctx_lengths;  // [rows] or null (n_ctx)
};

hipError_t launch_radix_select(const RadixArgs &a, hipStream_t stream);
// Dynamic LDS of the radix selection's launch for list size k (pool_keep
// slots kept in LDS for pooled rows, 0 otherwise).
size_t radix_lds_bytes(int k, int pool_keep);

// Sparse-attention decode over selected positions.
constexpr int kMaxDecodeDqk = 1024;
constexpr int kMaxDecodeDv = 1024;

struct DecodeArgs {
    const uint16_t *q;         // [rows][heads][dqk] bf16 bits, 16-byte aligned
    const uint16_t *kv;        // [n_kv][dqk] bf16 bits, 16-byte aligned; values = first dv
    const int32_t *idx;        // [rows][k]
    int64_t n_kv;
    int32_t rows;              // rows of this launch (partial kernel: grid z)
    int32_t row0;              // first row of this launch
    int32_t heads;             // multiple of 16
    int32_t k;
    int32_t dqk;               // multiple of 16, <= kMaxDecodeDqk
    int32_t dv;                // multiple of 64, <= min(dqk, kMaxDecodeDv)
    int32_t splits;            // workgroups per (row, 16 heads) along the k selected positions
    int32_t per_split;         // positions per split, a multiple of 32
    float scale;
    float *part_o;             // [rows][heads][splits][dv]
    float *part_ml;            // [rows][heads][splits][2] running max, sum
    float *out;                // [rows][heads][dv]
};

size_t decode_lds_bytes(int dqk);
hipError_t launch_decode_partial(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_decode_combine(const DecodeArgs &a, hipStream_t stream);


}  // namespace topk
