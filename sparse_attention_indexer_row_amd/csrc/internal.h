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
};

hipError_t launch_radix_select(const RadixArgs &a, hipStream_t stream);

// Selection inside a block pool: the pool's blocks in position order.  The
// order kernel sorts a row's slots in LDS (8 bytes per slot, rounded up to a
// power of two), so keep is at most TOPK_MAX_POOL_SLOTS (64 KiB).

struct PooledArgs {
    const float *pool_scores;  // [rows][keep * group]
    const int32_t *pool_idx;   // [rows][keep]
    const int32_t *lengths;    // [rows] or null
    int64_t n;                 // context length
    int64_t ld;                // row stride of `gathered` (>= keep * group)
    int32_t rows;              // rows handled by this launch
    int32_t row0;
    int32_t group;
    int32_t keep;              // pool slots per row, <= TOPK_MAX_POOL_SLOTS
    int32_t k;
    float *gathered;           // [rows][ld] scores in ascending position order
    int32_t *blocks;           // [rows][keep] block of each gathered group (ascending)
    int32_t *valid;            // [rows] gathered scores below the row length
    int32_t *out_idx;          // [rows][k] gathered offsets in, context positions out
};

hipError_t launch_pool_order(const PooledArgs &a, hipStream_t stream);
hipError_t launch_pool_positions(const PooledArgs &a, hipStream_t stream);

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
