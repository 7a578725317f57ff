// Interface of the streaming selection kernel and the fill and probe
// kernels built with it (select_kernel.hip); not exported.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace topk {

// Split rows merge in two levels: segments in groups of kMergeGroup, then
// the groups' lists.
constexpr int kMergeGroup = 8;

struct SelectArgs {
    const float *scores;       // [rows][n]
    const int32_t *lengths;    // [rows] or null
    int64_t n;                 // row stride and maximum length
    int32_t rows;              // rows handled by this launch
    int32_t row0;              // first row of this launch
    int32_t k;
    int32_t split;             // workgroups per row
    int32_t watermark;         // tray words that trigger a sort
    int32_t tray_words;        // tray capacity per wave
    float *out_vals;           // [rows][out_ld], first k slots of each row written
    int32_t *out_idx;          // [rows][out_ld]
    int64_t out_ld;            // output row stride in elements (>= k)
    uint64_t *ws_ctrl;         // [rows][2]: threshold word, arrival ticket (split > 1)
    uint32_t *ws_groups;       // [rows][groups] arrival tickets of segment groups (split > 1)
    uint64_t *ws_lists;        // [rows][split][list_words] (split > 1)
    unsigned long long *stats; // [rows][2] or null
    uint64_t seed;
    uint32_t flags;            // bit 0: no sampled estimate; bit 1: force the rerun path
};

// Launches the selection kernel for list capacity 64*E (E in 1..32).
hipError_t launch_select(const SelectArgs &a, int E, int waves, size_t lds_bytes,
                         hipStream_t stream);

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t stream);
hipError_t launch_probe_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream);
hipError_t launch_probe_read_cfg(const void *src, size_t per_group, size_t groups, int threads,
                                 int loads, bool nontemporal, size_t lds, uint32_t *sink,
                                 hipStream_t stream);
hipError_t launch_probe_copy(const void *src, void *dst, size_t bytes, hipStream_t stream);
size_t probe_read_groups(size_t bytes);

}  // namespace topk
