// C ABI of the selection library: argument checks, planning, workspace,
// launch.  Every argument is checked before the first HIP call, so an
// argument error never touches the device.
#include "../../include/topk_select.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>

#include "common.h"
#include "internal.h"

namespace {

using topk::kBlock;
using topk::kWave;

constexpr size_t kAlign = 256;
// Default waves per workgroup: when the rows alone do not outnumber the
// compute units, as many as the LDS holds trays for, up to eight (seven
// streamers and one sorter, one workgroup per compute unit); otherwise (and
// for lists of 2,048 words, whose registers allow one wave per SIMD) four
// waves, so more rows run at once.
constexpr int kDefaultWavesWide = 4;
constexpr int kDefaultWatermark = 256;
constexpr int kMaxDevices = 64;
constexpr int kAssumedCUs = 256;  // MI355X, used only when no device can be queried
constexpr int64_t kMaxGroupsPerLaunch = (int64_t)1 << 22;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int list_multiplier(int32_t k) {  // E: list capacity 64*E >= k
    int e = 1;
    while (64 * e < k) e *= 2;
    return e;
}

struct Plan {
    int E, waves, split, watermark, tray, cus;
    size_t lds, ws_bytes;
    size_t off_groups, off_lists;
};

// Workspace: per-row 16-byte control records (threshold word, ticket) at
// the front, then the per-(row, split) kept lists.  Every call leaves all of
// it zero again, so one zeroed buffer serves calls of any shape.
// Split-row workspace: per-row control records (threshold word, ticket),
// per-row group tickets, then the kept lists.
size_t workspace_layout(int64_t rows, int split, int list_words, size_t *off_groups,
                        size_t *off_lists) {
    const size_t ctrl = align_up((size_t)rows * 16, kAlign);
    const size_t groups_per_row = (size_t)((split + topk::kMergeGroup - 1) / topk::kMergeGroup);
    const size_t groups = align_up((size_t)rows * groups_per_row * 4, kAlign);
    const size_t lists = (size_t)rows * (size_t)split * (size_t)list_words * 8;
    if (off_groups) *off_groups = ctrl;
    if (off_lists) *off_lists = ctrl + groups;
    return ctrl + groups + lists;
}

int device_cus(int *cus) {
    static int cached[kMaxDevices] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TOPK_EDEVICE;
    if (cached[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            v <= 0)
            return TOPK_EDEVICE;
        cached[dev] = v;
    }
    *cus = cached[dev];
    return TOPK_OK;
}

bool misaligned(const void *p, size_t a) { return ((uintptr_t)p % a) != 0; }

// Argument checks shared by every selection entry point (no HIP calls).
int check_args(const float *scores, int32_t rows, int32_t n, int32_t k, const float *out_vals,
               const int32_t *out_idx, const int32_t *lengths) {
    if (rows < 0 || n < 1) return TOPK_EINVAL;
    if (k < 1 || k > TOPK_MAX_K) return TOPK_EK_RANGE;
    if (rows == 0) return TOPK_OK;
    if (!scores || !out_vals || !out_idx) return TOPK_EINVAL;
    if (misaligned(scores, 4) || misaligned(out_vals, 4) || misaligned(out_idx, 4) ||
        (lengths && misaligned(lengths, 4)))
        return TOPK_EINVAL;
    return TOPK_OK;
}

int check_options(const topk_options *o) {
    if (!o) return TOPK_OK;
    if (o->split < 0 || o->split > TOPK_MAX_SPLIT) return TOPK_ESPLIT;
    if (o->waves != 0 && (o->waves < 2 || o->waves > topk::kMaxWaves)) return TOPK_EINVAL;
    if (o->watermark < 0 || o->watermark > 4096) return TOPK_EINVAL;
    if (o->flags & ~(TOPK_FLAG_NO_ESTIMATE | TOPK_FLAG_FORCE_RERUN)) return TOPK_EINVAL;
    return TOPK_OK;
}

// A plan the kernel can launch: the widest lists run at most four waves
// (one per SIMD), and the dynamic LDS plus the kernel's own shared words must
// fit one workgroup's LDS.
constexpr size_t kLdsPerWorkgroup = 160 * 1024;
constexpr size_t kStaticLdsBound = 256;
int check_plan(const Plan &p) {
    const int max_waves = p.E >= 32 ? 4 : topk::kMaxWaves;
    if (p.waves > max_waves) return TOPK_EINVAL;
    if (p.lds + kStaticLdsBound > kLdsPerWorkgroup) return TOPK_EINVAL;
    return TOPK_OK;
}

// Plans a call.  `cus` is the compute-unit count to plan for.
Plan make_plan(int32_t rows, int32_t n, int32_t k, const topk_options *o, int cus) {
    Plan p{};
    p.cus = cus;
    p.E = list_multiplier(k);
    const int list_words = 64 * p.E;
    p.watermark = (o && o->watermark) ? o->watermark : kDefaultWatermark;
    if (p.watermark < 64) p.watermark = 64;
    p.tray = p.watermark + kBlock;  // a tray below the mark never overflows in one block
    // trays, then the sorter's candidate pool (list + one 1,024-word tray
    // piece), the end-of-pass selection's output list, gather buffer and three
    // key histograms
    auto lds_for = [&](int waves) {
        return (size_t)8 * (size_t)(2 * (waves - 1) * p.tray + 2 * list_words + 1024 + kWave) +
               4 * 3 * 256;
    };
    if (o && o->waves) {
        p.waves = o->waves;
    } else if (p.E >= 32 || rows > cus) {
        p.waves = kDefaultWavesWide;
    } else {
        p.waves = topk::kMaxWaves;
        while (p.waves > kDefaultWavesWide &&
               lds_for(p.waves) + kStaticLdsBound > kLdsPerWorkgroup) {
            --p.waves;
        }
    }
    p.lds = lds_for(p.waves);

    if (o && o->split) {
        p.split = o->split;
    } else {
        // Enough workgroups to fill every compute unit once (as many per
        // unit as its LDS holds), each segment at least max(16, nb/24)
        // blocks: every segment adds a list to the leader's merge, and on
        // 128K-1M-score rows smaller segments measured slower (1-4 rows of
        // 1M scores: 24 segments; of 256K: 16; of 128K: 8).  Past half the
        // chip's compute units, segments keep at least 32 blocks (16 rows of
        // 256K scores: 8 segments each beat 16 by 2 us).
        const int64_t nb = ((int64_t)n + 3 + kBlock - 1) / kBlock;
        const int64_t per_cu = std::max<int64_t>(
            1, (int64_t)((kLdsPerWorkgroup - kStaticLdsBound) / std::max<size_t>(p.lds, 1)));
        const int64_t target = per_cu * (int64_t)cus;
        int64_t s = rows > 0 ? (target + rows - 1) / rows : 1;
        int64_t cap = nb / std::max<int64_t>(16, nb / 24);
        if (cap < 1) cap = 1;
        if (s > cap) s = cap;
        if ((int64_t)rows * s * 2 > (int64_t)cus && s > 1 && nb / s < 32) {
            s = std::max<int64_t>(1, nb / 32);
        }
        if (s > TOPK_MAX_SPLIT) s = TOPK_MAX_SPLIT;
        if (s < 1) s = 1;
        p.split = (int)s;
    }
    p.ws_bytes = p.split > 1 ? workspace_layout(rows, p.split, list_words, &p.off_groups, &p.off_lists) : 0;
    return p;
}

int run(const float *scores, const int32_t *lengths, int32_t rows, int32_t n, int32_t k,
        float *out_vals, int32_t *out_idx, const Plan &pl, void *ws, uint64_t seed,
        uint32_t flags, unsigned long long *stats, hipStream_t stream, int64_t out_ld = 0) {
    topk::SelectArgs a{};
    a.out_ld = out_ld > 0 ? out_ld : k;
    a.scores = scores;
    a.lengths = lengths;
    a.n = n;
    a.k = k;
    a.split = pl.split;
    a.watermark = pl.watermark;
    a.tray_words = pl.tray;
    a.out_vals = out_vals;
    a.out_idx = out_idx;
    a.stats = stats;
    a.seed = seed;
    a.flags = flags;
    if (pl.split > 1) {
        char *base = static_cast<char *>(ws);
        a.ws_ctrl = reinterpret_cast<uint64_t *>(base);
        a.ws_groups = reinterpret_cast<uint32_t *>(base + pl.off_groups);
        a.ws_lists = reinterpret_cast<uint64_t *>(base + pl.off_lists);
    }
    // Keep each launch's work-item count well inside 32 bits.
    const int64_t rows_per_launch = kMaxGroupsPerLaunch / pl.split > 0 ? kMaxGroupsPerLaunch / pl.split : 1;
    for (int64_t r0 = 0; r0 < rows; r0 += rows_per_launch) {
        const int64_t nr = rows - r0 < rows_per_launch ? rows - r0 : rows_per_launch;
        a.row0 = (int32_t)r0;
        a.rows = (int32_t)nr;
        if (topk::launch_select(a, pl.E, pl.waves, pl.lds, stream) != hipSuccess)
            return TOPK_ELAUNCH;
    }
    return TOPK_OK;
}

// Library-owned device buffers: one grow-only buffer per device and purpose.
struct DeviceBuffers {
    std::mutex mutex;
    void *ptr[kMaxDevices] = {nullptr};
    size_t bytes[kMaxDevices] = {0};
};

// Returns a buffer of at least `need` bytes on the current device, growing
// it (after a device-wide synchronisation, since earlier calls may still use
// the old one) when it is too small.  With `zero`, a new buffer is cleared
// on `stream` before first use.
int grow_buffer(DeviceBuffers &b, size_t need, bool zero, hipStream_t stream, void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TOPK_EDEVICE;
    std::lock_guard<std::mutex> g(b.mutex);
    if (b.bytes[dev] < need) {
        if (b.ptr[dev]) {
            if (hipDeviceSynchronize() != hipSuccess) return TOPK_EDEVICE;
            (void)hipFree(b.ptr[dev]);
            b.ptr[dev] = nullptr;
            b.bytes[dev] = 0;
        }
        size_t bytes = align_up(need, (size_t)1 << 20);
        void *p = nullptr;
        if (hipMalloc(&p, bytes) != hipSuccess) return TOPK_EALLOC;
        if (zero && topk::launch_fill_zero(p, bytes, stream) != hipSuccess) {
            (void)hipFree(p);
            return TOPK_ELAUNCH;
        }
        b.ptr[dev] = p;
        b.bytes[dev] = bytes;
    }
    *out = b.ptr[dev];
    return TOPK_OK;
}

// Split-row workspace of topk_select (left zeroed by every call).
DeviceBuffers g_ws;
int internal_workspace(size_t need, hipStream_t stream, void **out) {
    return grow_buffer(g_ws, need, true, stream, out);
}

// Block maxima and older-block counts of topk_block_pool.
DeviceBuffers g_pool;
// Per-split partial results of topk_sparse_decode.
DeviceBuffers g_decode;

// Block-maxima rows hold ceil(n / group) floats padded to whole 256-byte
// lines, so every row starts aligned.
constexpr int64_t kPoolRowAlign = 64;
constexpr int32_t kMaxGridRows = 65535;

// Where topk_select takes the per-row radix selection instead of the
// streaming filter: every k above the filter's widest list, and, on rows no
// longer than 262,144 scores,
//   k > 512         always (the streaming lists of 1,024 words and more
//                   spend their time sorting; radix 0.7-0.9x the time),
//   256 < k <= 512  rows up to 65,536 scores; rows up to 131,072 once there
//                   are more than an eighth as many rows as compute units;
//                   any such row once there are half as many,
//   128 < k <= 256  rows up to 65,536 scores once there are more than a
//                   64th as many rows as compute units, or up to 131,072
//                   with half as many.
// Those are the shapes where one workgroup per row, the whole row read once
// into the candidate pass, beats the streaming path's fixed chain of
// estimate, trays, end-of-pass selection and merge (measured on MI355X over
// 1 to 256 rows of N(0,1) scores of 64K to 256K: radix 4-9 us faster there;
// on 1-16 rows of 131,072 scores at k = 384-512 the split streaming path is
// 2-6 us faster, and it always is on million-score rows).
bool prefer_radix(int32_t rows, int32_t n, int32_t k, int cus) {
    if (k > TOPK_MAX_K_STREAM) return true;   // wider than the streaming filter's lists
    if (n > 262144) return false;
    const bool many = (int64_t)rows * 2 >= cus;
    if (k > 512) return true;
    if (k > 256) return n <= 65536 || (n <= 131072 && (int64_t)rows * 8 > cus) || many;
    if (k > 128) return (n <= 65536 && (int64_t)rows * 64 > cus) || (n <= 131072 && many);
    return false;
}

// The radix selection over every row (one workgroup per row), in launches of
// at most kMaxGridRows rows.
int run_radix(const float *scores, const int32_t *lengths, int32_t rows, int32_t n, int32_t k,
              float *out_vals, int32_t *out_idx, hipStream_t stream) {
    topk::RadixArgs x{};
    x.vals = scores;
    x.count = lengths;
    x.ld = n;
    x.k = k;
    x.out_vals = out_vals;
    x.out_idx = out_idx;
    x.out_ld = k;
    for (int32_t r0 = 0; r0 < rows; r0 += kMaxGridRows) {
        x.row0 = r0;
        x.rows = std::min(kMaxGridRows, rows - r0);
        if (topk::launch_radix_select(x, stream) != hipSuccess) return TOPK_ELAUNCH;
    }
    return TOPK_OK;
}

// A radix plan (one workgroup of 16 waves per row, no workspace).
topk_plan_t radix_plan(int32_t k, int cus) {
    topk_plan_t p{};
    int32_t p2 = 2;
    while (p2 < k) p2 <<= 1;
    p.split = 1;
    p.waves = 16;
    p.list_words = p2;
    p.watermark = 0;
    p.tray_words = 0;
    p.lds_bytes = (int32_t)topk::radix_lds_bytes(k, 0);
    p.compute_units = cus;
    p.path = TOPK_PATH_RADIX;
    p.workspace_bytes = 0;
    return p;
}

// Device array behind topk_select_split_noalloc.  In host code `scratch`
// names a host-side stand-in, not device memory: its device address is
// looked up once per device (hipGetSymbolAddress, with that device current)
// and only that address is ever passed to kernels or fills.
static __device__ __align__(256) unsigned char scratch[TOPK_NOALLOC_SCRATCH_BYTES];

struct NoAllocScratch {
    std::mutex mutex;
    void *ptr[kMaxDevices] = {nullptr};
};
NoAllocScratch g_noalloc;

// The current device's copy of `scratch`, zeroed on `stream` on the
// device's first use (a fill kernel, no allocation).
int noalloc_scratch(hipStream_t stream, void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TOPK_EDEVICE;
    std::lock_guard<std::mutex> g(g_noalloc.mutex);
    if (!g_noalloc.ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TOPK_EDEVICE;
        if (topk::launch_fill_zero(p, TOPK_NOALLOC_SCRATCH_BYTES, stream) != hipSuccess)
            return TOPK_ELAUNCH;
        g_noalloc.ptr[dev] = p;
    }
    *out = g_noalloc.ptr[dev];
    return TOPK_OK;
}

// topk_select's visit-order seed: a per-device call counter run through
// splitmix64, so consecutive calls read a row's blocks in unrelated orders.
std::atomic<uint64_t> g_calls[kMaxDevices];

uint64_t next_seed() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
    const uint64_t c = g_calls[dev].fetch_add(1, std::memory_order_relaxed);
    return topk::splitmix64(c ^ ((uint64_t)dev << 56));
}

}  // namespace

extern "C" {

int topk_plan(int32_t rows, int32_t n, int32_t k, const topk_options *opts, topk_plan_t *out) {
    if (!out) return TOPK_EINVAL;
    if (rows < 0 || n < 1) return TOPK_EINVAL;
    if (k < 1 || k > TOPK_MAX_K) return TOPK_EK_RANGE;
    int st = check_options(opts);
    if (st != TOPK_OK) return st;
    int cus = kAssumedCUs;
    int dev_cus = 0;
    int count = 0;
    if (hipGetDeviceCount(&count) == hipSuccess && count > 0 && device_cus(&dev_cus) == TOPK_OK)
        cus = dev_cus;
    if (k > TOPK_MAX_K_STREAM || (!opts && prefer_radix(rows, n, k, cus))) {
        *out = radix_plan(k, cus);
        return TOPK_OK;
    }
    Plan p = make_plan(rows, n, k, opts, cus);
    st = check_plan(p);
    if (st != TOPK_OK) return st;
    out->split = p.split;
    out->waves = p.waves;
    out->list_words = 64 * p.E;
    out->watermark = p.watermark;
    out->tray_words = p.tray;
    out->lds_bytes = (int32_t)p.lds;
    out->compute_units = p.cus;
    out->path = TOPK_PATH_STREAM;
    out->workspace_bytes = p.ws_bytes;
    return TOPK_OK;
}

size_t topk_split_workspace_bytes(int32_t rows, int32_t n, int32_t k, int32_t split) {
    if (rows < 0 || n < 1 || k < 1 || k > TOPK_MAX_K_STREAM || split < 0 ||
        split > TOPK_MAX_SPLIT)
        return 0;
    topk_options o{};
    o.split = split;
    topk_plan_t pl;
    if (topk_plan(rows, n, k, &o, &pl) != TOPK_OK) return 0;
    return pl.workspace_bytes;
}

int topk_workspace_init(void *workspace, size_t workspace_bytes, void *stream) {
    if (!workspace || misaligned(workspace, kAlign)) return TOPK_EWORKSPACE;
    if (workspace_bytes == 0) return TOPK_OK;
    if (workspace_bytes % 16 != 0) return TOPK_EWORKSPACE;
    return topk::launch_fill_zero(workspace, workspace_bytes, (hipStream_t)stream) == hipSuccess
               ? TOPK_OK
               : TOPK_ELAUNCH;
}

int topk_select_ex(const float *scores, const int32_t *lengths, int32_t rows, int32_t n,
                   int32_t k, float *out_vals, int32_t *out_idx, const topk_options *opts,
                   void *workspace, size_t workspace_bytes, void *stream) {
    int st = check_args(scores, rows, n, k, out_vals, out_idx, lengths);
    if (st != TOPK_OK) return st;
    st = check_options(opts);
    if (st != TOPK_OK) return st;
    if (workspace && misaligned(workspace, kAlign)) return TOPK_EWORKSPACE;
    if (k > TOPK_MAX_K_STREAM) {
        // Wider than the streaming filter's lists: the radix selection.
        if (rows == 0) return TOPK_OK;
        return run_radix(scores, lengths, rows, n, k, out_vals, out_idx, (hipStream_t)stream);
    }
    // Whether the launch fits does not depend on the device's CU count, so
    // it is checked with the other arguments, before any HIP call.
    st = check_plan(make_plan(rows, n, k, opts, kAssumedCUs));
    if (st != TOPK_OK) return st;
    if (rows == 0) return TOPK_OK;
    int cus = 0;
    st = device_cus(&cus);
    if (st != TOPK_OK) return st;
    Plan pl = make_plan(rows, n, k, opts, cus);
    if (pl.split > 1 && (!workspace || workspace_bytes < pl.ws_bytes)) return TOPK_EWORKSPACE;
    return run(scores, lengths, rows, n, k, out_vals, out_idx, pl, workspace,
               opts ? opts->seed : 0, opts ? (uint32_t)opts->flags : 0u,
               opts ? opts->stats : nullptr, (hipStream_t)stream);
}

int topk_select_split(const float *scores, const int32_t *lengths, int32_t rows, int32_t n,
                      int32_t k, float *out_vals, int32_t *out_idx, int32_t split,
                      void *workspace, size_t workspace_bytes, void *stream) {
    if (split < 0 || split > TOPK_MAX_SPLIT) return TOPK_ESPLIT;
    topk_options o{};
    o.split = split;
    return topk_select_ex(scores, lengths, rows, n, k, out_vals, out_idx, &o, workspace,
                          workspace_bytes, stream);
}

int topk_select_split_noalloc(const float *scores, const int32_t *lengths, int32_t rows,
                              int32_t n, int32_t k, float *out_vals, int32_t *out_idx,
                              int32_t split, void *stream) {
    int st = check_args(scores, rows, n, k, out_vals, out_idx, lengths);
    if (st != TOPK_OK) return st;
    if (split < 0 || split > TOPK_MAX_SPLIT) return TOPK_ESPLIT;
    if (k > TOPK_MAX_K_STREAM) {
        if (rows == 0) return TOPK_OK;
        return run_radix(scores, lengths, rows, n, k, out_vals, out_idx, (hipStream_t)stream);
    }
    topk_options o{};
    o.split = split;
    // An explicit split fixes the workspace size without the device.
    if (split > 0) {
        const Plan fixed = make_plan(rows, n, k, &o, kAssumedCUs);
        st = check_plan(fixed);
        if (st != TOPK_OK) return st;
        if (fixed.ws_bytes > TOPK_NOALLOC_SCRATCH_BYTES) return TOPK_EWORKSPACE;
    }
    if (rows == 0) return TOPK_OK;
    int cus = 0;
    st = device_cus(&cus);
    if (st != TOPK_OK) return st;
    const Plan pl = make_plan(rows, n, k, &o, cus);
    st = check_plan(pl);
    if (st != TOPK_OK) return st;
    void *ws = nullptr;
    if (pl.split > 1) {
        if (pl.ws_bytes > TOPK_NOALLOC_SCRATCH_BYTES) return TOPK_EWORKSPACE;
        st = noalloc_scratch((hipStream_t)stream, &ws);
        if (st != TOPK_OK) return st;
    }
    return run(scores, lengths, rows, n, k, out_vals, out_idx, pl, ws, next_seed(), 0u, nullptr,
               (hipStream_t)stream);
}

int topk_select(const float *scores, const int32_t *lengths, int32_t rows, int32_t n, int32_t k,
                float *out_vals, int32_t *out_idx, void *stream) {
    int st = check_args(scores, rows, n, k, out_vals, out_idx, lengths);
    if (st != TOPK_OK) return st;
    if (rows == 0) return TOPK_OK;
    int cus = 0;
    st = device_cus(&cus);
    if (st != TOPK_OK) return st;
    if (prefer_radix(rows, n, k, cus))
        return run_radix(scores, lengths, rows, n, k, out_vals, out_idx, (hipStream_t)stream);
    Plan pl = make_plan(rows, n, k, nullptr, cus);
    void *ws = nullptr;
    if (pl.split > 1) {
        st = internal_workspace(pl.ws_bytes, (hipStream_t)stream, &ws);
        if (st != TOPK_OK) return st;
    }
    return run(scores, lengths, rows, n, k, out_vals, out_idx, pl, ws, next_seed(), 0u, nullptr,
               (hipStream_t)stream);
}

int topk_block_pool(const float *scores, const int32_t *lengths, int32_t rows, int32_t n,
                    int32_t group, int32_t keep, int32_t pinned, float *out_vals,
                    int32_t *out_idx, void *stream) {
    if (rows < 0 || n < 1 || group < 1 || keep < 1 || pinned < 0 || pinned > keep)
        return TOPK_EINVAL;
    const int32_t older_k = keep - pinned;
    if (older_k > TOPK_MAX_K) return TOPK_EK_RANGE;
    if (rows == 0) return TOPK_OK;
    if (!scores || !out_vals || !out_idx) return TOPK_EINVAL;
    if (misaligned(scores, 4) || misaligned(out_vals, 4) || misaligned(out_idx, 4) ||
        (lengths && misaligned(lengths, 4)))
        return TOPK_EINVAL;
    const int64_t nbk = ((int64_t)n + group - 1) / group;
    const int64_t bm_ld = (nbk + kPoolRowAlign - 1) / kPoolRowAlign * kPoolRowAlign;
    if (bm_ld > INT32_MAX) return TOPK_EINVAL;
    const size_t bm_bytes = align_up((size_t)rows * (size_t)bm_ld * 4, kAlign);
    void *scratch = nullptr;
    int st = grow_buffer(g_pool, bm_bytes + (size_t)rows * 4, false, (hipStream_t)stream, &scratch);
    if (st != TOPK_OK) return st;
    float *bm = static_cast<float *>(scratch);
    int32_t *older = reinterpret_cast<int32_t *>(static_cast<char *>(scratch) + bm_bytes);

    topk::PoolArgs a{};
    a.scores = scores;
    a.lengths = lengths;
    a.n = n;
    a.bm_ld = bm_ld;
    a.group = group;
    a.pinned = pinned;
    a.keep = keep;
    a.span = (int32_t)std::max<int64_t>(nbk, pinned);
    a.bm = bm;
    a.older = older;
    a.out_vals = out_vals;
    a.out_idx = out_idx;
    for (int32_t r0 = 0; r0 < rows; r0 += kMaxGridRows) {
        a.row0 = r0;
        a.rows = std::min(kMaxGridRows, rows - r0);
        if (topk::launch_block_max(a, (hipStream_t)stream) != hipSuccess) return TOPK_ELAUNCH;
    }
    if (older_k == 0) return TOPK_OK;
    // The best older blocks: an exact radix selection over each block-maxima
    // row cut at its older-block count, written behind the pinned slots.
    topk::RadixArgs x{};
    x.vals = bm;
    x.count = older;
    x.ld = bm_ld;
    x.k = older_k;
    x.out_vals = out_vals + pinned;
    x.out_idx = out_idx + pinned;
    x.out_ld = keep;
    for (int32_t r0 = 0; r0 < rows; r0 += kMaxGridRows) {
        x.row0 = r0;
        x.rows = std::min(kMaxGridRows, rows - r0);
        if (topk::launch_radix_select(x, (hipStream_t)stream) != hipSuccess) return TOPK_ELAUNCH;
    }
    return TOPK_OK;
}

int topk_select_radix(const float *scores, const int32_t *lengths, int32_t rows, int32_t n,
                      int32_t k, float *out_vals, int32_t *out_idx, void *stream) {
    if (rows < 0 || n < 1) return TOPK_EINVAL;
    if (k < 1 || k > TOPK_MAX_K_RADIX) return TOPK_EK_RANGE;
    if (rows == 0) return TOPK_OK;
    if (!scores || !out_vals || !out_idx) return TOPK_EINVAL;
    if (misaligned(scores, 4) || misaligned(out_vals, 4) || misaligned(out_idx, 4) ||
        (lengths && misaligned(lengths, 4)))
        return TOPK_EINVAL;
    return run_radix(scores, lengths, rows, n, k, out_vals, out_idx, (hipStream_t)stream);
}

int topk_sparse_decode(const void *q, const void *kv, const int32_t *idx, int32_t rows,
                       int32_t heads, int64_t n_kv, int32_t k, int32_t dqk, int32_t dv,
                       float scale, float *out, void *stream) {
    if (rows < 0 || heads < 16 || heads % 16 != 0 || n_kv < 1 || dqk < 16 || dqk % 16 != 0 ||
        dqk > topk::kMaxDecodeDqk || dv < 64 || dv % 64 != 0 || dv > dqk ||
        dv > topk::kMaxDecodeDv || !std::isfinite(scale))
        return TOPK_EINVAL;
    if (k < 1 || k > TOPK_MAX_K_RADIX) return TOPK_EK_RANGE;
    if ((int64_t)rows * heads > INT32_MAX) return TOPK_EINVAL;
    if (rows == 0) return TOPK_OK;
    if (!q || !kv || !idx || !out) return TOPK_EINVAL;
    if (misaligned(q, 16) || misaligned(kv, 16) || misaligned(idx, 4) || misaligned(out, 4))
        return TOPK_EINVAL;
    int cus = 0;
    int st = device_cus(&cus);
    if (st != TOPK_OK) return st;
    // Split the selected positions so that about two workgroups per compute
    // unit run, in multiples of 32 positions.
    const int64_t groups = (int64_t)rows * (heads / 16);
    int64_t splits = (2 * (int64_t)cus + groups - 1) / groups;
    const int64_t tiles = (k + 31) / 32;
    if (splits > tiles) splits = tiles;
    if (splits < 1) splits = 1;
    const int32_t per_split = (int32_t)(((tiles + splits - 1) / splits) * 32);
    splits = (k + per_split - 1) / per_split;
    const size_t part_o = align_up((size_t)rows * heads * splits * dv * 4, kAlign);
    const size_t part_ml = (size_t)rows * heads * splits * 2 * 4;
    void *scratch = nullptr;
    st = grow_buffer(g_decode, part_o + part_ml, false, (hipStream_t)stream, &scratch);
    if (st != TOPK_OK) return st;
    topk::DecodeArgs a{};
    a.q = static_cast<const uint16_t *>(q);
    a.kv = static_cast<const uint16_t *>(kv);
    a.idx = idx;
    a.n_kv = n_kv;
    a.heads = heads;
    a.k = k;
    a.dqk = dqk;
    a.dv = dv;
    a.splits = (int32_t)splits;
    a.per_split = per_split;
    a.scale = scale;
    a.part_o = static_cast<float *>(scratch);
    a.part_ml = reinterpret_cast<float *>(static_cast<char *>(scratch) + part_o);
    a.out = out;
    for (int32_t r0 = 0; r0 < rows; r0 += kMaxGridRows) {
        a.row0 = r0;
        a.rows = std::min(kMaxGridRows, rows - r0);
        if (topk::launch_decode_partial(a, (hipStream_t)stream) != hipSuccess) return TOPK_ELAUNCH;
    }
    a.row0 = 0;
    a.rows = rows;
    if (topk::launch_decode_combine(a, (hipStream_t)stream) != hipSuccess) return TOPK_ELAUNCH;
    return TOPK_OK;
}

int topk_pooled_select(const float *pool_scores, const int32_t *pool_idx,
                       const int32_t *lengths, int32_t rows, int32_t n, int32_t group,
                       int32_t keep, int32_t k, float *out_vals, int32_t *out_idx,
                       void *stream) {
    if (rows < 0 || n < 1 || group < 1 || keep < 1 || keep > TOPK_MAX_POOL_SLOTS)
        return TOPK_EINVAL;
    if (k < 1 || k > TOPK_MAX_K_POOLED) return TOPK_EK_RANGE;
    const int64_t total = (int64_t)keep * group;
    if (total > INT32_MAX) return TOPK_EINVAL;
    if (rows == 0) return TOPK_OK;
    if (!pool_scores || !pool_idx || !out_vals || !out_idx) return TOPK_EINVAL;
    if (misaligned(pool_scores, 4) || misaligned(pool_idx, 4) || misaligned(out_vals, 4) ||
        misaligned(out_idx, 4) || (lengths && misaligned(lengths, 4)))
        return TOPK_EINVAL;
    // One radix selection per row over the pooled scores, whose words
    // carry context positions (so equal values go to the lower position).
    topk::RadixArgs x{};
    x.vals = pool_scores;
    x.count = nullptr;
    x.ld = total;
    x.k = k;
    x.out_vals = out_vals;
    x.out_idx = out_idx;
    x.out_ld = k;
    x.pool = pool_idx;
    x.pool_keep = keep;
    x.group = group;
    x.n_ctx = n;
    x.ctx_lengths = lengths;
    for (int32_t r0 = 0; r0 < rows; r0 += kMaxGridRows) {
        x.row0 = r0;
        x.rows = std::min(kMaxGridRows, rows - r0);
        if (topk::launch_radix_select(x, (hipStream_t)stream) != hipSuccess) return TOPK_ELAUNCH;
    }
    return TOPK_OK;
}

const char *topk_strerror(int status) {
    switch (status) {
        case TOPK_OK: return "ok";
        case TOPK_EINVAL: return "invalid argument";
        case TOPK_EK_RANGE: return "k out of range";
        case TOPK_EWORKSPACE: return "workspace missing, misaligned or too small";
        case TOPK_ESPLIT: return "split out of range";
        case TOPK_ELAUNCH: return "kernel launch failed";
        case TOPK_EDEVICE: return "no usable device";
        case TOPK_EALLOC: return "workspace allocation failed";
        default: return "unknown status";
    }
}

int topk_visit_order(uint64_t seed, int32_t row, int32_t nblocks, int32_t *out) {
    if (nblocks < 0 || row < 0 || (nblocks > 0 && !out)) return TOPK_EINVAL;
    const topk::VisitOrder o = topk::make_visit_order(seed, (uint32_t)row, (uint32_t)nblocks);
    for (int32_t p = 0; p < nblocks; ++p) out[p] = (int32_t)topk::visit_block(o, (uint32_t)p);
    return TOPK_OK;
}

size_t topk_probe_sink_words(size_t bytes) { return topk::probe_read_groups(bytes); }

int topk_probe_read(const void *src, size_t bytes, uint32_t *sink, void *stream) {
    if (bytes == 0) return TOPK_OK;
    if (!src || !sink || bytes % 16 != 0 || misaligned(src, 16)) return TOPK_EINVAL;
    return topk::launch_probe_read(src, bytes, sink, (hipStream_t)stream) == hipSuccess
               ? TOPK_OK
               : TOPK_ELAUNCH;
}

int topk_probe_read_cfg(const void *src, size_t bytes_per_group, size_t groups, int32_t threads,
                        int32_t loads, int32_t nontemporal, size_t lds_bytes, uint32_t *sink,
                        void *stream) {
    if (threads != 256 && threads != 512 && threads != 1024) return TOPK_EINVAL;
    if (loads != 1 && loads != 2 && loads != 4 && loads != 8) return TOPK_EINVAL;
    if (lds_bytes > kLdsPerWorkgroup - kStaticLdsBound || groups > (size_t)INT32_MAX)
        return TOPK_EINVAL;
    if (groups == 0) return TOPK_OK;
    const size_t unit = (size_t)16 * (size_t)threads * (size_t)loads;
    if (!src || !sink || bytes_per_group == 0 || bytes_per_group % unit != 0 ||
        misaligned(src, 16))
        return TOPK_EINVAL;
    return topk::launch_probe_read_cfg(src, bytes_per_group, groups, threads, loads,
                                       nontemporal != 0, lds_bytes, sink,
                                       (hipStream_t)stream) == hipSuccess
               ? TOPK_OK
               : TOPK_ELAUNCH;
}

int topk_probe_copy(const void *src, void *dst, size_t bytes, void *stream) {
    if (bytes == 0) return TOPK_OK;
    if (!src || !dst || bytes % 16 != 0 || misaligned(src, 16) || misaligned(dst, 16))
        return TOPK_EINVAL;
    return topk::launch_probe_copy(src, dst, bytes, (hipStream_t)stream) == hipSuccess
               ? TOPK_OK
               : TOPK_ELAUNCH;
}

}  // extern "C"
