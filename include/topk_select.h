/*
 * topk_select.h -- exact per-row top-k selection on MI355X (gfx950).
 *
 * The operation ("The Secret GPU Kernel Behind DeepSeek V4.1 Flash",
 * transcript 2:40-4:20): for each query row of indexer scores, keep the k
 * largest of up to about a million fp32 scores and return their values and
 * positions.  The row is read once, in 1,024-element blocks visited in a
 * shuffled order drawn without looking at the data (3:30, 4:55-5:10); each
 * score meets one comparison against a threshold that only rises (3:18-4:08);
 * survivors go to a small tray that is sorted only when it passes its mark,
 * keeping the best k (3:55-4:08).  When there are too few rows to fill the
 * chip, one row is split across several compute units that each keep a local
 * top-k and a leader merges them (5:22-5:33).  Values come back bit-exact and
 * indices never repeat because every score travels as one 64-bit word holding
 * an order-preserving key above its index (kernelbench.com "DeepSeek V4.1
 * Flash", bitonic-selection paragraph).
 *
 * Result (identical for every schedule, seed and split):
 *   Row r holds positions [0, L_r), L_r = clamp(lengths[r], 0, n), or n when
 *   `lengths` is NULL.  Output row r has k slots.  The first min(k, L_r) hold
 *   the selected scores and their positions, ordered by value descending in
 *   IEEE-754 total order (-0.0 below +0.0), equal values by lower position.
 *   The remaining slots hold value -inf and index -1.  Values are bit copies
 *   of the input.  Positions >= L_r are never read or returned.
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers owned by the caller.
 *   - scores: fp32 [rows][n], row r starts at scores + r*n (any 4-byte
 *     alignment).  out_vals: fp32 [rows][k].  out_idx: int32 [rows][k].
 *     lengths: int32 [rows] or NULL.  Offsets are computed in 64 bits.
 *   - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *     Calls are asynchronous and stream-ordered.
 *   - Arguments are checked on the host before any HIP call.  On an argument
 *     error the call returns a negative status, launches nothing and writes
 *     nothing.  rows == 0 returns TOPK_OK and does nothing.
 *   - Device data is never an error: lengths outside [0, n] are clamped.
 *     NaN scores are a precondition violation: the output is then
 *     unspecified, but the call stays memory-safe and terminates.
 *   - A failed launch (hipGetLastError right after it) returns TOPK_ELAUNCH.
 */
#ifndef TOPK_SELECT_H
#define TOPK_SELECT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define TOPK_OK 0
#define TOPK_EINVAL (-1)     /* null pointer, rows < 0, n < 1, bad option    */
#define TOPK_EK_RANGE (-2)   /* k < 1 or k > TOPK_MAX_K                       */
#define TOPK_EWORKSPACE (-3) /* workspace missing, misaligned or too small    */
#define TOPK_ESPLIT (-4)     /* split outside [0, TOPK_MAX_SPLIT]             */
#define TOPK_ELAUNCH (-5)    /* the HIP launch failed                         */
#define TOPK_EDEVICE (-6)    /* no usable gfx950 device / runtime query failed */
#define TOPK_EALLOC (-7)     /* library-owned workspace allocation failed     */

/* Largest k of topk_select, topk_select_split and topk_select_ex: the
 * page's own kernel stops near k = 4,000 ("The Secret GPU Kernel Behind
 * DeepSeek V4.1 Flash", transcript 5:45).  Lists up to 2,048 words run the
 * streaming filter; wider lists (k > 2,048) run the per-row radix selection
 * of topk_select_radix, one workgroup per row, with the same result. */
#define TOPK_MAX_K 4096
/* Largest k the streaming filter itself takes (its kept lists sit in
 * registers); above it the calls take the radix path. */
#define TOPK_MAX_K_STREAM 2048
/* Largest number of workgroups one row may be split across. */
#define TOPK_MAX_SPLIT 1024

/*
 * topk_select -- top-k of every row, planned automatically ("The Secret GPU
 * Kernel Behind DeepSeek V4.1 Flash", transcript 2:40-4:20: keep the best k
 * of a row of indexer scores by one comparison per score against a rising
 * threshold; 5:45: k up to about 4,000).
 *
 * 1 <= k <= TOPK_MAX_K (TOPK_EK_RANGE otherwise).  Chooses one workgroup
 * per row or, when rows alone cannot fill the GPU, splits each row across
 * several workgroups (transcript 5:22-5:33).  It runs topk_select_radix
 * instead (same result) when k > TOPK_MAX_K_STREAM, and on rows of at most
 * 262,144 scores when k > 1024 with at least a quarter as many rows as
 * compute units, or k > 512 with at least half as many (measured faster
 * there).  A split call uses a library-owned, grow-only workspace per
 * device, allocated with hipMalloc on the first call that needs a larger one
 * (so the first such call is not graph-capturable; use topk_select_split
 * for capture).  Calls that share this internal workspace must be ordered
 * on one stream.  The visit order's seed changes from call to call (a
 * per-device counter), so the order in which a row's blocks are read cannot
 * be predicted from the input (transcript 4:55-5:10); the result never
 * depends on it.
 */
int topk_select(const float *scores, const int32_t *lengths, int32_t rows, int32_t n,
                int32_t k, float *out_vals, int32_t *out_idx, void *stream);

/*
 * topk_split_workspace_bytes -- device bytes topk_select_split needs for
 * the split-row mode ("The Secret GPU Kernel Behind DeepSeek V4.1 Flash",
 * transcript 5:22-5:33: when the batch is too small to fill the chip, one
 * row is spread over several compute units that each keep a local top-k,
 * and a leader merges their winners).  `split` == 0 means the automatic
 * choice.  Returns 0 when no workspace is needed (split 1, or k above
 * TOPK_MAX_K_STREAM) and for invalid arguments.  The workspace holds per-row
 * threshold and ticket words, one arrival ticket per group of eight of a
 * row's workgroups, and one k-list per (row, split) pair.
 */
size_t topk_split_workspace_bytes(int32_t rows, int32_t n, int32_t k, int32_t split);

/*
 * topk_workspace_init -- zero a caller-owned split-row workspace once,
 * before its first use, with a fill kernel on `stream` (no memset node, so it
 * can be captured).  The split path resets its tickets and shared
 * threshold words at the end of every call, so the workspace is all zero
 * again between calls (kernelbench.com "DeepSeek V4.1 Flash", Kimi-Linear
 * paragraph: an accumulator that is never reset corrupts the next launch).
 * `workspace` must be 256-byte aligned and workspace_bytes a multiple of 16
 * (TOPK_EWORKSPACE otherwise); workspace_bytes == 0 does nothing.
 */
int topk_workspace_init(void *workspace, size_t workspace_bytes, void *stream);

/*
 * topk_select_split -- top-k with each row split across `split` workgroups
 * (0 = automatic, 1 = no split), the split-row mode of "The Secret GPU
 * Kernel Behind DeepSeek V4.1 Flash", transcript 5:22-5:33.  Each workgroup
 * keeps a local top-k of its share of the row's blocks; workgroups of a row
 * share a rising threshold through the workspace.  The last of each group of
 * eight workgroups to finish (elected by an atomic ticket, as the split-KV
 * decode of kernelbench.com "DeepSeek V4.1 Flash" elects its merging
 * workgroup) merges the group's lists, and the last group to finish merges
 * the groups' lists and writes the row's output.  `workspace` is caller-owned
 * device memory of at least topk_split_workspace_bytes(...), 256-byte
 * aligned, zeroed once by topk_workspace_init.  Allocates nothing.  Two calls
 * that use one workspace must not run concurrently.  With
 * k > TOPK_MAX_K_STREAM the rows run the radix selection, one workgroup per
 * row: `split` is checked but not used and the workspace may be NULL (a
 * wide list leaves no room for several segments' lists in one workgroup's
 * registers; the radix path's own per-row time is short).
 */
int topk_select_split(const float *scores, const int32_t *lengths, int32_t rows, int32_t n,
                      int32_t k, float *out_vals, int32_t *out_idx, int32_t split,
                      void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of the device array behind topk_select_split_noalloc (per GPU). */
#define TOPK_NOALLOC_SCRATCH_BYTES (8u << 20)

/*
 * topk_select_split_noalloc -- topk_select_split without a workspace
 * argument and without any allocation, for callers that cannot allocate
 * (code under graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The split-row workspace is a file-scope device array of
 * TOPK_NOALLOC_SCRATCH_BYTES bytes; each GPU the library runs on holds its
 * own copy until the process ends.  Its address is looked up, and the array
 * zeroed with a fill kernel on `stream`, on the first call on each device;
 * every call leaves it zero again.  Same arguments and result as
 * topk_select_split (split 0 = automatic).  TOPK_EWORKSPACE when the plan
 * needs more than TOPK_NOALLOC_SCRATCH_BYTES (topk_split_workspace_bytes
 * gives the need; with split > 0 this is checked before any HIP call, with
 * split 0 after querying the device's compute units); k above
 * TOPK_MAX_K_STREAM needs no workspace.  Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (different streams, or host
 * threads) race and must be serialised by the caller.
 */
int topk_select_split_noalloc(const float *scores, const int32_t *lengths, int32_t rows,
                              int32_t n, int32_t k, float *out_vals, int32_t *out_idx,
                              int32_t split, void *stream);

/* Flags for topk_options.flags. */
/* Skip the sampled threshold estimate: filter with exact bounds only. */
#define TOPK_FLAG_NO_ESTIMATE 1
/* Testing aid: make the estimate admit nothing, so every row that uses an
 * estimate takes the verified re-stream path.  The result is unchanged. */
#define TOPK_FLAG_FORCE_RERUN 2

/* Tuning and instrumentation knobs.  Zero fields take the defaults. */
typedef struct {
    uint64_t seed;           /* visit-order and sample seed; the result never depends on it */
    int32_t split;           /* workgroups per row; 0 = automatic                */
    int32_t waves;           /* waves per workgroup, 2..8 (2..4 when k > 1024), as long
                              * as the trays fit in LDS: one sorts, the rest stream;
                              * TOPK_EINVAL otherwise                                */
    int32_t watermark;       /* tray words that trigger a hand-off; 0 = default  */
    int32_t flags;           /* TOPK_FLAG_* bits; 0 = default behaviour          */
    /* Optional device array [rows][2] of uint64, accumulated into (zero it
     * first): [0] scores that entered a tray (the only ones that ever meet
     * more than one comparison), [1] threshold-raising selections run over
     * trays.  NULL turns the counters off. */
    unsigned long long *stats;
} topk_options;

/*
 * topk_select_ex -- topk_select_split with explicit options: the visit
 * order's seed ("The Secret GPU Kernel Behind DeepSeek V4.1 Flash",
 * transcript 4:55-5:10: blocks visited in a shuffled order that does not
 * depend on the data), the split (5:22-5:33), the waves per workgroup, the
 * tray watermark (3:55-4:08: the tray is sorted only once it passes its
 * mark), the sampled estimate (10:57-11:09 and 11:47-12:10: start from an
 * estimated threshold and still return the exact answer) and per-row counts
 * of scores that entered a tray (4:45-4:55: the bound on elements that ever
 * reach a sort).  `workspace` may be NULL when the plan has split == 1.
 * Every option is range-checked for every k.  With k > TOPK_MAX_K_STREAM
 * the rows run the radix selection, where seed, split, waves, watermark and
 * the flags do not apply and `stats` is left untouched.
 */
int topk_select_ex(const float *scores, const int32_t *lengths, int32_t rows, int32_t n,
                   int32_t k, float *out_vals, int32_t *out_idx, const topk_options *opts,
                   void *workspace, size_t workspace_bytes, void *stream);

/* Paths a plan can take. */
#define TOPK_PATH_STREAM 0   /* the streaming threshold filter (select_kernel) */
#define TOPK_PATH_RADIX 1    /* the per-row radix selection (topk_select_radix) */

/*
 * topk_plan -- the plan a call would use (host only, no launch): the
 * split-row choice ("The Secret GPU Kernel Behind DeepSeek V4.1 Flash",
 * transcript 5:22-5:33), the tray and its watermark (3:55-4:08) and the
 * LDS they take.  With opts == NULL it is topk_select's plan (including its
 * routing to the radix path); otherwise topk_select_ex's with those options.
 * A radix plan has split 1, waves 16, list_words = the winners' sort size
 * (k rounded up to a power of two), watermark and tray_words 0, and no
 * workspace.  Status codes as for topk_select_ex.
 */
typedef struct {
    int32_t split;           /* workgroups per row                      */
    int32_t waves;           /* waves per workgroup                     */
    int32_t list_words;      /* kept-list capacity: k rounded up to 64*2^j */
    int32_t watermark;       /* tray words that trigger a sort          */
    int32_t tray_words;      /* tray capacity per wave                  */
    int32_t lds_bytes;       /* dynamic LDS per workgroup               */
    int32_t compute_units;   /* compute units the plan assumed          */
    int32_t path;            /* TOPK_PATH_STREAM or TOPK_PATH_RADIX     */
    size_t workspace_bytes;  /* 0 when split == 1                       */
} topk_plan_t;

int topk_plan(int32_t rows, int32_t n, int32_t k, const topk_options *opts, topk_plan_t *out);

/*
 * topk_block_pool -- block-max pooled pre-selection ("The Secret GPU Kernel
 * Behind DeepSeek V4.1 Flash", transcript 7:22-7:46): while a layer holds a
 * row's scores it also keeps a pool of position blocks for the layers above,
 * chosen by each block's best score, with the newest blocks always in.
 *
 *   Row r holds positions [0, L_r) as for topk_select.  Block b covers
 *   positions [b*group, (b+1)*group) cut at L_r; the row has
 *   nb_r = ceil(L_r / group) blocks.  A block's score is its largest valid
 *   score in IEEE-754 total order (-0.0 below +0.0).
 *   Output row r has `keep` slots:
 *     - slots [0, P_r), P_r = min(pinned, nb_r): the newest blocks
 *       nb_r-1, nb_r-2, ... whatever their scores;
 *     - then the best min(keep - P_r, nb_r - P_r) older blocks (blocks
 *       [0, nb_r - P_r)), by block score descending, equal scores to the
 *       lower block;
 *     - the remaining slots: value -inf, index -1.
 *   out_vals holds bit copies of the block scores, out_idx the block
 *   indices (multiply by `group` for the first position of a block).
 *   The pages do not say how many tokens are pinned; here the caller gives a
 *   block count.
 *
 * group >= 1, keep >= 1, 0 <= pinned <= keep, keep - pinned <= TOPK_MAX_K
 * (TOPK_EINVAL / TOPK_EK_RANGE otherwise; the page keeps 2,000 blocks).  out_vals: fp32 [rows][keep],
 * out_idx: int32 [rows][keep], device pointers owned by the caller.
 * Work: one pass over the scores writing ceil(n / group) block maxima per row
 * into a library-owned, grow-only device buffer, then the radix selection of
 * topk_select_radix over those maxima, written behind the pinned slots.
 * Like topk_select, the first call that needs a larger library buffer
 * allocates it (not graph-capturable), and calls that share the library's
 * buffers must be ordered on one stream.
 */
int topk_block_pool(const float *scores, const int32_t *lengths, int32_t rows, int32_t n,
                    int32_t group, int32_t keep, int32_t pinned, float *out_vals,
                    int32_t *out_idx, void *stream);

/* Largest k of topk_select_radix. */
#define TOPK_MAX_K_RADIX 8192

/*
 * topk_select_radix -- the same result as topk_select (see the top of this
 * file) for 1 <= k <= TOPK_MAX_K_RADIX, by an exact per-row radix selection
 * instead of the streaming filter.  The pages test the selection up to
 * vocabulary-sized rows and k = 1,000, and the page's own kernel stops near
 * k = 4,000 ("The Secret GPU Kernel Behind DeepSeek V4.1 Flash", transcript
 * 5:45 and 8:00-8:14); this entry point serves larger k.
 *
 * One workgroup per row: an evenly spread 4,096-score sample gives a
 * threshold a little below the k-th score; one pass over the row copies
 * every score at or above it into LDS; an 11-bit-digit radix selection in
 * LDS finds the k-th (value, position) word exactly, and the winners are
 * sorted in LDS.  When the sample's threshold admits fewer than k scores or
 * more than the LDS holds, the row is instead narrowed digit by digit with
 * passes over it.  Rows of any length and 4-byte alignment; nothing past a
 * row's length is read.  Allocates nothing, launches one kernel; status
 * codes as for topk_select (TOPK_EK_RANGE for k outside [1, 8192]).
 */
int topk_select_radix(const float *scores, const int32_t *lengths, int32_t rows, int32_t n,
                      int32_t k, float *out_vals, int32_t *out_idx, void *stream);

/*
 * topk_sparse_decode -- attention over the selected positions only, the
 * consumer of the indices ("The Secret GPU Kernel Behind DeepSeek V4.1
 * Flash", transcript 1:48-2:13: the indexer chooses which positions the
 * expensive attention reads; "The Full-Stack Optimization of DeepSeek-V4-Flash
 * on Blackwell GPUs", chunk 68.0 summary: a sparse-MLA decode kernel splits
 * the top-k dimension and merges the parts by log-sum-exp).
 *
 *   q:   bf16 [rows][heads][dqk] (raw bits, 16-byte aligned)
 *   kv:  bf16 [n_kv][dqk], one latent cache shared by every head (16-byte
 *        aligned); a head's values are the first dv channels of each entry
 *   idx: int32 [rows][k], the selected positions (e.g. topk_select's out_idx);
 *        entries < 0 or >= n_kv select nothing, a repeated entry counts twice
 *   out: fp32 [rows][heads][dv]:
 *        out[r][h] = sum_j softmax_j(scale * q[r][h] . kv[j]) * kv[j][0:dv]
 *        over the selected j; rows with nothing selected give zeros.
 * Arithmetic: bf16 products summed in fp32 on MFMA; weights rounded to bf16
 * for the value product (the running sums add the rounded weights).
 * heads a multiple of 16; dqk a multiple of 16, <= 1024; dv a multiple of
 * 64, <= min(dqk, 1024); 1 <= k <= TOPK_MAX_K_RADIX (TOPK_EK_RANGE
 * otherwise); scale finite.  Partial results go to a library-owned,
 * grow-only device buffer (same rules as topk_block_pool).
 */
int topk_sparse_decode(const void *q, const void *kv, const int32_t *idx, int32_t rows,
                       int32_t heads, int64_t n_kv, int32_t k, int32_t dqk, int32_t dv,
                       float scale, float *out, void *stream);

/* Most pool slots topk_pooled_select takes per row, and its largest k (its
 * radix selection keeps the pool's slots in LDS beside the winners). */
#define TOPK_MAX_POOL_SLOTS 8192
#define TOPK_MAX_K_POOLED 2048

/*
 * topk_pooled_select -- top-k inside a block pool ("The Secret GPU Kernel
 * Behind DeepSeek V4.1 Flash", transcript 7:46-8:00): the indexers above the
 * pooling layer score only the pooled positions and keep their own top-k.
 *
 *   pool_idx: int32 [rows][keep], a row's pooled block indices (as written by
 *   topk_block_pool; negative = empty slot).  Slot s covers context positions
 *   pool_idx[r][s]*group + j, j < group.
 *   pool_scores: fp32 [rows][keep*group]; [r][s*group + j] is the score of
 *   that position.
 *   Row r of the context has length L_r = clamp(lengths[r], 0, n) (n when
 *   `lengths` is NULL); positions >= L_r are not candidates.
 *   Output row r has k slots: the top-k candidates by value descending in
 *   IEEE-754 total order, equal values to the LOWER CONTEXT POSITION
 *   (whatever their slot order), then (-inf, -1).  out_idx holds context
 *   positions, out_vals bit copies of the scores.
 *
 * Precondition: a row's block indices are distinct and below 2^31 / group
 * (a pool never repeats a block); otherwise the output is unspecified but
 * the call stays memory-safe.  1 <= keep <= TOPK_MAX_POOL_SLOTS, group >= 1
 * (TOPK_EINVAL otherwise), 1 <= k <= TOPK_MAX_K_POOLED (TOPK_EK_RANGE).
 * Work: one kernel, the radix selection of topk_select_radix, one workgroup
 * per row, with each pooled score's word carrying its context position (so
 * ties resolve by position without reordering the pool).  Allocates nothing.
 */
int topk_pooled_select(const float *pool_scores, const int32_t *pool_idx,
                       const int32_t *lengths, int32_t rows, int32_t n, int32_t group,
                       int32_t keep, int32_t k, float *out_vals, int32_t *out_idx,
                       void *stream);

/* Human-readable text for a status code (static storage); the codes are the
 * argument checks every entry point above makes before any HIP call. */
const char *topk_strerror(int status);

/*
 * topk_visit_order -- host-side copy of the block visit order ("The Secret
 * GPU Kernel Behind DeepSeek V4.1 Flash", transcript 3:30 and 4:55-5:10:
 * 1,024-element blocks visited in a shuffled order drawn without looking at
 * the data) for row `row` of a row with `nblocks` blocks: out[p] = block
 * visited at step p.  A diagnostic for tests; it is the same function the
 * kernel uses.  TOPK_EINVAL for negative sizes or a NULL `out`.
 */
int topk_visit_order(uint64_t seed, int32_t row, int32_t nblocks, int32_t *out);

/*
 * Streaming probes used to measure the machine, not part of the selection
 * (kernelbench.com "DeepSeek V4.1 Flash", split-KV decode paragraph: a
 * bandwidth roof taken from a weak measured read sits well short of what
 * the GPU delivers, so the roof here is measured, over a sweep of read
 * shapes):
 * topk_probe_read reads `src` once in whole 4 MiB workgroup shares (the
 * floor(bytes / 4 MiB) of them; `bytes` a multiple of 16) with the best
 * shape of the sweep on MI355X -- 1,024 threads, four nontemporal 16-byte
 * loads in flight per thread -- and writes one word per workgroup into
 * `sink` (at least topk_probe_sink_words(bytes) uint32 words), so the read
 * cannot be elided.  topk_probe_read_cfg reads `groups` workgroup shares of
 * `bytes_per_group` bytes (a multiple of 16 * threads * loads) with
 * `threads` in {256, 512, 1024}, `loads` in {1, 2, 4, 8} loads in flight per
 * thread, plain or nontemporal loads, and `lds_bytes` (<= 160 KiB) of LDS
 * reserved per workgroup (a large reservation keeps one workgroup per
 * compute unit, so `groups` sets the active compute units); sink: `groups`
 * words.  topk_probe_copy copies `bytes` (multiple of 16) from src to dst.
 * All return TOPK_OK or an error status (TOPK_EINVAL for shapes outside
 * these sets, NULL or misaligned pointers).
 */
size_t topk_probe_sink_words(size_t bytes);
int topk_probe_read(const void *src, size_t bytes, uint32_t *sink, void *stream);
int topk_probe_read_cfg(const void *src, size_t bytes_per_group, size_t groups, int32_t threads,
                        int32_t loads, int32_t nontemporal, size_t lds_bytes, uint32_t *sink,
                        void *stream);
int topk_probe_copy(const void *src, void *dst, size_t bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TOPK_SELECT_H */
