// Internal interface between the host control plane (host.cpp) and the
// gfx950 kernels (kernels.hip).  Not part of the public ABI.
//
// Per-head arrays (lengths, group_of_head, slot_of_head) are passed already
// offset to the layer being processed; lengths rows are `lstride` entries
// apart (the KV heads of all layers), so entry (s, h) is lengths[s*lstride + h].
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nup {

constexpr int kPage = 16;           // tokens per page
constexpr int kWavesPerBlock = 4;   // split-K workers per 256-thread workgroup

// Where the partial kernel reads K/V from.
constexpr int kModePaged = 0;     // pool through the page tables, plan rows
constexpr int kModeStaged = 1;    // contiguous staging [Bmax*Hkv][K][D], equal split
constexpr int kModeIndexed = 2;   // pool rows named by top-K indices, equal split
constexpr int kModeGang = 3;      // shared pages, one plan row per wave, four sharers per workgroup (D = 128)
constexpr int kGangDepth = 8;     // pages in flight per workgroup in gang mode
constexpr int kMaxTopkChunk = 2048;  // entries per top-K worker (LDS row ids)

// Split-K decode attention.  One wave is one worker.  In table mode a
// worker walks rows[worker_start[w] .. worker_start[w+1]) of (head, t0, t1);
// in top-K mode worker w takes chunk w % splits of head w / splits of a
// contiguous staging buffer holding topk_k rows per head.  A head covered by
// one row is written to out directly; otherwise each row leaves a partial
// (o, m, l) for the merge kernel.
struct PartialArgs {
    const uint16_t *q;          // bf16 [Bmax][Hq][D]
    const uint16_t *kbase;      // K pool [pages][Gh][16][D] or staging [Bmax*Hkv][K][D]
    const uint16_t *vbase;
    const int32_t *page_table;  // [ng][Bmax][max_pages] (paged)
    const int32_t *active;      // [Bmax]
    const int32_t *lengths;     // this layer's lengths: entry (s, h) at s*lstride + h (paged)
    const int32_t *group_of_head;
    const int32_t *slot_of_head;
    const int32_t *rows;        // [n][4] (sh, t0, t1, s*lstride + h) (paged)
    const int32_t *worker_start;// [W+1] (paged)
    const int32_t *idx;         // [Bmax*Hkv][K] logical positions (indexed top-K)
    int32_t *err;               // latched error word (indexed top-K)
    const int32_t *head_row_start; // [Bmax*Hkv+1] (paged); top-K rows of head sh are sh*splits..
    float *ws_o;                // [rows][gqa][D]
    float *ws_ml;               // [rows][gqa][2]  (max in log2 units, sum)
    float *out;                 // fp32 [Bmax][Hq][D]
    float *lse;                 // fp32 [Bmax][Hq] or NULL
    int32_t bmax, hkv, gh, max_pages, n_workers;
    int32_t lstride;            // length-row stride: KV heads of all layers
    int32_t topk_k, topk_splits, topk_chunk;
    float scale_log2;           // softmax scale * log2(e)
    // fused append (paged mode; k_new NULL: none): the new token's rows
    // [Bmax][Hkv][D] are stored at each head's position L and attended to;
    // the merge kernel then advances L
    const uint16_t *k_new, *v_new;
    const int32_t *caps;        // this layer's budgets, indexed like lengths
    // share-aware plans (paged and gang modes; NULL otherwise)
    const int32_t *worker_skip; // [W]: 1 if the worker's first row runs in gang mode instead
    const int32_t *gang_rows;   // [4 * blocks]: the plan rows of workgroup b's four waves
    const int32_t *gang_blocks; // workgroups that have a chunk (device, read at run time)
    // In-launch merge (arrive non-NULL; plans whose head rows are contiguous,
    // i.e. not the share-aware plan): partials are written at device scope,
    // every row of a split head then counts itself in arrive[head], and the
    // row that counts last merges the head's partials itself.  With the fused
    // append, the wave that finishes a head (that last row, or an unsplit
    // head's only row) advances its length.  NULL: a merge launch follows.
    int32_t *arrive;            // [Bmax*Hkv] this layer's counts; zero between launches
    int32_t *lengths_w;         // fused append + in-launch merge: lengths to advance (as lengths)
    uint32_t ws_o_bytes, ws_ml_bytes;   // sizes of the partial areas (buffer range checks)
};

struct MergeArgs {
    const float *ws_o;
    const float *ws_ml;
    const int32_t *head_row_start; // [Bmax*Hkv+1] (table mode) or NULL
    const int32_t *head_rows;      // partial slot of each head's rows, by head (NULL: the row index itself)
    int32_t uniform_splits;        // rows of head sh are sh*splits.. (when table NULL)
    float *out;                    // fp32 [Bmax][Hq][D]
    float *lse;                    // fp32 [Bmax][Hq] or NULL
    int32_t hkv;
    int32_t n_pairs;               // (slot, query head) pairs; set by the launcher
    // fused append: advance each active head's length (NULL: no append)
    int32_t *lengths;
    const int32_t *caps, *active;
    int32_t *err;                  // latched error word (bit 2: a head was full)
    int32_t lstride;
};

// Top-K selection.  score_kernel walks the committed plan like the paged
// attention and writes, for every retained position of every active head,
// the largest q.k over the head's query rows into scores[sh * stride + t].
// The select kernels keep the `window` most recent positions and the
// K - window highest-scoring older ones (ties to the lower position) and
// write them in ascending order.
constexpr int kSelBins = 2048;      // histogram of the top 11 key bits
constexpr int kSelSplit = 16;       // slices (workgroups) per head in the parallel select kernels
constexpr int kSelCap = 8192;       // threshold-bin entries the select keeps in LDS
constexpr int kSelHistStride = kSelBins + 64;   // a head's histogram row; word kSelBins counts candidates

struct ScoreArgs {
    const uint16_t *q, *kbase;
    const int32_t *page_table, *lengths, *group_of_head, *slot_of_head, *rows, *worker_start;
    float *scores;
    uint32_t *hist;             // [heads][kSelHistStride]: cleared by each head's first row (or NULL)
    int32_t bmax, hkv, gh, max_pages, n_workers, stride, lstride;
};

struct SelectArgs {
    const float *scores;
    const int32_t *active, *lengths;
    int32_t *idx_out;              // [Bmax*Hkv][K]
    uint32_t *hist;                // [heads][kSelHistStride]: bins, then the candidate count
    uint32_t *cand_key;            // [heads][kSelCap]: entries of the threshold's top bin
    int32_t *cand_pos;             // [heads][kSelCap]
    int32_t *slice_gt;             // [heads][kSelSplit]: entries above the threshold's top bin
    int32_t *thr;                  // [heads][2]: threshold key, ties taken
    int32_t *cnt;                  // [heads][kSelSplit][2]: per slice, above and equal
    int32_t hkv, stride, k, window, lstride;
};

// Top-K selection through key clusters.  centroid_score_kernel writes, for
// every active head, the largest q.c over its query rows for each of its C
// centroids into cscore[sh * C + c]; cluster_select_kernel takes clusters
// whole in descending score (ties to the lower id) until K - window older
// positions are covered, the cut cluster giving its lowest positions, and
// writes them in order followed by the window.
constexpr int kMaxClusters = 8192;          // clusters per head (LDS sort)
constexpr int kMaxSelectPositions = 262144; // older positions per head (LDS bitmap)

struct CentroidArgs {
    const uint16_t *q;              // bf16 [Bmax][Hq][D]
    const uint16_t *centroids;      // bf16 [Bmax*Hkv][C][D]
    const int32_t *active, *lengths;
    const int32_t *cl_start;        // [Bmax*Hkv][C+1] member-list offsets
    const int32_t *cl_pos;          // [Bmax*Hkv][P] positions, ascending within a cluster
    float *cscore;                  // [Bmax*Hkv][C]
    int32_t *idx_out;               // [Bmax*Hkv][K]
    int32_t *err;                   // latched error word
    int32_t hkv, lstride, C, P, k, window;
};

struct AppendArgs {
    uint16_t *k_pool, *v_pool;
    const uint16_t *k_new, *v_new; // [Bmax][Hkv][D]
    const int32_t *page_table, *active, *group_of_head, *slot_of_head;
    int32_t *lengths;
    const int32_t *caps;           // each head's budget: an append at L == cap is dropped
    int32_t *err;                  // latched error word (bit 2: a head was full)
    int32_t bmax, hkv, gh, max_pages, lstride;
};

struct GatherIndexArgs {
    const uint16_t *k_pool, *v_pool;
    const int32_t *page_table, *active, *lengths, *group_of_head, *slot_of_head;
    const int32_t *idx;            // [Bmax*Hkv][K]
    uint16_t *k_out, *v_out;       // [Bmax*Hkv][K][D]
    int32_t *phys_out;             // [Bmax*Hkv][K] or NULL
    int32_t *err;                  // latched error word
    int32_t bmax, hkv, gh, max_pages, k, lstride;
};

struct GatherRunsArgs {
    const uint16_t *k_pool, *v_pool;
    const int32_t *runs;           // [n_runs][4] (slot*ng+g, phys, pages, logical)
    const int32_t *run_prefix;     // [n_runs+1] page prefix sums
    const int32_t *active, *lengths, *head_of_gslot;  // head_of_gslot: all layers' heads
    const int64_t *row_off;        // [Bmax*Hkv]
    uint16_t *k_out, *v_out;       // packed rows of D
    int32_t *phys_out;             // packed like the rows, or NULL
    int32_t n_runs, ng, gh, hkv, lstride;
    int32_t layer_base;            // first head of this layer in head_of_gslot numbering
};

// Split-K scratch of the allocation-free entry point: a device array of
// this many bytes in kernels.hip, one copy per GPU for the life of the
// process.  scratch_buffer() gives the calling thread's current device's
// copy; `device` must be that current device (checked).  The address is
// looked up once per device and kept.
constexpr size_t kScratchBytes = (size_t)32 << 20;
hipError_t scratch_buffer(int device, void **ptr);

bool supported_shape(int head_dim, int gqa);
int partial_blocks_per_cu(int head_dim, int gqa, int mode);

hipError_t launch_partial(const PartialArgs &a, int head_dim, int gqa, int mode, hipStream_t st);
hipError_t launch_merge(const MergeArgs &a, int head_dim, int gqa, int n_heads, hipStream_t st);
hipError_t launch_append(const AppendArgs &a, int head_dim, hipStream_t st);
hipError_t launch_score(const ScoreArgs &a, int head_dim, int gqa, hipStream_t st);
hipError_t launch_select(const SelectArgs &a, int n_heads, hipStream_t st);
hipError_t launch_centroid_select(const CentroidArgs &a, int head_dim, int gqa, int n_heads, hipStream_t st);
hipError_t launch_gather_index(const GatherIndexArgs &a, int head_dim, hipStream_t st);
hipError_t launch_gather_runs(const GatherRunsArgs &a, int head_dim, int total_pages, hipStream_t st);
hipError_t launch_fill(int32_t *p, int n, int32_t value, hipStream_t st);
hipError_t launch_apply_patches(int32_t *page_table, const int32_t *hdr, const int32_t *data,
                                int n_patches, int max_pages, hipStream_t st);
hipError_t launch_probe_copy(const void *src, void *dst, size_t bytes, hipStream_t st);
hipError_t launch_probe_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t st);

}  // namespace nup
