/*
 * nupaged.h -- C ABI of libnupaged.so: non-uniform paged decode attention on
 * AMD Instinct MI355X (gfx950).
 *
 * The path: single-token decode attention over a paged bf16 KV cache whose
 * KV heads each keep a different, fixed number of tokens; heads are
 * clustered into groups that each own a page table; a split-K work table is
 * computed ahead of time from the budgets; scattered pages or top-K entries
 * can be gathered into contiguous staging.
 *   - Tangram (Unlocking Non-Uniform KV Cache): fixed per-head budgets,
 *     Head Group Page (Fig 8), ahead-of-time load balancing (Fig 4c, Fig 5,
 *     Fig 13).
 *   - KV-RM (Regularizing KV-Cache Movement): block pager with Reserve /
 *     Trim edits, one committed descriptor per decode step through a
 *     shadow-to-active swap, descriptor merging into few large transfers
 *     (Fig 2, Fig 3).
 *   - KVDrive (multi-tier KV cache): attention over selected critical
 *     entries (Fig 1).
 *
 * Conventions
 *   Status.   Every call returns an nup_status; no exception crosses the ABI.
 *             nup_last_error() gives the message of the last failure on a
 *             context.  Host-state mutators are all-or-nothing: on error the
 *             pager state is unchanged.
 *   Memory.   The caller owns every device buffer: the K and V pools, the
 *             descriptor arena, q, out, lse, staging and workspace.  The
 *             library never allocates device memory.  It owns its host state
 *             and two pinned host staging buffers (hipHostMalloc) used to
 *             upload the descriptor.
 *   Streams.  `stream` is a hipStream_t passed as void*.  Every launch and
 *             copy is asynchronous on that stream.  All calls on one context
 *             must be ordered on one stream (the active descriptor is shared
 *             state on the device).  Device-side faults surface at the
 *             caller's next synchronisation; NUP_E_HIP reports launch-time
 *             failures only.  Data errors found by kernels (bad top-K
 *             indices) are latched in the arena and read by
 *             nup_device_errors().
 *   Threads.  A context is not thread-safe; use one context per thread.
 *   Layouts.  bf16 values are passed as raw 16-bit words.
 *     K/V pool:    bf16 [num_pages][heads_per_group][page_size][head_dim]
 *                  (one pool for K, one for V; a page holds page_size tokens
 *                  of every head of one group, each head's rows contiguous)
 *     q:           bf16 [max_batch][num_q_heads][head_dim]
 *     out:         fp32 [max_batch][num_q_heads][head_dim]
 *     lse:         fp32 [max_batch][num_q_heads], natural log; may be NULL
 *     GQA:         query head r reads KV head r / (num_q_heads/num_kv_heads)
 *     page table:  int32 [num_groups][max_batch][max_pages], -1 padded
 *   Inactive sequence slots (never allocated, or freed) produce out = 0 and
 *   lse = -inf.
 */
#ifndef NUPAGED_H
#define NUPAGED_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t nup_status;
enum {
    NUP_OK = 0,
    NUP_E_ARG = 1,      /* bad argument or unsupported shape */
    NUP_E_NOPAGES = 2,  /* not enough free pages for a Reserve */
    NUP_E_CAPACITY = 3, /* append past a head's fixed budget */
    NUP_E_STATE = 4,    /* slot busy / not active, or uncommitted edits */
    NUP_E_HIP = 5,      /* a HIP call failed at launch or copy time */
    NUP_E_INDEX = 6     /* a top-K index is out of range, unsorted or repeated */
};

/* Split-K planning policy. */
enum {
    /* Tangram's ahead-of-time balance: the pages of all heads, concatenated,
     * are cut into num_workers equal contiguous shares (rows split at head
     * boundaries); every worker is resident for the whole launch. */
    NUP_PLAN_BALANCED = 0,
    /* The uniform split Tangram measures against (Fig 4c): every head is cut
     * into the same number of chunks regardless of its length, one chunk
     * per worker, scheduled by the hardware. */
    NUP_PLAN_UNIFORM = 1,
    /* The balanced plan made aware of Alias (KV-RM, Fig 3): for head-group
     * pages that several forked sequences map at the same logical positions,
     * every sharer's copy of a chunk is the first row of its own worker, and
     * a chunk's workers sit on one XCD, so they read the same blocks together
     * and all but the first read can be served from that XCD's L2.  Rows are
     * stored in worker order; nup_get_plan_head_rows() lists each head's rows.
     * Without shared pages (or with more sharer rows than workers) it equals
     * NUP_PLAN_BALANCED.  The result is the same attention either way. */
    NUP_PLAN_SHARED = 2
};

/* Where the partial results of a head split over several work rows are
 * merged (the log-sum-exp merge of split-K decoding).  Both give the same
 * bits. */
enum {
    NUP_MERGE_AUTO = 0,     /* the library's choice: the merge launch, which
                               measured faster on MI355X everywhere */
    NUP_MERGE_LAUNCH = 1,   /* a merge launch after the split-K launch */
    NUP_MERGE_IN_SPLIT = 2  /* inside the split-K launch: partials are written
                               at device scope and counted per head, and the
                               row of a head that counts last merges it; with
                               the fused append it also advances the length.
                               Not under NUP_PLAN_SHARED, which keeps the
                               merge launch. */
};

typedef struct nup_ctx nup_ctx;

typedef struct nup_config {
    int32_t num_kv_heads;   /* H_kv */
    int32_t num_q_heads;    /* H_q, a multiple of H_kv; H_q/H_kv in {1,2,4,5,8} */
    int32_t head_dim;       /* D: 64 or 128 */
    int32_t page_size;      /* P: must be 16 */
    int32_t num_groups;     /* n_g, divides V = num_layers * H_kv; heads per group
                               G_h = V / n_g (a group may span layers) */
    int32_t max_batch;      /* B_max: sequence slots in the fixed-shape descriptor */
    int32_t num_pages;      /* physical pages in each pool */
    int32_t max_pages;      /* logical pages per (slot, group): page-table row length */
    int32_t num_workers;    /* split-K workers (waves); 0 = chosen from the device */
    int32_t plan_mode;      /* NUP_PLAN_BALANCED, NUP_PLAN_UNIFORM or NUP_PLAN_SHARED */
    int32_t uniform_splits; /* chunks per head for NUP_PLAN_UNIFORM (0 = 8) */
    int32_t num_layers;     /* layers sharing the pager (0 or 1: a single layer).
                               The pager's heads are the V = num_layers * H_kv
                               (layer, KV head) pairs, numbered layer * H_kv + h:
                               grouping, capacities and lengths are per pair
                               (Tangram, Fig 11: group sizes beyond one layer's
                               heads).  Per-layer calls act on the layer chosen
                               by nup_set_layer(). */
    int32_t merge_mode;     /* NUP_MERGE_AUTO, NUP_MERGE_LAUNCH or NUP_MERGE_IN_SPLIT */
    void *k_pool;           /* device, bf16 pool for K (caller-owned) */
    void *v_pool;           /* device, bf16 pool for V (caller-owned) */
    void *desc;             /* device, descriptor arena of nup_desc_bytes() bytes,
                               256-byte aligned (caller-owned) */
    const int32_t *free_list_init; /* host, [num_pages] permutation giving the
                               initial free-list order, or NULL for 0..N-1; copied */
} nup_config;

/* Bytes of the device descriptor arena a configuration needs (active
 * descriptor with every layer's plan at a fixed place, page tables, error
 * word).  Host only; no device call. */
nup_status nup_desc_bytes(const nup_config *cfg, size_t *bytes);

/*
 * nup_create -- set up the block pager over caller-owned physical storage
 * (KV-RM, abstract: logical KV histories decoupled from physical storage
 * and tracked by a block pager; Fig 2: the KV pager of the control plane).
 * The K and V pools are the physical pages, the FIFO free list starts as
 * cfg->free_list_init (or 0..num_pages-1), every slot is inactive and no
 * head is grouped yet.
 *   cfg   host; read, not kept (free_list_init is copied)
 *   out   host; receives the new context (NULL on failure)
 * The arena is not touched until the first nup_commit().  cfg->k_pool /
 * v_pool / desc may be NULL for host-only use (pager, planner and
 * coalescer queries); device calls on such a context fail with
 * NUP_E_STATE.  The library keeps the device pointers but never frees
 * them.  Errors: NUP_E_ARG (a shape the kernels do not support, sizes out
 * of range, an arena not 256-byte aligned, a free_list_init that is not a
 * permutation), NUP_E_HIP (device buffers given but no HIP device); the
 * reason goes to stderr, and nothing is kept on failure. */
nup_status nup_create(const nup_config *cfg, nup_ctx **out);
/* nup_destroy -- release the context's host state and pinned staging
 * buffers (the end of the pager of nup_create; KV-RM, abstract), after
 * waiting for the commits that still read those buffers.  The caller's
 * device buffers are left alone; kernels still queued that read the arena
 * or pools must finish before the caller frees them.  NULL is a no-op. */
void nup_destroy(nup_ctx *ctx);
const char *nup_last_error(const nup_ctx *ctx);

/*
 * nup_set_layer -- choose the layer that the per-layer calls act on:
 * kv_append, kv_gather_compact, kv_gather_trains_dma, the attention calls,
 * kv_select_topk and nup_get_plan.  Host state, read when a call is made (a
 * captured graph keeps the layer of each captured call).  Reserve, Alias,
 * Trim and nup_commit cover all layers at once: one frame per step carries
 * every layer's split-K plan.  Errors: NUP_E_ARG (layer outside
 * [0, num_layers)).
 */
nup_status nup_set_layer(nup_ctx *ctx, int32_t layer);

/*
 * kv_alloc_groups -- Reserve (KV-RM, Fig 3) for n sequence slots under fixed
 * per-head budgets (Tangram, abstract: a static footprint per head).
 * "Head" below is a (layer, KV head) pair: V = num_layers * H_kv of them.
 *   slots [n]           slot ids in [0, B_max), distinct, currently inactive
 *   cap   [n][V]        capacity in tokens per (slot, head): the head's
 *                       fixed budget plus any decode headroom; <= max_pages*P
 *   len   [n][V]        tokens already present (0..cap), or NULL for 0
 *   group_of_head_out [V] or NULL: receives each head's group
 * On the first successful call the heads are grouped (Tangram, Fig 8):
 * ordered by the sum of their capacities over this call's slots (ties by
 * head index) and cut into n_g equal groups; the grouping is fixed after
 * that.  Each (slot, group) receives ceil(max cap over the group / P) pages,
 * popped from the front of the FIFO free list in (slot, group, logical page)
 * order.  The shadow descriptor and the split-K plan are updated; nothing
 * reaches the device before nup_commit().
 * Errors: NUP_E_ARG, NUP_E_STATE (slot active), NUP_E_NOPAGES. */
nup_status kv_alloc_groups(nup_ctx *ctx, int32_t n, const int32_t *slots,
                           const int32_t *cap, const int32_t *len,
                           int32_t *group_of_head_out);

/*
 * kv_alias -- Alias (KV-RM, Fig 3: a mapping edit next to Reserve and Trim):
 * reserve new slots whose leading pages are the physical pages of a live
 * source sequence, e.g. a shared prompt prefix.  Sequence i gets, in every
 * group g, page-table entries 0..share_pages[i][g]-1 equal to those of
 * src_slots[i] (each such page's reference count grows by one); the rest of
 * its ceil(max cap over the group / P) pages are popped from the free list
 * as kv_alloc_groups does.
 *   slots       [n] new slots (inactive, distinct, none of them a source)
 *   src_slots   [n] active source slots (repeats allowed)
 *   share_pages [n][n_g] whole pages shared per group (>= 0)
 *   cap, len    [n][V] as for kv_alloc_groups; len is required
 * Shared pages must be full in both sequences: for every head h of group g,
 * share_pages*P <= len (new) and <= the source's current length, so that no
 * append ever writes a shared page.  The K/V rows of shared positions are
 * the source's; rows at len.. of unshared pages are the caller's to fill.
 * Checks run in this order: arguments (NUP_E_ARG), slot states
 * (NUP_E_STATE), the shares against both lengths (NUP_E_ARG), free pages
 * for the unshared rest (NUP_E_NOPAGES); nothing changes on failure. */
nup_status kv_alias(nup_ctx *ctx, int32_t n, const int32_t *slots, const int32_t *src_slots,
                    const int32_t *share_pages, const int32_t *cap, const int32_t *len);

/* kv_free_seqs -- Trim (KV-RM, Fig 3; EOS absorbed by the pager): drop the
 * slots' page references in (group, logical page) order, pushing a page to
 * the back of the free list when its last reference goes, and mark the
 * slots inactive.  Errors: NUP_E_ARG, NUP_E_STATE (not active). */
nup_status kv_free_seqs(nup_ctx *ctx, int32_t n, const int32_t *slots);

/* nup_commit -- seal the step (KV-RM, Fig 3: one Frame commit through a
 * shadow-to-active descriptor swap).  One host-to-device copy of the packed
 * shadow (activity and lengths; when they changed, also the budgets, the
 * split-K plans, the trains and page-table row patches) into the arena,
 * then, if rows changed, one small kernel that applies the patches.  Kernels
 * enqueued earlier on the stream see the previous descriptor.
 * Every argument that the decode calls (kv_append, the attention calls,
 * kv_select_topk) derive from the descriptor -- plan, lengths and
 * page-table addresses, worker counts -- is the same after every commit of
 * a context.  So a decode step captured into a HIP graph once stays valid
 * while commits between its replays change the mapping (KV-RM, abstract and
 * Fig 2: a fixed-shape decoder over a per-step descriptor).  The trains
 * gathers size their launches from the current trains and refuse capture
 * (NUP_E_STATE).  The commit itself always runs eagerly: NUP_E_STATE on a
 * capturing stream.  Errors: NUP_E_STATE, NUP_E_HIP. */
nup_status nup_commit(nup_ctx *ctx, void *stream);

/*
 * kv_append -- the decode step's write (KV-RM, Fig 3: one decode step
 * under the pager's contract, whose new token lands in the mapping sealed
 * by the frame commit; Tangram, abstract: the head's footprint is fixed, so
 * the write must fit its budget): for every active (slot, KV head),
 * store the new token's K and V rows at logical position L (page table
 * entry L / P of the head's group, row L % P of the head's slot) and
 * advance L by one, on the device and in the shadow.
 *   k_new, v_new   device bf16 [B_max][H_kv][D], the current layer's new
 *                  rows; rows of inactive slots ignored.  Only the current
 *                  layer's heads advance.
 * Requires a committed descriptor (NUP_E_STATE if edits are pending).
 * NUP_E_CAPACITY, checked on the host before launch, if any active head
 * has L == cap (a fixed budget is never exceeded; nothing is written).
 * On a stream under graph capture the call only records the launch: the
 * host check and the shadow's advance are skipped, since the kernel runs at
 * each replay.  The kernel itself drops the token of a head at L == cap and
 * latches NUP_E_CAPACITY for nup_device_errors(); the other heads advance.
 * Report the replays with nup_note_appends before the next edit. */
nup_status kv_append(nup_ctx *ctx, const void *k_new, const void *v_new, void *stream);

/*
 * nup_note_appends -- bring the shadow lengths up to date after `steps`
 * replays of a graph that holds kv_append for `layer` (-1: every layer):
 * each active head of those layers advances by steps, stopping at its
 * budget exactly as the replayed kernel did.  Host only.  Call it after
 * the replays and before any Reserve / Alias / Trim, since the next commit
 * sends the shadow lengths to the device.  NUP_E_CAPACITY if a head
 * reached its budget (the lengths are still updated, matching the
 * device); NUP_E_STATE if edits are pending; NUP_E_ARG on a bad layer or
 * steps < 0. */
nup_status nup_note_appends(nup_ctx *ctx, int32_t layer, int32_t steps);

/*
 * kv_gather_compact -- copy cache rows into contiguous staging (KV-RM,
 * Fig 2: coalesced transfers feeding the attention kernel; KVDrive, Fig 1:
 * fetch of critical entries).  Bit-exact copies of K and V rows.
 *   mode 0 (trains): for every active (s, h), rows 0..L-1 go to
 *        k_out/v_out rows row_off[s*H_kv + h] .. + L - 1.  The copy walks the
 *        committed trains (maximal runs of physically consecutive pages).
 *        row_off: device int64 [B_max*H_kv]; idx ignored.
 *   mode 1 (indices): staging[s][h][k] = row of logical position
 *        idx[s][h][k], k < K; idx: device int32 [B_max][H_kv][K],
 *        ascending, distinct, 0 <= idx < L.  k_out/v_out: bf16
 *        [B_max][H_kv][K][D].  A violating index is not read: its staging
 *        row is zero-filled and NUP_E_INDEX is latched for nup_device_errors().
 *   phys_out: optional device int32 receiving each copied row's physical
 *        row id (page * G_h * P + slot * P + t % P), laid out like the
 *        staging rows; NULL to skip.
 * Rows of inactive slots are not written.  Errors: NUP_E_ARG, NUP_E_STATE, NUP_E_HIP. */
nup_status kv_gather_compact(nup_ctx *ctx, int32_t mode, const int32_t *idx, int32_t K,
                             void *k_out, void *v_out, const int64_t *row_off,
                             int32_t *phys_out, void *stream);

/*
 * kv_gather_trains_dma -- the train copy of kv_gather_compact mode 0 moved by
 * the copy engines instead of a kernel (KV-RM, Fig 2: the transport turns
 * the mapping into coalesced transfers for the DMA engine).  Same rows and
 * destination layout: for every active (s, h), rows 0..L-1 go to k_out/v_out
 * rows row_off[s*H_kv + h] .. + L - 1, bit-exact.
 *   row_off   HOST int64 [B_max*H_kv] (the host issues the copies, so it
 *             needs the offsets; the destination rows must not overlap)
 *   n_copies  optional host int32: receives the number of copies enqueued
 * The copies are enqueued on `stream` as device-to-device copies that ask
 * for no compute units.  With one head per group (G_h = 1) a train's rows
 * of a head are one byte range: one linear copy per (train, head) and K/V,
 * which the runtime hands to the SDMA engines when it is large (about
 * 1 MiB and up; small ones run as its blit kernels).  With G_h > 1 the heads
 * interleave page by page: one strided copy of the full pages (source pitch
 * G_h pages) plus one for a partial last page, which the runtime runs as
 * blit kernels, not on the SDMA engines.  Reads
 * the host's view of the trains and lengths, so it needs a committed
 * descriptor with no pending edits (NUP_E_STATE).  Errors: NUP_E_ARG,
 * NUP_E_STATE, NUP_E_HIP. */
nup_status kv_gather_trains_dma(nup_ctx *ctx, void *k_out, void *v_out, const int64_t *row_off,
                                int32_t *n_copies, void *stream);

/* Workspace bytes attn_decode_nonuniform / attn_decode_topk need for split-K
 * partial results at this configuration (K = top-K count, 0 for the paged
 * call).  Host only. */
nup_status nup_workspace_bytes(const nup_ctx *ctx, int32_t K, size_t *bytes);

/*
 * attn_decode_nonuniform -- decode attention of one query token per active
 * slot over each KV head's own retained length, read through its group's
 * page table (Tangram, abstract and Fig 8), split ahead of time by the
 * committed work table (Tangram, Fig 13) and merged by log-sum-exp
 * (the split-K decoding scheme Tangram builds on).
 *   q        device bf16 [B_max][H_q][D]
 *   out      device fp32 [B_max][H_q][D];  lse device fp32 [B_max][H_q] or NULL
 *   scale    softmax scale (1/sqrt(D) is the usual choice)
 *   workspace device, >= nup_workspace_bytes(ctx, 0) bytes, 256-byte aligned
 * Uses the active descriptor: the state of the last nup_commit() plus the
 * appends since.  Errors: NUP_E_ARG, NUP_E_STATE, NUP_E_HIP. */
nup_status attn_decode_nonuniform(nup_ctx *ctx, const void *q, float *out, float *lse,
                                  float scale, void *workspace, size_t ws_bytes,
                                  void *stream);

/*
 * attn_decode_nonuniform_noalloc -- attn_decode_nonuniform without a
 * workspace argument and without any allocation, for callers that cannot
 * allocate device memory around the call: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same kernels, same
 * results, bit for bit.  The split-K partials go to a scratch array of
 * NUP_NOALLOC_SCRATCH_BYTES (32 MiB) that the library holds per GPU for the
 * life of the process; its address is looked up at nup_create.  The call
 * makes no hipMalloc / hipFree and creates no events (nup_set_timing does
 * not time it).
 *   q, out, lse, scale, stream   as for attn_decode_nonuniform
 * Every call on one GPU shares that GPU's scratch, from every context:
 * calls that may overlap on one GPU (several streams, several threads)
 * race and must be ordered by the caller.  Nothing in the scratch needs to
 * start at zero; each launch writes what it reads.
 * Errors: NUP_E_ARG if this context's partials exceed the scratch (the
 * message gives both sizes; nothing is launched), NUP_E_STATE (no device
 * buffers, no committed descriptor, or a current device other than the
 * one the context was created on), NUP_E_HIP. */
#define NUP_NOALLOC_SCRATCH_BYTES (32u << 20)
nup_status attn_decode_nonuniform_noalloc(nup_ctx *ctx, const void *q, float *out, float *lse,
                                          float scale, void *stream);

/*
 * attn_decode_nonuniform_append -- kv_append followed by
 * attn_decode_nonuniform for the current layer, in two launches instead of
 * three (the decode step of KV-RM, abstract: the step's write and the
 * fixed-shape attention over the committed mapping).  The split-K worker
 * whose work row holds a head's position L stores the new K and V rows
 * there before it reads the row's pages, every row of the head reads up to
 * L + 1, and the merge launch advances L.  Results, pools and lengths are
 * bit-identical to the two calls made separately.
 *   k_new, v_new   device bf16 [B_max][H_kv][D], as for kv_append
 *   q, out, lse, scale, workspace as for attn_decode_nonuniform
 * Capacity and capture behave as for kv_append: NUP_E_CAPACITY on the host
 * if any active head is at its budget (nothing launched); under graph
 * capture the device drops the token of a full head, latches
 * NUP_E_CAPACITY, and nup_note_appends reports the replays.
 * Errors: NUP_E_ARG, NUP_E_STATE, NUP_E_CAPACITY, NUP_E_HIP. */
nup_status attn_decode_nonuniform_append(nup_ctx *ctx, const void *k_new, const void *v_new,
                                         const void *q, float *out, float *lse, float scale,
                                         void *workspace, size_t ws_bytes, void *stream);

/*
 * attn_decode_topk -- decode attention over K gathered entries per active
 * (slot, KV head) held contiguously (KVDrive, Fig 1: sparse attention over
 * critical entries), e.g. the output of kv_gather_compact mode 1.
 *   k_stage, v_stage  device bf16 [B_max][H_kv][K][D]
 *   out / lse / scale / workspace as for attn_decode_nonuniform, with
 *   workspace >= nup_workspace_bytes(ctx, K).
 * Activity comes from the active descriptor.  Errors: NUP_E_ARG, NUP_E_STATE, NUP_E_HIP. */
nup_status attn_decode_topk(nup_ctx *ctx, const void *q, const void *k_stage,
                            const void *v_stage, int32_t K, float *out, float *lse,
                            float scale, void *workspace, size_t ws_bytes, void *stream);

/*
 * attn_decode_topk_paged -- the same attention as attn_decode_topk, read in
 * place: each of the K entries of an active (slot, KV head) is taken from the
 * paged pool through its logical position and the head group's page table,
 * with no staging copy (KVDrive, Fig 1: attention over the fetched critical
 * entries; here the fetch and the attention are one pass over HBM).
 *   idx      device int32 [B_max][H_kv][K]: logical positions, ascending,
 *            distinct, 0 <= idx < L (as for kv_gather_compact mode 1)
 *   out / lse / scale / workspace as for attn_decode_topk (workspace >=
 *   nup_workspace_bytes(ctx, K)).
 * An entry outside 0..L-1 is not read: it is left out of the softmax and
 * NUP_E_INDEX is latched for nup_device_errors(); an out-of-order entry is
 * read but also latched.  Errors: NUP_E_ARG, NUP_E_STATE, NUP_E_HIP. */
nup_status attn_decode_topk_paged(nup_ctx *ctx, const void *q, const int32_t *idx, int32_t K,
                                  float *out, float *lse, float scale, void *workspace,
                                  size_t ws_bytes, void *stream);

/*
 * kv_select_topk -- choose each active (slot, KV head)'s K critical entries
 * (KVDrive, Fig 1: critical entries fetched at each decode step; Fig 3:
 * critical KV windows).  The score of position t is the largest q.k over the
 * head's query rows (fp32 from exact bf16 products).  The `window` most
 * recent positions L-window .. L-1 are always kept; the other K - window are
 * the highest-scoring positions of 0 .. L-window-1, ties to the lower
 * position.  The list is written in ascending order, ready for
 * kv_gather_compact mode 1 or attn_decode_topk_paged.
 *   q          device bf16 [B_max][H_q][D]
 *   idx_out    device int32 [B_max][H_kv][K]; rows of inactive slots untouched
 *   workspace  device, >= nup_select_workspace_bytes() bytes, 256-byte aligned
 *              (fp32 scores, then the selection's histograms and counts)
 * Requires a committed descriptor and L >= K for every active head (checked
 * on the host; for a captured call the check covers the lengths at capture,
 * and the caller keeps L >= K through the replays).  Errors: NUP_E_ARG,
 * NUP_E_STATE, NUP_E_HIP. */
nup_status kv_select_topk(nup_ctx *ctx, const void *q, int32_t K, int32_t window, int32_t *idx_out,
                          void *workspace, size_t ws_bytes, void *stream);
/* Workspace bytes for kv_select_topk: B_max * H_kv * max_pages * P fp32
 * scores, plus per head a 2048-bin histogram, a threshold and per-slice counts. */
nup_status nup_select_workspace_bytes(const nup_ctx *ctx, size_t *bytes);

/* ---- host-side queries (no device call; for tests and reports) ---------- */

/*
 * kv_select_topk_centroids -- approximate selection through key clusters
 * (KVDrive, Fig 18 and Fig 19 vary the number of centroids, 2048 to 8192).
 * The older positions of each (slot, KV head) of the current layer are
 * partitioned into C clusters, given by a centroid key each and a member
 * list (the clustering happens before decode).  A cluster's score is the
 * largest q.c over the head's query rows (fp32 from bf16 products).
 * Clusters are taken whole in descending score, ties to the lower cluster
 * id, until K - window positions below L - window are covered; the cluster
 * that crosses the count gives its lowest positions.  The list is written
 * ascending, followed by the window L-window .. L-1 (as kv_select_topk).
 *   centroids  device bf16 [B_max][H_kv][C][D]
 *   cl_start   device int32 [B_max][H_kv][C+1]: cluster c's members are
 *              cl_pos[... + cl_start[c] .. cl_start[c+1]), with
 *              0 <= cl_start[c] <= cl_start[c+1] <= P
 *   cl_pos     device int32 [B_max][H_kv][P]: positions, ascending within a
 *              cluster, each older position in at most one cluster;
 *              members at or past L - window are ignored
 *   C          1 .. 8192;  max_pages * P must not exceed 262144
 *   idx_out    device int32 [B_max][H_kv][K]; rows of inactive slots untouched
 *   workspace  device, >= nup_centroid_workspace_bytes(ctx, C) bytes
 * A head whose lists are malformed or hold fewer than K - window older
 * positions latches NUP_E_INDEX (nup_device_errors) and gets -1 for its
 * selected entries, which attn_decode_topk_paged masks.  Requires a
 * committed descriptor with no pending edits and L >= K for every active
 * head (host checks).  Errors: NUP_E_ARG, NUP_E_STATE, NUP_E_HIP. */
nup_status kv_select_topk_centroids(nup_ctx *ctx, const void *q, const void *centroids, int32_t C,
                                    const int32_t *cl_start, const int32_t *cl_pos, int32_t P,
                                    int32_t K, int32_t window, int32_t *idx_out, void *workspace,
                                    size_t ws_bytes, void *stream);
/* Workspace bytes for kv_select_topk_centroids: B_max * H_kv * C fp32 cluster scores. */
nup_status nup_centroid_workspace_bytes(const nup_ctx *ctx, int32_t C, size_t *bytes);

/* Shadow page table int32 [n_g][B_max][max_pages]. */
nup_status nup_get_page_table(const nup_ctx *ctx, int32_t *out);
/* Shadow lengths int32 [B_max][V] (0 for inactive slots). */
nup_status nup_get_lengths(const nup_ctx *ctx, int32_t *out);
/* group_of_head / slot_of_head int32 [V] each (-1 before the first Reserve). */
nup_status nup_get_groups(const nup_ctx *ctx, int32_t *group_of_head, int32_t *slot_of_head);
/* Free list front to back: int32 [num_pages] capacity, count in *n. */
nup_status nup_get_free_list(const nup_ctx *ctx, int32_t *out, int32_t *n);
/* Reference count of every physical page (host shadow): int32 [num_pages]. */
nup_status nup_get_refcounts(const nup_ctx *ctx, int32_t *out);

/* Trains of the shadow page tables: int32 [max_runs][5] rows of
 * (slot, group, first physical page, pages, first logical page) in (slot,
 * group, logical page) order; count in *n (NUP_E_ARG if max_runs is short). */
nup_status nup_get_runs(const nup_ctx *ctx, int32_t *out, int32_t max_runs, int32_t *n);
/* Split-K plan of the shadow for the current layer: counts first (any pointer may be NULL).
 *   rows           int32 [n_rows][4] = (slot*H_kv + head, t0, t1, slot*V + head);
 *                  the last word indexes the head's length from the current
 *                  layer's first head, length rows being V apart
 *   worker_start   int32 [n_workers + 1]: worker w runs rows worker_start[w] ..
 *                  worker_start[w+1] - 1, in that order
 *   head_row_start int32 [B_max*H_kv + 1]: head sh has head_row_start[sh+1] -
 *                  head_row_start[sh] rows; they are those rows of the table
 *                  except under NUP_PLAN_SHARED (see nup_get_plan_head_rows) */
nup_status nup_get_plan(const nup_ctx *ctx, int32_t *n_rows, int32_t *n_workers,
                        int32_t *rows, int32_t *worker_start, int32_t *head_row_start);
/* Row ids of each head in the current layer's plan, int32 [n_rows]: head
 * sh's rows are head_rows[head_row_start[sh] .. head_row_start[sh+1]), in
 * token order.  Under NUP_PLAN_SHARED the rows table is in worker order and
 * this is the index the merge uses; under the other modes a head's rows are
 * contiguous and this is 0, 1, ..., n_rows - 1.  Errors: NUP_E_ARG. */
nup_status nup_get_plan_head_rows(const nup_ctx *ctx, int32_t *head_rows);
/* The gang launch of the current layer's NUP_PLAN_SHARED plan (head_dim 128):
 * *n_blocks workgroups whose four waves hold one chunk of shared pages for
 * four sharers; gang_rows int32 [4 * n_blocks] are their plan rows (the first
 * row of each of those workers), run by the split-K kernel's gang mode, where
 * the four waves load each page once between them through LDS; worker_skip
 * int32 [n_workers] is 1 for the workers whose first row is run there (the
 * main launch skips it).  Any pointer may be NULL; zero blocks under the
 * other modes.  Errors: NUP_E_ARG. */
nup_status nup_get_plan_gangs(const nup_ctx *ctx, int32_t *n_blocks, int32_t *gang_rows, int32_t *worker_skip);

/* ---- measurement helpers ------------------------------------------------ */

/* When enabled, the library brackets each split-K partial-attention launch
 * with HIP events on the caller's stream, created without the system-scope
 * fence (hipEventDisableSystemFence: timing only, so the interval holds the
 * launch and no cache writeback); nup_kernel_time() returns the summed
 * milliseconds and launch count since the last reset (synchronises on the
 * recorded events).  Launches recorded into a graph are not timed. */
nup_status nup_set_timing(nup_ctx *ctx, int32_t enable);
nup_status nup_kernel_time(nup_ctx *ctx, double *partial_ms, int32_t *launches, int32_t reset);

/* Read and clear the latched device error word (synchronises the stream).
 * *code receives NUP_OK, NUP_E_INDEX (a bad top-K index or cluster list) or
 * NUP_E_CAPACITY (a replayed append found a head at its budget), the
 * former when both were latched. */
nup_status nup_device_errors(nup_ctx *ctx, void *stream, int32_t *code);

/* Plain streaming copy of `bytes` (a multiple of 16) from src to dst with
 * 16-byte loads and stores: the calibration kernel for HBM counters and the
 * achievable-bandwidth ceiling.  Errors: NUP_E_ARG, NUP_E_HIP. */
nup_status nup_probe_copy(const void *src, void *dst, size_t bytes, void *stream);

/* Plain streaming read of `bytes` (a multiple of 16) from src: 2048 waves,
 * each reading its own contiguous share with 16-byte nontemporal loads, four
 * per lane in flight.  `sink` is a device word the kernel may write (it keeps
 * the loads alive).  The achievable read-bandwidth ceiling the decode kernel
 * is compared with.  Errors: NUP_E_ARG, NUP_E_HIP. */
nup_status nup_probe_read(const void *src, size_t bytes, void *sink, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* NUPAGED_H */
