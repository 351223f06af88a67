// Host control plane and C ABI of libnupaged.so.
//
//  * Head grouping and the head-group block pager (Tangram, Fig 8 Head Group
//    Page; KV-RM, Fig 3 Reserve / Trim): a FIFO free list of physical pages,
//    one dense int32 page table per (group, sequence slot).
//  * Ahead-of-time split-K plan (Tangram, Fig 4c / Fig 13): computed from the
//    reserved capacities whenever the batch composition changes, never per
//    decode step.
//  * Trains (KV-RM, Fig 3 descriptor merging): maximal runs of physically
//    consecutive pages per (slot, group).
//  * Frame commit (KV-RM, Fig 3 shadow-to-active swap): the host shadow is
//    packed into a pinned buffer and reaches the device in one copy; page
//    table rows that changed travel as patches applied by one small kernel.
//    What the decode kernels read (lengths, budgets, every layer's plan, the
//    page tables) sits at fixed places in the arena, so their arguments never
//    change for a context and a decode step captured into a HIP graph once
//    replays correctly across commits (KV-RM's static-graph decoder); calls
//    made under capture leave the host shadow to nup_note_appends.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <numeric>
#include <string>
#include <utility>
#include <vector>

#include "../../include/nupaged.h"
#include "kernels.h"

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }

// Byte sizes of the packed descriptor sections, all int32 words.
struct Sizes {
    size_t fixed;        // active[B] lengths[B*V] goh[V] soh[V] head_of_gslot[V] (V = layers*H)
    size_t caps;         // cap[B*V], sent with the plan (both change only on Reserve / Alias / Trim)
    size_t plan_max;     // per layer: worker_start[W+1] head_row_start[B*H+1] rows[R][4]
    size_t plan_layer;   // one layer's plan section (each layer's sits at a fixed offset)
    size_t runs_max;     // runs[N][4] run_prefix[N+1]
    size_t patches_max;  // hdr[ng*B][4] data[ng*B*max_pages]
    size_t inbox;        // fixed + plan_max + runs_max + patches_max (aligned)
    size_t pt;           // page table bytes
    size_t err;          // error word (padded)
    size_t arrive;       // in-launch merge: arrival counts [NL][B*H], zero between launches
    size_t total;        // inbox + pt + error word + arrival counts
    int max_rows;
    int max_workers;
};

// One split-K wave per SIMD (a four-wave workgroup per CU) on MI355X's 256
// CUs: measured faster than the two waves per SIMD the registers allow
// (Qwen2.5-32B batch 447 against 470 us on one box; the 36-layer Qwen3-4B
// step 0.63 against 0.74 ms at 1k context, 3.52 against 3.61 ms at 16k).
int default_workers_hostonly() { return 1024; }

bool valid_gqa(int g) { return g == 1 || g == 2 || g == 4 || g == 5 || g == 8; }

nup_status validate(const nup_config *c, std::string *why) {
    auto bad = [&](const char *m) { if (why) *why = m; return NUP_E_ARG; };
    if (!c) return bad("config is NULL");
    if (c->num_kv_heads <= 0 || c->num_q_heads <= 0) return bad("head counts must be positive");
    if (c->num_q_heads % c->num_kv_heads) return bad("num_q_heads must be a multiple of num_kv_heads");
    if (!valid_gqa(c->num_q_heads / c->num_kv_heads)) return bad("num_q_heads/num_kv_heads must be 1, 2, 4, 5 or 8");
    if (c->head_dim != 64 && c->head_dim != 128) return bad("head_dim must be 64 or 128");
    if (c->page_size != nup::kPage) return bad("page_size must be 16");
    if (c->num_layers < 0) return bad("num_layers must be >= 0");
    const long long nl = c->num_layers > 0 ? c->num_layers : 1;
    if (nl > 4096) return bad("num_layers too large");
    if (c->num_groups <= 0 || (nl * c->num_kv_heads) % c->num_groups)
        return bad("num_groups must divide num_layers * num_kv_heads");
    if (c->max_batch <= 0 || c->num_pages <= 0 || c->max_pages <= 0) return bad("max_batch, num_pages, max_pages must be positive");
    if ((long long)c->num_pages * (nl * c->num_kv_heads / c->num_groups) * nup::kPage > 0x7fffffffLL)
        return bad("pool too large for 32-bit row ids");
    if ((long long)c->max_pages * nup::kPage > 0x7fffffffLL) return bad("max_pages too large");
    if (c->num_workers < 0) return bad("num_workers must be >= 0");
    if (c->plan_mode != NUP_PLAN_BALANCED && c->plan_mode != NUP_PLAN_UNIFORM && c->plan_mode != NUP_PLAN_SHARED)
        return bad("unknown plan_mode");
    if (c->uniform_splits < 0) return bad("uniform_splits must be >= 0");
    if (c->merge_mode != NUP_MERGE_AUTO && c->merge_mode != NUP_MERGE_LAUNCH && c->merge_mode != NUP_MERGE_IN_SPLIT)
        return bad("unknown merge_mode");
    return NUP_OK;
}

Sizes compute_sizes(const nup_config &c, int workers) {
    Sizes z{};
    const size_t B = c.max_batch, H = c.num_kv_heads, ng = c.num_groups;
    const size_t NL = c.num_layers > 0 ? c.num_layers : 1, V = NL * H;
    const int splits = c.uniform_splits > 0 ? c.uniform_splits : 8;
    if (c.plan_mode == NUP_PLAN_UNIFORM) {
        z.max_rows = (int)(B * H * splits);
        z.max_workers = z.max_rows;
    } else if (c.plan_mode == NUP_PLAN_SHARED) {
        // at most one gang row per worker, plus the balanced bound
        z.max_rows = 2 * workers + 2 * (int)(B * H);
        z.max_workers = workers;
    } else {
        z.max_rows = workers + 2 * (int)(B * H);
        z.max_workers = workers;
    }
    z.fixed = align_up(4 * (B + B * V + 3 * V));
    z.caps = align_up(4 * B * V);
    z.plan_layer = align_up(4 * ((size_t)z.max_workers + 1)) + align_up(4 * (B * H + 1)) +
                   align_up(16 * (size_t)z.max_rows);
    // the shared plan's rows are in worker order; head_rows lists each
    // head's rows for the merge
    // and the gang launch's rows (four per workgroup), its workgroup count and
    // which workers skip their first row
    if (c.plan_mode == NUP_PLAN_SHARED)
        z.plan_layer += align_up(4 * (size_t)z.max_rows) + 2 * align_up(4 * (size_t)z.max_workers) + kAlign;
    z.plan_max = NL * z.plan_layer;
    // every train covers at least one live page-table entry; with Alias the
    // entries (not the physical pages) are what bounds their number
    const size_t entries = ng * B * (size_t)c.max_pages;
    z.runs_max = align_up(16 * entries) + align_up(4 * (entries + 1));
    z.patches_max = align_up(16 * ng * B) + align_up(4 * ng * B * (size_t)c.max_pages);
    z.inbox = z.fixed + z.caps + z.plan_max + z.runs_max + z.patches_max;
    z.pt = align_up(4 * ng * B * (size_t)c.max_pages);
    z.err = kAlign;
    z.arrive = align_up(4 * NL * B * H);
    z.total = z.inbox + z.pt + z.err + z.arrive;
    return z;
}

}  // namespace

// FIFO free list of physical pages: a ring over a fixed array of num_pages
// entries (the list never holds more), so Reserve takes its pages with at
// most two block copies.
struct PageRing {
    std::vector<int32_t> a;
    size_t head = 0, n = 0;
    void init(size_t cap) { a.assign(cap, 0); head = n = 0; }
    size_t size() const { return n; }
    void push_back(int32_t v) {
        size_t i = head + n;
        if (i >= a.size()) i -= a.size();
        a[i] = v;
        ++n;
    }
    // moves the first k entries to out (k <= size())
    void pop_front(int32_t *out, size_t k) {
        const size_t first = std::min(k, a.size() - head);
        std::memcpy(out, a.data() + head, first * sizeof(int32_t));
        if (k > first) std::memcpy(out + first, a.data(), (k - first) * sizeof(int32_t));
        head += k;
        if (head >= a.size()) head -= a.size();
        n -= k;
    }
    void copy_to(int32_t *out) const {
        const size_t first = std::min(n, a.size() - head);
        std::memcpy(out, a.data() + head, first * sizeof(int32_t));
        if (n > first) std::memcpy(out + first, a.data(), (n - first) * sizeof(int32_t));
    }
};

struct nup_ctx {
    nup_config cfg{};
    int H = 0, Hq = 0, D = 0, P = 0, ng = 0, gh = 0, B = 0, num_pages = 0, max_pages = 0, gqa = 0;
    int NL = 1, V = 0;    // layers, and KV heads of all layers (V = NL*H): the pager's heads
    int layer = 0;        // the layer per-layer calls act on
    int workers = 0;      // balanced-plan worker count
    Sizes sz{};
    std::string err;
    bool has_device = false;
    int device = -1;              // the HIP device current at nup_create (device contexts)

    // pager shadow
    PageRing free_list;
    std::vector<int32_t> pt;       // [ng][B][max_pages]
    std::vector<int32_t> npages;   // [ng][B]
    std::vector<int32_t> len, cap; // [B][V]
    std::vector<int32_t> active;   // [B]
    std::vector<int32_t> ref;      // [num_pages]: page-table entries mapping each page
    std::vector<int32_t> goh, soh, head_of_gslot;
    bool grouped = false;

    // trains of each page-table row, rebuilt only for rows that changed
    std::vector<std::vector<int32_t>> row_runs;  // [ng*B]: (phys, pages, logical) triples
    std::vector<uint8_t> runs_stale;             // [ng*B]

    // edits since the last commit
    std::vector<int32_t> dirty_count;  // [ng*B]: page-table entries to send, 0 = clean
    bool plan_dirty = true;
    bool pending = true;               // no commit yet, or edits since

    // plan of each layer (shadow)
    struct Plan {
        std::vector<int32_t> rows;           // [n][4] (s*H + h, t0, t1, 0)
        std::vector<int32_t> worker_start;   // [W+1]
        std::vector<int32_t> head_row_start; // [B*H+1]
        std::vector<int32_t> head_rows;      // shared plan: row ids by head (empty: identity)
        std::vector<int32_t> gang_rows;      // shared plan: rows of the gang launch, four per workgroup
        std::vector<int32_t> worker_skip;    // shared plan: [W] 1 if the worker's first row is in gang_rows
    };
    std::vector<Plan> plan;                  // [NL]
    std::vector<long long> plan_base, plan_bound;   // the balanced planner's scratch

    // active descriptor on the device (offsets into the inbox, in bytes)
    bool committed = false;
    std::vector<size_t> off_ws, off_hrs, off_rows, off_hr, off_skip, off_gang, off_gn;   // [NL]
    std::vector<int> dev_workers, dev_rows;          // [NL]
    size_t off_runs = 0, off_runpre = 0;
    int dev_runs = 0, dev_run_pages = 0;

    // device pointers
    char *desc = nullptr;
    uint16_t *kpool = nullptr, *vpool = nullptr;

    // pinned staging for commits
    char *pinned[2] = {nullptr, nullptr};
    hipEvent_t pinned_ev[2] = {nullptr, nullptr};
    bool pinned_used[2] = {false, false};
    int pinned_next = 0;

    // timing
    bool timing = false;
    std::vector<std::pair<hipEvent_t, hipEvent_t>> tev;
    double acc_ms = 0.0;
    int launches = 0;

    int32_t *inbox_i32(size_t off) { return reinterpret_cast<int32_t *>(desc + off); }
    int32_t *d_active() { return inbox_i32(0); }
    int32_t *d_len() { return inbox_i32(4 * (size_t)B); }
    int32_t *d_goh() { return inbox_i32(4 * ((size_t)B + (size_t)B * V)); }
    int32_t *d_soh() { return d_goh() + V; }
    int32_t *d_hog() { return d_goh() + 2 * V; }
    int32_t *d_cap() { return inbox_i32(sz.fixed); }
    // this layer's view of the per-head arrays (rows of lengths are V apart)
    size_t lbase() const { return (size_t)layer * H; }
    int32_t *d_pt() { return reinterpret_cast<int32_t *>(desc + sz.inbox); }
    int32_t *d_err() { return reinterpret_cast<int32_t *>(desc + sz.inbox + sz.pt); }
    int32_t *d_arrive() { return reinterpret_cast<int32_t *>(desc + sz.inbox + sz.pt + sz.err); }
};

namespace {

nup_status fail(nup_ctx *c, nup_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    c->err = buf;
    return st;
}

bool capturing(hipStream_t st) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    return hipStreamIsCapturing(st, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone;
}

nup_status hip_fail(nup_ctx *c, hipError_t e, const char *what) {
    return fail(c, NUP_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ---- grouping (Tangram, Fig 8) --------------------------------------------
void group_heads(nup_ctx *c, int n, const int32_t *cap) {
    std::vector<long long> key(c->V, 0);
    for (int i = 0; i < n; ++i)
        for (int h = 0; h < c->V; ++h) key[h] += cap[(size_t)i * c->V + h];
    std::vector<int> order(c->V);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return key[a] < key[b]; });
    for (int rank = 0; rank < c->V; ++rank) {
        const int h = order[rank];
        c->goh[h] = rank / c->gh;
        c->soh[h] = rank % c->gh;
        c->head_of_gslot[rank] = h;
    }
    c->grouped = true;
}

// ---- ahead-of-time split-K plan -------------------------------------------
// Balanced plan: the pages of all active heads, concatenated in (slot, head)
// order, are cut into `workers` equal contiguous shares; a share is split
// into rows at head boundaries.  A head with no pages gets one empty row on
// the worker at its position, so that its (zero) output is written too.
// Rows come out sorted by head and, within that, by worker.  A row is
// (s*H + h, t0, t1, s*V + h): the last word indexes the head's length in
// the layer's view of the lengths (rows V apart), so the kernels read it
// without a division.
void plan_balanced(nup_ctx *c, int layer, nup_ctx::Plan &pl) {
    const int B = c->B, H = c->H, W = c->workers;
    const int32_t *capl = c->cap.data() + (size_t)layer * H;   // row s at capl + s*V
    const int NH = B * H;
    static_assert(nup::kPage == 16, "page arithmetic below uses shifts");
    // 64-bit page positions: with Alias the summed head pages are not
    // bounded by the pool
    std::vector<long long> &base = c->plan_base;    // first page of each head
    std::vector<long long> &bound = c->plan_bound;  // first page of each worker's share
    base.resize((size_t)NH + 1);
    base[0] = 0;
    for (int s = 0, sh = 0; s < B; ++s) {
        const int32_t *cr = capl + (size_t)s * c->V;
        const bool act = c->active[s] != 0;
        for (int h = 0; h < H; ++h, ++sh) base[sh + 1] = base[sh] + (act ? (cr[h] + 15) >> 4 : 0);
    }
    const long long T = base[NH];
    // share boundaries floor(T*w/W), built without divisions in the loop; a
    // sentinel past the last one ends every forward scan
    bound.resize((size_t)W + 2);
    {
        const long long q = T / W, r = T % W;
        long long acc = 0, b = 0;
        for (int w = 0; w <= W; ++w) {
            bound[w] = b;
            b += q;
            acc += r;
            if (acc >= W) {
                acc -= W;
                ++b;
            }
        }
        bound[(size_t)W + 1] = LLONG_MAX;
    }
    const size_t max_rows = (size_t)W + 2 * (size_t)NH;
    if (pl.rows.size() < 4 * max_rows) pl.rows.resize(4 * max_rows);
    pl.head_row_start.resize((size_t)NH + 1);
    pl.worker_start.resize((size_t)W + 1);
    int32_t *rw = pl.rows.data();
    int32_t *wst = pl.worker_start.data();
    int32_t *hrs = pl.head_row_start.data();
    const long long *bd = bound.data();
    int32_t n = 0;
    int w = 0;      // worker holding the current page; only moves forward
    int next = 0;   // first worker whose start row is not set yet
    // the row about to be written belongs to worker `o`: it starts every
    // worker up to o that has no row yet (owners never decrease)
    auto own = [&](int o) {
        while (next <= o) wst[next++] = n;
    };
    for (int sh = 0, s = 0, h = 0; sh < NH; ++sh, (++h == H ? (h = 0, ++s) : 0)) {
        hrs[sh] = n;
        const long long lo = base[sh], hi = base[sh + 1];
        const int32_t li = s * c->V + h;
        int32_t *r = rw + 4 * (size_t)n;
        if (lo == hi) {
            int ow;
            if (T > 0) {
                const long long pos = std::min(lo, T - 1);
                while (bd[w + 1] <= pos) ++w;
                ow = w;
            } else {
                ow = (int)((long long)sh * W / NH);
            }
            own(ow);
            r[0] = sh;
            r[1] = 0;
            r[2] = 0;
            r[3] = li;
            ++n;
            continue;
        }
        const long long cap = capl[(size_t)s * c->V + h];
        long long p = lo;
        while (p < hi) {
            while (bd[w + 1] <= p) ++w;
            const long long end = std::min(hi, bd[w + 1]);
            own(w);
            r[0] = sh;
            r[1] = (int32_t)((p - lo) << 4);
            r[2] = (int32_t)std::min((end - lo) << 4, cap);
            r[3] = li;
            r += 4;
            ++n;
            p = end;
        }
    }
    hrs[NH] = n;
    pl.rows.resize(4 * (size_t)n);
    while (next <= W) wst[next++] = n;
}

// The uniform split (the control): every head is cut into the same number of
// page-aligned chunks regardless of its length, one chunk per worker.
void plan_uniform(nup_ctx *c, int layer, nup_ctx::Plan &pl) {
    const int B = c->B, H = c->H, P = c->P;
    const int S = c->cfg.uniform_splits > 0 ? c->cfg.uniform_splits : 8;
    pl.rows.clear();
    pl.head_row_start.assign((size_t)B * H + 1, 0);
    for (int sh = 0; sh < B * H; ++sh) {
        const int s = sh / H;
        const int cap = c->active[s] ? c->cap[(size_t)s * c->V + (size_t)layer * H + sh % H] : 0;
        int nr = 0;
        if (cap > 0) {
            const long long chunk = (long long)P * ((((long long)cap + S - 1) / S + P - 1) / P);
            for (long long t0 = 0; t0 < cap; t0 += chunk) {
                pl.rows.insert(pl.rows.end(), {sh, (int32_t)t0, (int32_t)std::min<long long>(t0 + chunk, cap),
                                               s * c->V + sh % H});
                ++nr;
            }
        } else {
            pl.rows.insert(pl.rows.end(), {sh, 0, 0, s * c->V + sh % H});
            nr = 1;
        }
        pl.head_row_start[sh + 1] = pl.head_row_start[sh] + nr;
    }
    const int n = (int)(pl.rows.size() / 4);
    pl.worker_start.resize(n + 1);
    std::iota(pl.worker_start.begin(), pl.worker_start.end(), 0);
}

// Share-aware plan (KV-RM, Fig 3: Alias).  Sequences forked from one source
// map the same physical pages at the same logical positions, so those
// tokens hold the same K/V for every sharer.  The balanced plan reads them
// once per sharer at unrelated points of the pass, far too far apart for any
// cache to keep them.  Here every sharer's copy of a shared chunk is the
// first row of its own worker, and the workers of one chunk ("a gang") sit
// on one XCD: they start together and read the same blocks within a short
// window, so after the first read the others can hit in that XCD's L2.
//  * Sharing sets: per head group, active slots whose page-table rows begin
//    with the same page, provided that page has more than one reference.
//    The set's shared range is the pages all its rows have in common,
//    capped at every member head's capacity.
//  * Gangs: every (set, head of this layer in the group) range is cut into
//    near-equal chunks of at most c pages, c the smallest size for which
//    all chunks' rows (one per sharer) fit one per worker.
//  * The rest of every head (everything, for heads in no set) is cut like
//    the balanced plan, with each worker's share reduced by its gang row.
// Rows are stored in worker order; head_rows lists each head's rows for the
// merge.  No sharing, more sharer rows than workers, or a chunk longer than
// a worker's share gives exactly the balanced plan.  Correctness never depends on the sharing: every head's
// [0, cap) is still covered exactly once.
void plan_shared(nup_ctx *c, int layer, nup_ctx::Plan &pl) {
    const int B = c->B, H = c->H, W = c->workers;
    const int NH = B * H;
    const int32_t *capl = c->cap.data() + (size_t)layer * H;
    auto pages_of = [&](int s, int h) -> long long {
        return c->active[s] ? ((long long)capl[(size_t)s * c->V + h] + 15) >> 4 : 0;
    };
    // -- sharing sets and their shared page counts
    struct Gang { int g, h; long long len; int first, n; };   // members: mem[first .. first+n)
    std::vector<int32_t> mem;
    std::vector<Gang> gangs;
    std::vector<long long> shared0((size_t)NH, 0);   // first unshared page of each head
    {
        std::vector<std::pair<int32_t, int32_t>> keys;   // (first page, slot)
        for (int g = 0; g < c->ng; ++g) {
            std::vector<int> heads;
            for (int h = 0; h < H; ++h)
                if (c->goh[(size_t)layer * H + h] == g) heads.push_back(h);
            if (heads.empty()) continue;
            keys.clear();
            for (int s = 0; s < B; ++s) {
                const size_t ri = (size_t)g * B + s;
                if (!c->active[s] || c->npages[ri] == 0) continue;
                const int32_t p0 = c->pt[ri * c->max_pages];
                if (p0 >= 0 && c->ref[p0] > 1) keys.emplace_back(p0, s);
            }
            std::sort(keys.begin(), keys.end());
            for (size_t i = 0; i < keys.size();) {
                size_t j = i;
                while (j < keys.size() && keys[j].first == keys[i].first) ++j;
                if (j - i >= 2) {
                    const int32_t *r0 = &c->pt[((size_t)g * B + keys[i].second) * c->max_pages];
                    long long len = c->npages[(size_t)g * B + keys[i].second];
                    for (size_t k = i + 1; k < j; ++k) {
                        const size_t rk = (size_t)g * B + keys[k].second;
                        const int32_t *r = &c->pt[rk * c->max_pages];
                        long long m = 0;
                        const long long lim = std::min<long long>(len, c->npages[rk]);
                        while (m < lim && r[m] == r0[m]) ++m;
                        len = m;
                    }
                    // Only whole pages below every member head's current
                    // length: shared pages are full (kv_alias checks it) and
                    // lengths only grow, so this cap changes nothing today,
                    // but it states at the point of use what the gang launch
                    // relies on: a gang chunk never holds a head's append
                    // position, whose token only the main launch stores.
                    const int32_t *lenl = c->len.data() + (size_t)layer * H;
                    for (int h : heads)
                        for (size_t k = i; k < j; ++k) {
                            const size_t sk = (size_t)keys[k].second * c->V + h;
                            len = std::min(len, (long long)capl[sk] >> 4);
                            len = std::min(len, (long long)lenl[sk] >> 4);
                        }
                    if (len > 0) {
                        for (int h : heads) {
                            gangs.push_back({g, h, len, (int)mem.size(), (int)(j - i)});
                            for (size_t k = i; k < j; ++k) shared0[(size_t)keys[k].second * H + h] = len;
                        }
                        for (size_t k = i; k < j; ++k) mem.push_back(keys[k].second);
                    }
                }
                i = j;
            }
        }
    }
    long long T = 0;
    for (int s = 0; s < B; ++s)
        for (int h = 0; h < H; ++h) T += pages_of(s, h);
    const long long Aq = W > 0 ? (T + W - 1) / W : 0;
    long long maxlen = 0, nsum = 0;
    for (const Gang &gg : gangs) {
        maxlen = std::max(maxlen, gg.len);
        nsum += gg.n;
    }
    auto gang_rows = [&](long long cc) {
        long long r = 0;
        for (const Gang &gg : gangs) r += (long long)gg.n * ((gg.len + cc - 1) / cc);
        return r;
    };
    long long chunk = 0;
    if (!gangs.empty() && nsum <= W && T > 0) {
        long long lo = 1, hi = maxlen;   // gang_rows(maxlen) = nsum <= W
        while (lo < hi) {
            const long long mid = (lo + hi) / 2;
            if (gang_rows(mid) <= W) hi = mid;
            else lo = mid + 1;
        }
        chunk = lo;
        if (chunk > Aq) chunk = 0;   // a chunk longer than a worker's share would straggle
    }
    pl.gang_rows.clear();
    pl.worker_skip.clear();
    if (chunk == 0) {
        pl.head_rows.clear();
        plan_balanced(c, layer, pl);
        return;
    }
    // -- gang rows: virtual worker v, XCD-major, so that consecutive v share
    //    an XCD (workgroups go to the XCDs round robin, kWavesPerBlock waves each)
    constexpr int kXcd = 8;
    const int per_xcd = W / kXcd;
    const bool xcd_map = W % (kXcd * nup::kWavesPerBlock) == 0;
    auto phys = [&](int v) -> int {
        if (!xcd_map) return v;
        const int x = v / per_xcd, j = v % per_xcd;
        return ((j / nup::kWavesPerBlock) * kXcd + x) * nup::kWavesPerBlock + j % nup::kWavesPerBlock;
    };
    std::vector<int32_t> grow((size_t)W * 4, -1);   // the gang row of each physical worker
    std::vector<int32_t> gpiece((size_t)W, 0);      // its chunk's index within the head's range
    std::vector<long long> gchunk((size_t)W, -1);   // which chunk (numbered over all gangs)
    std::vector<int32_t> gcount((size_t)NH, 0);     // gang rows of each head
    std::vector<long long> gload((size_t)W, 0);
    {
        int v = 0;
        long long chunk_id = 0;
        for (const Gang &gg : gangs) {
            const long long k = (gg.len + chunk - 1) / chunk;
            for (long long i = 0; i < k; ++i, ++chunk_id) {
                const long long p0 = gg.len * i / k, p1 = gg.len * (i + 1) / k;
                for (int m = 0; m < gg.n; ++m, ++v) {
                    const int s = mem[(size_t)gg.first + m];
                    const int w = phys(v);
                    int32_t *r = &grow[(size_t)w * 4];
                    r[0] = s * H + gg.h;
                    r[1] = (int32_t)(p0 << 4);
                    r[2] = (int32_t)(p1 << 4);
                    r[3] = s * c->V + gg.h;
                    gload[w] = p1 - p0;
                    gpiece[w] = (int32_t)i;
                    gchunk[w] = chunk_id;
                    gcount[(size_t)s * H + gg.h]++;
                }
            }
        }
    }
    // -- workgroups whose four waves hold one chunk run it in the gang launch
    //    (the split-K kernel's gang mode: the four waves load each page once
    //    between them, through LDS); their workers skip that row in the main
    //    launch, so it takes no room there
    constexpr int kG = nup::kWavesPerBlock;
    std::vector<uint8_t> coop((size_t)W / kG, 0);
    if (xcd_map && c->D == 128) {
        for (int b = 0; b < W / kG; ++b) {
            const long long id = gchunk[(size_t)b * kG];
            bool same = id >= 0;
            for (int j = 1; j < kG && same; ++j) same = gchunk[(size_t)b * kG + j] == id;
            if (same) {
                coop[b] = 1;
                for (int j = 0; j < kG; ++j) gload[(size_t)b * kG + j] = 0;
            }
        }
    }
    // -- the rest, cut into shares proportional to each worker's room
    std::vector<long long> ubase((size_t)NH + 1, 0);
    for (int sh = 0; sh < NH; ++sh) {
        const long long hp = pages_of(sh / H, sh % H);
        ubase[sh + 1] = ubase[sh] + std::max(0LL, hp - shared0[sh]);
    }
    const long long U = ubase[NH];
    // share boundaries floor(U * room_before(w) / room_total), carried as a
    // quotient and remainder: a room value's own quotient and remainder are
    // computed once (rooms take few distinct values), not one 128-bit
    // division per worker
    std::vector<long long> bound((size_t)W + 2);
    {
        long long R = 0;
        for (int w = 0; w < W; ++w) R += std::max(0LL, Aq - gload[w]);
        std::vector<std::pair<long long, long long>> per_room((size_t)std::min<long long>(Aq + 1, 1 << 16), {-1, 0});
        auto step_of = [&](long long d) -> std::pair<long long, long long> {
            auto calc = [&]() {
                const __int128 x = (__int128)U * d;
                return std::make_pair((long long)(x / R), (long long)(x % R));
            };
            if (d < (long long)per_room.size()) {
                if (per_room[d].first < 0) per_room[d] = calc();
                return per_room[d];
            }
            return calc();
        };
        long long q = 0, r = 0;   // U * room_before(w) = q * R + r
        for (int w = 0; w <= W; ++w) {
            bound[w] = R ? q : (w ? U : 0);
            if (w < W && R) {
                const auto st = step_of(std::max(0LL, Aq - gload[w]));
                q += st.first;
                r += st.second;
                if (r >= R) {
                    r -= R;
                    ++q;
                }
            }
        }
        bound[W] = U;
        bound[(size_t)W + 1] = LLONG_MAX;
    }
    // rest rows in head order; owners never decrease
    std::vector<int32_t> rest;     // [n][4]
    std::vector<int32_t> owner;    // [n]
    rest.reserve(4 * ((size_t)NH + W + 1));
    owner.reserve((size_t)NH + W + 1);
    auto push_row = [&](int32_t a0, int32_t a1, int32_t a2, int32_t a3) {
        rest.push_back(a0);
        rest.push_back(a1);
        rest.push_back(a2);
        rest.push_back(a3);
    };
    {
        int w = 0;
        for (int sh = 0; sh < NH; ++sh) {
            const int s = sh / H, h = sh % H;
            const long long lo = ubase[sh], hi = ubase[sh + 1];
            const int32_t li = s * c->V + h;
            if (lo == hi) {
                if (shared0[sh] > 0) continue;   // covered by its gang rows
                int ow;
                if (U > 0) {
                    const long long pos = std::min(lo, U - 1);
                    while (bound[w + 1] <= pos) ++w;
                    ow = w;
                } else {
                    ow = std::max(w, (int)((long long)sh * W / NH));
                }
                push_row(sh, 0, 0, li);
                owner.push_back(ow);
                continue;
            }
            const long long cap = capl[(size_t)s * c->V + h];
            const long long off = shared0[sh];
            long long p = lo;
            while (p < hi) {
                while (bound[w + 1] <= p) ++w;
                const long long end = std::min(hi, bound[w + 1]);
                push_row(sh, (int32_t)((p - lo + off) << 4), (int32_t)std::min((end - lo + off) << 4, cap), li);
                owner.push_back(w);
                p = end;
            }
        }
    }
    // -- the table in worker order: each worker's gang row, then its rest
    const size_t nrest = owner.size();
    size_t ngang = 0;
    for (int w = 0; w < W; ++w) ngang += grow[(size_t)w * 4] >= 0;
    const size_t n = nrest + ngang;
    if (n > (size_t)c->sz.max_rows) {   // not expected (bounded above); stay valid
        pl.head_rows.clear();
        plan_balanced(c, layer, pl);
        return;
    }
    pl.rows.resize(4 * n);
    pl.worker_start.resize((size_t)W + 1);
    {
        size_t k = 0, ri = 0;
        for (int w = 0; w < W; ++w) {
            pl.worker_start[w] = (int32_t)k;
            if (grow[(size_t)w * 4] >= 0) {
                std::copy(&grow[(size_t)w * 4], &grow[(size_t)w * 4] + 4, &pl.rows[4 * k]);
                ++k;
            }
            while (ri < nrest && owner[ri] == w) {
                std::copy(&rest[4 * ri], &rest[4 * ri] + 4, &pl.rows[4 * k]);
                ++k;
                ++ri;
            }
        }
        pl.worker_start[W] = (int32_t)k;
        if (ri != nrest || k != n) {   // owners out of order: not expected; stay valid
            pl.head_rows.clear();
            plan_balanced(c, layer, pl);
            return;
        }
    }
    // -- each head's rows, in token order: its gang rows by chunk index, then
    //    its rest rows, which were made in token order and all start later
    pl.head_row_start.assign((size_t)NH + 1, 0);
    for (size_t k = 0; k < n; ++k) pl.head_row_start[pl.rows[4 * k] + 1]++;
    for (int sh = 0; sh < NH; ++sh) pl.head_row_start[sh + 1] += pl.head_row_start[sh];
    pl.head_rows.resize(n);
    {
        std::vector<int32_t> next_rest((size_t)NH);
        for (int sh = 0; sh < NH; ++sh) next_rest[sh] = pl.head_row_start[sh] + gcount[sh];
        for (int w = 0; w < W; ++w) {
            int32_t k = pl.worker_start[w];
            const int32_t ke = pl.worker_start[w + 1];
            if (k < ke && grow[(size_t)w * 4] >= 0) {   // the worker's gang row
                pl.head_rows[pl.head_row_start[grow[(size_t)w * 4]] + gpiece[w]] = k;
                ++k;
            }
            for (; k < ke; ++k) pl.head_rows[next_rest[pl.rows[4 * (size_t)k]]++] = k;
        }
    }
    // -- the gang launch: each cooperating workgroup's four gang rows (the
    //    first row of each of its workers)
    pl.worker_skip.assign((size_t)W, 0);
    for (int b = 0; b < W / kG; ++b) {
        if (!coop[b]) continue;
        for (int j = 0; j < kG; ++j) {
            const int w = b * kG + j;
            pl.gang_rows.push_back(pl.worker_start[w]);
            pl.worker_skip[w] = 1;
        }
    }
}

void replan(nup_ctx *c) {
    for (int l = 0; l < c->NL; ++l) {
        if (c->cfg.plan_mode == NUP_PLAN_UNIFORM) plan_uniform(c, l, c->plan[l]);
        else if (c->cfg.plan_mode == NUP_PLAN_SHARED) plan_shared(c, l, c->plan[l]);
        else plan_balanced(c, l, c->plan[l]);
    }
}

// ---- trains (KV-RM, Fig 3) --------------------------------------------------
// Maximal runs of physically consecutive pages in one page-table row.
void row_trains(const int32_t *row, int n, std::vector<int32_t> &out) {
    out.clear();
    int i = 0;
    while (i < n) {
        const int start = i;
        while (i + 1 < n && row[i + 1] == row[i] + 1) ++i;
        out.insert(out.end(), {row[start], i - start + 1, start});
        ++i;
    }
}

// Appends (slot, group, first physical page, pages, first logical page) for
// every active slot in (slot, group, logical page) order.
const std::vector<int32_t> &runs_of_row(nup_ctx *c, size_t ri) {
    if (c->runs_stale[ri]) {
        row_trains(&c->pt[ri * c->max_pages], c->npages[ri], c->row_runs[ri]);
        c->runs_stale[ri] = 0;
    }
    return c->row_runs[ri];
}

void build_runs(nup_ctx *c, std::vector<int32_t> &out) {
    out.clear();
    for (int s = 0; s < c->B; ++s) {
        if (!c->active[s]) continue;
        for (int g = 0; g < c->ng; ++g) {
            const std::vector<int32_t> &rr = runs_of_row(c, (size_t)g * c->B + s);
            for (size_t k = 0; k < rr.size(); k += 3) out.insert(out.end(), {s, g, rr[k], rr[k + 1], rr[k + 2]});
        }
    }
}

// Bring slot s to life with need[g] pages per group.  The first share[g] of
// them are the pages source slot `src` holds at the same logical positions
// (Alias, KV-RM Fig 3: their counts grow by one); the rest are popped from
// the front of the free list.  cap/len: this slot's [H] rows (len NULL = 0).
// The caller has checked everything, including the free-page count.
void install(nup_ctx *c, int s, const int32_t *need, int src, const int32_t *share,
             const int32_t *cap, const int32_t *len) {
    for (int g = 0; g < c->ng; ++g) {
        const int np = need[g];
        const int shared = share ? share[g] : 0;
        const size_t ri = (size_t)g * c->B + s;
        int32_t *row = &c->pt[ri * c->max_pages];
        const int32_t *src_row = src >= 0 ? &c->pt[((size_t)g * c->B + src) * c->max_pages] : nullptr;
        for (int j = 0; j < shared; ++j) {
            row[j] = src_row[j];
            ++c->ref[row[j]];
        }
        if (np > shared) {
            c->free_list.pop_front(row + shared, (size_t)(np - shared));
            for (int j = shared; j < np; ++j) c->ref[row[j]] = 1;
        }
        c->dirty_count[ri] = std::max(c->dirty_count[ri], np);
        c->npages[ri] = np;
        c->runs_stale[ri] = 1;
    }
    for (int h = 0; h < c->V; ++h) {
        c->cap[(size_t)s * c->V + h] = cap[h];
        c->len[(size_t)s * c->V + h] = len ? len[h] : 0;
    }
    c->active[s] = 1;
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

nup_status nup_desc_bytes(const nup_config *cfg, size_t *bytes) {
    if (!bytes) return NUP_E_ARG;
    if (validate(cfg, nullptr) != NUP_OK) return NUP_E_ARG;
    int workers = cfg->num_workers > 0 ? cfg->num_workers : 0;
    if (workers == 0) {
        // largest default the library may pick: every CU at the highest occupancy
        int dev = 0;
        hipDeviceProp_t prop;
        if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess)
            workers = prop.multiProcessorCount * 32;
        else
            workers = default_workers_hostonly();
    }
    *bytes = compute_sizes(*cfg, workers).total;
    return NUP_OK;
}

nup_status nup_create(const nup_config *cfg, nup_ctx **out) {
    if (!out) return NUP_E_ARG;
    *out = nullptr;
    std::string why;
    if (validate(cfg, &why) != NUP_OK) {
        fprintf(stderr, "nup_create: %s\n", why.c_str());
        return NUP_E_ARG;
    }
    nup_ctx *c = new (std::nothrow) nup_ctx();
    if (!c) return NUP_E_ARG;
    c->cfg = *cfg;
    c->H = cfg->num_kv_heads;
    c->Hq = cfg->num_q_heads;
    c->D = cfg->head_dim;
    c->P = cfg->page_size;
    c->ng = cfg->num_groups;
    c->NL = cfg->num_layers > 0 ? cfg->num_layers : 1;
    c->V = c->NL * c->H;
    c->gh = c->V / c->ng;
    c->B = cfg->max_batch;
    c->num_pages = cfg->num_pages;
    c->max_pages = cfg->max_pages;
    c->gqa = c->Hq / c->H;
    c->has_device = cfg->k_pool && cfg->v_pool && cfg->desc;
    c->kpool = static_cast<uint16_t *>(cfg->k_pool);
    c->vpool = static_cast<uint16_t *>(cfg->v_pool);
    c->desc = static_cast<char *>(cfg->desc);
    if (c->has_device && (reinterpret_cast<uintptr_t>(c->desc) % kAlign)) {
        delete c;
        fprintf(stderr, "nup_create: descriptor arena must be 256-byte aligned\n");
        return NUP_E_ARG;
    }
    if (cfg->num_workers > 0) {
        c->workers = cfg->num_workers;
    } else if (!c->has_device) {
        c->workers = default_workers_hostonly();
    } else {
        int dev = 0;
        hipDeviceProp_t prop;
        if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            delete c;
            fprintf(stderr, "nup_create: no HIP device for a device context\n");
            return NUP_E_HIP;
        }
        // one workgroup of kWavesPerBlock workers per CU: one wave per SIMD
        if (nup::partial_blocks_per_cu(c->D, c->gqa, nup::kModePaged) < 1) {
            delete c;
            fprintf(stderr, "nup_create: the split-K kernel does not fit a compute unit\n");
            return NUP_E_HIP;
        }
        // The share-aware plan keeps two waves per SIMD: its gang launch
        // wants the larger worker count (forked batch: 46 + 375 us against
        // 77 + 382 us with one wave per SIMD).
        c->workers = prop.multiProcessorCount * nup::kWavesPerBlock * (c->cfg.plan_mode == NUP_PLAN_SHARED ? 2 : 1);
    }
    if (c->has_device) {
        // set-up of the allocation-free entry point: look up this device's
        // scratch address now, with the device current (a failure is kept
        // and reported by that entry point)
        if (hipGetDevice(&c->device) != hipSuccess) {
            delete c;
            fprintf(stderr, "nup_create: no HIP device for a device context\n");
            return NUP_E_HIP;
        }
        void *scratch = nullptr;
        (void)nup::scratch_buffer(c->device, &scratch);
    }
    c->sz = compute_sizes(c->cfg, c->workers);
    c->free_list.init((size_t)c->num_pages);
    if (cfg->free_list_init) {
        std::vector<char> seen(c->num_pages, 0);
        for (int i = 0; i < c->num_pages; ++i) {
            const int32_t p = cfg->free_list_init[i];
            if (p < 0 || p >= c->num_pages || seen[p]) {
                delete c;
                fprintf(stderr, "nup_create: free_list_init is not a permutation\n");
                return NUP_E_ARG;
            }
            seen[p] = 1;
            c->free_list.push_back(p);
        }
    } else {
        for (int i = 0; i < c->num_pages; ++i) c->free_list.push_back(i);
    }
    c->pt.assign((size_t)c->ng * c->B * c->max_pages, -1);
    c->npages.assign((size_t)c->ng * c->B, 0);
    c->len.assign((size_t)c->B * c->V, 0);
    c->cap.assign((size_t)c->B * c->V, 0);
    c->active.assign(c->B, 0);
    c->ref.assign(c->num_pages, 0);
    c->goh.assign(c->V, -1);
    c->soh.assign(c->V, -1);
    c->head_of_gslot.assign(c->V, -1);
    c->plan.assign(c->NL, {});
    // each layer's plan at a fixed place in the inbox, so that the kernels'
    // plan pointers never change for a context (a captured decode graph
    // stays valid across commits)
    c->off_ws.assign(c->NL, 0);
    c->off_hrs.assign(c->NL, 0);
    c->off_rows.assign(c->NL, 0);
    c->off_hr.assign(c->NL, 0);
    c->off_skip.assign(c->NL, 0);
    c->off_gang.assign(c->NL, 0);
    c->off_gn.assign(c->NL, 0);
    for (int l = 0; l < c->NL; ++l) {
        c->off_ws[l] = c->sz.fixed + c->sz.caps + (size_t)l * c->sz.plan_layer;
        c->off_hrs[l] = c->off_ws[l] + align_up(4 * ((size_t)c->sz.max_workers + 1));
        c->off_rows[l] = c->off_hrs[l] + align_up(4 * ((size_t)c->B * c->H + 1));
        c->off_hr[l] = c->off_rows[l] + align_up(16 * (size_t)c->sz.max_rows);
        c->off_skip[l] = c->off_hr[l] + align_up(4 * (size_t)c->sz.max_rows);
        c->off_gang[l] = c->off_skip[l] + align_up(4 * (size_t)c->sz.max_workers);
        c->off_gn[l] = c->off_gang[l] + align_up(4 * (size_t)c->sz.max_workers);
    }
    c->dev_workers.assign(c->NL, 0);
    c->dev_rows.assign(c->NL, 0);
    c->dirty_count.assign((size_t)c->ng * c->B, 0);
    c->row_runs.assign((size_t)c->ng * c->B, {});
    c->runs_stale.assign((size_t)c->ng * c->B, 0);
    replan(c);
    *out = c;
    return NUP_OK;
}

void nup_destroy(nup_ctx *c) {
    if (!c) return;
    for (int i = 0; i < 2; ++i) {
        if (c->pinned_ev[i]) {
            (void)hipEventSynchronize(c->pinned_ev[i]);
            (void)hipEventDestroy(c->pinned_ev[i]);
        }
        if (c->pinned[i]) (void)hipHostFree(c->pinned[i]);
    }
    for (auto &e : c->tev) {
        (void)hipEventDestroy(e.first);
        (void)hipEventDestroy(e.second);
    }
    delete c;
}

const char *nup_last_error(const nup_ctx *c) { return c ? c->err.c_str() : "null context"; }

nup_status kv_alloc_groups(nup_ctx *c, int32_t n, const int32_t *slots, const int32_t *cap,
                           const int32_t *len, int32_t *group_of_head_out) {
    if (!c) return NUP_E_ARG;
    if (n < 0) return fail(c, NUP_E_ARG, "n < 0");
    if (n == 0) {
        if (group_of_head_out && c->grouped) std::copy(c->goh.begin(), c->goh.end(), group_of_head_out);
        return NUP_OK;
    }
    if (!slots || !cap) return fail(c, NUP_E_ARG, "slots and cap are required");
    std::vector<char> seen(c->B, 0);
    for (int i = 0; i < n; ++i) {
        const int s = slots[i];
        if (s < 0 || s >= c->B) return fail(c, NUP_E_ARG, "slot %d out of range", s);
        if (seen[s]) return fail(c, NUP_E_ARG, "slot %d repeated", s);
        seen[s] = 1;
        for (int h = 0; h < c->V; ++h) {
            const long long cp = cap[(size_t)i * c->V + h];
            const long long ln = len ? len[(size_t)i * c->V + h] : 0;
            if (cp < 0 || cp > (long long)c->max_pages * c->P)
                return fail(c, NUP_E_ARG, "cap %lld of slot %d head %d outside [0, %lld]", cp, s, h,
                            (long long)c->max_pages * c->P);
            if (ln < 0 || ln > cp) return fail(c, NUP_E_ARG, "len %lld of slot %d head %d outside [0, cap]", ln, s, h);
        }
    }
    for (int i = 0; i < n; ++i)
        if (c->active[slots[i]]) return fail(c, NUP_E_STATE, "slot %d is already active", slots[i]);

    // grouping of this call (fixed only once the call succeeds)
    std::vector<int32_t> goh = c->goh;
    if (!c->grouped) {
        nup_ctx tmp;  // reuse group_heads on a scratch context
        tmp.H = c->H;
        tmp.V = c->V;
        tmp.gh = c->gh;
        tmp.goh.assign(c->V, 0);
        tmp.soh.assign(c->V, 0);
        tmp.head_of_gslot.assign(c->V, 0);
        group_heads(&tmp, n, cap);
        goh = tmp.goh;
    }
    std::vector<int32_t> need((size_t)n * c->ng, 0);
    long long total = 0;
    for (int i = 0; i < n; ++i)
        for (int h = 0; h < c->V; ++h) {
            int32_t &x = need[(size_t)i * c->ng + goh[h]];
            x = std::max<int32_t>(x, (cap[(size_t)i * c->V + h] + c->P - 1) / c->P);
        }
    for (int32_t x : need) total += x;
    if (total > (long long)c->free_list.size())
        return fail(c, NUP_E_NOPAGES, "need %lld pages, %zu free", total, c->free_list.size());

    if (!c->grouped) group_heads(c, n, cap);
    for (int i = 0; i < n; ++i)
        install(c, slots[i], &need[(size_t)i * c->ng], -1, nullptr, cap + (size_t)i * c->V,
                len ? len + (size_t)i * c->V : nullptr);
    c->plan_dirty = true;
    c->pending = true;
    if (group_of_head_out) std::copy(c->goh.begin(), c->goh.end(), group_of_head_out);
    return NUP_OK;
}

nup_status kv_alias(nup_ctx *c, int32_t n, const int32_t *slots, const int32_t *src_slots,
                    const int32_t *share_pages, const int32_t *cap, const int32_t *len) {
    if (!c) return NUP_E_ARG;
    if (n < 0) return fail(c, NUP_E_ARG, "n < 0");
    if (n == 0) return NUP_OK;
    if (!slots || !src_slots || !share_pages || !cap || !len)
        return fail(c, NUP_E_ARG, "slots, src_slots, share_pages, cap and len are required");
    std::vector<char> seen(c->B, 0);
    for (int i = 0; i < n; ++i) {
        const int s = slots[i];
        if (s < 0 || s >= c->B) return fail(c, NUP_E_ARG, "slot %d out of range", s);
        if (seen[s]) return fail(c, NUP_E_ARG, "slot %d repeated", s);
        seen[s] = 1;
    }
    for (int i = 0; i < n; ++i) {
        const int src = src_slots[i];
        if (src < 0 || src >= c->B) return fail(c, NUP_E_ARG, "source slot %d out of range", src);
        if (seen[src]) return fail(c, NUP_E_ARG, "source slot %d is also a new slot", src);
    }
    for (int i = 0; i < n; ++i) {
        for (int h = 0; h < c->V; ++h) {
            const long long cp = cap[(size_t)i * c->V + h];
            const long long ln = len[(size_t)i * c->V + h];
            if (cp < 0 || cp > (long long)c->max_pages * c->P)
                return fail(c, NUP_E_ARG, "cap %lld of slot %d head %d outside [0, %lld]", cp, slots[i], h,
                            (long long)c->max_pages * c->P);
            if (ln < 0 || ln > cp)
                return fail(c, NUP_E_ARG, "len %lld of slot %d head %d outside [0, cap]", ln, slots[i], h);
        }
        for (int g = 0; g < c->ng; ++g)
            if (share_pages[(size_t)i * c->ng + g] < 0)
                return fail(c, NUP_E_ARG, "negative share for slot %d group %d", slots[i], g);
    }
    for (int i = 0; i < n; ++i) {
        if (c->active[slots[i]]) return fail(c, NUP_E_STATE, "slot %d is already active", slots[i]);
        if (!c->active[src_slots[i]]) return fail(c, NUP_E_STATE, "source slot %d is not active", src_slots[i]);
    }
    // shared pages must be full in both sequences, so that no append writes them
    for (int i = 0; i < n; ++i)
        for (int h = 0; h < c->V; ++h) {
            const long long tokens = (long long)share_pages[(size_t)i * c->ng + c->goh[h]] * c->P;
            if (tokens > len[(size_t)i * c->V + h] || tokens > c->len[(size_t)src_slots[i] * c->V + h])
                return fail(c, NUP_E_ARG, "share of %lld tokens exceeds a length of slot %d or source %d (head %d)",
                            tokens, slots[i], src_slots[i], h);
        }
    std::vector<int32_t> need((size_t)n * c->ng, 0);
    long long fresh = 0;
    for (int i = 0; i < n; ++i) {
        for (int h = 0; h < c->V; ++h) {
            int32_t &x = need[(size_t)i * c->ng + c->goh[h]];
            x = std::max<int32_t>(x, (cap[(size_t)i * c->V + h] + c->P - 1) / c->P);
        }
        for (int g = 0; g < c->ng; ++g) fresh += need[(size_t)i * c->ng + g] - share_pages[(size_t)i * c->ng + g];
    }
    if (fresh > (long long)c->free_list.size())
        return fail(c, NUP_E_NOPAGES, "need %lld pages, %zu free", fresh, c->free_list.size());
    for (int i = 0; i < n; ++i)
        install(c, slots[i], &need[(size_t)i * c->ng], src_slots[i], share_pages + (size_t)i * c->ng,
                cap + (size_t)i * c->V, len + (size_t)i * c->V);
    c->plan_dirty = true;
    c->pending = true;
    return NUP_OK;
}

nup_status kv_free_seqs(nup_ctx *c, int32_t n, const int32_t *slots) {
    if (!c) return NUP_E_ARG;
    if (n < 0 || (n > 0 && !slots)) return fail(c, NUP_E_ARG, "bad slot list");
    std::vector<char> seen(c->B, 0);
    for (int i = 0; i < n; ++i) {
        const int s = slots[i];
        if (s < 0 || s >= c->B) return fail(c, NUP_E_ARG, "slot %d out of range", s);
        if (seen[s]) return fail(c, NUP_E_ARG, "slot %d repeated", s);
        seen[s] = 1;
    }
    for (int i = 0; i < n; ++i)
        if (!c->active[slots[i]]) return fail(c, NUP_E_STATE, "slot %d is not active", slots[i]);
    if (n == 0) return NUP_OK;
    for (int i = 0; i < n; ++i) {
        const int s = slots[i];
        for (int g = 0; g < c->ng; ++g) {
            const size_t ri = (size_t)g * c->B + s;
            int32_t *row = &c->pt[ri * c->max_pages];
            for (int j = 0; j < c->npages[ri]; ++j) {
                if (--c->ref[row[j]] == 0) c->free_list.push_back(row[j]);
                row[j] = -1;
            }
            c->dirty_count[ri] = std::max(c->dirty_count[ri], c->npages[ri]);
            c->npages[ri] = 0;
            c->runs_stale[ri] = 1;
        }
        for (int h = 0; h < c->V; ++h) {
            c->cap[(size_t)s * c->V + h] = 0;
            c->len[(size_t)s * c->V + h] = 0;
        }
        c->active[s] = 0;
    }
    c->plan_dirty = true;
    c->pending = true;
    return NUP_OK;
}

nup_status nup_commit(nup_ctx *c, void *stream) {
    if (!c) return NUP_E_ARG;
    if (!c->has_device) return fail(c, NUP_E_STATE, "context has no device buffers");
    hipStream_t st = static_cast<hipStream_t>(stream);
    // a captured copy would replay this call's staging buffer, which later
    // commits rewrite: the commit always runs eagerly, between replays
    if (capturing(st)) return fail(c, NUP_E_STATE, "nup_commit cannot be captured into a graph");
    // Nothing edited since the last commit: the device already holds this
    // frame (appends advance the device lengths themselves), so the commit
    // sends nothing.
    if (c->committed && !c->pending) return NUP_OK;
    const int i = c->pinned_next;
    if (!c->pinned[i]) {
        hipError_t e = hipHostMalloc(reinterpret_cast<void **>(&c->pinned[i]), c->sz.inbox, hipHostMallocDefault);
        if (e != hipSuccess) return hip_fail(c, e, "hipHostMalloc");
        e = hipEventCreateWithFlags(&c->pinned_ev[i], hipEventDisableTiming);
        if (e != hipSuccess) return hip_fail(c, e, "hipEventCreate");
    }
    if (c->pinned_used[i]) {
        hipError_t e = hipEventSynchronize(c->pinned_ev[i]);
        if (e != hipSuccess) return hip_fail(c, e, "hipEventSynchronize");
    }
    char *blob = c->pinned[i];
    int32_t *w = reinterpret_cast<int32_t *>(blob);
    const size_t B = c->B, V = c->V;
    for (size_t s = 0; s < B; ++s) w[s] = c->active[s];
    for (size_t k = 0; k < B * V; ++k) w[B + k] = c->active[k / V] ? c->len[k] : 0;
    std::copy(c->goh.begin(), c->goh.end(), w + B + B * V);
    std::copy(c->soh.begin(), c->soh.end(), w + B + B * V + V);
    std::copy(c->head_of_gslot.begin(), c->head_of_gslot.end(), w + B + B * V + 2 * V);
    size_t used = c->sz.fixed;
    int n_patches = 0;
    size_t off_hdr = 0, off_data = 0;
    if (c->plan_dirty || !c->committed) {
        int32_t *cw = reinterpret_cast<int32_t *>(blob + c->sz.fixed);
        for (size_t k = 0; k < B * V; ++k) cw[k] = c->active[k / V] ? c->cap[k] : 0;
        // plan (once per commit, however many Reserve / Trim edits came before)
        replan(c);
        for (int l = 0; l < c->NL; ++l) {
            const nup_ctx::Plan &pl = c->plan[l];
            const int nr = (int)(pl.rows.size() / 4);
            int32_t *wsd = reinterpret_cast<int32_t *>(blob + c->off_ws[l]);
            std::memcpy(wsd, pl.worker_start.data(), 4 * pl.worker_start.size());
            // the launch always has max_workers workers (the balanced plan
            // has exactly that many; the uniform one's surplus get no rows),
            // so a captured launch stays valid when the plan changes
            for (size_t w = pl.worker_start.size(); w <= (size_t)c->sz.max_workers; ++w) wsd[w] = nr;
            std::memcpy(blob + c->off_hrs[l], pl.head_row_start.data(), 4 * pl.head_row_start.size());
            if (nr) std::memcpy(blob + c->off_rows[l], pl.rows.data(), 16 * (size_t)nr);
            if (c->cfg.plan_mode == NUP_PLAN_SHARED) {
                int32_t *hr = reinterpret_cast<int32_t *>(blob + c->off_hr[l]);
                if (pl.head_rows.empty()) std::iota(hr, hr + nr, 0);
                else std::memcpy(hr, pl.head_rows.data(), 4 * (size_t)nr);
                int32_t *sk = reinterpret_cast<int32_t *>(blob + c->off_skip[l]);
                std::fill(sk, sk + c->sz.max_workers, 0);
                if (!pl.worker_skip.empty()) std::memcpy(sk, pl.worker_skip.data(), 4 * pl.worker_skip.size());
                if (!pl.gang_rows.empty())
                    std::memcpy(blob + c->off_gang[l], pl.gang_rows.data(), 4 * pl.gang_rows.size());
                *reinterpret_cast<int32_t *>(blob + c->off_gn[l]) = (int32_t)(pl.gang_rows.size() / nup::kWavesPerBlock);
            }
            c->dev_workers[l] = c->sz.max_workers;
            c->dev_rows[l] = nr;
        }
        size_t off = c->sz.fixed + c->sz.caps + c->sz.plan_max;
        // trains
        std::vector<int32_t> runs5;
        build_runs(c, runs5);
        const int nruns = (int)(runs5.size() / 5);
        if ((size_t)nruns > (size_t)c->ng * c->B * c->max_pages)
            return fail(c, NUP_E_STATE, "internal: %d trains exceed the page-table entries", nruns);
        c->off_runs = off;
        int32_t *rw = reinterpret_cast<int32_t *>(blob + off);
        for (int r = 0; r < nruns; ++r) {
            rw[r * 4 + 0] = runs5[r * 5 + 0] * c->ng + runs5[r * 5 + 1];
            rw[r * 4 + 1] = runs5[r * 5 + 2];
            rw[r * 4 + 2] = runs5[r * 5 + 3];
            rw[r * 4 + 3] = runs5[r * 5 + 4];
        }
        off = align_up(off + 16 * (size_t)nruns);
        c->off_runpre = off;
        int32_t *pre = reinterpret_cast<int32_t *>(blob + off);
        pre[0] = 0;
        for (int r = 0; r < nruns; ++r) pre[r + 1] = pre[r] + runs5[r * 5 + 3];
        off = align_up(off + 4 * ((size_t)nruns + 1));
        // page-table patches
        off_hdr = off;
        int32_t *hdr = reinterpret_cast<int32_t *>(blob + off);
        for (size_t ri = 0; ri < c->dirty_count.size(); ++ri)
            if (c->dirty_count[ri] > 0) ++n_patches;
        off = align_up(off + 16 * (size_t)n_patches);
        off_data = off;
        int32_t *data = reinterpret_cast<int32_t *>(blob + off);
        size_t dpos = 0;
        int p = 0;
        for (size_t ri = 0; ri < c->dirty_count.size(); ++ri) {
            const int cnt = c->dirty_count[ri];
            if (cnt <= 0) continue;
            hdr[p * 4 + 0] = (int32_t)ri;
            hdr[p * 4 + 1] = cnt;
            hdr[p * 4 + 2] = (int32_t)dpos;
            hdr[p * 4 + 3] = 0;
            std::memcpy(data + dpos, &c->pt[ri * c->max_pages], 4 * (size_t)cnt);
            dpos += cnt;
            ++p;
        }
        used = off + 4 * dpos;
        c->dev_runs = nruns;
        c->dev_run_pages = pre[nruns];
    }
    hipError_t e;
    if (!c->committed) {  // the latched device error word and the arrival counts start clear
        e = nup::launch_fill(c->d_err(), 1, 0, st);
        if (e != hipSuccess) return hip_fail(c, e, "clear device error word");
        e = nup::launch_fill(c->d_arrive(), c->NL * c->B * c->H, 0, st);
        if (e != hipSuccess) return hip_fail(c, e, "clear arrival counts");
    }
    e = hipMemcpyAsync(c->desc, blob, used, hipMemcpyHostToDevice, st);
    if (e != hipSuccess) return hip_fail(c, e, "hipMemcpyAsync (commit)");
    if (n_patches > 0) {
        e = nup::launch_apply_patches(c->d_pt(), reinterpret_cast<const int32_t *>(c->desc + off_hdr),
                                      reinterpret_cast<const int32_t *>(c->desc + off_data), n_patches,
                                      c->max_pages, st);
        if (e != hipSuccess) return hip_fail(c, e, "apply_patches launch");
    }
    e = hipEventRecord(c->pinned_ev[i], st);
    if (e != hipSuccess) return hip_fail(c, e, "hipEventRecord");
    c->pinned_used[i] = true;
    c->pinned_next = 1 - i;
    std::fill(c->dirty_count.begin(), c->dirty_count.end(), 0);
    c->plan_dirty = false;
    c->pending = false;
    c->committed = true;
    return NUP_OK;
}

nup_status kv_append(nup_ctx *c, const void *k_new, const void *v_new, void *stream) {
    if (!c) return NUP_E_ARG;
    if (!c->has_device) return fail(c, NUP_E_STATE, "context has no device buffers");
    if (!k_new || !v_new) return fail(c, NUP_E_ARG, "k_new and v_new are required");
    if (!c->committed || c->pending) return fail(c, NUP_E_STATE, "edits pending: nup_commit first");
    const bool cap_mode = capturing(static_cast<hipStream_t>(stream));
    for (int s = 0; s < c->B && !cap_mode; ++s) {
        if (!c->active[s]) continue;
        for (int h = 0; h < c->H; ++h) {
            const size_t k = (size_t)s * c->V + c->lbase() + h;
            if (c->len[k] >= c->cap[k])
                return fail(c, NUP_E_CAPACITY, "slot %d layer %d head %d is at its budget (%d tokens)", s,
                            c->layer, h, c->cap[k]);
        }
    }
    nup::AppendArgs a{};
    a.k_pool = c->kpool;
    a.v_pool = c->vpool;
    a.k_new = static_cast<const uint16_t *>(k_new);
    a.v_new = static_cast<const uint16_t *>(v_new);
    a.page_table = c->d_pt();
    a.active = c->d_active();
    a.group_of_head = c->d_goh() + c->lbase();
    a.slot_of_head = c->d_soh() + c->lbase();
    a.lengths = c->d_len() + c->lbase();
    a.caps = c->d_cap() + c->lbase();
    a.err = c->d_err();
    a.bmax = c->B;
    a.hkv = c->H;
    a.gh = c->gh;
    a.max_pages = c->max_pages;
    a.lstride = c->V;
    hipError_t e = nup::launch_append(a, c->D, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(c, e, "append launch");
    // a captured append runs at each replay, after this call: the caller
    // reports the replays with nup_note_appends
    if (cap_mode) return NUP_OK;
    for (int s = 0; s < c->B; ++s)
        if (c->active[s])
            for (int h = 0; h < c->H; ++h) c->len[(size_t)s * c->V + c->lbase() + h]++;
    return NUP_OK;
}

nup_status kv_gather_compact(nup_ctx *c, int32_t mode, const int32_t *idx, int32_t K, void *k_out,
                             void *v_out, const int64_t *row_off, int32_t *phys_out, void *stream) {
    if (!c) return NUP_E_ARG;
    if (!c->has_device) return fail(c, NUP_E_STATE, "context has no device buffers");
    if (!c->committed) return fail(c, NUP_E_STATE, "no committed descriptor");
    if (!k_out || !v_out) return fail(c, NUP_E_ARG, "k_out and v_out are required");
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (mode == 1) {
        if (!idx || K <= 0) return fail(c, NUP_E_ARG, "index mode needs idx and K > 0");
        nup::GatherIndexArgs a{};
        a.k_pool = c->kpool;
        a.v_pool = c->vpool;
        a.page_table = c->d_pt();
        a.active = c->d_active();
        a.lengths = c->d_len() + c->lbase();
        a.group_of_head = c->d_goh() + c->lbase();
        a.slot_of_head = c->d_soh() + c->lbase();
        a.lstride = c->V;
        a.idx = idx;
        a.k_out = static_cast<uint16_t *>(k_out);
        a.v_out = static_cast<uint16_t *>(v_out);
        a.phys_out = phys_out;
        a.err = c->d_err();
        a.bmax = c->B;
        a.hkv = c->H;
        a.gh = c->gh;
        a.max_pages = c->max_pages;
        a.k = K;
        e = nup::launch_gather_index(a, c->D, st);
    } else if (mode == 0) {
        if (!row_off) return fail(c, NUP_E_ARG, "train mode needs row_off");
        // the launch is sized by the current trains, which the next commit changes
        if (capturing(st)) return fail(c, NUP_E_STATE, "the trains gather cannot be captured into a graph");
        nup::GatherRunsArgs a{};
        a.k_pool = c->kpool;
        a.v_pool = c->vpool;
        a.runs = c->inbox_i32(c->off_runs);
        a.run_prefix = c->inbox_i32(c->off_runpre);
        a.active = c->d_active();
        a.lengths = c->d_len() + c->lbase();
        a.lstride = c->V;
        a.layer_base = (int32_t)c->lbase();
        a.head_of_gslot = c->d_hog();
        a.row_off = row_off;
        a.k_out = static_cast<uint16_t *>(k_out);
        a.v_out = static_cast<uint16_t *>(v_out);
        a.phys_out = phys_out;
        a.n_runs = c->dev_runs;
        a.ng = c->ng;
        a.gh = c->gh;
        a.hkv = c->H;
        e = nup::launch_gather_runs(a, c->D, c->dev_run_pages, st);
    } else {
        return fail(c, NUP_E_ARG, "mode must be 0 (trains) or 1 (indices)");
    }
    if (e != hipSuccess) return hip_fail(c, e, "gather launch");
    return NUP_OK;
}

nup_status kv_gather_trains_dma(nup_ctx *c, void *k_out, void *v_out, const int64_t *row_off,
                                int32_t *n_copies, void *stream) {
    if (!c) return NUP_E_ARG;
    if (!c->has_device) return fail(c, NUP_E_STATE, "context has no device buffers");
    if (!c->committed || c->pending) return fail(c, NUP_E_STATE, "needs a committed descriptor and no pending edits");
    if (!k_out || !v_out || !row_off) return fail(c, NUP_E_ARG, "k_out, v_out and row_off are required");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (capturing(st)) return fail(c, NUP_E_STATE, "copies of the current trains cannot be captured into a graph");
    const size_t row_bytes = (size_t)c->D * 2, page_rows = (size_t)c->P;
    const size_t page_bytes = page_rows * row_bytes;          // one head's rows of one page
    const size_t src_pitch = (size_t)c->gh * page_bytes;      // next physical page, same head slot
    int32_t copies = 0;
    for (int s = 0; s < c->B; ++s) {
        if (!c->active[s]) continue;
        for (int g = 0; g < c->ng; ++g) {
            const std::vector<int32_t> &rr = runs_of_row(c, (size_t)g * c->B + s);
            for (size_t k = 0; k < rr.size(); k += 3) {
                const int64_t phys = rr[k], pages = rr[k + 1], logical = rr[k + 2];
                for (int j = 0; j < c->gh; ++j) {
                    const int h = c->head_of_gslot[g * c->gh + j] - (int)c->lbase();  // this layer's?
                    if (h < 0 || h >= c->H) continue;
                    const int64_t L = c->len[(size_t)s * c->V + c->lbase() + h];
                    const int64_t rows = std::min<int64_t>(std::max<int64_t>(L - logical * c->P, 0), pages * c->P);
                    if (rows == 0) continue;
                    const int64_t full = rows / c->P, tail = rows % c->P;
                    const size_t src_off = ((size_t)phys * c->gh + j) * page_bytes;
                    const size_t dst_off = (size_t)(row_off[(size_t)s * c->H + h] + logical * c->P) * row_bytes;
                    for (int kv = 0; kv < 2; ++kv) {
                        const char *src = reinterpret_cast<const char *>(kv ? c->vpool : c->kpool) + src_off;
                        char *dst = static_cast<char *>(kv ? v_out : k_out) + dst_off;
                        hipError_t e = hipSuccess;
                        if (c->gh == 1) {
                            // one head per page: the train's rows of this head are one range
                            e = hipMemcpyAsync(dst, src, rows * row_bytes, hipMemcpyDeviceToDeviceNoCU, st);
                            ++copies;
                        } else {
                            // G_h heads interleave page by page: a strided copy of the
                            // full pages, then the partial last page
                            if (full > 0)
                                e = hipMemcpy2DAsync(dst, page_bytes, src, src_pitch, page_bytes, full,
                                                     hipMemcpyDeviceToDeviceNoCU, st);
                            if (e == hipSuccess && tail > 0)
                                e = hipMemcpyAsync(dst + full * page_bytes, src + full * src_pitch, tail * row_bytes,
                                                   hipMemcpyDeviceToDeviceNoCU, st);
                            copies += (full > 0) + (tail > 0);
                        }
                        if (e != hipSuccess) return hip_fail(c, e, "copy-engine train");
                    }
                }
            }
        }
    }
    if (n_copies) *n_copies = copies;
    return NUP_OK;
}

// Top-K split: every head holds K rows, so a plain equal split balances it.
// About one worker per SIMD, as for the paged plan: a top-K head is short,
// and more splits cost more in the merge than they gain in parallelism
// (measured on the Llama-3-8B shape, 64 heads x 2048 rows: 1024 workers
// 20.4 us per layer, 2048 workers 22.7 us, 512 workers 25.6 us).
static void topk_split(const nup_ctx *c, int K, int *splits, int *chunk) {
    const int heads = c->B * c->H;
    const int pages = (K + nup::kPage - 1) / nup::kPage;
    // one per SIMD: the context's worker count, which the share-aware plan doubles
    const int target = std::max(1, c->cfg.plan_mode == NUP_PLAN_SHARED && c->cfg.num_workers <= 0 ? c->workers / 2
                                                                                                  : c->workers);
    int S = std::max(1, (target + heads - 1) / heads);
    S = std::max(S, (K + nup::kMaxTopkChunk - 1) / nup::kMaxTopkChunk);  // chunk <= LDS row-id room
    S = std::min(S, pages);
    const int ch = nup::kPage * ((pages + S - 1) / S);
    S = (K + ch - 1) / ch;
    *splits = S;
    *chunk = ch;
}

nup_status nup_workspace_bytes(const nup_ctx *c, int32_t K, size_t *bytes) {
    if (!c || !bytes || K < 0) return NUP_E_ARG;
    long long rows;
    if (K > 0) {
        int S, ch;
        topk_split(c, K, &S, &ch);
        rows = (long long)c->B * c->H * S;
    } else {
        rows = c->sz.max_rows;
    }
    *bytes = align_up((size_t)rows * c->gqa * c->D * 4) + align_up((size_t)rows * c->gqa * 2 * 4);
    return NUP_OK;
}

static nup_status attn_common(nup_ctx *c, const void *q, float *out, float *lse, float scale, void *ws,
                              size_t ws_bytes, void *stream, int mode, const void *ks, const void *vs,
                              const int32_t *idx, int K, const void *k_new = nullptr,
                              const void *v_new = nullptr, bool may_time = true) {
    const bool topk = mode != nup::kModePaged;
    if (!c) return NUP_E_ARG;
    if (!c->has_device) return fail(c, NUP_E_STATE, "context has no device buffers");
    if (!c->committed) return fail(c, NUP_E_STATE, "no committed descriptor");
    if (!q || !out || !ws) return fail(c, NUP_E_ARG, "q, out and workspace are required");
    if (!(scale > 0.0f) || !std::isfinite(scale)) return fail(c, NUP_E_ARG, "scale must be positive and finite");
    size_t need = 0;
    nup_workspace_bytes(c, topk ? K : 0, &need);
    if (ws_bytes < need) return fail(c, NUP_E_ARG, "workspace %zu bytes < %zu needed", ws_bytes, need);
    hipStream_t st = static_cast<hipStream_t>(stream);
    nup::PartialArgs a{};
    a.q = static_cast<const uint16_t *>(q);
    a.active = c->d_active();
    a.lengths = c->d_len() + c->lbase();
    a.group_of_head = c->d_goh() + c->lbase();
    a.slot_of_head = c->d_soh() + c->lbase();
    a.lstride = c->V;
    a.bmax = c->B;
    a.hkv = c->H;
    a.gh = c->gh;
    a.max_pages = c->max_pages;
    a.scale_log2 = scale * 1.4426950408889634f;
    int rows_max;
    int splits = 0;
    if (topk) {
        int ch;
        topk_split(c, K, &splits, &ch);
        if (mode == nup::kModeStaged) {
            a.kbase = static_cast<const uint16_t *>(ks);
            a.vbase = static_cast<const uint16_t *>(vs);
        } else {
            a.kbase = c->kpool;
            a.vbase = c->vpool;
            a.page_table = c->d_pt();
            a.idx = idx;
            a.err = c->d_err();
        }
        a.topk_k = K;
        a.topk_splits = splits;
        a.topk_chunk = ch;
        a.n_workers = c->B * c->H * splits;
        rows_max = a.n_workers;
    } else {
        a.kbase = c->kpool;
        a.vbase = c->vpool;
        a.page_table = c->d_pt();
        a.rows = c->inbox_i32(c->off_rows[c->layer]);
        a.worker_start = c->inbox_i32(c->off_ws[c->layer]);
        a.n_workers = c->dev_workers[c->layer];
        rows_max = c->sz.max_rows;
        a.k_new = static_cast<const uint16_t *>(k_new);
        a.v_new = static_cast<const uint16_t *>(v_new);
        a.caps = c->d_cap() + c->lbase();
        a.err = c->d_err();
    }
    float *wso = static_cast<float *>(ws);
    float *wsml = reinterpret_cast<float *>(static_cast<char *>(ws) +
                                            align_up((size_t)rows_max * c->gqa * c->D * 4));
    a.ws_o = wso;
    a.ws_ml = wsml;
    a.out = out;
    a.lse = lse;
    a.head_row_start = topk ? nullptr : c->inbox_i32(c->off_hrs[c->layer]);
    hipError_t e;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    // a graph's launches are not timed, nor the allocation-free call's
    // (creating events is an allocation)
    const bool timed = may_time && c->timing && !capturing(st);
    if (timed) {
        // timing-only events: no system-scope fence when recorded, so the
        // interval holds the launch and not a writeback of the caches
        if ((e = hipEventCreateWithFlags(&e0, hipEventDisableSystemFence)) != hipSuccess ||
            (e = hipEventCreateWithFlags(&e1, hipEventDisableSystemFence)) != hipSuccess)
            return hip_fail(c, e, "hipEventCreate");
        if ((e = hipEventRecord(e0, st)) != hipSuccess) return hip_fail(c, e, "hipEventRecord");
    }
    const bool gang = !topk && c->cfg.plan_mode == NUP_PLAN_SHARED && c->D == 128 &&
                      c->sz.max_workers % nup::kWavesPerBlock == 0;
    // The merge inside the split-K launch, when asked for: it needs each
    // head's rows contiguous in the table (the share-aware plan keeps its
    // merge launch) and partial areas that 32-bit buffer offsets reach.  The
    // default is the merge launch: on MI355X the device-scope round trips of
    // the in-launch merge (store, count, reload) cost more than the launch.
    const size_t o_bytes = align_up((size_t)rows_max * c->gqa * c->D * 4);
    const size_t ml_bytes = (size_t)rows_max * c->gqa * 2 * 4;
    const bool in_split = c->cfg.merge_mode == NUP_MERGE_IN_SPLIT && (topk || c->cfg.plan_mode != NUP_PLAN_SHARED) &&
                          o_bytes < 0x80000000ull;
    if (in_split) {
        a.arrive = c->d_arrive() + (size_t)c->layer * c->B * c->H;
        a.ws_o_bytes = (uint32_t)o_bytes;
        a.ws_ml_bytes = (uint32_t)ml_bytes;
        if (k_new) {
            a.lengths_w = c->d_len() + c->lbase();
            a.active = c->d_active();
        }
    }
    if (gang) {
        // the share-aware plan's gang launch first: workgroups of four
        // sharers of one chunk (the count is read on the device, so a
        // captured launch follows the plan); no appends there
        nup::PartialArgs g = a;
        g.k_new = nullptr;
        g.v_new = nullptr;
        g.gang_rows = c->inbox_i32(c->off_gang[c->layer]);
        g.gang_blocks = c->inbox_i32(c->off_gn[c->layer]);
        e = nup::launch_partial(g, c->D, c->gqa, nup::kModeGang, st);
        if (e != hipSuccess) return hip_fail(c, e, "gang attention launch");
        a.worker_skip = c->inbox_i32(c->off_skip[c->layer]);
    }
    e = nup::launch_partial(a, c->D, c->gqa, mode, st);
    if (e != hipSuccess) return hip_fail(c, e, "partial attention launch");
    if (timed) {
        if ((e = hipEventRecord(e1, st)) != hipSuccess) return hip_fail(c, e, "hipEventRecord");
        c->tev.emplace_back(e0, e1);
    }
    if (in_split) return NUP_OK;
    nup::MergeArgs m{};
    m.ws_o = wso;
    m.ws_ml = wsml;
    m.head_row_start = a.head_row_start;
    m.head_rows = (!topk && c->cfg.plan_mode == NUP_PLAN_SHARED) ? c->inbox_i32(c->off_hr[c->layer]) : nullptr;
    m.uniform_splits = splits;
    m.out = out;
    m.lse = lse;
    m.hkv = c->H;
    if (k_new) {
        m.lengths = c->d_len() + c->lbase();
        m.caps = c->d_cap() + c->lbase();
        m.active = c->d_active();
        m.err = c->d_err();
        m.lstride = c->V;
    }
    e = nup::launch_merge(m, c->D, c->gqa, c->B * c->H, st);
    if (e != hipSuccess) return hip_fail(c, e, "merge launch");
    return NUP_OK;
}

nup_status attn_decode_nonuniform(nup_ctx *c, const void *q, float *out, float *lse, float scale,
                                  void *workspace, size_t ws_bytes, void *stream) {
    return attn_common(c, q, out, lse, scale, workspace, ws_bytes, stream, nup::kModePaged, nullptr,
                       nullptr, nullptr, 0);
}

static_assert(nup::kScratchBytes == (size_t)NUP_NOALLOC_SCRATCH_BYTES, "scratch size in the header");

nup_status attn_decode_nonuniform_noalloc(nup_ctx *c, const void *q, float *out, float *lse, float scale,
                                          void *stream) {
    if (!c) return NUP_E_ARG;
    if (!c->has_device) return fail(c, NUP_E_STATE, "context has no device buffers");
    size_t need = 0;
    nup_workspace_bytes(c, 0, &need);
    if (need > nup::kScratchBytes)
        return fail(c, NUP_E_ARG,
                    "split-K partials of this context need %zu bytes; the allocation-free call holds at most "
                    "%zu (use attn_decode_nonuniform with a workspace)",
                    need, nup::kScratchBytes);
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != c->device)
        return fail(c, NUP_E_STATE, "current device %d is not the context's device %d", dev, c->device);
    void *ws = nullptr;
    const hipError_t e = nup::scratch_buffer(c->device, &ws);
    if (e != hipSuccess || !ws) return hip_fail(c, e != hipSuccess ? e : hipErrorInvalidSymbol, "scratch lookup");
    return attn_common(c, q, out, lse, scale, ws, nup::kScratchBytes, stream, nup::kModePaged, nullptr, nullptr,
                       nullptr, 0, nullptr, nullptr, /*may_time=*/false);
}

nup_status attn_decode_nonuniform_append(nup_ctx *c, const void *k_new, const void *v_new, const void *q,
                                         float *out, float *lse, float scale, void *workspace, size_t ws_bytes,
                                         void *stream) {
    if (!c) return NUP_E_ARG;
    if (!c->has_device) return fail(c, NUP_E_STATE, "context has no device buffers");
    if (!k_new || !v_new) return fail(c, NUP_E_ARG, "k_new and v_new are required");
    if (!c->committed || c->pending) return fail(c, NUP_E_STATE, "edits pending: nup_commit first");
    const bool cap_mode = capturing(static_cast<hipStream_t>(stream));
    for (int s = 0; s < c->B && !cap_mode; ++s) {
        if (!c->active[s]) continue;
        for (int h = 0; h < c->H; ++h) {
            const size_t k = (size_t)s * c->V + c->lbase() + h;
            if (c->len[k] >= c->cap[k])
                return fail(c, NUP_E_CAPACITY, "slot %d layer %d head %d is at its budget (%d tokens)", s,
                            c->layer, h, c->cap[k]);
        }
    }
    nup_status r = attn_common(c, q, out, lse, scale, workspace, ws_bytes, stream, nup::kModePaged, nullptr,
                               nullptr, nullptr, 0, k_new, v_new);
    if (r != NUP_OK || cap_mode) return r;
    for (int s = 0; s < c->B; ++s)
        if (c->active[s])
            for (int h = 0; h < c->H; ++h) c->len[(size_t)s * c->V + c->lbase() + h]++;
    return NUP_OK;
}

nup_status attn_decode_topk(nup_ctx *c, const void *q, const void *k_stage, const void *v_stage, int32_t K,
                            float *out, float *lse, float scale, void *workspace, size_t ws_bytes,
                            void *stream) {
    if (!c) return NUP_E_ARG;
    if (K <= 0 || !k_stage || !v_stage) return fail(c, NUP_E_ARG, "top-K needs K > 0 and staging buffers");
    return attn_common(c, q, out, lse, scale, workspace, ws_bytes, stream, nup::kModeStaged, k_stage,
                       v_stage, nullptr, K);
}

nup_status attn_decode_topk_paged(nup_ctx *c, const void *q, const int32_t *idx, int32_t K, float *out,
                                  float *lse, float scale, void *workspace, size_t ws_bytes, void *stream) {
    if (!c) return NUP_E_ARG;
    if (K <= 0 || !idx) return fail(c, NUP_E_ARG, "top-K needs K > 0 and an index list");
    return attn_common(c, q, out, lse, scale, workspace, ws_bytes, stream, nup::kModeIndexed, nullptr,
                       nullptr, idx, K);
}

// Selection workspace: scores [heads][max_pages*P] fp32, then the select
// kernels' histogram [heads][kSelBins], thresholds [heads][2] and per-slice
// counts [heads][kSelSplit][2].
struct SelectWs { size_t hist, ckey, cpos, sgt, thr, cnt, total; };
static SelectWs select_ws(const nup_ctx *c) {
    const size_t heads = (size_t)c->B * c->H;
    SelectWs w;
    w.hist = align_up(heads * (size_t)c->max_pages * nup::kPage * 4);
    w.ckey = w.hist + align_up(heads * nup::kSelHistStride * 4);
    w.cpos = w.ckey + align_up(heads * nup::kSelCap * 4);
    w.sgt = w.cpos + align_up(heads * nup::kSelCap * 4);
    w.thr = w.sgt + align_up(heads * nup::kSelSplit * 4);
    w.cnt = w.thr + align_up(heads * 2 * 4);
    w.total = w.cnt + align_up(heads * nup::kSelSplit * 2 * 4);
    return w;
}

nup_status nup_select_workspace_bytes(const nup_ctx *c, size_t *bytes) {
    if (!c || !bytes) return NUP_E_ARG;
    *bytes = select_ws(c).total;
    return NUP_OK;
}

nup_status kv_select_topk(nup_ctx *c, const void *q, int32_t K, int32_t window, int32_t *idx_out,
                          void *workspace, size_t ws_bytes, void *stream) {
    if (!c) return NUP_E_ARG;
    if (!c->has_device) return fail(c, NUP_E_STATE, "context has no device buffers");
    if (!c->committed || c->pending) return fail(c, NUP_E_STATE, "edits pending: nup_commit first");
    if (!q || !idx_out || !workspace) return fail(c, NUP_E_ARG, "q, idx_out and workspace are required");
    if (K <= 0 || window < 0 || window > K) return fail(c, NUP_E_ARG, "need K > 0 and 0 <= window <= K");
    size_t need = 0;
    nup_select_workspace_bytes(c, &need);
    if (ws_bytes < need) return fail(c, NUP_E_ARG, "workspace %zu bytes < %zu needed", ws_bytes, need);
    for (int s = 0; s < c->B; ++s) {
        if (!c->active[s]) continue;
        for (int h = 0; h < c->H; ++h)
            if (c->len[(size_t)s * c->V + c->lbase() + h] < K)
                return fail(c, NUP_E_ARG, "slot %d head %d retains %d < K = %d entries", s, h,
                            c->len[(size_t)s * c->V + c->lbase() + h], K);
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    nup::ScoreArgs sa{};
    sa.q = static_cast<const uint16_t *>(q);
    sa.kbase = c->kpool;
    sa.page_table = c->d_pt();
    sa.lengths = c->d_len() + c->lbase();
    sa.group_of_head = c->d_goh() + c->lbase();
    sa.slot_of_head = c->d_soh() + c->lbase();
    sa.lstride = c->V;
    sa.rows = c->inbox_i32(c->off_rows[c->layer]);
    sa.worker_start = c->inbox_i32(c->off_ws[c->layer]);
    sa.scores = static_cast<float *>(workspace);
    sa.hist = reinterpret_cast<uint32_t *>(static_cast<char *>(workspace) + select_ws(c).hist);
    sa.bmax = c->B;
    sa.hkv = c->H;
    sa.gh = c->gh;
    sa.max_pages = c->max_pages;
    sa.n_workers = c->dev_workers[c->layer];
    sa.stride = c->max_pages * nup::kPage;
    hipError_t e = nup::launch_score(sa, c->D, c->gqa, st);
    if (e != hipSuccess) return hip_fail(c, e, "score launch");
    const SelectWs sw = select_ws(c);
    nup::SelectArgs sl{};
    sl.scores = sa.scores;
    sl.hist = reinterpret_cast<uint32_t *>(static_cast<char *>(workspace) + sw.hist);
    sl.cand_key = reinterpret_cast<uint32_t *>(static_cast<char *>(workspace) + sw.ckey);
    sl.cand_pos = reinterpret_cast<int32_t *>(static_cast<char *>(workspace) + sw.cpos);
    sl.slice_gt = reinterpret_cast<int32_t *>(static_cast<char *>(workspace) + sw.sgt);
    sl.thr = reinterpret_cast<int32_t *>(static_cast<char *>(workspace) + sw.thr);
    sl.cnt = reinterpret_cast<int32_t *>(static_cast<char *>(workspace) + sw.cnt);
    sl.active = c->d_active();
    sl.lengths = c->d_len() + c->lbase();
    sl.lstride = c->V;
    sl.idx_out = idx_out;
    sl.hkv = c->H;
    sl.stride = sa.stride;
    sl.k = K;
    sl.window = window;
    e = nup::launch_select(sl, c->B * c->H, st);
    if (e != hipSuccess) return hip_fail(c, e, "select launch");
    return NUP_OK;
}

nup_status nup_centroid_workspace_bytes(const nup_ctx *c, int32_t C, size_t *bytes) {
    if (!c || !bytes || C <= 0) return NUP_E_ARG;
    *bytes = align_up((size_t)c->B * c->H * (size_t)C * 4);
    return NUP_OK;
}

nup_status kv_select_topk_centroids(nup_ctx *c, const void *q, const void *centroids, int32_t C,
                                    const int32_t *cl_start, const int32_t *cl_pos, int32_t P, int32_t K,
                                    int32_t window, int32_t *idx_out, void *workspace, size_t ws_bytes,
                                    void *stream) {
    if (!c) return NUP_E_ARG;
    if (!c->has_device) return fail(c, NUP_E_STATE, "context has no device buffers");
    if (!c->committed || c->pending) return fail(c, NUP_E_STATE, "edits pending: nup_commit first");
    if (!q || !centroids || !cl_start || !cl_pos || !idx_out || !workspace)
        return fail(c, NUP_E_ARG, "q, centroids, cluster lists, idx_out and workspace are required");
    if (C <= 0 || C > nup::kMaxClusters) return fail(c, NUP_E_ARG, "C = %d outside [1, %d]", C, nup::kMaxClusters);
    if (P < 0) return fail(c, NUP_E_ARG, "P < 0");
    if (K <= 0 || window < 0 || window > K) return fail(c, NUP_E_ARG, "need K > 0 and 0 <= window <= K");
    if ((long long)c->max_pages * c->P > nup::kMaxSelectPositions)
        return fail(c, NUP_E_ARG, "max_pages * P = %lld exceeds the %d positions the cluster select holds",
                    (long long)c->max_pages * c->P, nup::kMaxSelectPositions);
    size_t need = 0;
    nup_centroid_workspace_bytes(c, C, &need);
    if (ws_bytes < need) return fail(c, NUP_E_ARG, "workspace %zu bytes < %zu needed", ws_bytes, need);
    for (int s = 0; s < c->B; ++s) {
        if (!c->active[s]) continue;
        for (int h = 0; h < c->H; ++h)
            if (c->len[(size_t)s * c->V + c->lbase() + h] < K)
                return fail(c, NUP_E_ARG, "slot %d head %d retains %d < K = %d entries", s, h,
                            c->len[(size_t)s * c->V + c->lbase() + h], K);
    }
    nup::CentroidArgs a{};
    a.q = static_cast<const uint16_t *>(q);
    a.centroids = static_cast<const uint16_t *>(centroids);
    a.active = c->d_active();
    a.lengths = c->d_len() + c->lbase();
    a.cl_start = cl_start;
    a.cl_pos = cl_pos;
    a.cscore = static_cast<float *>(workspace);
    a.idx_out = idx_out;
    a.err = c->d_err();
    a.hkv = c->H;
    a.lstride = c->V;
    a.C = C;
    a.P = P;
    a.k = K;
    a.window = window;
    hipError_t e = nup::launch_centroid_select(a, c->D, c->gqa, c->B * c->H, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(c, e, "centroid select launch");
    return NUP_OK;
}

nup_status nup_get_page_table(const nup_ctx *c, int32_t *out) {
    if (!c || !out) return NUP_E_ARG;
    std::copy(c->pt.begin(), c->pt.end(), out);
    return NUP_OK;
}

nup_status nup_get_lengths(const nup_ctx *c, int32_t *out) {
    if (!c || !out) return NUP_E_ARG;
    for (size_t k = 0; k < c->len.size(); ++k) out[k] = c->active[k / c->V] ? c->len[k] : 0;
    return NUP_OK;
}

nup_status nup_get_groups(const nup_ctx *c, int32_t *goh, int32_t *soh) {
    if (!c) return NUP_E_ARG;
    if (goh) std::copy(c->goh.begin(), c->goh.end(), goh);
    if (soh) std::copy(c->soh.begin(), c->soh.end(), soh);
    return NUP_OK;
}

nup_status nup_get_free_list(const nup_ctx *c, int32_t *out, int32_t *n) {
    if (!c || !n) return NUP_E_ARG;
    *n = (int32_t)c->free_list.size();
    if (out) c->free_list.copy_to(out);
    return NUP_OK;
}

nup_status nup_get_refcounts(const nup_ctx *c, int32_t *out) {
    if (!c || !out) return NUP_E_ARG;
    std::copy(c->ref.begin(), c->ref.end(), out);
    return NUP_OK;
}

nup_status nup_get_runs(const nup_ctx *c, int32_t *out, int32_t max_runs, int32_t *n) {
    if (!c || !n) return NUP_E_ARG;
    std::vector<int32_t> runs;
    build_runs(const_cast<nup_ctx *>(c), runs);  // refreshes the per-row cache only
    *n = (int32_t)(runs.size() / 5);
    if (!out) return NUP_OK;
    if (*n > max_runs) return NUP_E_ARG;
    std::copy(runs.begin(), runs.end(), out);
    return NUP_OK;
}

nup_status nup_get_plan(const nup_ctx *c, int32_t *n_rows, int32_t *n_workers, int32_t *rows,
                        int32_t *worker_start, int32_t *head_row_start) {
    if (!c) return NUP_E_ARG;
    if (c->plan_dirty) replan(const_cast<nup_ctx *>(c));  // the plan of the shadow
    const nup_ctx::Plan &pl = c->plan[c->layer];
    if (n_rows) *n_rows = (int32_t)(pl.rows.size() / 4);
    if (n_workers) *n_workers = (int32_t)pl.worker_start.size() - 1;
    if (rows) std::copy(pl.rows.begin(), pl.rows.end(), rows);
    if (worker_start) std::copy(pl.worker_start.begin(), pl.worker_start.end(), worker_start);
    if (head_row_start) std::copy(pl.head_row_start.begin(), pl.head_row_start.end(), head_row_start);
    return NUP_OK;
}

nup_status nup_get_plan_head_rows(const nup_ctx *c, int32_t *head_rows) {
    if (!c || !head_rows) return NUP_E_ARG;
    if (c->plan_dirty) replan(const_cast<nup_ctx *>(c));
    const nup_ctx::Plan &pl = c->plan[c->layer];
    const int32_t n = (int32_t)(pl.rows.size() / 4);
    if (pl.head_rows.empty()) std::iota(head_rows, head_rows + n, 0);
    else std::copy(pl.head_rows.begin(), pl.head_rows.end(), head_rows);
    return NUP_OK;
}

nup_status nup_get_plan_gangs(const nup_ctx *c, int32_t *n_blocks, int32_t *gang_rows, int32_t *worker_skip) {
    if (!c) return NUP_E_ARG;
    if (c->plan_dirty) replan(const_cast<nup_ctx *>(c));
    const nup_ctx::Plan &pl = c->plan[c->layer];
    if (n_blocks) *n_blocks = (int32_t)(pl.gang_rows.size() / nup::kWavesPerBlock);
    if (gang_rows) std::copy(pl.gang_rows.begin(), pl.gang_rows.end(), gang_rows);
    if (worker_skip) {
        const size_t W = pl.worker_start.empty() ? 0 : pl.worker_start.size() - 1;
        std::fill(worker_skip, worker_skip + W, 0);
        std::copy(pl.worker_skip.begin(), pl.worker_skip.end(), worker_skip);
    }
    return NUP_OK;
}

nup_status nup_note_appends(nup_ctx *c, int32_t layer, int32_t steps) {
    if (!c) return NUP_E_ARG;
    if (layer < -1 || layer >= c->NL) return fail(c, NUP_E_ARG, "layer %d outside [-1, %d)", layer, c->NL);
    if (steps < 0) return fail(c, NUP_E_ARG, "steps must be >= 0");
    if (!c->committed || c->pending)
        return fail(c, NUP_E_STATE, "appends are reported before any edit of the next step");
    const int l0 = layer < 0 ? 0 : layer, l1 = layer < 0 ? c->NL : layer + 1;
    int full = 0;
    for (int s = 0; s < c->B; ++s) {
        if (!c->active[s]) continue;
        for (size_t k = (size_t)s * c->V + (size_t)l0 * c->H; k < (size_t)s * c->V + (size_t)l1 * c->H; ++k) {
            // the replayed kernel stops a head at its budget, as this does
            const long long n = (long long)c->len[k] + steps;
            if (n > c->cap[k]) ++full;
            c->len[k] = (int32_t)std::min<long long>(n, c->cap[k]);
        }
    }
    if (full)
        return fail(c, NUP_E_CAPACITY, "%d heads reached their budget; their extra tokens were not stored", full);
    return NUP_OK;
}

nup_status nup_set_layer(nup_ctx *c, int32_t layer) {
    if (!c) return NUP_E_ARG;
    if (layer < 0 || layer >= c->NL) return fail(c, NUP_E_ARG, "layer %d outside [0, %d)", layer, c->NL);
    c->layer = layer;
    return NUP_OK;
}

nup_status nup_set_timing(nup_ctx *c, int32_t enable) {
    if (!c) return NUP_E_ARG;
    c->timing = enable != 0;
    return NUP_OK;
}

nup_status nup_kernel_time(nup_ctx *c, double *partial_ms, int32_t *launches, int32_t reset) {
    if (!c) return NUP_E_ARG;
    for (auto &ev : c->tev) {
        hipError_t e = hipEventSynchronize(ev.second);
        if (e != hipSuccess) return hip_fail(c, e, "hipEventSynchronize");
        float ms = 0.f;
        e = hipEventElapsedTime(&ms, ev.first, ev.second);
        if (e != hipSuccess) return hip_fail(c, e, "hipEventElapsedTime");
        c->acc_ms += ms;
        c->launches++;
        (void)hipEventDestroy(ev.first);
        (void)hipEventDestroy(ev.second);
    }
    c->tev.clear();
    if (partial_ms) *partial_ms = c->acc_ms;
    if (launches) *launches = c->launches;
    if (reset) {
        c->acc_ms = 0.0;
        c->launches = 0;
    }
    return NUP_OK;
}

nup_status nup_device_errors(nup_ctx *c, void *stream, int32_t *code) {
    if (!c || !code) return NUP_E_ARG;
    if (!c->has_device) return fail(c, NUP_E_STATE, "context has no device buffers");
    hipStream_t st = static_cast<hipStream_t>(stream);
    int32_t h = 0;
    hipError_t e = hipMemcpyAsync(&h, c->d_err(), 4, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(c, e, "read device error word");
    const int32_t zero = 0;
    e = hipMemcpyAsync(c->d_err(), &zero, 4, hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(c, e, "clear device error word");
    *code = (h & 1) ? NUP_E_INDEX : (h & 2) ? NUP_E_CAPACITY : NUP_OK;
    return NUP_OK;
}

nup_status nup_probe_copy(const void *src, void *dst, size_t bytes, void *stream) {
    if (!src || !dst || bytes % 16) return NUP_E_ARG;
    hipError_t e = nup::launch_probe_copy(src, dst, bytes, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NUP_OK : NUP_E_HIP;
}

nup_status nup_probe_read(const void *src, size_t bytes, void *sink, void *stream) {
    if (!src || !sink || bytes % 16) return NUP_E_ARG;
    hipError_t e = nup::launch_probe_read(src, bytes, static_cast<uint32_t *>(sink),
                                          static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NUP_OK : NUP_E_HIP;
}

}  // extern "C"
