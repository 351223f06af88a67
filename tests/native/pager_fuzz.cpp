// Random Reserve / Alias / Trim / plan / train sequences through the C ABI on a
// host-only context, for the sanitizer build.  Prints "ok" and the number of
// operations; any sanitizer report aborts with a non-zero status.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "../../include/nupaged.h"

int main(int argc, char **argv) {
    const unsigned seed = argc > 1 ? (unsigned)atoi(argv[1]) : 1u;
    std::mt19937 rng(seed);
    long ops = 0, aliased = 0;
    for (int trial = 0; trial < 40; ++trial) {
        const int Hl = 1 << (rng() % 4);              // 1, 2, 4, 8 KV heads per layer
        const int NL = 1 + rng() % 3;                 // layers sharing the pager
        const int H = NL * Hl;                        // the pager's heads
        const int ng = 1 << (rng() % 4);
        if (H % ng) continue;
        nup_config c{};
        c.num_kv_heads = Hl;
        c.num_layers = NL;
        c.num_q_heads = Hl * (int[]){1, 2, 4, 5, 8}[rng() % 5];
        c.head_dim = rng() % 2 ? 128 : 64;
        c.page_size = 16;
        c.num_groups = ng;
        c.max_batch = 1 + rng() % 24;
        c.num_pages = 1 + rng() % 400;
        c.max_pages = 1 + rng() % 40;
        c.num_workers = 1 + rng() % 300;
        c.plan_mode = rng() % 4 == 0 ? NUP_PLAN_UNIFORM : NUP_PLAN_BALANCED;
        c.uniform_splits = rng() % 5;
        std::vector<int32_t> perm(c.num_pages);
        for (int i = 0; i < c.num_pages; ++i) perm[i] = i;
        std::shuffle(perm.begin(), perm.end(), rng);
        c.free_list_init = rng() % 2 ? perm.data() : nullptr;
        nup_ctx *ctx = nullptr;
        if (nup_create(&c, &ctx) != NUP_OK) return 2;
        std::vector<int32_t> pt((size_t)ng * c.max_batch * c.max_pages), fl(c.num_pages);
        std::vector<int32_t> runs((size_t)5 * c.num_pages + 5);
        std::vector<char> live(c.max_batch, 0);  // tracked from the return codes
        for (int step = 0; step < 60; ++step, ++ops) {
            const int n = 1 + rng() % 4;
            std::vector<int32_t> slots(n), cap((size_t)n * H), len((size_t)n * H);
            for (int i = 0; i < n; ++i) slots[i] = rng() % (c.max_batch + 1) - (rng() % 16 == 0);  // some invalid
            for (auto &x : cap) x = rng() % (c.max_pages * 16 + 2);
            for (size_t i = 0; i < len.size(); ++i) len[i] = cap[i] ? rng() % (cap[i] + 1) : 0;
            const int op = rng() % 3;
            if (op == 0) {
                if (kv_alloc_groups(ctx, n, slots.data(), cap.data(), rng() % 2 ? len.data() : nullptr,
                                    nullptr) == NUP_OK)
                    for (int32_t s : slots) live[s] = 1;
            } else if (op == 1) {
                std::vector<int32_t> idle, busy;
                for (int s = 0; s < c.max_batch; ++s) (live[s] ? busy : idle).push_back(s);
                if (!idle.empty() && !busy.empty() && rng() % 4) {
                    std::shuffle(idle.begin(), idle.end(), rng);
                    slots.assign(idle.begin(), idle.begin() + std::min<size_t>(n, idle.size()));
                }
                // Alias: sources and shares mostly within what the lengths allow
                std::vector<int32_t> src(n), share((size_t)n * ng), lens(c.max_batch * H);
                nup_get_lengths(ctx, lens.data());
                for (int i = 0; i < n; ++i)
                    src[i] = !busy.empty() && rng() % 4 ? busy[rng() % busy.size()]
                                                        : (int32_t)(rng() % (c.max_batch + 1)) - (rng() % 16 == 0);
                for (int i = 0; i < n; ++i)
                    for (int g = 0; g < ng; ++g) {
                        int most = 1 << 30;
                        const int s = src[i] >= 0 && src[i] < c.max_batch ? src[i] : 0;
                        for (int h = g * (H / ng); h < (g + 1) * (H / ng); ++h)
                            most = std::min(most, lens[(size_t)s * H + h] / 16);
                        share[(size_t)i * ng + g] = rng() % (most + 2) - (rng() % 32 == 0);
                        for (int h = g * (H / ng); h < (g + 1) * (H / ng); ++h) {
                            const int lo = 16 * std::max(0, share[(size_t)i * ng + g]);
                            const int room = std::max(0, c.max_pages * 16 - lo);
                            cap[(size_t)i * H + h] = lo + rng() % (room + 1) + (rng() % 32 == 0);
                            len[(size_t)i * H + h] = lo + rng() % (cap[(size_t)i * H + h] - lo + 1);
                        }
                    }
                if (kv_alias(ctx, (int)slots.size(), slots.data(), src.data(), share.data(), cap.data(),
                             len.data()) == NUP_OK) {
                    ++aliased;
                    for (int32_t s : slots) live[s] = 1;
                }
            } else {
                if (kv_free_seqs(ctx, n, slots.data()) == NUP_OK)
                    for (int32_t s : slots) live[s] = 0;
            }
            int32_t nr = 0, nw = 0, nruns = 0, nfree = 0;
            nup_set_layer(ctx, (int32_t)(rng() % (NL + 1)) - (rng() % 16 == 0));   // sometimes invalid
            nup_note_appends(ctx, (int32_t)(rng() % (NL + 2)) - 1, (int32_t)(rng() % 40) - (rng() % 16 == 0));
            nup_get_plan(ctx, &nr, &nw, nullptr, nullptr, nullptr);
            std::vector<int32_t> rows((size_t)4 * nr + 4), ws(nw + 1), hrs((size_t)c.max_batch * Hl + 1);
            nup_get_plan(ctx, nullptr, nullptr, rows.data(), ws.data(), hrs.data());
            nup_get_runs(ctx, runs.data(), c.num_pages + 1, &nruns);
            nup_get_page_table(ctx, pt.data());
            nup_get_free_list(ctx, fl.data(), &nfree);
            nup_get_refcounts(ctx, fl.data());
            size_t wsb = 0;
            nup_workspace_bytes(ctx, rng() % 3 ? 0 : 1 + rng() % 3000, &wsb);
        }
        nup_destroy(ctx);
    }
    printf("ok %ld ops, %ld aliases\n", ops, aliased);
    return 0;
}
