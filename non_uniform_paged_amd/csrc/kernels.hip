// gfx950 kernels of the non-uniform paged decode path.
//
// Data layout (see nupaged.h): K and V pools are bf16
// [num_pages][heads_per_group][16][head_dim]: a page holds 16 tokens of every
// head of one head group (Tangram, Fig 8: Head Group Page), and a head's 16
// rows are one contiguous 4 KB block at head_dim 128.
//
// Decode attention is bound by HBM bandwidth: every cached byte is read
// once and feeds GQA multiply-adds, far below the matrix-core ridge.  The
// partial kernel therefore keeps the arithmetic on the vector ALU in fp32
// (q.k with the packed bf16 dot2 instruction, whose products are exact and
// whose sum is kept in fp32), and spends its effort on keeping enough
// 16-byte loads in flight: each wave streams a page (K and V) ahead of the
// one it computes.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kernels.h"

namespace nup {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// The running maximum of a lane is only raised when a score exceeds it by
// this many powers of two, which keeps every exp2 argument at most 8 and
// skips almost all rescaling of the accumulators.
constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
// DPP controls: quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror,
// row_ror:8.
constexpr int kQuadSwap1 = 0xB1;
constexpr int kQuadSwap2 = 0x4E;
constexpr int kHalfMirror = 0x141;
constexpr int kRowRor8 = 0x128;

// Sum over the 8 lanes of an aligned group (lanes 8k .. 8k+7).
__device__ __forceinline__ float sum8(float x) {
    x += dpp<kQuadSwap1>(x);
    x += dpp<kQuadSwap2>(x);
    x += dpp<kHalfMirror>(x);
    return x;
}

// Across the 8 groups that share a lane position inside their group
// (lanes e, e+8, ..., e+56).
__device__ __forceinline__ float max_groups(float x) {
    x = fmaxf(x, dpp<kRowRor8>(x));
    x = fmaxf(x, __shfl_xor(x, 16));
    x = fmaxf(x, __shfl_xor(x, 32));
    return x;
}
__device__ __forceinline__ float sum_groups(float x) {
    x += dpp<kRowRor8>(x);
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

// ---------------------------------------------------------------------------
// Split-K partial attention.
//
// Lane layout inside a wave (64 lanes): lane = 8*tq + e.  For a 16-token
// page the lane owns tokens tq and tq+8 and, of each, the 16-byte pieces
// e and e+8 of the row (dims 8e..8e+7 and 64+8e..64+8e+7 at head_dim 128).
// Eight consecutive lanes thus read 128 contiguous bytes of one row, and a
// wave-wide load instruction covers eight rows: every load is a full
// 16-byte, fully coalesced access.  q.k is finished with three DPP adds
// across the 8 lanes of a token; the softmax state and the output
// accumulator are kept per lane (per token subset) and combined once per
// row at the end.
// ---------------------------------------------------------------------------
template <int D, int GQA, bool TOPK>
struct Partial {
    static constexpr int NH = D / 64;  // 16-byte pieces per token per lane

    float o[GQA][NH * 8];
    float m[GQA], l[GQA];

    // qs: this wave's q rows in LDS, bf16 [GQA][D]; read one row at a time
    // so that q occupies no registers across the page loop.
    __device__ __forceinline__ void compute(const uint4 (&k)[2][NH], const uint4 (&v)[2][NH],
                                            const uint4 *qs, int e, bool valid0, bool valid1,
                                            float scale_log2) {
        float sc[2][GQA];
#pragma unroll
        for (int r = 0; r < GQA; ++r) {
            uint4 qv[NH];
#pragma unroll
            for (int hh = 0; hh < NH; ++hh) qv[hh] = qs[r * (D / 8) + e + 8 * hh];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                float acc = 0.f;
#pragma unroll
                for (int hh = 0; hh < NH; ++hh) {
                    acc = dot2(qv[hh].x, k[i][hh].x, acc);
                    acc = dot2(qv[hh].y, k[i][hh].y, acc);
                    acc = dot2(qv[hh].z, k[i][hh].z, acc);
                    acc = dot2(qv[hh].w, k[i][hh].w, acc);
                }
                sc[i][r] = acc;
            }
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < GQA; ++r) sc[i][r] = sum8(sc[i][r]) * scale_log2;

#pragma unroll
        for (int r = 0; r < GQA; ++r) {
            const float s0 = valid0 ? sc[0][r] : -INFINITY;
            const float s1 = valid1 ? sc[1][r] : -INFINITY;
            const float mx = fmaxf(s0, s1);
            if (mx > m[r] + kRescaleSlack) {
                const float a = exp2f(m[r] - mx);
                m[r] = mx;
                l[r] *= a;
#pragma unroll
                for (int d = 0; d < NH * 8; ++d) o[r][d] *= a;
            }
            const float p0 = valid0 ? exp2f(s0 - m[r]) : 0.f;
            const float p1 = valid1 ? exp2f(s1 - m[r]) : 0.f;
            l[r] += p0 + p1;
#pragma unroll
            for (int hh = 0; hh < NH; ++hh) {
                const uint32_t w0[4] = {v[0][hh].x, v[0][hh].y, v[0][hh].z, v[0][hh].w};
                const uint32_t w1[4] = {v[1][hh].x, v[1][hh].y, v[1][hh].z, v[1][hh].w};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    float *od = &o[r][hh * 8 + 2 * c];
                    od[0] = fmaf(p1, bf16lo(w1[c]), fmaf(p0, bf16lo(w0[c]), od[0]));
                    od[1] = fmaf(p1, bf16hi(w1[c]), fmaf(p0, bf16hi(w0[c]), od[1]));
                }
            }
        }
    }
};

template <int D, int GQA, bool TOPK>
__global__ __launch_bounds__(256) void partial_attn_kernel(PartialArgs a) {
    using W = Partial<D, GQA, TOPK>;
    constexpr int NH = W::NH;
    const int lane = threadIdx.x & 63;
    const int w = blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (w >= a.n_workers) return;
    const int tq = lane >> 3, e = lane & 7;

    int rb, re;
    if (TOPK) {
        rb = w;
        re = w + 1;
    } else {
        rb = a.worker_start[w];
        re = a.worker_start[w + 1];
    }
    __shared__ uint4 q_lds[kWavesPerBlock][GQA * D / 8];
    uint4 *qs = q_lds[threadIdx.x >> 6];
    W st;
    for (int row = rb; row < re; ++row) {
        int sh, t0, t1;
        if (TOPK) {
            sh = row / a.topk_splits;
            t0 = (row - sh * a.topk_splits) * a.topk_chunk;
            const int L = a.active[sh / a.hkv] ? a.topk_k : 0;
            t1 = min(t0 + a.topk_chunk, L);
        } else {
            sh = a.rows[row * 4 + 0];
            t0 = a.rows[row * 4 + 1];
            t1 = min(a.rows[row * 4 + 2], a.lengths[sh]);
        }
        const int s = sh / a.hkv, h = sh - s * a.hkv;
        float *ml = a.ws_ml + (size_t)row * GQA * 2;
        if (t0 >= t1) {
            if (lane < GQA) {
                ml[lane * 2 + 0] = -INFINITY;
                ml[lane * 2 + 1] = 0.f;
            }
            continue;
        }
        // q rows of this KV head -> this wave's LDS slot (the wave's own
        // in-order LDS queue orders these writes before the reads below)
        const uint4 *qh = reinterpret_cast<const uint4 *>(
            a.q + ((size_t)s * a.hkv * GQA + (size_t)h * GQA) * D);
        __builtin_amdgcn_wave_barrier();
        for (int c = lane; c < GQA * D / 8; c += 64) qs[c] = qh[c];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int r = 0; r < GQA; ++r) {
            st.m[r] = -INFINITY;
            st.l[r] = 0.f;
#pragma unroll
            for (int d = 0; d < NH * 8; ++d) st.o[r][d] = 0.f;
        }

        const int32_t *ptrow = nullptr;
        size_t slot_off = 0;
        if (!TOPK) {
            ptrow = a.page_table +
                    ((size_t)a.group_of_head[h] * a.bmax + s) * (size_t)a.max_pages;
            slot_off = (size_t)a.slot_of_head[h] * kPage * D;
        }
        const size_t head_base = TOPK ? (size_t)sh * a.topk_k * D : 0;
        const int p0 = t0 / kPage, p1 = (t1 - 1) / kPage;  // inclusive page range

        auto page_base = [&](int pi) -> size_t {
            if (TOPK) return head_base + (size_t)pi * kPage * D;
            return (size_t)ptrow[pi] * a.gh * kPage * D + slot_off;
        };
        auto load = [&](int pi, size_t base, uint4 (&k)[2][NH], uint4 (&v)[2][NH]) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                int j = tq + 8 * i;
                j = min(pi * kPage + j, t1 - 1) - pi * kPage;  // clamp past the end
                const size_t off = base + (size_t)j * D;
                const uint4 *kp = reinterpret_cast<const uint4 *>(a.kbase + off);
                const uint4 *vp = reinterpret_cast<const uint4 *>(a.vbase + off);
#pragma unroll
                for (int hh = 0; hh < NH; ++hh) {
                    k[i][hh] = kp[e + 8 * hh];
                    v[i][hh] = vp[e + 8 * hh];
                }
            }
        };

        uint4 kA[2][NH], vA[2][NH], kB[2][NH], vB[2][NH];
        size_t baseB = 0;
        load(p0, page_base(p0), kA, vA);
        if (p0 + 1 <= p1) baseB = page_base(p0 + 1);
        for (int pi = p0; pi <= p1; pi += 2) {
            const bool hasB = pi + 1 <= p1;
            if (hasB) load(pi + 1, baseB, kB, vB);
            size_t baseA = 0;
            if (pi + 2 <= p1) baseA = page_base(pi + 2);
            st.compute(kA, vA, qs, e, pi * kPage + tq < t1, pi * kPage + tq + 8 < t1, a.scale_log2);
            if (!hasB) break;
            if (pi + 2 <= p1) load(pi + 2, baseA, kA, vA);
            if (pi + 3 <= p1) baseB = page_base(pi + 3);
            st.compute(kB, vB, qs, e, (pi + 1) * kPage + tq < t1, (pi + 1) * kPage + tq + 8 < t1,
                       a.scale_log2);
        }

        // Combine the eight token groups of the wave.
        float *wo = a.ws_o + (size_t)row * GQA * D;
#pragma unroll
        for (int r = 0; r < GQA; ++r) {
            const float mm = max_groups(st.m[r]);
            const float f = (st.m[r] == -INFINITY) ? 0.f : exp2f(st.m[r] - mm);
            const float lt = sum_groups(st.l[r] * f);
            float ot[NH * 8];
#pragma unroll
            for (int d = 0; d < NH * 8; ++d) ot[d] = sum_groups(st.o[r][d] * f);
            if (tq == r) {
#pragma unroll
                for (int hh = 0; hh < NH; ++hh) {
                    float4 *dst = reinterpret_cast<float4 *>(wo + (size_t)r * D + 8 * e + 64 * hh);
                    dst[0] = make_float4(ot[hh * 8 + 0], ot[hh * 8 + 1], ot[hh * 8 + 2], ot[hh * 8 + 3]);
                    dst[1] = make_float4(ot[hh * 8 + 4], ot[hh * 8 + 5], ot[hh * 8 + 6], ot[hh * 8 + 7]);
                }
                if (e == 0) {
                    ml[r * 2 + 0] = mm;
                    ml[r * 2 + 1] = lt;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of split-K partials: one 64-lane block per (slot, KV head).
// ---------------------------------------------------------------------------
template <int D, int GQA>
__global__ __launch_bounds__(64) void merge_kernel(MergeArgs a) {
    constexpr int NJ = D / 64;
    const int sh = blockIdx.x;
    const int lane = threadIdx.x;
    const int s = sh / a.hkv, h = sh - s * a.hkv;
    int rb, re;
    if (a.head_row_start) {
        rb = a.head_row_start[sh];
        re = a.head_row_start[sh + 1];
    } else {
        rb = sh * a.uniform_splits;
        re = rb + a.uniform_splits;
    }
    const int hq = a.hkv * GQA;
#pragma unroll
    for (int r = 0; r < GQA; ++r) {
        float M = -INFINITY;
        for (int i = rb; i < re; ++i) M = fmaxf(M, a.ws_ml[((size_t)i * GQA + r) * 2]);
        float L = 0.f, acc[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[j] = 0.f;
        if (M != -INFINITY) {
            for (int i = rb; i < re; ++i) {
                const float mi = a.ws_ml[((size_t)i * GQA + r) * 2];
                if (mi == -INFINITY) continue;
                const float wgt = exp2f(mi - M);
                L = fmaf(wgt, a.ws_ml[((size_t)i * GQA + r) * 2 + 1], L);
                const float *oi = a.ws_o + ((size_t)i * GQA + r) * D;
#pragma unroll
                for (int j = 0; j < NJ; ++j) acc[j] = fmaf(wgt, oi[lane + 64 * j], acc[j]);
            }
        }
        const size_t qr = (size_t)s * hq + (size_t)h * GQA + r;
        const float inv = (M != -INFINITY) ? 1.0f / L : 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) a.out[qr * D + lane + 64 * j] = acc[j] * inv;
        if (a.lse && lane == 0) a.lse[qr] = (M != -INFINITY) ? (M + log2f(L)) * kLn2 : -INFINITY;
    }
}

// ---------------------------------------------------------------------------
// Append: one token per active (slot, KV head).  2*(D/8) lanes per head: the
// first half copies the K row, the second the V row, 16 bytes per lane.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
    constexpr int LPR = D / 8;
    constexpr int PER = 2 * LPR;
    const int local = threadIdx.x / PER, sub = threadIdx.x % PER;
    const int sh = blockIdx.x * (256 / PER) + local;
    const bool ok = sh < a.bmax * a.hkv;
    const int s = ok ? sh / a.hkv : 0, h = ok ? sh - s * a.hkv : 0;
    const bool act = ok && a.active[s];
    int L = 0;
    if (act) {
        L = a.lengths[sh];
        const int pid = a.page_table[((size_t)a.group_of_head[h] * a.bmax + s) * a.max_pages + L / kPage];
        const size_t rowid = ((size_t)pid * a.gh + a.slot_of_head[h]) * kPage + L % kPage;
        const bool isv = sub >= LPR;
        const int c = sub - (isv ? LPR : 0);
        const uint4 *src = reinterpret_cast<const uint4 *>((isv ? a.v_new : a.k_new) + (size_t)sh * D) + c;
        uint4 *dst = reinterpret_cast<uint4 *>((isv ? a.v_pool : a.k_pool) + rowid * D) + c;
        *dst = *src;
    }
    __syncthreads();
    if (act && sub == 0) a.lengths[sh] = L + 1;
}

// ---------------------------------------------------------------------------
// Gather, index mode: staging[s][h][k] = row of logical position idx[s][h][k].
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void gather_index_kernel(GatherIndexArgs a) {
    constexpr int LPR = D / 8;
    constexpr int PER = 2 * LPR;
    const int local = threadIdx.x / PER, sub = threadIdx.x % PER;
    const long long gr = (long long)blockIdx.x * (256 / PER) + local;  // staging row
    const long long nrows = (long long)a.bmax * a.hkv * a.k;
    if (gr >= nrows) return;
    const int sh = (int)(gr / a.k), kk = (int)(gr - (long long)sh * a.k);
    const int s = sh / a.hkv, h = sh - s * a.hkv;
    if (!a.active[s]) return;
    const int t = a.idx[gr];
    const int L = a.lengths[sh];
    const bool bad = t < 0 || t >= L || (kk > 0 && a.idx[gr - 1] >= t);
    const bool isv = sub >= LPR;
    const int c = sub - (isv ? LPR : 0);
    uint4 *dst = reinterpret_cast<uint4 *>((isv ? a.v_out : a.k_out) + (size_t)gr * D) + c;
    if (bad) {
        *dst = make_uint4(0, 0, 0, 0);
        if (sub == 0) {
            if (a.phys_out) a.phys_out[gr] = -1;
            atomicOr(a.err, 1);
        }
        return;
    }
    const int pid = a.page_table[((size_t)a.group_of_head[h] * a.bmax + s) * a.max_pages + t / kPage];
    const size_t rowid = ((size_t)pid * a.gh + a.slot_of_head[h]) * kPage + t % kPage;
    *dst = reinterpret_cast<const uint4 *>((isv ? a.v_pool : a.k_pool) + rowid * D)[c];
    if (a.phys_out && sub == 0) a.phys_out[gr] = (int32_t)rowid;
}

// ---------------------------------------------------------------------------
// Gather, train mode: one block per physical page of the committed trains.
// Consecutive blocks walk physically consecutive pages of a train.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void gather_runs_kernel(GatherRunsArgs a) {
    constexpr int LPR = D / 8;
    const int b = blockIdx.x;
    // find the train holding page b (uniform binary search over prefix sums)
    int lo = 0, hi = a.n_runs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.run_prefix[mid] <= b) lo = mid; else hi = mid - 1;
    }
    const int r = lo;
    const int sg = a.runs[r * 4 + 0];
    const int s = sg / a.ng, g = sg - s * a.ng;
    const int in_run = b - a.run_prefix[r];
    const int pid = a.runs[r * 4 + 1] + in_run;
    const int lp = a.runs[r * 4 + 3] + in_run;
    const int chunks = a.gh * kPage * LPR;  // 16-byte pieces per pool per page
    for (int c = threadIdx.x; c < 2 * chunks; c += 256) {
        const bool isv = c >= chunks;
        const int cc = c - (isv ? chunks : 0);
        const int j = cc / (kPage * LPR);             // slot in the group
        const int row = (cc / LPR) % kPage;           // row in the page
        const int piece = cc % LPR;
        const int h = a.head_of_gslot[g * a.gh + j];
        const int sh = s * a.hkv + h;
        const int t = lp * kPage + row;
        if (t >= a.lengths[sh]) continue;
        const size_t rowid = ((size_t)pid * a.gh + j) * kPage + row;
        const uint4 v = reinterpret_cast<const uint4 *>((isv ? a.v_pool : a.k_pool) + rowid * D)[piece];
        const long long dr = a.row_off[sh] + t;
        reinterpret_cast<uint4 *>((isv ? a.v_out : a.k_out) + (size_t)dr * D)[piece] = v;
        if (a.phys_out && !isv && piece == 0) a.phys_out[dr] = (int32_t)rowid;
    }
}

__global__ __launch_bounds__(256) void apply_patches_kernel(int32_t *pt, const int32_t *hdr,
                                                            const int32_t *data, int max_pages) {
    const int p = blockIdx.x;
    const int row = hdr[p * 4 + 0], count = hdr[p * 4 + 1], off = hdr[p * 4 + 2];
    for (int i = threadIdx.x; i < count; i += 256) pt[(size_t)row * max_pages + i] = data[off + i];
}

__global__ __launch_bounds__(256) void probe_copy_kernel(const uint4 *src, uint4 *dst, size_t n) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

template <int D, int GQA, bool TOPK>
void *partial_fn() { return reinterpret_cast<void *>(&partial_attn_kernel<D, GQA, TOPK>); }

template <int D, bool TOPK>
void *partial_fn_gqa(int gqa) {
    switch (gqa) {
        case 1: return partial_fn<D, 1, TOPK>();
        case 2: return partial_fn<D, 2, TOPK>();
        case 4: return partial_fn<D, 4, TOPK>();
        case 5: return partial_fn<D, 5, TOPK>();
        case 8: return partial_fn<D, 8, TOPK>();
        default: return nullptr;
    }
}

void *partial_ptr(int d, int gqa, bool topk) {
    if (d == 64) return topk ? partial_fn_gqa<64, true>(gqa) : partial_fn_gqa<64, false>(gqa);
    if (d == 128) return topk ? partial_fn_gqa<128, true>(gqa) : partial_fn_gqa<128, false>(gqa);
    return nullptr;
}

template <int D>
void *merge_fn_gqa(int gqa) {
    switch (gqa) {
        case 1: return reinterpret_cast<void *>(&merge_kernel<D, 1>);
        case 2: return reinterpret_cast<void *>(&merge_kernel<D, 2>);
        case 4: return reinterpret_cast<void *>(&merge_kernel<D, 4>);
        case 5: return reinterpret_cast<void *>(&merge_kernel<D, 5>);
        case 8: return reinterpret_cast<void *>(&merge_kernel<D, 8>);
        default: return nullptr;
    }
}

// Launch a kernel whose single parameter is the struct at `arg`.
hipError_t launch_raw(void *fn, dim3 grid, dim3 block, void *arg, size_t arg_size, hipStream_t st) {
    (void)arg_size;
    void *args[] = {arg};
    return hipLaunchKernel(fn, grid, block, args, 0, st);
}

}  // namespace

bool supported_shape(int head_dim, int gqa) { return partial_ptr(head_dim, gqa, false) != nullptr; }

int partial_blocks_per_cu(int head_dim, int gqa, bool topk) {
    void *fn = partial_ptr(head_dim, gqa, topk);
    if (!fn) return 0;
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, 256, 0) != hipSuccess) return 0;
    return nb;
}

hipError_t launch_partial(const PartialArgs &a, int head_dim, int gqa, bool topk, hipStream_t st) {
    void *fn = partial_ptr(head_dim, gqa, topk);
    if (!fn) return hipErrorInvalidValue;
    if (a.n_workers <= 0) return hipSuccess;
    const unsigned blocks = (unsigned)((a.n_workers + kWavesPerBlock - 1) / kWavesPerBlock);
    PartialArgs copy = a;
    return launch_raw(fn, dim3(blocks), dim3(256), &copy, sizeof(copy), st);
}

hipError_t launch_merge(const MergeArgs &a, int head_dim, int gqa, int n_heads, hipStream_t st) {
    void *fn = head_dim == 64 ? merge_fn_gqa<64>(gqa) : head_dim == 128 ? merge_fn_gqa<128>(gqa) : nullptr;
    if (!fn) return hipErrorInvalidValue;
    if (n_heads <= 0) return hipSuccess;
    MergeArgs copy = a;
    return launch_raw(fn, dim3(n_heads), dim3(64), &copy, sizeof(copy), st);
}

hipError_t launch_append(const AppendArgs &a, int head_dim, hipStream_t st) {
    const int per = 2 * (head_dim / 8);
    const int n = a.bmax * a.hkv;
    const unsigned blocks = (unsigned)((n + 256 / per - 1) / (256 / per));
    AppendArgs copy = a;
    if (head_dim == 64) return launch_raw((void *)&append_kernel<64>, dim3(blocks), dim3(256), &copy, sizeof(copy), st);
    if (head_dim == 128) return launch_raw((void *)&append_kernel<128>, dim3(blocks), dim3(256), &copy, sizeof(copy), st);
    return hipErrorInvalidValue;
}

hipError_t launch_gather_index(const GatherIndexArgs &a, int head_dim, hipStream_t st) {
    const int per = 2 * (head_dim / 8);
    const long long n = (long long)a.bmax * a.hkv * a.k;
    const long long blocks = (n + 256 / per - 1) / (256 / per);
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    GatherIndexArgs copy = a;
    if (head_dim == 64) return launch_raw((void *)&gather_index_kernel<64>, dim3((unsigned)blocks), dim3(256), &copy, sizeof(copy), st);
    if (head_dim == 128) return launch_raw((void *)&gather_index_kernel<128>, dim3((unsigned)blocks), dim3(256), &copy, sizeof(copy), st);
    return hipErrorInvalidValue;
}

hipError_t launch_gather_runs(const GatherRunsArgs &a, int head_dim, int total_pages, hipStream_t st) {
    if (total_pages <= 0 || a.n_runs <= 0) return hipSuccess;
    GatherRunsArgs copy = a;
    if (head_dim == 64) return launch_raw((void *)&gather_runs_kernel<64>, dim3(total_pages), dim3(256), &copy, sizeof(copy), st);
    if (head_dim == 128) return launch_raw((void *)&gather_runs_kernel<128>, dim3(total_pages), dim3(256), &copy, sizeof(copy), st);
    return hipErrorInvalidValue;
}

hipError_t launch_apply_patches(int32_t *page_table, const int32_t *hdr, const int32_t *data,
                                int n_patches, int max_pages, hipStream_t st) {
    if (n_patches <= 0) return hipSuccess;
    hipLaunchKernelGGL(apply_patches_kernel, dim3(n_patches), dim3(256), 0, st, page_table, hdr, data, max_pages);
    return hipGetLastError();
}

hipError_t launch_probe_copy(const void *src, void *dst, size_t bytes, hipStream_t st) {
    const size_t n = bytes / 16;
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 256 * 64) blocks = 256 * 64;
    hipLaunchKernelGGL(probe_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                       static_cast<const uint4 *>(src), static_cast<uint4 *>(dst), n);
    return hipGetLastError();
}

}  // namespace nup
