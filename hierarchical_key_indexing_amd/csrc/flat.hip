// Flat search over the leaves of the cluster tree (gfx950).
//
// Instead of descending the tree, the query is compared against every cluster
// centroid ("Latent sparse attention", bdtechtalks.com, section "How latent
// sparse attention works": flat search against hierarchical search).  The
// clusters are the tree's leaves: every non-empty leaf is scored, the leaves
// are visited in (score desc, id asc) order and the keys are retrieved exactly
// as in the top-down selection (retrieval range, k, sinks and window).
//
// Five kernels per batch of rows; a leaf's key is the 64-bit (orderable
// score, ~leaf id), so keys are distinct and descend in visiting order:
//   k_flat_latent    u = fl32(fl32(mean of the group's query heads) . W_g) per
//                    (row, KV head);
//   k_flat_score     1024 leaves x up to 64 rows of one KV head per workgroup:
//                    a leaf's centroid row is loaded once into registers and
//                    scored against every row's u (double accumulation in
//                    ascending index order, four rows at a time, u read
//                    widened through scalar loads), and its
//                    members in each row's retrieval range are counted; writes
//                    the score and min(count, k) of every (row, leaf), and the
//                    keys of every S-th leaf as a sample;
//   k_flat_threshold one workgroup per (row, KV head): sorts the sample and
//                    takes as threshold T the key where the sample's weight
//                    reaches 8k / S, an estimate of where the full weight
//                    reaches 8k;
//   k_flat_collect   4096 leaves of one (row, KV head) per workgroup: every key
//                    >= T goes to the row's list, with its weight;
//   k_flat_finish    one workgroup per (row, KV head): when the list weighs at
//                    least k (so the k-th retrieved key is in it) and fits, it
//                    is sorted and filled in order; otherwise an exact weighted
//                    radix selection (up to 11 bits a round) over all leaves
//                    narrows the boundary to a bucket that fits, and those keys
//                    are sorted and filled.
#include <algorithm>
#include <atomic>

#include "common.h"
#include "internal.h"

namespace lsa {

namespace {

constexpr int kFlatLeaves = 1024;   // leaves per scoring workgroup
constexpr int kFlatRows = 64;       // rows per scoring workgroup
constexpr int kFlatList = 16384;    // keys collected per (row, KV head) in LDS
constexpr int kFlatBins = 2048;     // radix digits of up to 11 bits
constexpr int64_t kFlatBatch = 512; // rows per batch the workspace query sizes for
constexpr int kSampleMax = 1024;    // sampled keys per (row, KV head)
constexpr int kCollect = 4096;      // leaves per collecting workgroup

struct FlatArgs {
    const void *Q;              // the batch's first row
    int h_q, h_kv, d, r;
    int64_t mb;                 // rows in the batch
    const int32_t *q_pos;       // the batch's positions
    int64_t n, nleaf;
    const float *C;             // leaf centroids [h_kv][nleaf][r]
    const int32_t *cnt;         // leaf member counts [h_kv][nleaf]
    const int32_t *leaf_off;    // [h_kv][nleaf + 1]
    const int32_t *perm;        // [h_kv][n]
    const float *W;
    int k, n_sink, window, row;
    float *U;                   // [mb][h_kv][r]
    double *Ud;                 // [mb][h_kv][r]: U widened (read by the scoring through scalar loads)
    uint32_t *sc;               // [mb][h_kv][nleaf] orderable scores
    uint16_t *wt;               // [mb][h_kv][nleaf] min(members in range, k); 0: not a candidate
    int64_t S;                  // sample stride (0: no sample, every candidate is collected)
    int ns;                     // sampled leaves (0, S, 2S, ...)
    uint64_t *smp;              // [mb][h_kv][kSampleMax] sampled keys (0: not a candidate)
    uint64_t *thr;              // [mb][h_kv] threshold key T
    int32_t *lcnt, *lwt;        // [mb][h_kv] collected keys and their weight
    int32_t *fail;              // [mb][h_kv] 1: the list does not decide the row (exact selection)
    int2 *fl;                   // [h_kv][nleaf] first and last member of each leaf (0, 0: empty)
    uint64_t *lst;              // [mb][h_kv][kFlatList] collected keys
    int32_t *sel, *sel_count;   // the batch's rows
    float *sel_cutoff;
};

// W_g is staged in LDS 64 input rows (16 KB) at a time; the sum over the
// input dimension continues in order across them.
template <typename T>
__global__ __launch_bounds__(256) void k_flat_latent(FlatArgs A) {
    __shared__ float qbar_s[256];
    __shared__ __attribute__((aligned(16))) float w_s[64 * 64];
    const int64_t i = blockIdx.x;
    const int g = blockIdx.y;
    const int G = A.h_q / A.h_kv, d = A.d, r = A.r;
    const T *Q = (const T *)A.Q;
    for (int t = threadIdx.x; t < d; t += blockDim.x) {
        double s = 0.0;
        for (int h = 0; h < G; ++h) s = s + (double)to_float(Q[((size_t)i * A.h_q + (size_t)g * G + h) * d + t]);
        qbar_s[t] = (float)(s / (double)G);
    }
    const float *Wg = A.W + (size_t)g * d * r;
    double s = 0.0;
    for (int t0 = 0; t0 < d; t0 += 64) {
        const int nt = min(64, d - t0);
        if (((nt * r) & 3) == 0 && (((size_t)g * d * r + (size_t)t0 * r) & 3) == 0) g2s_rows<4>(w_s, nt * r, Wg + (size_t)t0 * r, nt * r, nt * r);
        else for (int e = threadIdx.x; e < nt * r; e += blockDim.x) w_s[e] = Wg[(size_t)t0 * r + e];
        __syncthreads();
        if ((int)threadIdx.x < r)
            for (int t = 0; t < nt; ++t) s = fma((double)qbar_s[t0 + t], (double)w_s[t * r + threadIdx.x], s);
        __syncthreads();
    }
    if ((int)threadIdx.x < r) {
        A.U[((size_t)i * A.h_kv + g) * r + threadIdx.x] = (float)s;
        A.Ud[((size_t)i * A.h_kv + g) * r + threadIdx.x] = (double)(float)s;
    }
}

// u . c in double, ascending index (u from LDS, 64-float padded; c in registers)
template <int RC>
LSA_DEV double dot_row(const float *u, const float (&c)[64], int r) {
    double s = 0.0;
    if constexpr (RC == 64) {
        const f4_t *u4 = reinterpret_cast<const f4_t *>(u);
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            const f4_t a = u4[x];
            s = fma((double)a.x, (double)c[4 * x + 0], s);
            s = fma((double)a.y, (double)c[4 * x + 1], s);
            s = fma((double)a.z, (double)c[4 * x + 2], s);
            s = fma((double)a.w, (double)c[4 * x + 3], s);
        }
    } else {
#pragma unroll
        for (int x = 0; x < 64; ++x)
            if (x < r) s = fma((double)u[x], (double)c[x], s);
    }
    return s;
}

// u . c for four rows at once, u read from memory through uniform addresses
// (scalar loads: every lane uses the same value, as one operand of the fp64
// FMA), c in registers widened once per step: four independent chains, each
// in ascending index order.
typedef __attribute__((address_space(4))) const double const_f64;   // read-only, scalar-loadable

LSA_DEV const_f64 *as_const(const double *p) { return (const_f64 *)(uintptr_t)p; }

LSA_DEV void dot4_uniform(const_f64 *u0, const_f64 *u1, const_f64 *u2, const_f64 *u3, const float (&c)[64],
                          double (&s)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) s[q] = 0.0;
#pragma unroll
    for (int x0 = 0; x0 < 64; x0 += 8) {
#pragma unroll
        for (int x = x0; x < x0 + 8; ++x) {
            const double cx = (double)c[x];
            s[0] = fma(u0[x], cx, s[0]);
            s[1] = fma(u1[x], cx, s[1]);
            s[2] = fma(u2[x], cx, s[2]);
            s[3] = fma(u3[x], cx, s[3]);
        }
        asm volatile("" : "+v"(s[0]), "+v"(s[1]), "+v"(s[2]), "+v"(s[3]));
    }
}

// members of a leaf (ascending, pm[0..len), first and last given) in [rlo, rhi]
LSA_DEV int members_in(const int32_t *pm, int len, int32_t first, int32_t last, int32_t rlo, int32_t rhi) {
    if (first >= rlo && last <= rhi) return len;
    if (last < rlo || first > rhi) return 0;
    return max(0, count_le(pm, len, rhi) - count_le(pm, len, rlo - 1));
}

template <int RC>
__global__ __launch_bounds__(256, 2) void k_flat_score(FlatArgs A) {
    // r = 64: u read widened from memory (A.Ud); otherwise staged as float in LDS
    constexpr bool kWide = RC == 64;
    __shared__ __attribute__((aligned(16))) float u_s[kWide ? 4 : kFlatRows * 64];
    __shared__ int32_t rlo_s[kFlatRows], rhi_s[kFlatRows];
    const int64_t v0 = (int64_t)blockIdx.x * kFlatLeaves;
    const int64_t i0 = (int64_t)blockIdx.y * kFlatRows;
    const int g = blockIdx.z;
    const int r = RC > 0 ? RC : A.r;
    const int nr = (int)min<int64_t>(kFlatRows, A.mb - i0);
    if constexpr (!kWide) {
        for (int e = threadIdx.x; e < nr * r; e += blockDim.x)
            u_s[(e / r) * 64 + e % r] = A.U[((size_t)(i0 + e / r) * A.h_kv + g) * r + e % r];
    }
    if ((int)threadIdx.x < nr) {
        const AttnSet as = attn_set(A.q_pos[i0 + threadIdx.x], A.n, A.n_sink, A.window);
        rlo_s[threadIdx.x] = as.rlo;
        rhi_s[threadIdx.x] = as.rhi;
    }
    __syncthreads();
    const float *Cg = A.C + (size_t)g * A.nleaf * r;
    const int32_t *cn = A.cnt + (size_t)g * A.nleaf;
    const int32_t *lo = A.leaf_off + (size_t)g * (A.nleaf + 1);
    const int32_t *pm = A.perm + (size_t)g * A.n;
    const size_t rs = (size_t)A.h_kv * A.nleaf;              // stride between rows
#pragma unroll 1
    for (int j = 0; j < kFlatLeaves / 256; ++j) {
        const int64_t v = v0 + j * 256 + threadIdx.x;
        if (v >= A.nleaf) break;
        const size_t o = ((size_t)i0 * A.h_kv + g) * A.nleaf + v;
        const int c = cn[v];
        const bool sampled = A.S > 0 && v % A.S == 0;
        uint64_t *sp = A.smp + ((size_t)i0 * A.h_kv + g) * kSampleMax + (sampled ? v / A.S : 0);
        const size_t ss = (size_t)A.h_kv * kSampleMax;           // sample stride between rows
        if (c <= 0) {
            for (int rr = 0; rr < nr; ++rr) {
                A.wt[o + rr * rs] = 0;
                if (sampled) sp[rr * ss] = 0ull;
            }
            continue;
        }
        const int32_t a0 = lo[v], a1 = lo[v + 1];
        const int32_t first = pm[a0], last = pm[a1 - 1];
        if constexpr (kWide) {
            float cw[64];
            const f4_t *c4 = reinterpret_cast<const f4_t *>(Cg + (size_t)v * 64);
#pragma unroll
            for (int x = 0; x < 16; ++x) {
                const f4_t t = c4[x];
                cw[4 * x] = t.x; cw[4 * x + 1] = t.y; cw[4 * x + 2] = t.z; cw[4 * x + 3] = t.w;
            }
#pragma unroll 1
            for (int rr = 0; rr < nr; rr += 4) {
                // (the row stays float and is widened at each use: widened once
                // it would take 128 registers and cost occupancy)
#pragma unroll
                for (int x = 0; x < 64; ++x) asm volatile("" : "+v"(cw[x]));
                int eq[4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    eq[q] = rr + q < nr ? members_in(pm + a0, a1 - a0, first, last, rlo_s[rr + q], rhi_s[rr + q]) : 0;
                double sq[4];
                const double *ub = A.Ud + ((size_t)i0 * A.h_kv + g) * 64;
                const size_t us = (size_t)A.h_kv * 64;       // between rows (rows past nr repeat the last)
                dot4_uniform(as_const(ub + (size_t)min(rr, nr - 1) * us), as_const(ub + (size_t)min(rr + 1, nr - 1) * us),
                             as_const(ub + (size_t)min(rr + 2, nr - 1) * us),
                             as_const(ub + (size_t)min(rr + 3, nr - 1) * us), cw, sq);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (rr + q < nr) {
                        const int e = eq[q];
                        const uint32_t oq = e > 0 ? orderable((float)sq[q]) : 0u;
                        A.sc[o + (rr + q) * rs] = oq;
                        A.wt[o + (rr + q) * rs] = (uint16_t)min(e, A.k);
                        if (sampled) sp[(rr + q) * ss] = e > 0 ? ((uint64_t)oq << 32) | (uint64_t)(~(uint32_t)v) : 0ull;
                    }
                }
            }
            continue;
        }
        float cr[64];
        if constexpr (RC == 64) {
            const f4_t *c4 = reinterpret_cast<const f4_t *>(Cg + (size_t)v * 64);
#pragma unroll
            for (int x = 0; x < 16; ++x) {
                const f4_t t = c4[x];
                cr[4 * x] = t.x; cr[4 * x + 1] = t.y; cr[4 * x + 2] = t.z; cr[4 * x + 3] = t.w;
            }
        } else {
#pragma unroll
            for (int x = 0; x < 64; ++x) cr[x] = (x < r) ? Cg[(size_t)v * r + x] : 0.0f;
        }
        for (int rr = 0; rr < nr; rr += 2) {
            const bool two = rr + 1 < nr;
            const int e0 = members_in(pm + a0, a1 - a0, first, last, rlo_s[rr], rhi_s[rr]);
            const int e1 = two ? members_in(pm + a0, a1 - a0, first, last, rlo_s[rr + 1], rhi_s[rr + 1]) : 0;
            // two independent accumulation chains
            const double s0 = dot_row<RC>(u_s + rr * 64, cr, r);
            const double s1 = two ? dot_row<RC>(u_s + (rr + 1) * 64, cr, r) : 0.0;
            const uint32_t o0 = e0 > 0 ? orderable((float)s0) : 0u, o1 = e1 > 0 ? orderable((float)s1) : 0u;
            A.sc[o + rr * rs] = o0;
            A.wt[o + rr * rs] = (uint16_t)min(e0, A.k);
            if (sampled) sp[rr * ss] = e0 > 0 ? ((uint64_t)o0 << 32) | (uint64_t)(~(uint32_t)v) : 0ull;
            if (two) {
                A.sc[o + (rr + 1) * rs] = o1;
                A.wt[o + (rr + 1) * rs] = (uint16_t)min(e1, A.k);
                if (sampled) sp[(rr + 1) * ss] = e1 > 0 ? ((uint64_t)o1 << 32) | (uint64_t)(~(uint32_t)v) : 0ull;
            }
        }
    }
}

// r = 64 and at least kFlatMfmaRows rows: the scores from the fp64 matrix
// cores, in three passes that write no full (row, leaf) table:
//   MODE 1  the sample: leaves 0, S, 2S, ... (the sample index is the leaf
//           space here), their keys to the sample and weights to the table;
//   MODE 2  every leaf: the keys at or above the row's threshold T go to the
//           row's list (through 32-key segments per row in LDS, one global
//           reservation per row and workgroup), their weights to the table
//           and to the row's list weight;
//   MODE 3  every leaf, for the rows whose list does not decide them only:
//           every score and weight to the table (the exact selection's input).
// Wave w takes rows 16 w .. 16 w + 15 of the tile (the product's rows: u
// widened once) against the workgroup's leaves, 16 at a time (the columns:
// lane (k, c) leaf c).  A block's 16 leaf rows are staged once for the
// workgroup in LDS, widened and in operand order, and the next block's are
// loaded while it is multiplied.  Lane (k, c) then owns rows k + 4 e
// against leaf c.
constexpr int kFlatMfmaRows = 16;
constexpr int kFlatSeg = 32;        // list keys per row staged in LDS by a collecting workgroup

template <int MODE>
__global__ __launch_bounds__(256) void k_flat_score_mfma(FlatArgs A) {
    constexpr int SR = MODE == 2 ? kFlatRows : 1;
    constexpr int LPW = MODE == 1 ? 64 : kFlatLeaves;        // leaves per workgroup
    __shared__ int32_t rlo_s[kFlatRows], rhi_s[kFlatRows];
    __shared__ uint64_t thr_s[SR];
    __shared__ int cnt_s[SR], wsum_s[SR];
    __shared__ uint64_t seg_s[SR][MODE == 2 ? kFlatSeg : 1];
    __shared__ int fail_s[MODE == 3 ? kFlatRows : 1];
    __shared__ int any_s;
    // a step of two 16-leaf blocks, twice: their rows widened in operand
    // order (dim 4 blk + k of leaf c of block h at [h][blk][k][c]) and member
    // count, first offset, first and last member
    __shared__ double bs[2][2][16][4][16];
    __shared__ int4 meta_s[2][32];
    const int64_t v0 = (int64_t)blockIdx.x * LPW;
    const int64_t i0 = (int64_t)blockIdx.y * kFlatRows;
    const int g = blockIdx.z;
    const int tid = threadIdx.x;
    const int nr = (int)min<int64_t>(kFlatRows, A.mb - i0);
    if (tid == 0) any_s = 0;
    __syncthreads();
    if (tid < nr) {
        const AttnSet as = attn_set(A.q_pos[i0 + tid], A.n, A.n_sink, A.window);
        rlo_s[tid] = as.rlo;
        rhi_s[tid] = as.rhi;
        const int64_t gi = (i0 + tid) * A.h_kv + g;
        if constexpr (MODE == 2) { thr_s[tid] = A.thr[gi]; cnt_s[tid] = 0; wsum_s[tid] = 0; }
        if constexpr (MODE == 3) {
            fail_s[tid] = A.fail[gi];
            if (fail_s[tid]) any_s = 1;
        }
    }
    __syncthreads();
    if (MODE == 3 && !any_s) return;                         // (uniform in the workgroup)
    const int wv = tid / kWave, lane = lane_id();
    const int col = lane & 15, kk = lane >> 4;
    const int rb = 16 * wv;                                  // the wave's first row in the tile
    const bool wave_on = rb < nr;                            // (uniform in the wave)
    // the workgroup's leaf range; in the sample pass leaf x stands for leaf x S
    const int64_t span = MODE == 1 ? (int64_t)A.ns : A.nleaf;
    const int64_t vend = min<int64_t>(v0 + LPW, span);
    const float *Cg = A.C + (size_t)g * A.nleaf * 64;
    const int32_t *lo = A.leaf_off + (size_t)g * (A.nleaf + 1);
    const int32_t *pm = A.perm + (size_t)g * A.n;
    const int2 *fl = A.fl + (size_t)g * A.nleaf;
    // staging: thread t loads dims 4 (t / 16) .. + 3 of leaf t % 16 of both
    // blocks (a half-wave's stores: consecutive doubles), threads below 32
    // also leaf t's member range (clamped leaves: in bounds)
    const int sc_leaf = tid % 16, sq = tid / 16;
    auto leaf_of = [&](int64_t x) -> int64_t {
        const int64_t xc = min<int64_t>(x, span - 1);
        return MODE == 1 ? xc * A.S : xc;
    };
    struct Stage { f4_t v[2]; int4 meta; };
    auto stage_load = [&](Stage &st, int64_t vb) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t v = leaf_of(vb + 16 * h + sc_leaf);
            st.v[h] = *reinterpret_cast<const f4_t *>(Cg + (size_t)v * 64 + 4 * sq);
        }
        if (tid < 32) {
            const int64_t vm = leaf_of(vb + tid);
            const int2 f = fl[vm];
            const int32_t a0 = lo[vm];
            st.meta = int4{lo[vm + 1] - a0, a0, f.x, f.y};
        }
    };
    auto stage_store = [&](int p, const Stage &st) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            bs[p][h][sq][0][sc_leaf] = (double)st.v[h].x;
            bs[p][h][sq][1][sc_leaf] = (double)st.v[h].y;
            bs[p][h][sq][2][sc_leaf] = (double)st.v[h].z;
            bs[p][h][sq][3][sc_leaf] = (double)st.v[h].w;
        }
        if (tid < 32) meta_s[p][tid] = st.meta;
    };
    double ua[16];
    int rlo[4], rhi[4];
    uint64_t thr[4] = {0ull, 0ull, 0ull, 0ull};
    if (wave_on) {
        f4_t t[4];
        load_row_mfma(A.U + ((size_t)(i0 + min(rb + col, nr - 1)) * A.h_kv + g) * 64, kk, t);
        widen_row_mfma(t, ua);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int rr = min(rb + kk + 4 * e, nr - 1);
            rlo[e] = rlo_s[rr];
            rhi[e] = rhi_s[rr];
            if constexpr (MODE == 2) thr[e] = thr_s[rr];
        }
    }
    // the step of 32 leaves at vb, from buffer p
    auto compute_step = [&](int64_t vb, int p) {
        if (!wave_on) return;
        // two independent chains (one a block), each over the dims in order
        d4_t acc2[2] = {{0.0, 0.0, 0.0, 0.0}, {0.0, 0.0, 0.0, 0.0}};
#pragma unroll
        for (int blk = 0; blk < 16; ++blk)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                acc2[h] = __builtin_amdgcn_mfma_f64_16x16x4f64(ua[blk], bs[p][h][blk][kk][col], acc2[h], 0, 0, 0);
        if constexpr (MODE == 2) {
            // which of the lane's eight keys reach their row's threshold (a
            // bit each), then rounds that take one hit per lane, every lane
            // with a hit together: a round per hit of the busiest lane rather
            // than a branch per (block, element) with any hit in the wave
            uint32_t ok[8];
            uint32_t hits = 0;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int64_t x = vb + 16 * h + col;
                const int c = meta_s[p][16 * h + col].x;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    ok[4 * h + e] = orderable((float)acc2[h][e]);
                    const uint64_t key = ((uint64_t)ok[4 * h + e] << 32) | (uint64_t)(~(uint32_t)x);
                    if (x < vend && rb + kk + 4 * e < nr && c > 0 && key >= thr[e]) hits |= 1u << (4 * h + e);
                }
            }
            while (__ballot(hits != 0)) {
                if (hits != 0) {
                    const int bi = __builtin_ctz(hits);
                    hits &= hits - 1;
                    const int h = bi >> 2, e = bi & 3;
                    uint32_t o32 = ok[0];
#pragma unroll
                    for (int t = 1; t < 8; ++t) o32 = bi == t ? ok[t] : o32;
                    const int rr = rb + kk + 4 * e;
                    const int64_t x = vb + 16 * h + col;
                    const int4 mt = meta_s[p][16 * h + col];     // member count, first offset, first, last
                    const int eq = members_in(pm + mt.y, mt.x, mt.z, mt.w, rlo_s[rr], rhi_s[rr]);
                    if (eq > 0) {
                        const int64_t gi = (i0 + rr) * A.h_kv + g;
                        const int w = min(eq, A.k);
                        A.wt[(size_t)gi * A.nleaf + x] = (uint16_t)w;
                        atomicAdd(&wsum_s[rr], w);
                        const uint64_t key = ((uint64_t)o32 << 32) | (uint64_t)(~(uint32_t)x);
                        const int pos = atomicAdd(&cnt_s[rr], 1);
                        if (pos < kFlatSeg) {
                            seg_s[rr][pos] = key;
                        } else {
                            const int gp = atomicAdd(A.lcnt + gi, 1);
                            if (gp < kFlatList) A.lst[(size_t)gi * kFlatList + gp] = key;
                        }
                    }
                }
            }
            return;
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const d4_t acc = acc2[h];
            const int64_t x = vb + 16 * h + col, v = MODE == 1 ? x * A.S : x;
            const int4 mt = meta_s[p][16 * h + col];         // member count, first offset, first, last
            const int c = mt.x, a0 = mt.y;
            const int32_t first = mt.z, last = mt.w;
            if (x >= vend) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int rr = rb + kk + 4 * e;
                if (rr >= nr) continue;
                if (MODE == 3 && !fail_s[rr]) continue;
                const int64_t gi = (i0 + rr) * A.h_kv + g;
                const size_t o = (size_t)gi * A.nleaf + v;
                const int eq = c > 0 ? members_in(pm + a0, c, first, last, rlo[e], rhi[e]) : 0;
                const uint32_t oq = eq > 0 ? orderable((float)acc[e]) : 0u;
                if constexpr (MODE == 1) {
                    A.wt[o] = (uint16_t)min(eq, A.k);
                    A.smp[(size_t)gi * kSampleMax + x] =
                        eq > 0 ? ((uint64_t)oq << 32) | (uint64_t)(~(uint32_t)v) : 0ull;
                } else {
                    A.sc[o] = oq;
                    A.wt[o] = (uint16_t)min(eq, A.k);
                }
            }
        }
    };
    // steps two at a time: the loads of a step are issued two steps ahead
    // and stored to LDS at the end of the step before it
    Stage s0 = {}, s1 = {};
    stage_load(s0, v0);
    stage_store(0, s0);
    __syncthreads();
    if (v0 + 32 < vend) stage_load(s1, v0 + 32);
#pragma unroll 1
    for (int64_t vb = v0; vb < vend; vb += 64) {
        if (vb + 64 < vend) stage_load(s0, vb + 64);
        compute_step(vb, 0);
        if (vb + 32 < vend) stage_store(1, s1);
        __syncthreads();
        if (vb + 32 >= vend) break;
        if (vb + 96 < vend) stage_load(s1, vb + 96);
        compute_step(vb + 32, 1);
        if (vb + 64 < vend) stage_store(0, s0);
        __syncthreads();
    }
    if constexpr (MODE == 2) {
        // every row's segment into its list (one reservation) and its weight
        __syncthreads();
        if (tid < nr) {
            const int64_t gi = (i0 + tid) * A.h_kv + g;
            const int nseg = min(cnt_s[tid], kFlatSeg);
            if (nseg > 0) {
                const int base = atomicAdd(A.lcnt + gi, nseg);
                for (int e = 0; e < nseg; ++e)
                    if (base + e < kFlatList) A.lst[(size_t)gi * kFlatList + base + e] = seg_s[tid][e];
            }
            if (wsum_s[tid] > 0) atomicAdd(A.lwt + gi, wsum_s[tid]);
        }
    }
}

// Whether a row's list decides it: the list holds every key >= T, so it
// holds the k-th retrieved key when it weighs >= k or holds every candidate
// (T = 1), provided it did not overflow.
LSA_DEV bool list_decides(const FlatArgs &A, int64_t gi) {
    return A.lcnt[gi] <= kFlatList && (A.lwt[gi] >= A.k || A.thr[gi] == 1ull);
}

// Every leaf's first and last member (ascending lists), for the scoring's
// retrieval-range counts.
__global__ __launch_bounds__(256) void k_flat_bounds(FlatArgs A) {
    const int64_t tot = (int64_t)A.h_kv * A.nleaf;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < tot; e += (int64_t)gridDim.x * blockDim.x) {
        const int g = (int)(e / A.nleaf);
        const int64_t v = e % A.nleaf;
        const int32_t *lo = A.leaf_off + (size_t)g * (A.nleaf + 1);
        const int32_t *pm = A.perm + (size_t)g * A.n;
        const int32_t a0 = lo[v], a1 = lo[v + 1];
        A.fl[e] = a1 > a0 ? int2{pm[a0], pm[a1 - 1]} : int2{0, 0};
    }
}

__global__ __launch_bounds__(256) void k_flat_check(FlatArgs A) {
    const int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gi < A.mb * A.h_kv) A.fail[gi] = list_decides(A, gi) ? 0 : 1;
}

// ---------------------------------------------------------------- threshold
__global__ __launch_bounds__(256) void k_flat_threshold(FlatArgs A) {
    __shared__ __attribute__((aligned(16))) uint64_t sk[256 * 4];
    __shared__ int scr[8];
    __shared__ uint64_t t_s;
    const int64_t gi = blockIdx.x;
    const int tid = threadIdx.x;
    if (A.S == 0) {                                   // few leaves: collect every candidate
        if (tid == 0) { A.thr[gi] = 1ull; A.lcnt[gi] = 0; A.lwt[gi] = 0; }
        return;
    }
    // thread t: sorted ranks 4t .. 4t + 3
    uint64_t kk[4];
    const uint64_t *sp = A.smp + (size_t)gi * kSampleMax;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int e = 4 * tid + u;
        kk[u] = e < A.ns ? sp[e] : 0ull;
    }
    block_sort_desc<4>(kk, sk);
    const uint16_t *wt = A.wt + (size_t)gi * A.nleaf;
    int w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) w[u] = kk[u] ? (int)wt[~(uint32_t)kk[u]] : 0;
    const int local = w[0] + w[1] + w[2] + w[3];
    int total;
    int run = block_excl_scan(local, scr, &total);
    const int target = (int)std::min<int64_t>((8 * (int64_t)A.k + A.S - 1) / A.S, INT32_MAX);
    if (tid == 0) t_s = 1ull;                         // sample too light: collect every candidate
    __syncthreads();
    if (run < target && run + local >= target) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            run += w[u];
            if (run >= target) { t_s = kk[u]; break; }
        }
    }
    __syncthreads();
    if (tid == 0) { A.thr[gi] = t_s; A.lcnt[gi] = 0; A.lwt[gi] = 0; }
}

// ---------------------------------------------------------------- collect
__global__ __launch_bounds__(256) void k_flat_collect(FlatArgs A) {
    __shared__ uint64_t lk[kCollect];
    __shared__ int n_s, w_s, base_s;
    const int64_t gi = blockIdx.y;
    const int64_t v0 = (int64_t)blockIdx.x * kCollect;
    const int tid = threadIdx.x;
    const uint64_t T = A.thr[gi];
    const uint32_t *sc = A.sc + (size_t)gi * A.nleaf;
    const uint16_t *wt = A.wt + (size_t)gi * A.nleaf;
    if (tid == 0) { n_s = 0; w_s = 0; }
    __syncthreads();
    int wloc = 0;
    auto take = [&](int64_t v, uint32_t s, int w) {
        const uint64_t key = ((uint64_t)s << 32) | (uint64_t)(~(uint32_t)v);
        if (w == 0 || key < T) return;
        lk[atomicAdd(&n_s, 1)] = key;
        wloc += w;
    };
    if ((A.nleaf & 7) == 0) {
        // two steps of eight leaves per thread; every load issued before use
        // (clamped indices; the rows start 16-byte aligned)
        const int64_t nq = A.nleaf / 8, q0 = v0 / 8;
        uint4 wv[2], s0[2], s1[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int64_t q = min(q0 + tid + 256 * u, nq - 1);
            wv[u] = reinterpret_cast<const uint4 *>(wt)[q];
            s0[u] = reinterpret_cast<const uint4 *>(sc)[2 * q];
            s1[u] = reinterpret_cast<const uint4 *>(sc)[2 * q + 1];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int64_t q = q0 + tid + 256 * u;
            if (q >= nq) break;
            const uint32_t ww[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
            const uint32_t ss[8] = {s0[u].x, s0[u].y, s0[u].z, s0[u].w, s1[u].x, s1[u].y, s1[u].z, s1[u].w};
#pragma unroll
            for (int x = 0; x < 8; ++x) take(8 * q + x, ss[x], (int)((ww[x >> 1] >> (16 * (x & 1))) & 0xffffu));
        }
    } else {
        for (int64_t v = v0 + tid; v < min<int64_t>(v0 + kCollect, A.nleaf); v += blockDim.x) take(v, sc[v], wt[v]);
    }
    atomicAdd(&w_s, wloc);
    __syncthreads();
    if (tid == 0) {
        base_s = n_s > 0 ? atomicAdd(A.lcnt + gi, n_s) : 0;
        if (w_s > 0) atomicAdd(A.lwt + gi, w_s);
    }
    __syncthreads();
    uint64_t *dst = A.lst + (size_t)gi * kFlatList;
    for (int e = tid; e < n_s; e += blockDim.x)
        if (base_s + e < kFlatList) dst[base_s + e] = lk[e];
}

// ---------------------------------------------------------------- finish
// Fill the row from the nl descending keys lst[0..nl) (LDS), in rounds of 256
// ranks, one per thread: a block scan of the weights gives each leaf its
// offset, and every thread copies its leaf's members (eight loads in flight).
// Rounds stop once k keys are placed.
LSA_DEV void fill_rounds(const FlatArgs &A, const uint64_t *lst, int nl, int *scr, float *cut_s) {
    const int64_t gi = blockIdx.x;
    const int64_t i = gi / A.h_kv;
    const int g = (int)(gi % A.h_kv);
    const int tid = threadIdx.x;
    const uint16_t *wt = A.wt + (size_t)gi * A.nleaf;
    const int32_t *lo = A.leaf_off + (size_t)g * (A.nleaf + 1);
    const int32_t *pm = A.perm + (size_t)g * A.n;
    const AttnSet as = attn_set(A.q_pos[i], A.n, A.n_sink, A.window);
    int32_t *out = A.sel + (size_t)gi * A.row;
    int carry = 0;
    for (int base = 0; base < nl && carry < A.k; base += blockDim.x) {
        const int e = base + tid;
        const uint64_t key = e < nl ? lst[e] : 0ull;
        const uint32_t v = key ? ~(uint32_t)key : 0u;
        const int w = key ? (int)wt[v] : 0;
        const int32_t a0 = lo[v], a1 = lo[v + 1];
        int tot;
        const int run = carry + block_excl_scan(w, scr, &tot);
        if (w > 0 && run < A.k) {
            const int take = min(w, A.k - run);
            int f, c;
            in_range(as, pm + a0, a1 - a0, f, c);
            const int32_t *src = pm + a0 + f;
            for (int t0 = 0; t0 < take; t0 += 8) {
                int32_t x[8];
#pragma unroll
                for (int t = 0; t < 8; ++t) x[t] = src[min(t0 + t, take - 1)];       // clamped: in the leaf
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    if (t0 + t < take) out[run + t0 + t] = x[t];
            }
            if (run + w >= A.k) *cut_s = unorderable((uint32_t)(key >> 32));
        }
        carry += tot;
    }
    const int count = min(A.k, carry);
    for (int t = tid; t < as.nloc; t += blockDim.x) out[count + t] = local_key(as, t);
    for (int t = count + as.nloc + tid; t < A.row; t += blockDim.x) out[t] = -1;
    __syncthreads();
    if (tid == 0) {
        A.sel_count[gi] = count + as.nloc;
        if (A.sel_cutoff) A.sel_cutoff[gi] = *cut_s;
    }
}

// Bitonic sort, descending, of keys[0..N) in LDS (N a power of two) by the
// block; each thread's eight compare-exchanges of a stage are loaded before
// any is stored.  Loops rather than unrolled stages keep the code small.
LSA_DEV void lds_sort_desc(uint64_t *keys, int N) {
    for (int size = 2; size <= N; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int t0 = threadIdx.x; t0 < (N >> 1); t0 += 8 * blockDim.x) {
                uint64_t a[8], b[8];
                int lo[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int t = min(t0 + u * (int)blockDim.x, (N >> 1) - 1);      // clamped: in bounds
                    lo[u] = 2 * t - (t & (stride - 1));
                    a[u] = keys[lo[u]];
                    b[u] = keys[lo[u] + stride];
                }
                __builtin_amdgcn_sched_barrier(0);   // every load issued before the first store
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    if (t0 + u * (int)blockDim.x >= (N >> 1)) break;
                    const bool desc = (lo[u] & size) == 0;     // segment sorted descending
                    const bool sw = desc ? (b[u] > a[u]) : (a[u] > b[u]);
                    if (sw) { keys[lo[u]] = b[u]; keys[lo[u] + stride] = a[u]; }
                }
            }
            __syncthreads();
        }
    }
}

// Sort the nl keys of src (global memory or LDS) descending into lst (LDS, at
// least kFlatList keys; may be src) and fill the row from them.  Up to 1024
// keys are sorted in registers (four per thread), more in LDS.
LSA_DEV void sort_and_fill_any(const FlatArgs &A, const uint64_t *src, int nl, uint64_t *lst, int *scr, float *cut_s) {
    if (nl <= 1024) {
        uint64_t kk[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = 4 * (int)threadIdx.x + u;
            kk[u] = e < nl ? src[e] : 0ull;
        }
        block_sort_desc<4>(kk, lst);
        __syncthreads();
#pragma unroll
        for (int u = 0; u < 4; ++u) lst[4 * threadIdx.x + u] = kk[u];
        __syncthreads();
    } else {
        const int np2 = next_pow2(nl);
        if (src != lst)
            for (int e = threadIdx.x; e < nl; e += blockDim.x) lst[e] = src[e];
        for (int e = nl + threadIdx.x; e < np2; e += blockDim.x) lst[e] = 0ull;
        __syncthreads();
        lds_sort_desc(lst, np2);
    }
    fill_rounds(A, lst, nl, scr, cut_s);
}

// Every key at or above the boundary bucket into lst (LDS), their number to
// *nlist: exact weighted radix selection over all of the row's leaves.
LSA_DEV void exact_boundary_list(const FlatArgs &A, uint64_t *lst, int *hw, int *hc, int *scr, int *res_s,
                                 int *nlist) {
    const int64_t gi = blockIdx.x;
    const int tid = threadIdx.x;
    // ---- exact boundary by weighted radix selection: the top `fixed` bits
    // `prefix` of the key whose inclusion brings the weight of the keys above
    // it to k, refined until the keys above the bucket and the bucket itself
    // fit in LDS (at 64 bits the bucket is one key: the keys are distinct)
    const uint32_t *sc = A.sc + (size_t)gi * A.nleaf;
    const uint16_t *wt = A.wt + (size_t)gi * A.nleaf;
    auto keyof = [&](int64_t v) -> uint64_t { return ((uint64_t)sc[v] << 32) | (uint64_t)(~(uint32_t)v); };
    uint64_t prefix = 0;
    int fixed = 0, want = A.k, nabove = 0;
    bool take_all = false;
    for (int lv = 0; lv < 6; ++lv) {
        const int D = (lv % 3 == 2) ? 10 : 11;
        const int nb = 1 << D, shift = 64 - fixed - D;
        for (int e = tid; e < nb; e += blockDim.x) { hw[e] = 0; hc[e] = 0; }
        __syncthreads();
        for (int64_t v = tid; v < A.nleaf; v += blockDim.x) {
            const int w = wt[v];
            if (w == 0) continue;
            const uint64_t key = keyof(v);
            if (fixed > 0 && (key >> (64 - fixed)) != prefix) continue;
            const int dg = (int)((key >> shift) & (uint64_t)(nb - 1));
            atomicAdd(&hw[dg], w);
            atomicAdd(&hc[dg], 1);
        }
        __syncthreads();
        // thread t owns the digits nb-1-t*per .. nb-t*per-per (descending):
        // the weight of larger digits is an exclusive scan in thread order
        const int per = nb / 256;
        int sw = 0, sn = 0;
        for (int q = 0; q < per; ++q) {
            const int dg = nb - 1 - (tid * per + q);
            sw += hw[dg];
            sn += hc[dg];
        }
        int tw, tn;
        const int bw = block_excl_scan(sw, scr, &tw);
        const int bn = block_excl_scan(sn, scr, &tn);
        if (lv == 0 && tw < want) { take_all = true; break; }    // every candidate is taken
        {
            int run = bw, runn = bn;
            for (int q = 0; q < per; ++q) {
                const int dg = nb - 1 - (tid * per + q);
                const int h = hw[dg];
                if (h > 0 && run < want && run + h >= want) {
                    res_s[0] = dg; res_s[1] = want - run; res_s[2] = runn; res_s[3] = hc[dg];
                }
                run += h;
                runn += hc[dg];
            }
        }
        __syncthreads();
        const int dg = res_s[0];
        want = res_s[1];
        nabove += res_s[2];
        const int nbucket = res_s[3];
        prefix = (prefix << D) | (uint64_t)dg;
        fixed += D;
        __syncthreads();
        if (nabove + nbucket <= kFlatList) break;
    }
    // the keys above the bucket and in it (all candidates when their total
    // weight is below k: fewer than k of them)
    const uint64_t lo_key = take_all ? 1ull : prefix << (64 - fixed);
    if (tid == 0) *nlist = 0;
    __syncthreads();
    for (int64_t v = tid; v < A.nleaf; v += blockDim.x) {
        if (wt[v] == 0) continue;
        const uint64_t key = keyof(v);
        if (key < lo_key) continue;
        const int at = atomicAdd(nlist, 1);
        if (at < kFlatList) lst[at] = key;
    }
    __syncthreads();
}

// The smallest key B of the nl keys lst[0..nl) (LDS) such that the keys >= B
// weigh at least k, widened to a bucket of the key's top bits that holds at
// most 1024 keys (with every key above it) where the bits allow: the keys at
// or above the returned value include every key retrieval reaches.  1 when the
// whole list weighs less than k.  Weighted radix selection from the first bit
// where the list's keys differ, up to 11 bits a round.
LSA_DEV uint64_t narrow_list(const FlatArgs &A, const uint64_t *lst, int nl, int *hw, int *hc, int *scr, int *res_s,
                             unsigned long long *red_s) {
    const int64_t gi = blockIdx.x;
    const int tid = threadIdx.x;
    const uint16_t *wt = A.wt + (size_t)gi * A.nleaf;
    if (tid == 0) { red_s[0] = 0ull; red_s[1] = ~0ull; }
    __syncthreads();
    unsigned long long mx = 0ull, mn = ~0ull;
    for (int e = tid; e < nl; e += blockDim.x) { mx = max(mx, (unsigned long long)lst[e]); mn = min(mn, (unsigned long long)lst[e]); }
    atomicMax(red_s, mx);
    atomicMin(red_s + 1, mn);
    __syncthreads();
    mx = red_s[0];
    mn = red_s[1];
    __syncthreads();
    if (nl == 0) return 1ull;
    int fixed = (mx == mn) ? 64 : __clzll((long long)(mx ^ mn));
    uint64_t prefix = fixed == 0 ? 0ull : (uint64_t)mx >> (64 - fixed);
    int want = A.k, nabove = 0;
    bool first = true;
    while (fixed < 64) {
        const int D = min(11, 64 - fixed);
        const int nb = 1 << D, shift = 64 - fixed - D;
        for (int e = tid; e < nb; e += blockDim.x) { hw[e] = 0; hc[e] = 0; }
        __syncthreads();
        for (int e0 = tid; e0 < nl; e0 += 8 * blockDim.x) {
            uint64_t key[8];
            int w[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int e = e0 + u * (int)blockDim.x;
                key[u] = e < nl ? lst[e] : 0ull;
                const bool in = key[u] != 0ull && (fixed == 0 || (key[u] >> (64 - fixed)) == prefix);
                w[u] = in ? (int)wt[~(uint32_t)key[u]] : 0;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (w[u] == 0) continue;
                const int dg = (int)((key[u] >> shift) & (uint64_t)(nb - 1));
                atomicAdd(&hw[dg], w[u]);
                atomicAdd(&hc[dg], 1);
            }
        }
        __syncthreads();
        // thread t owns digits nb-1-t*per .. (descending), per >= 1
        const int per = max(1, nb / (int)blockDim.x);
        int sw = 0, sn = 0;
        for (int q = 0; q < per; ++q) {
            const int dg = nb - 1 - (tid * per + q);
            if (dg >= 0) { sw += hw[dg]; sn += hc[dg]; }
        }
        int totw, totn;
        const int bw = block_excl_scan(sw, scr, &totw);
        const int bn = block_excl_scan(sn, scr, &totn);
        if (first && totw < want) return 1ull;                   // the whole list is taken
        first = false;
        {
            int run = bw, runn = bn;
            for (int q = 0; q < per; ++q) {
                const int dg = nb - 1 - (tid * per + q);
                if (dg < 0) break;
                const int h = hw[dg];
                if (h > 0 && run < want && run + h >= want) {
                    res_s[0] = dg; res_s[1] = want - run; res_s[2] = runn; res_s[3] = hc[dg];
                }
                run += h;
                runn += hc[dg];
            }
        }
        __syncthreads();
        const int dg = res_s[0];
        want = res_s[1];
        nabove += res_s[2];
        const int nbucket = res_s[3];
        prefix = (prefix << D) | (uint64_t)dg;
        fixed += D;
        __syncthreads();
        if (nabove + nbucket <= 1024) break;
    }
    return prefix << (64 - fixed);
}

__global__ __launch_bounds__(256) void k_flat_finish(FlatArgs A) {
    extern __shared__ __attribute__((aligned(16))) uint64_t lst[];   // [kFlatList] keys
    int *hw = reinterpret_cast<int *>(lst + kFlatList);               // [kFlatBins] weight per digit
    int *hc = hw + kFlatBins;                                          // [kFlatBins] keys per digit
    __shared__ int scr[8], nlist_s, res_s[4];
    __shared__ unsigned long long red_s[2];
    __shared__ float cut_s;
    const int64_t gi = blockIdx.x;                 // row * h_kv + KV head, within the batch
    const int tid = threadIdx.x;
    if (tid == 0) cut_s = -INFINITY;
    const int nl0 = A.lcnt[gi];
    uint64_t *glst = A.lst + (size_t)gi * kFlatList;
    // the list decides the row (list_decides), or the exact radix selection
    // over every leaf builds it
    int nl;
    if (list_decides(A, gi)) {
        for (int e = tid; e < nl0; e += blockDim.x) lst[e] = glst[e];
        nl = nl0;
        __syncthreads();
    } else {
        exact_boundary_list(A, lst, hw, hc, scr, res_s, &nlist_s);
        nl = min(nlist_s, kFlatList);
    }
    // keep the keys at or above the list's own boundary (in the row's global
    // list, any order), then sort them and fill
    const uint64_t lo_key = narrow_list(A, lst, nl, hw, hc, scr, res_s, red_s);
    if (tid == 0) nlist_s = 0;
    __syncthreads();
    for (int e = tid; e < nl; e += blockDim.x) {
        const uint64_t key = lst[e];
        if (key >= lo_key) glst[atomicAdd(&nlist_s, 1)] = key;
    }
    __syncthreads();
    const int nk = nlist_s;
    __syncthreads();
    sort_and_fill_any(A, glst, nk, lst, scr, &cut_s);
}

inline size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

struct FlatWs {
    float *U; double *Ud; uint32_t *sc; uint16_t *wt; uint64_t *smp, *thr; int32_t *lcnt, *lwt, *fail; uint64_t *lst;
    int2 *fl; size_t bytes;
};

// (after the workspace's reserved prefix, which this path never writes)
FlatWs carve_flat_ws(char *base, int64_t mb, int h_kv, int r, int64_t nleaf) {
    size_t cur = (size_t)ws_reserved_bytes();
    FlatWs w{};
    auto take = [&](size_t n) { char *p = base ? base + cur : nullptr; cur = a256(cur + n); return p; };
    const size_t groups = (size_t)mb * h_kv;
    w.fl = (int2 *)take(sizeof(int2) * (size_t)h_kv * nleaf);     // first: the same place for every batch size
    w.U = (float *)take(sizeof(float) * groups * r);
    w.Ud = (double *)take(sizeof(double) * groups * r);
    w.sc = (uint32_t *)take(sizeof(uint32_t) * groups * nleaf);
    w.wt = (uint16_t *)take(sizeof(uint16_t) * groups * nleaf);
    w.smp = (uint64_t *)take(sizeof(uint64_t) * groups * kSampleMax);
    w.thr = (uint64_t *)take(sizeof(uint64_t) * groups);
    w.lcnt = (int32_t *)take(sizeof(int32_t) * groups);
    w.lwt = (int32_t *)take(sizeof(int32_t) * groups);
    w.fail = (int32_t *)take(sizeof(int32_t) * groups);
    w.lst = (uint64_t *)take(sizeof(uint64_t) * groups * kFlatList);
    w.bytes = cur;
    return w;
}

}  // namespace

int64_t flat_workspace_bytes(int64_t m, int h_kv, int r, int64_t nleaf) {
    return (int64_t)carve_flat_ws(nullptr, std::max<int64_t>(1, std::min(m, kFlatBatch)), h_kv, r, nleaf).bytes;
}

int64_t flat_batch_rows(int64_t m, int h_kv, int r, int64_t nleaf, int64_t ws_bytes) {
    int64_t mb = std::min(m, kFlatBatch);
    while (mb > 0 && (int64_t)carve_flat_ws(nullptr, mb, h_kv, r, nleaf).bytes > ws_bytes) mb >>= 1;
    return mb;
}

hipError_t select_flat(const void *Q, int dtype, int64_t m, int h_q, int d, const int32_t *q_pos, const char *index,
                       int64_t n, int h_kv, int r, int64_t nleaf, int64_t leaf_c_off, int64_t leaf_cnt_off,
                       int64_t leaf_off_off, int64_t perm_off, const float *W, int k, int n_sink, int window,
                       int32_t *sel, int32_t *sel_count, float *sel_cutoff, void *ws, int64_t ws_bytes,
                       hipStream_t st) {
    const int64_t mb = flat_batch_rows(m, h_kv, r, nleaf, ws_bytes);
    if (mb < 1) return hipErrorInvalidValue;
    // the attribute is set once per device (setting it twice is harmless)
    static std::atomic<int> attr_set[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    const size_t shm = sizeof(uint64_t) * kFlatList + sizeof(int) * 2 * kFlatBins;
    if (!attr_set[dev].load(std::memory_order_acquire)) {
        hipError_t e = hipFuncSetAttribute((const void *)k_flat_finish, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)shm);
        if (e != hipSuccess) return e;
        attr_set[dev].store(1, std::memory_order_release);
    }
    const int row = k + n_sink + window;
    const size_t esz = dtype == 0 ? 4 : 2;
    // sample stride: none when every candidate fits the list, else at least
    // 64 and at most kSampleMax samples
    const int64_t S = nleaf <= kFlatList ? 0 : std::max<int64_t>(64, (nleaf + kSampleMax - 1) / kSampleMax);
    for (int64_t i0 = 0; i0 < m; i0 += mb) {
        const int64_t nb = std::min(mb, m - i0);
        FlatWs w = carve_flat_ws((char *)ws, nb, h_kv, r, nleaf);
        FlatArgs A{};
        A.Q = (const char *)Q + (size_t)i0 * h_q * d * esz;
        A.h_q = h_q; A.h_kv = h_kv; A.d = d; A.r = r; A.mb = nb; A.q_pos = q_pos + i0;
        A.n = n; A.nleaf = nleaf;
        A.C = (const float *)(index + leaf_c_off);
        A.cnt = (const int32_t *)(index + leaf_cnt_off);
        A.leaf_off = (const int32_t *)(index + leaf_off_off);
        A.perm = (const int32_t *)(index + perm_off);
        A.W = W; A.k = k; A.n_sink = n_sink; A.window = window; A.row = row;
        A.U = w.U; A.Ud = w.Ud; A.sc = w.sc; A.wt = w.wt;
        A.S = S; A.ns = S > 0 ? (int)((nleaf + S - 1) / S) : 0;
        A.smp = w.smp; A.thr = w.thr; A.lcnt = w.lcnt; A.lwt = w.lwt; A.fail = w.fail; A.lst = w.lst; A.fl = w.fl;
        A.sel = sel + (size_t)i0 * h_kv * row;
        A.sel_count = sel_count + (size_t)i0 * h_kv;
        A.sel_cutoff = sel_cutoff ? sel_cutoff + (size_t)i0 * h_kv : nullptr;
        const unsigned groups = (unsigned)(nb * h_kv);
        if (dtype == 0) hipLaunchKernelGGL(k_flat_latent<float>, dim3((unsigned)nb, (unsigned)h_kv), dim3(256), 0, st, A);
        else hipLaunchKernelGGL(k_flat_latent<bf16_t>, dim3((unsigned)nb, (unsigned)h_kv), dim3(256), 0, st, A);
        const dim3 sgrid((unsigned)((nleaf + kFlatLeaves - 1) / kFlatLeaves), (unsigned)((nb + kFlatRows - 1) / kFlatRows),
                         (unsigned)h_kv);
        if (r == 64 && nb >= kFlatMfmaRows) {
            // threshold from the sample, the list from one scoring pass, the
            // full table only for the rows the list does not decide
            // every leaf's first and last member, once per call
            if (i0 == 0)
                hipLaunchKernelGGL(k_flat_bounds, dim3((unsigned)std::min<int64_t>((h_kv * nleaf + 255) / 256, 8192)),
                                   dim3(256), 0, st, A);
            if (S > 0) {
                const dim3 pgrid((unsigned)((A.ns + 63) / 64), sgrid.y, sgrid.z);
                hipLaunchKernelGGL(k_flat_score_mfma<1>, pgrid, dim3(256), 0, st, A);
            }
            hipLaunchKernelGGL(k_flat_threshold, dim3(groups), dim3(256), 0, st, A);
            hipLaunchKernelGGL(k_flat_score_mfma<2>, sgrid, dim3(256), 0, st, A);
            hipLaunchKernelGGL(k_flat_check, dim3((groups + 255) / 256), dim3(256), 0, st, A);
            hipLaunchKernelGGL(k_flat_score_mfma<3>, sgrid, dim3(256), 0, st, A);
        } else {
            if (r == 64) hipLaunchKernelGGL(k_flat_score<64>, sgrid, dim3(256), 0, st, A);
            else hipLaunchKernelGGL(k_flat_score<0>, sgrid, dim3(256), 0, st, A);
            hipLaunchKernelGGL(k_flat_threshold, dim3(groups), dim3(256), 0, st, A);
            hipLaunchKernelGGL(k_flat_collect, dim3((unsigned)((nleaf + kCollect - 1) / kCollect), groups), dim3(256),
                               0, st, A);
        }
        hipLaunchKernelGGL(k_flat_finish, dim3(groups), dim3(256), shm, st, A);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace lsa
