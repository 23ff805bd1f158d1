// Index build: latent projection and top-down k-means tree (gfx950).
//
// Method: keys are projected into a learned latent space and grouped by a
// tree whose root holds every key and whose levels split clusters further,
// like hierarchical k-means ("Latent Sparse Attention Breaks Through the
// Million-Token Context Bottleneck", kongchang.com, section "How LSA Sidesteps
// Per-Key Scoring with Hierarchical Clustering"); each cluster is a centroid
// stored with references to its keys ("Latent sparse attention",
// bdtechtalks.com, section "How latent sparse attention works").
//
// Work layout.  Per level, the keys sit in `perm` grouped by their parent
// node, ascending within a parent.  A parent's range is cut into pieces of
// kPiece positions (one workgroup each), so every piece belongs to exactly one
// parent and can stage that parent's child centroids in LDS.  One Lloyd round
// is: assign (nearest child, plus the key's stable rank among the piece's keys
// with the same child), a per-parent prefix over pieces, a scatter that
// regroups the keys by child in ascending position, and a fixed-order mean.
// Distances, projection sums and means are accumulated in double in ascending
// dimension / key order with no fused multiply-add where a product is
// inexact, so the tree does not depend on scheduling.
#include "common.h"
#include "internal.h"

namespace lsa {

constexpr int kPiece = 256;   // keys per piece = threads per assign workgroup

struct Piece { int32_t u, start, len; };

// ---------------------------------------------------------------- projection
// z[g][j][c] = fl32(sum_i K[g][j][i] * W[g][i][c]), i ascending.  Each product
// of a bf16/fp32 key element with an fp32 weight is exact in double, so a
// fused multiply-add rounds exactly like a multiply followed by an add.
template <typename T>
__global__ __launch_bounds__(256) void k_project(const T *__restrict__ K, const float *__restrict__ W,
                                                 float *__restrict__ Z, int64_t n, int d, int r) {
    constexpr int KT = 32;    // keys per workgroup
    constexpr int IC = 64;    // input dimensions staged per pass
    __shared__ float Ws[IC * 64];
    __shared__ float Ks[KT * IC];
    const int g = blockIdx.y;
    const int64_t key0 = (int64_t)blockIdx.x * KT;
    const int c = threadIdx.x & 63;
    const int q = threadIdx.x >> 6;            // 0..3
    const T *Kg = K + (size_t)g * n * d;
    const float *Wg = W + (size_t)g * d * r;
    double acc[KT / 4];
#pragma unroll
    for (int t = 0; t < KT / 4; ++t) acc[t] = 0.0;
    for (int i0 = 0; i0 < d; i0 += IC) {
        const int ic = min(IC, d - i0);
        for (int idx = threadIdx.x; idx < ic * r; idx += blockDim.x)
            Ws[(idx / r) * 64 + (idx % r)] = Wg[(size_t)(i0 + idx / r) * r + (idx % r)];
        for (int idx = threadIdx.x; idx < KT * ic; idx += blockDim.x) {
            const int kk = idx / ic, ii = idx % ic;
            const int64_t j = key0 + kk;
            Ks[kk * IC + ii] = (j < n) ? to_float(Kg[(size_t)j * d + i0 + ii]) : 0.0f;
        }
        __syncthreads();
        if (c < r) {
            for (int ii = 0; ii < ic; ++ii) {
                const double w = (double)Ws[ii * 64 + c];
#pragma unroll
                for (int t = 0; t < KT / 4; ++t)
                    acc[t] = fma((double)Ks[(q + 4 * t) * IC + ii], w, acc[t]);
            }
        }
        __syncthreads();
    }
    if (c < r) {
#pragma unroll
        for (int t = 0; t < KT / 4; ++t) {
            const int64_t j = key0 + q + 4 * t;
            if (j < n) Z[((size_t)g * n + j) * r + c] = (float)acc[t];
        }
    }
}

// The same projection on the fp64 matrix cores (r = 64, d a multiple of 8,
// d <= 256): a workgroup takes KB 16-key blocks, wave w the latent columns
// 16 w .. 16 w + 15.  v_mfma_f64_16x16x4_f64 adds the four exact products of
// dims 4 blk .. 4 blk + 3 in order, each addition rounded as a separate fma
// would be, so the chain over blk ascending gives the same double sum bit for
// bit.  The key tile is staged in LDS transposed ([dim][key], padded rows) as
// floats.  NQ = d / 4 when fixed at compile time (the lane's weights, dims
// 4 blk + l / 16 of its column, then sit in registers before the tile is
// staged); NQ = 0 takes d at run time and loads a weight per block.
constexpr int kPjMaxD = 256;
template <typename T, int KB, int NQ>
__global__ __launch_bounds__(256) void k_project_mfma(const T *__restrict__ K, const float *__restrict__ W,
                                                      float *__restrict__ Z, int64_t n, int d) {
    constexpr int r = 64, KT = 16 * KB, ST = KT + 1;
    extern __shared__ float Kt[];                 // [d][ST]
    const int g = blockIdx.y;
    const int64_t key0 = (int64_t)blockIdx.x * KT;
    const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
    const int lr = lane % 16, lk = lane / 16;
    const T *Kg = K + (size_t)g * n * d;
    const float *wcol = W + (size_t)g * d * r + 16 * w + lr;
    const int nq = NQ > 0 ? NQ : d / 4;
    float wv[NQ > 0 ? NQ : 1];
    if constexpr (NQ > 0) {
#pragma unroll
        for (int blk = 0; blk < NQ; ++blk) wv[blk] = wcol[(size_t)(4 * blk + lk) * r];
    }
    // the tile: key row kk, dims 8 x .. 8 x + 7 per 16-byte (bf16) or two
    // 16-byte (fp32) loads, stored transposed
    for (int idx = tid; idx < KT * (d / 8); idx += blockDim.x) {
        const int kk = idx / (d / 8), x = idx % (d / 8);
        const int64_t j = key0 + kk;
        float v[8];
        load8(Kg, j < n ? (size_t)j * d + 8 * x : 0, v);
#pragma unroll
        for (int u = 0; u < 8; ++u) Kt[(8 * x + u) * ST + kk] = j < n ? v[u] : 0.0f;
    }
    __syncthreads();
    d4_t acc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) acc[kb] = d4_t{0.0, 0.0, 0.0, 0.0};
#pragma unroll(NQ > 0 ? NQ : 1)
    for (int blk = 0; blk < nq; ++blk) {
        double b;
        if constexpr (NQ > 0) b = (double)wv[blk];
        else b = (double)wcol[(size_t)(4 * blk + lk) * r];
        const float *krow = Kt + (4 * blk + lk) * ST + lr;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            acc[kb] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)krow[16 * kb], b, acc[kb], 0, 0, 0);
    }
    // element e of lane l: key 16 kb + l / 16 + 4 e, column 16 w + l % 16
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t j = key0 + 16 * kb + lk + 4 * e;
            if (j < n) Z[((size_t)g * n + j) * r + 16 * w + lr] = (float)acc[kb][e];
        }
}

// ---------------------------------------------------------------- level setup
__global__ void k_iota(int32_t *perm, int64_t n, int h) {
    const int64_t tot = n * h;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < tot; i += (int64_t)gridDim.x * blockDim.x)
        perm[i] = (int32_t)(i % n);
}

__global__ void k_root_off(int32_t *off, int64_t n, int h) {
    for (int g = threadIdx.x; g < h; g += blockDim.x) { off[2 * g] = 0; off[2 * g + 1] = (int32_t)n; }
}

// pieces per parent: np[g][u] = ceil(m_u / kPiece)
__global__ void k_piece_count(const int32_t *__restrict__ off_prev, int32_t *__restrict__ np, int64_t S, int h) {
    const int64_t tot = S * h;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < tot; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t g = i / S, u = i % S;
        const int32_t *o = off_prev + g * (S + 1);
        const int32_t m = o[u + 1] - o[u];
        np[i] = (m + kPiece - 1) / kPiece;
    }
}

// exclusive scan of np per head (one workgroup of 1024 threads per head)
__global__ __launch_bounds__(1024) void k_scan_heads(const int32_t *__restrict__ in, int32_t *__restrict__ out,
                                                     int32_t *__restrict__ total, int64_t S) {
    __shared__ int scratch[17];
    const int g = blockIdx.x;
    const int32_t *a = in + (size_t)g * S;
    int32_t *o = out + (size_t)g * S;
    const int64_t chunk = (S + blockDim.x - 1) / blockDim.x;
    const int64_t s = threadIdx.x * chunk, e = min(S, s + chunk);
    int local = 0;
    for (int64_t i = s; i < e; ++i) local += a[i];
    int tot;
    int run = block_excl_scan(local, scratch, &tot);
    for (int64_t i = s; i < e; ++i) { const int v = a[i]; o[i] = run; run += v; }
    if (threadIdx.x == 0) total[g] = tot;
}

__global__ void k_piece_fill(const int32_t *__restrict__ pbase, const int32_t *__restrict__ np,
                             const int32_t *__restrict__ off_prev, const int32_t *__restrict__ total,
                             Piece *__restrict__ pieces, int64_t S, int64_t NPmax) {
    const int g = blockIdx.y;
    const int64_t p = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (p >= total[g]) return;
    const int32_t *pb = pbase + (size_t)g * S;
    // largest u with pb[u] <= p
    int64_t lo = 0, hi = S;   // invariant: pb[lo] <= p, answer in [lo, hi)
    while (hi - lo > 1) {
        const int64_t mid = (lo + hi) >> 1;
        if (pb[mid] <= p) lo = mid; else hi = mid;
    }
    const int64_t u = lo;
    const int32_t *o = off_prev + (size_t)g * (S + 1);
    const int32_t m = o[u + 1] - o[u];
    const int32_t t = (int32_t)(p - pb[u]);
    Piece pc;
    pc.u = (int32_t)u;
    pc.start = o[u] + t * kPiece;
    pc.len = min(kPiece, m - t * kPiece);
    pieces[(size_t)g * NPmax + p] = pc;
    (void)np;
}

// Child seeds: child c < a = min(b, m) of parent u starts at the member of
// rank floor(c*m/a); the other children are zero and stay empty.
__global__ void k_init(const int32_t *__restrict__ off_prev, const int32_t *__restrict__ perm_prev,
                       const float *__restrict__ Z, float *__restrict__ C, int64_t S, int b, int r, int64_t n, int h) {
    // one thread per (node, latent dimension)
    const int64_t tot = (int64_t)h * S * b * r;
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < tot; e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = e / r;
        const int x = (int)(e % r);
        const int64_t g = i / (S * b);
        const int64_t v = i % (S * b);
        const int64_t u = v / b;
        const int c = (int)(v % b);
        const int32_t *o = off_prev + g * (S + 1);
        const int64_t m = o[u + 1] - o[u];
        const int a = (int)min((int64_t)b, m);
        float val = 0.0f;
        if (c < a) {
            const int32_t j = perm_prev[g * n + o[u] + ((int64_t)c * m) / a];
            val = Z[((size_t)g * n + j) * r + x];
        }
        C[(size_t)i * r + x] = val;
    }
}

// ---------------------------------------------------------------- Lloyd round
// Squared distances of z to four centroids (four independent chains), the
// same arithmetic as sq_dist2.
LSA_DEV void sq_dist4(const double (&z)[64], const double *c0, int r, double (&d)[4]) {
#pragma clang fp contract(off)
    double s[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int x = 0; x < 64; x += 2) {
        if (x < r) {
            double2 a[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) a[q] = *reinterpret_cast<const double2 *>(c0 + q * 64 + x);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const double e = z[x] - a[q].x;
                const double p = e * e;
                s[q] = s[q] + p;
            }
            if (x + 1 < r) {                 // (LDS entries at and beyond r are never written)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const double e = z[x + 1] - a[q].y;
                    const double p = e * e;
                    s[q] = s[q] + p;
                }
            }
        }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) d[q] = s[q];
}

// Squared distances of z to two centroids: per dimension, in ascending order,
// diff = z - c, then diff * diff and the running sum as separate roundings
// (no fused multiply-add); the same arithmetic as widening each float when
// it is used.
LSA_DEV void sq_dist2(const double (&z)[64], const double *c0, const double *c1, int r, double &d0, double &d1) {
#pragma clang fp contract(off)
    double s0 = 0.0, s1 = 0.0;
#pragma unroll
    for (int x = 0; x < 64; x += 2) {
        if (x < r) {
            const double2 a = *reinterpret_cast<const double2 *>(c0 + x);
            const double2 b = *reinterpret_cast<const double2 *>(c1 + x);
            const double e0 = z[x] - a.x, e1 = z[x] - b.x;
            const double q0 = e0 * e0, q1 = e1 * e1;
            s0 = s0 + q0;
            s1 = s1 + q1;
            if (x + 1 < r) {                 // (LDS entries at and beyond r are never written)
                const double f0 = z[x + 1] - a.y, f1 = z[x + 1] - b.y;
                const double p0 = f0 * f0, p1 = f1 * f1;
                s0 = s0 + p0;
                s1 = s1 + p1;
            }
        }
    }
    d0 = s0;
    d1 = s1;
}

__global__ __launch_bounds__(kPiece) void k_assign(const Piece *__restrict__ pieces, const int32_t *__restrict__ total,
                                                   const int32_t *__restrict__ off_prev,
                                                   const int32_t *__restrict__ perm_prev, const float *__restrict__ Z,
                                                   const float *__restrict__ C, uint8_t *__restrict__ child,
                                                   uint8_t *__restrict__ lrank, int32_t *__restrict__ hist, int64_t S,
                                                   int64_t NPmax, int b, int r, int64_t n) {
    __shared__ __attribute__((aligned(16))) double Cs[64 * 64];     // child centroids, widened once
    __shared__ int wcnt[kPiece / kWave][64];
    const int g = blockIdx.y;
    const int64_t p = blockIdx.x;
    if (p >= total[g]) return;
    const Piece pc = pieces[(size_t)g * NPmax + p];
    const int32_t *o = off_prev + (size_t)g * (S + 1);
    const int64_t m = o[pc.u + 1] - o[pc.u];
    const int a = (int)min((int64_t)b, m);
    const float *Cu = C + ((size_t)g * S * b + (size_t)pc.u * b) * r;
    for (int idx = threadIdx.x; idx < a * r; idx += blockDim.x) Cs[(idx / r) * 64 + idx % r] = (double)Cu[idx];
    for (int idx = threadIdx.x; idx < (kPiece / kWave) * 64; idx += blockDim.x) (&wcnt[0][0])[idx] = 0;
    __syncthreads();

    const bool valid = threadIdx.x < pc.len;
    const int64_t posn = (int64_t)pc.start + threadIdx.x;
    int best = 0;
    if (valid) {
        const int32_t j = perm_prev[(size_t)g * n + posn];
        const float *zr = Z + ((size_t)g * n + j) * r;
        double z[64];
#pragma unroll
        for (int x = 0; x < 64; ++x) z[x] = (x < r) ? (double)zr[x] : 0.0;
        double bestd = 0.0;
        int c = 0;
        // four, then two children per step (independent chains), compared in
        // child order
        for (; c + 4 <= a; c += 4) {
            double dq[4];
            sq_dist4(z, Cs + c * 64, r, dq);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if ((c + q == 0) || dq[q] < bestd) { bestd = dq[q]; best = c + q; }
        }
        for (; c + 2 <= a; c += 2) {
            double d0, d1;
            sq_dist2(z, Cs + c * 64, Cs + (c + 1) * 64, r, d0, d1);
            if (c == 0 || d0 < bestd) { bestd = d0; best = c; }
            if (d1 < bestd) { bestd = d1; best = c + 1; }
        }
        if (c < a) {
            double d0, d1;
            sq_dist2(z, Cs + c * 64, Cs + c * 64, r, d0, d1);
            if (c == 0 || d0 < bestd) { bestd = d0; best = c; }
        }
    }
    // stable rank among this wave's lanes with the same child (6-bit match)
    uint64_t eq = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 6; ++bit) {
        const bool on = (best >> bit) & 1;
        const uint64_t bb = __ballot(valid && on);
        eq &= on ? bb : ~bb;
    }
    const int w = threadIdx.x / kWave;
    const int rw = __popcll(eq & lanemask_lt());
    if (valid && rw == 0) wcnt[w][best] = __popcll(eq);
    __syncthreads();
    if (valid) {
        int rank = rw;
        for (int w2 = 0; w2 < w; ++w2) rank += wcnt[w2][best];
        child[(size_t)g * n + posn] = (uint8_t)best;
        lrank[(size_t)g * n + posn] = (uint8_t)rank;
    }
    if (threadIdx.x < b) {
        int s = 0;
        for (int w2 = 0; w2 < kPiece / kWave; ++w2) s += wcnt[w2][threadIdx.x];
        hist[((size_t)g * NPmax + p) * b + threadIdx.x] = s;
    }
}

// One wave per parent, lane = child: prefix of the child histograms over the
// parent's pieces, child counts, and child offsets into the regrouped perm.
__global__ __launch_bounds__(256) void k_seg_prefix(const int32_t *__restrict__ pbase, const int32_t *__restrict__ np,
                                                    const int32_t *__restrict__ hist, int32_t *__restrict__ pref,
                                                    const int32_t *__restrict__ off_prev, int32_t *__restrict__ off_new,
                                                    int32_t *__restrict__ cnt, int64_t S, int64_t NPmax, int b,
                                                    int64_t n) {
    const int g = blockIdx.y;
    const int64_t u = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (u >= S) return;
    const int c = lane_id();
    const int32_t base = pbase[(size_t)g * S + u];
    const int32_t cntp = np[(size_t)g * S + u];
    const bool act = c < b;
    const size_t row0 = ((size_t)g * NPmax + base) * b + c;
    int run = 0;
    int q = 0;
    for (; q + 32 <= cntp; q += 32) {
        int hv[32];
#pragma unroll
        for (int t = 0; t < 32; ++t) hv[t] = act ? hist[row0 + (size_t)(q + t) * b] : 0;
#pragma unroll
        for (int t = 0; t < 32; ++t) {
            if (act) pref[row0 + (size_t)(q + t) * b] = run;
            run += hv[t];
        }
    }
    for (; q < cntp; ++q) {
        const int hv = act ? hist[row0 + (size_t)q * b] : 0;
        if (act) pref[row0 + (size_t)q * b] = run;
        run += hv;
    }
    const int incl = wave_incl_scan_add(act ? run : 0);
    const int ex = incl - (act ? run : 0);
    const int64_t nodes = S * b;
    if (act) {
        cnt[(size_t)g * nodes + u * b + c] = run;
        off_new[(size_t)g * (nodes + 1) + u * b + c] = off_prev[(size_t)g * (S + 1) + u] + ex;
    }
    if (u == S - 1 && c == 0) off_new[(size_t)g * (nodes + 1) + nodes] = (int32_t)n;
}

__global__ __launch_bounds__(kPiece) void k_scatter(const Piece *__restrict__ pieces, const int32_t *__restrict__ total,
                                                    const uint8_t *__restrict__ child, const uint8_t *__restrict__ lrank,
                                                    const int32_t *__restrict__ pref, const int32_t *__restrict__ off_new,
                                                    const int32_t *__restrict__ perm_prev, int32_t *__restrict__ perm_new,
                                                    int64_t S, int64_t NPmax, int b, int64_t n) {
    const int g = blockIdx.y;
    const int64_t p = blockIdx.x;
    if (p >= total[g]) return;
    const Piece pc = pieces[(size_t)g * NPmax + p];
    if (threadIdx.x >= pc.len) return;
    const int64_t posn = (int64_t)pc.start + threadIdx.x;
    const int c = child[(size_t)g * n + posn];
    const int64_t nodes = S * b;
    const int64_t dest = (int64_t)off_new[(size_t)g * (nodes + 1) + (int64_t)pc.u * b + c] +
                         pref[((size_t)g * NPmax + p) * b + c] + lrank[(size_t)g * n + posn];
    perm_new[(size_t)g * n + dest] = perm_prev[(size_t)g * n + posn];
}

// Centroid = fl32(sum of member latents / count), members in ascending key
// order, double accumulation, lane = latent dimension.  A node without
// members keeps its centroid.
//
// mean_span: one wave walks the consecutive nodes v0 .. v0+nv-1 (one node, or
// all children of one parent), whose members are contiguous in perm.  Members
// come 64 at a time: one coalesced load of their perm entries, then 64 row
// loads in flight, staged in the wave's LDS slice `zs` (lane x keeps column
// x, so only the lane itself reads back what it wrote) and added in a rolled
// loop.  Node boundaries (at most 65) are held one per lane and read with
// readlane, so crossing one costs no load.
LSA_DEV void mean_span(const int32_t *__restrict__ o, const int32_t *__restrict__ pm, const float *__restrict__ Zg,
                       float *__restrict__ Cg, int64_t v0, int nv, int r, float *zs) {
    const int x = lane_id();
    const int32_t t_begin = o[v0];
    const int32_t t_end = o[v0 + nv];
    // lane c: start of node v0 + c (lane nv and above: the end of the span)
    const int32_t ol = (x < nv) ? o[v0 + x] : t_end;
    int cur = 0;                                         // node being summed (relative to v0)
    int32_t start = t_begin;
    int32_t end = __builtin_amdgcn_readlane(ol, min(1, 63));
    if (nv == 1) end = t_end;
    double acc = 0.0;
    auto finish = [&]() {
        if (end > start && x < r) Cg[(size_t)(v0 + cur) * r + x] = (float)(acc / (double)(end - start));
        acc = 0.0;
        ++cur;
        start = end;
        end = (cur + 1 < nv) ? __builtin_amdgcn_readlane(ol, cur + 1) : t_end;
    };
    while (cur < nv && end == start) finish();          // leading empty nodes
    for (int32_t t0 = t_begin; t0 < t_end; t0 += 64) {
        const int nb = min(64, t_end - t0);
        const int32_t jl = (x < nb) ? pm[t0 + x] : 0;
        float zv[64];
#pragma unroll
        for (int q = 0; q < 64; ++q) {
            const int32_t j = __builtin_amdgcn_readlane(jl, q);
            zv[q] = (q < nb && x < r) ? Zg[(size_t)j * r + x] : 0.0f;
        }
#pragma unroll
        for (int q = 0; q < 64; ++q) zs[q * 64 + x] = zv[q];
        for (int q = 0; q < nb; ++q) {
            acc = acc + (double)zs[q * 64 + x];
            if (t0 + q + 1 == end) {
                finish();
                while (cur < nv && end == start) finish();   // empty nodes in between
            }
        }
    }
}

// Waves over spans: parent mode, one wave per parent (its b children);
// otherwise one wave per node.
__global__ __launch_bounds__(256) void k_mean(const int32_t *__restrict__ off_new, const int32_t *__restrict__ cnt,
                                              const int32_t *__restrict__ perm_new, const float *__restrict__ Z,
                                              float *__restrict__ C, int64_t S, int b, int r, int64_t n, int parent_mode) {
    __shared__ float zs[4][64 * 64];
    const int g = blockIdx.y;
    const int64_t wv = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    const int64_t nodes = S * b;
    const int32_t *o = off_new + (size_t)g * (nodes + 1);
    const int32_t *pm = perm_new + (size_t)g * n;
    const float *Zg = Z + (size_t)g * n * r;
    float *Cg = C + (size_t)g * nodes * r;
    (void)cnt;
    if (parent_mode) {
        if (wv >= S) return;
        mean_span(o, pm, Zg, Cg, wv * b, b, r, zs[threadIdx.x / kWave]);
    } else {
        if (wv >= nodes) return;
        mean_span(o, pm, Zg, Cg, wv, 1, r, zs[threadIdx.x / kWave]);
    }
}

// One workgroup per node, for levels whose nodes hold thousands of members.
// Waves 1..3 gather 192 member rows a round (perm entries fetched one round
// ahead) into LDS; wave 0 adds the previous round's rows in member order
// while the next round's loads are in flight.
constexpr int kMeanRound = 3 * 64;

__global__ __launch_bounds__(256) void k_mean_wg(const int32_t *__restrict__ off_new, const int32_t *__restrict__ cnt,
                                                 const int32_t *__restrict__ perm_new, const float *__restrict__ Z,
                                                 float *__restrict__ C, int64_t nodes, int r, int64_t n) {
    __shared__ float buf[kMeanRound * 64];
    const int g = blockIdx.y;
    const int64_t v = blockIdx.x;
    const int32_t cv = cnt[(size_t)g * nodes + v];
    if (cv <= 0) return;
    const int32_t s0 = off_new[(size_t)g * (nodes + 1) + v];
    const int32_t *pm = perm_new + (size_t)g * n + s0;
    const float *Zg = Z + (size_t)g * n * r;
    const int w = threadIdx.x / kWave, x = lane_id();
    const int rounds = (cv + kMeanRound - 1) / kMeanRound;
    float zr[64];
    auto perm_of = [&](int k) -> int32_t {
        const int e = k * kMeanRound + (w - 1) * 64 + x;
        return (w > 0 && e < cv) ? pm[e] : 0;
    };
    auto load_rows = [&](int k, int32_t jl) {
        const int nb = min(64, cv - (k * kMeanRound + (w - 1) * 64));
#pragma unroll
        for (int q = 0; q < 64; ++q) {
            const int32_t j = __builtin_amdgcn_readlane(jl, q);
            zr[q] = (q < nb && x < r) ? Zg[(size_t)j * r + x] : 0.0f;
        }
    };
    int32_t jnext = 0;
    if (w > 0) {
        const int32_t j0 = perm_of(0);
        jnext = perm_of(1);
        load_rows(0, j0);
    }
    double acc = 0.0;
    for (int k = 0; k < rounds; ++k) {
        if (w > 0) {
#pragma unroll
            for (int q = 0; q < 64; ++q) buf[((w - 1) * 64 + q) * 64 + x] = zr[q];
        }
        __syncthreads();
        if (w > 0 && k + 1 < rounds) {
            const int32_t jl = jnext;
            jnext = perm_of(k + 2);
            load_rows(k + 1, jl);
        }
        if (w == 0) {
            const int nb = min(kMeanRound, cv - k * kMeanRound);
            int q = 0;
            for (; q + 8 <= nb; q += 8) {
                float t[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) t[u] = buf[(q + u) * 64 + x];
#pragma unroll
                for (int u = 0; u < 8; ++u) acc = acc + (double)t[u];
            }
            for (; q < nb; ++q) acc = acc + (double)buf[q * 64 + x];
        }
        __syncthreads();
    }
    if (w == 0 && x < r) C[((size_t)g * nodes + v) * r + x] = (float)(acc / (double)cv);
}

// ---------------------------------------------------------------- host driver
static inline int64_t ipow64(int64_t b, int e) { int64_t v = 1; while (e-- > 0) v *= b; return v; }
static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct BuildWs {
    float *Z;
    int32_t *permA, *permB, *offA, *offB, *np, *pbase, *total, *hist, *pref;
    uint8_t *child, *lrank;
    Piece *pieces;
    size_t bytes;
};

static BuildWs carve_build_ws(char *base, int64_t n, int h, int r, int b, int L) {
    const int64_t Smax = ipow64(b, L - 1);
    const int64_t NPmax = (n + kPiece - 1) / kPiece + Smax;
    size_t cur = 0;
    BuildWs w{};
    auto take = [&](size_t bytes) { char *p = base ? base + cur : nullptr; cur = align256(cur + bytes); return p; };
    w.Z = (float *)take(sizeof(float) * (size_t)h * n * r);
    w.permA = (int32_t *)take(sizeof(int32_t) * (size_t)h * n);
    w.permB = (int32_t *)take(sizeof(int32_t) * (size_t)h * n);
    w.offA = (int32_t *)take(sizeof(int32_t) * (size_t)h * (Smax + 1));
    w.offB = (int32_t *)take(sizeof(int32_t) * (size_t)h * (Smax + 1));
    w.np = (int32_t *)take(sizeof(int32_t) * (size_t)h * Smax);
    w.pbase = (int32_t *)take(sizeof(int32_t) * (size_t)h * Smax);
    w.total = (int32_t *)take(sizeof(int32_t) * (size_t)h);
    w.pieces = (Piece *)take(sizeof(Piece) * (size_t)h * NPmax);
    w.hist = (int32_t *)take(sizeof(int32_t) * (size_t)h * NPmax * b);
    w.pref = (int32_t *)take(sizeof(int32_t) * (size_t)h * NPmax * b);
    w.child = (uint8_t *)take((size_t)h * n);
    w.lrank = (uint8_t *)take((size_t)h * n);
    w.bytes = cur;
    return w;
}

int64_t build_workspace_bytes(int64_t n, int h, int r, int b, int L) {
    return (int64_t)carve_build_ws(nullptr, n, h, r, b, L).bytes;
}

static inline unsigned grid1(int64_t tot, int bs) {
    int64_t g = (tot + bs - 1) / bs;
    if (g > (1 << 20)) g = 1 << 20;
    if (g < 1) g = 1;
    return (unsigned)g;
}

// The matrix-core projection: d = 128 with the weights in registers and
// 128 keys a workgroup (66 KB of LDS: two workgroups a compute unit), other
// d with 64 keys a workgroup.
template <typename T, int KB, int NQ>
static hipError_t launch_project_mfma(const T *K, int64_t n, int h, int d, const float *W, float *Z,
                                      hipStream_t st) {
    const size_t lds = sizeof(float) * (size_t)d * (16 * KB + 1);
    if (lds > 65536) {
        const hipError_t e = hipFuncSetAttribute((const void *)k_project_mfma<T, KB, NQ>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    const dim3 grid((unsigned)((n + 16 * KB - 1) / (16 * KB)), (unsigned)h);
    hipLaunchKernelGGL((k_project_mfma<T, KB, NQ>), grid, dim3(256), lds, st, K, W, Z, n, d);
    return hipSuccess;
}

static hipError_t project_mfma(const void *K, int dtype, int64_t n, int h, int d, const float *W, float *Z,
                               hipStream_t st) {
    if (dtype == 0)
        return d == 128 ? launch_project_mfma<float, 8, 32>((const float *)K, n, h, d, W, Z, st)
                        : launch_project_mfma<float, 4, 0>((const float *)K, n, h, d, W, Z, st);
    return d == 128 ? launch_project_mfma<bf16_t, 8, 32>((const bf16_t *)K, n, h, d, W, Z, st)
                    : launch_project_mfma<bf16_t, 4, 0>((const bf16_t *)K, n, h, d, W, Z, st);
}

hipError_t build_index(const void *K, int dtype, int64_t n, int h, int d, const float *W, int r, int b, int L,
                       int iters, char *index, const int64_t *centroid_off, const int64_t *count_off,
                       int64_t leaf_off_off, int64_t perm_off, void *ws, hipStream_t st) {
    BuildWs w = carve_build_ws((char *)ws, n, h, r, b, L);
    const dim3 pg((unsigned)((n + 31) / 32), (unsigned)h);
    if (r == 64 && d % 8 == 0 && d <= kPjMaxD) {
        const hipError_t e = project_mfma(K, dtype, n, h, d, W, w.Z, st);
        if (e != hipSuccess) return e;
    } else if (dtype == 0) {
        hipLaunchKernelGGL(k_project<float>, pg, dim3(256), 0, st, (const float *)K, W, w.Z, n, d, r);
    } else {
        hipLaunchKernelGGL(k_project<bf16_t>, pg, dim3(256), 0, st, (const bf16_t *)K, W, w.Z, n, d, r);
    }
    hipLaunchKernelGGL(k_iota, dim3(grid1(n * h, 256)), dim3(256), 0, st, w.permA, n, h);
    hipLaunchKernelGGL(k_root_off, dim3(1), dim3(64), 0, st, w.offA, n, h);
    int32_t *prev_perm = w.permA, *prev_off = w.offA;
    int32_t *idx_perm = (int32_t *)(index + perm_off);
    int32_t *idx_leaf = (int32_t *)(index + leaf_off_off);
    for (int l = 1; l <= L; ++l) {
        const int64_t S = ipow64(b, l - 1);
        const int64_t nodes = S * b;
        const int64_t NPmax = (n + kPiece - 1) / kPiece + S;
        int32_t *next_perm = (l == L) ? idx_perm : (prev_perm == w.permA ? w.permB : w.permA);
        int32_t *next_off = (l == L) ? idx_leaf : (prev_off == w.offA ? w.offB : w.offA);
        float *C = (float *)(index + centroid_off[l]);
        int32_t *cnt = (int32_t *)(index + count_off[l]);
        hipLaunchKernelGGL(k_piece_count, dim3(grid1(S * h, 256)), dim3(256), 0, st, prev_off, w.np, S, h);
        hipLaunchKernelGGL(k_scan_heads, dim3(h), dim3(1024), 0, st, w.np, w.pbase, w.total, S);
        hipLaunchKernelGGL(k_piece_fill, dim3((unsigned)((NPmax + 255) / 256), (unsigned)h), dim3(256), 0, st, w.pbase,
                           w.np, prev_off, w.total, w.pieces, S, NPmax);
        hipLaunchKernelGGL(k_init, dim3(grid1(nodes * h * r, 256)), dim3(256), 0, st, prev_off, prev_perm, w.Z, C, S, b,
                           r, n, h);
        const bool parent_mode = S * h >= 1024;
        const int64_t mean_waves = parent_mode ? S : nodes;
        const bool wg_mean = n >= 2048 * nodes;        // thousands of members per node
        for (int t = 0; t < iters; ++t) {
            hipLaunchKernelGGL(k_assign, dim3((unsigned)NPmax, (unsigned)h), dim3(kPiece), 0, st, w.pieces, w.total,
                               prev_off, prev_perm, w.Z, C, w.child, w.lrank, w.hist, S, NPmax, b, r, n);
            hipLaunchKernelGGL(k_seg_prefix, dim3((unsigned)((S + 3) / 4), (unsigned)h), dim3(256), 0, st, w.pbase, w.np,
                               w.hist, w.pref, prev_off, next_off, cnt, S, NPmax, b, n);
            hipLaunchKernelGGL(k_scatter, dim3((unsigned)NPmax, (unsigned)h), dim3(kPiece), 0, st, w.pieces, w.total,
                               w.child, w.lrank, w.pref, next_off, prev_perm, next_perm, S, NPmax, b, n);
            if (wg_mean)
                hipLaunchKernelGGL(k_mean_wg, dim3((unsigned)nodes, (unsigned)h), dim3(256), 0, st, next_off, cnt,
                                   next_perm, w.Z, C, nodes, r, n);
            else
                hipLaunchKernelGGL(k_mean, dim3((unsigned)((mean_waves + 3) / 4), (unsigned)h), dim3(256), 0, st,
                                   next_off, cnt, next_perm, w.Z, C, S, b, r, n, parent_mode ? 1 : 0);
        }
        prev_perm = next_perm;
        prev_off = next_off;
    }
    return hipGetLastError();
}

}  // namespace lsa
