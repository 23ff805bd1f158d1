// Incremental insertion of appended keys into the cluster tree (gfx950).
//
// The key index is precomputed and then updated as the context grows ("Latent
// Sparse Attention Breaks Through the Million-Token Context Bottleneck",
// kongchang.com, section "How LSA Sidesteps Per-Key Scoring with Hierarchical
// Clustering").  A batch of m keys (positions n .. n + m - 1) is inserted:
//   * each key's latent (the build's projection) descends from the root to the
//     nearest non-empty child at every level (squared distance in double,
//     ties to the smaller child) against the centroids before the batch;
//   * every node on a path takes its new keys: c its old count and S the
//     double sum of their latents (keys ascending),
//     centroid = fl32((c * centroid + S) / (c + #new)), count = c + #new;
//   * each leaf's member list becomes its old members followed by its new
//     keys, and the member array's per-head stride grows from n to n + m.
//
// Kernels, in stream order:
//   k_ins_small    batches of up to kInsSmall keys: one workgroup per head
//                  stages W_g in LDS, descends every key (a wave per key,
//                  lane c scoring child c), then updates the nodes on the
//                  paths level by level (the batch's (node, key) pairs ranked
//                  in LDS, a wave per node and a lane per dimension) and
//                  places the new keys;
//   (larger batches) k_ins_descend, one wave per new key, k_ins_update, one
//                  workgroup per (level, head), and k_ins_place for the new
//                  keys' positions;
//   k_ins_move     the leaf offsets rewritten in place (old offset plus the
//                  new keys in earlier leaves), and the member array moved in
//                  place to its [h][n + m] layout: every member moves to a
//                  slot at or above its old one, so the array is cut into
//                  chunks taken from the top down; a workgroup reads a
//                  chunk's sources into registers, marks the chunk read, and
//                  writes it once the chunks above that read from its range
//                  are marked.
#include <algorithm>
#include <atomic>

#include "common.h"
#include "internal.h"

namespace lsa {

namespace {

constexpr int kInsMax = 4096;      // keys per batch (the update kernel sorts them in LDS)
constexpr int kInsSmall = 16;      // batches up to this size take k_ins_small
constexpr int kInsRS = 68;         // row stride of k_ins_small's child-row tiles (floats)
constexpr int kMvPer = 32;         // members a thread of k_ins_move carries
constexpr int kMvChunk = 256 * kMvPer;
constexpr int kMvSpin = 1 << 24;   // bound of a chunk's wait for the chunks above it

struct InsArgs {
    int64_t m, n;                  // new keys, old keys
    int h, r, b, L;
    int64_t nleaf;
    char *index;
    int64_t nodes[8], centroid_off[8], count_off[8];
    int64_t leaf_off_off, perm_off;
    const void *K;                 // [h][m][d] the new keys
    int d, dtype;
    const float *W;                // [h][d][r]
    float *Z;                      // [h][m][r] latents of the new keys
    int32_t *path;                 // [h][m][L] node of each new key per level
    uint64_t *slist;               // [h][kInsMax] (leaf << 32 | key) sorted, level L
    int32_t *qpos, *qid;           // [h][kInsMax] new position and key id of each sorted new key
    int32_t *flags;                // [nchunks] chunk-read marks of k_ins_move (cleared by the kernel before it)
    int64_t nchunks;
};

// the rows of a node's children (lane c: child c; 16-byte loads when r = 64)
LSA_DEV void ins_child_row(const float *C, int64_t child, int r, float (&row)[64]) {
    if (r == 64) {
        const f4_t *c4 = reinterpret_cast<const f4_t *>(C + (size_t)child * 64);
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            const f4_t t4 = c4[x];
            row[4 * x] = t4.x; row[4 * x + 1] = t4.y; row[4 * x + 2] = t4.z; row[4 * x + 3] = t4.w;
        }
    } else {
#pragma unroll
        for (int x = 0; x < 64; ++x) row[x] = x < r ? C[(size_t)child * r + x] : 0.0f;
    }
}

// The key's latent in registers: 16-byte LDS reads of the row every lane
// shares (the row 16-byte aligned), issued together, so the distance chains
// below wait on no LDS read.
LSA_DEV void ins_load_z(const float *z, float (&zr)[64]) {
    const f4_t *z4 = reinterpret_cast<const f4_t *>(z);
#pragma unroll
    for (int x = 0; x < 16; ++x) {
        const f4_t t = z4[x];
        zr[4 * x] = t.x; zr[4 * x + 1] = t.y; zr[4 * x + 2] = t.z; zr[4 * x + 3] = t.w;
    }
}

// Squared distance in double, dimensions ascending, each difference and
// square rounded once (the build's assignment distance).
LSA_DEV double ins_sq_dist(const float (&z)[64], const float (&cs)[64], int r) {
#pragma clang fp contract(off)
    double dist = 0.0;
#pragma unroll
    for (int x = 0; x < 64; ++x) {
        if (x < r) {
            const double diff = (double)z[x] - (double)cs[x];
            const double sq = diff * diff;
            dist = dist + sq;
        }
    }
    return dist;
}

// The wave's nearest child: lane c holds child c's row (`ok`: a non-empty
// child); squared distance in double, ties to the smaller child.
LSA_DEV int ins_nearest(const float (&z)[64], const float (&row)[64], int r, bool ok) {
    const int lane = lane_id();
    // distances are >= 0, so their bit patterns order like the values
    uint64_t key = ok ? (uint64_t)__double_as_longlong(ins_sq_dist(z, row, r)) : ~0ull;
    int best = lane;
#pragma unroll
    for (int s = 1; s < kWave; s <<= 1) {
        uint64_t ok2;
        int ob;
        switch (s) {
            case 1: ok2 = xor_lane64<1>(key); ob = xor_lane_i<1>(best); break;
            case 2: ok2 = xor_lane64<2>(key); ob = xor_lane_i<2>(best); break;
            case 4: ok2 = xor_lane64<4>(key); ob = xor_lane_i<4>(best); break;
            case 8: ok2 = xor_lane64<8>(key); ob = xor_lane_i<8>(best); break;
            case 16: ok2 = xor_lane64<16>(key); ob = xor_lane_i<16>(best); break;
            default: ok2 = xor_lane64<32>(key); ob = xor_lane_i<32>(best); break;
        }
        if (ok2 < key || (ok2 == key && ob < best)) { key = ok2; best = ob; }
    }
    return best;
}

template <typename T>
__global__ __launch_bounds__(256) void k_ins_descend(InsArgs A) {
    __shared__ __attribute__((aligned(16))) float z_s[4][64];
    __shared__ __attribute__((aligned(16))) float k_s[4][256];
    const int g = blockIdx.y, wv = threadIdx.x / kWave, lane = lane_id();
    const int64_t j = (int64_t)blockIdx.x * 4 + wv;
    if (j >= A.m) return;                                   // whole waves only
    const int r = A.r, b = A.b, d = A.d;
    // Every load that does not depend on the key's path is issued first: the
    // level-1 children (the root's, the same for every key), the key and W.
    const float *C1 = (const float *)(A.index + A.centroid_off[1]) + (size_t)g * A.nodes[1] * r;
    const int32_t *cn1 = (const int32_t *)(A.index + A.count_off[1]) + (size_t)g * A.nodes[1];
    const int64_t child1 = min<int64_t>(lane, A.nodes[1] - 1);      // clamped: in bounds
    float row[64];
    ins_child_row(C1, child1, r, row);
    const int cnt1 = cn1[child1];
    // the latent, as the build projects keys: lane c sums k_i * W[i][c] in
    // double over i ascending (each product exact), rounded once.  W's first
    // 128 input rows are loaded before the key (clamped: in bounds).
    const float *Wg = A.W + (size_t)g * d * r + min(lane, r - 1);
    float wl[128];
#pragma unroll
    for (int u = 0; u < 128; ++u) wl[u] = Wg[(size_t)min(u, d - 1) * r];
    const T *kr = (const T *)A.K + ((size_t)g * A.m + j) * d;
    for (int i = lane; i < d; i += kWave) k_s[wv][i] = to_float(kr[i]);
    wave_sync();
    if (lane < r) {
        double acc = 0.0;
        for (int i0 = 0; i0 < d; i0 += 128) {
            if (i0 > 0) {
#pragma unroll
                for (int u = 0; u < 128; ++u) wl[u] = Wg[(size_t)min(i0 + u, d - 1) * r];
            }
#pragma unroll
            for (int u = 0; u < 128; ++u)
                if (i0 + u < d) acc = fma((double)k_s[wv][i0 + u], (double)wl[u], acc);
        }
        z_s[wv][lane] = (float)acc;
        A.Z[((size_t)g * A.m + j) * r + lane] = (float)acc;
    }
    wave_sync();
    float zr[64];
    ins_load_z(z_s[wv], zr);
    int64_t u = 0;
    for (int l = 1; l <= A.L; ++l) {
        const float *C = (const float *)(A.index + A.centroid_off[l]) + (size_t)g * A.nodes[l] * r;
        const int32_t *cn = (const int32_t *)(A.index + A.count_off[l]) + (size_t)g * A.nodes[l];
        const int64_t child = min<int64_t>(u * b + lane, A.nodes[l] - 1);      // clamped: in bounds
        int cnt = cnt1;
        if (l > 1) {
            ins_child_row(C, child, r, row);
            cnt = cn[child];
        }
        u = u * b + ins_nearest(zr, row, r, lane < b && cnt > 0);
        if (lane == 0) A.path[((size_t)g * A.m + j) * A.L + (l - 1)] = (int32_t)u;
    }
}

__global__ __launch_bounds__(256) void k_ins_update(InsArgs A) {
#pragma clang fp contract(off)
    __shared__ uint64_t ks[kInsMax];
    __shared__ int nseg_s;
    __shared__ int seg_s[kInsMax];
    const int l = blockIdx.x + 1, g = blockIdx.y, t = threadIdx.x;
    const int m = (int)A.m, r = A.r;
    const int N = next_pow2(max(m, 2));
    for (int e = t; e < N; e += blockDim.x)
        ks[e] = e < m ? ((uint64_t)(uint32_t)A.path[((size_t)g * m + e) * A.L + (l - 1)] << 32) | (uint32_t)e : ~0ull;
    if (t == 0) nseg_s = 0;
    __syncthreads();
    block_bitonic_sort<uint64_t, false>(ks, N);
    // runs of equal nodes (keys ascending inside a run)
    for (int e = t; e < m; e += blockDim.x)
        if (e == 0 || (ks[e] >> 32) != (ks[e - 1] >> 32)) seg_s[atomicAdd(&nseg_s, 1)] = e;
    if (l == A.L)
        for (int e = t; e < m; e += blockDim.x) A.slist[(size_t)g * kInsMax + e] = ks[e];
    __syncthreads();
    float *C = (float *)(A.index + A.centroid_off[l]) + (size_t)g * A.nodes[l] * r;
    int32_t *cn = (int32_t *)(A.index + A.count_off[l]) + (size_t)g * A.nodes[l];
    // one wave per run (node), lane x: dimension x
    const int wv = t / kWave, lane = lane_id();
    for (int q = wv; q < nseg_s; q += blockDim.x / kWave) {
        const int e0 = seg_s[q];
        const uint32_t v = (uint32_t)(ks[e0] >> 32);
        int e1 = e0 + 1;
        while (e1 < m && (uint32_t)(ks[e1] >> 32) == v) ++e1;
        const int c0 = cn[v];
        const double cd = (double)c0, cnew = (double)(c0 + (e1 - e0));
        if (lane < r) {
            double S = 0.0;
            for (int e = e0; e < e1; ++e) S = S + (double)A.Z[((size_t)g * m + (uint32_t)ks[e]) * r + lane];
            const double num = cd * (double)C[(size_t)v * r + lane] + S;
            C[(size_t)v * r + lane] = (float)(num / cnew);
        }
        wave_sync();
        if (lane == 0) cn[v] = c0 + (e1 - e0);
    }
}


// Positions of the sorted new keys of head g (k_ins_update wrote them to
// slist): the end of the key's leaf in the old member list plus the new keys
// before it; and the move's chunk marks cleared.
__global__ __launch_bounds__(256) void k_ins_place(InsArgs A) {
    const int g = blockIdx.y;
    const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g == 0)
        for (int64_t e = v; e < A.nchunks; e += (int64_t)gridDim.x * blockDim.x) A.flags[e] = 0;
    if (v >= A.m) return;
    const uint64_t *sl = A.slist + (size_t)g * kInsMax;
    const int32_t *lo = (const int32_t *)(A.index + A.leaf_off_off) + (size_t)g * (A.nleaf + 1);
    const uint32_t leaf = (uint32_t)(sl[v] >> 32);
    A.qpos[(size_t)g * kInsMax + v] = lo[leaf + 1] + (int32_t)v;
    A.qid[(size_t)g * kInsMax + v] = (int32_t)(A.n + (uint32_t)sl[v]);
}

// A batch of at most kInsSmall keys, one workgroup per head: descent (a wave
// per key), then per level the nodes on the paths updated (their (node, key)
// pairs ranked in LDS; a wave per node, lane = dimension, new keys summed in
// ascending key order), and the new keys' positions.  Same arithmetic as
// k_ins_descend and k_ins_update.
template <typename T>
__global__ __launch_bounds__(256) void k_ins_small(InsArgs A) {
#pragma clang fp contract(off)
    extern __shared__ __attribute__((aligned(16))) float dsm[];     // W_g [d][r], then a row tile per wave
    __shared__ __attribute__((aligned(16))) float k_s[4][256];
    __shared__ __attribute__((aligned(16))) float zl[kInsSmall][64];
    __shared__ int32_t path_s[kInsSmall][LSA_MAX_LEVELS];
    __shared__ uint64_t ks[LSA_MAX_LEVELS][kInsSmall];
    __shared__ int32_t seg_s[LSA_MAX_LEVELS][kInsSmall + 1];
    __shared__ int nseg_s[LSA_MAX_LEVELS + 1];
    const int g = blockIdx.x, tid = threadIdx.x, wv = tid / kWave, lane = lane_id();
    const int m = (int)A.m, r = A.r, b = A.b, d = A.d, L = A.L;
    float *Wsm = dsm;
    float *rt = dsm + (((size_t)d * r + 3) & ~(size_t)3) + (size_t)wv * 64 * kInsRS;   // this wave's row tile
    // the move's chunk marks, cleared before it runs
    for (int64_t e = (int64_t)g * blockDim.x + tid; e < A.nchunks; e += (int64_t)gridDim.x * blockDim.x) A.flags[e] = 0;
    // W_g into LDS (16-byte loads when they fit), the level-1 children's rows
    // issued behind them
    {
        const float *Wg = A.W + (size_t)g * d * r;
        const int nw = d * r;
        if ((nw & 3) == 0) {
            // eight 16-byte loads a thread in flight before their stores
            const f4_t *w4 = reinterpret_cast<const f4_t *>(Wg);
            f4_t *s4 = reinterpret_cast<f4_t *>(Wsm);
            const int n4 = nw / 4;
            for (int e0 = tid; e0 < n4; e0 += 8 * (int)blockDim.x) {
                f4_t t[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) t[u] = w4[min(e0 + u * (int)blockDim.x, n4 - 1)];   // (clamped: in bounds)
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (e0 + u * (int)blockDim.x < n4) s4[e0 + u * (int)blockDim.x] = t[u];
            }
        } else {
            for (int e = tid; e < nw; e += blockDim.x) Wsm[e] = Wg[e];
        }
    }
    const float *C1 = (const float *)(A.index + A.centroid_off[1]) + (size_t)g * A.nodes[1] * r;
    const int32_t *cn1 = (const int32_t *)(A.index + A.count_off[1]) + (size_t)g * A.nodes[1];
    const int64_t child1 = min<int64_t>(lane, A.nodes[1] - 1);      // clamped: in bounds
    float row1[64];
    ins_child_row(C1, child1, r, row1);
    const int cnt1 = cn1[child1];
    __syncthreads();
    for (int j = wv; j < m; j += 4) {
        const T *kr = (const T *)A.K + ((size_t)g * A.m + j) * d;
        for (int i = lane; i < d; i += kWave) k_s[wv][i] = to_float(kr[i]);
        wave_sync();
        // the latent, as the build projects keys: lane c sums k_i * W[i][c]
        // in double over i ascending (each product exact), rounded once
        if (lane < r) {
            double acc = 0.0;
            if (d % 16 == 0) {
                // 16 dims a round: the key's four 16-byte LDS reads (every
                // lane the same address) and the column's 16 reads issued
                // before the round's FMAs, the next round's during them
                const f4_t *k4 = reinterpret_cast<const f4_t *>(k_s[wv]);
                for (int i0 = 0; i0 < d; i0 += 16) {
                    f4_t kv[4];
                    float wc[16];
#pragma unroll
                    for (int q = 0; q < 4; ++q) kv[q] = k4[i0 / 4 + q];
#pragma unroll
                    for (int u = 0; u < 16; ++u) wc[u] = Wsm[(i0 + u) * r + lane];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        acc = fma((double)kv[q].x, (double)wc[4 * q], acc);
                        acc = fma((double)kv[q].y, (double)wc[4 * q + 1], acc);
                        acc = fma((double)kv[q].z, (double)wc[4 * q + 2], acc);
                        acc = fma((double)kv[q].w, (double)wc[4 * q + 3], acc);
                    }
                }
            } else {
                for (int i = 0; i < d; ++i) acc = fma((double)k_s[wv][i], (double)Wsm[i * r + lane], acc);
            }
            zl[j][lane] = (float)acc;
        }
        wave_sync();
        float zr[64];
        ins_load_z(zl[j], zr);
        int64_t u = 0;
        for (int l = 1; l <= L; ++l) {
            const float *C = (const float *)(A.index + A.centroid_off[l]) + (size_t)g * A.nodes[l] * r;
            const int32_t *cn = (const int32_t *)(A.index + A.count_off[l]) + (size_t)g * A.nodes[l];
            const int64_t child = min<int64_t>(u * b + lane, A.nodes[l] - 1);      // clamped: in bounds
            float row[64];
            int cnt;
            if (l == 1) {
#pragma unroll
                for (int x = 0; x < 64; ++x) row[x] = row1[x];
                cnt = cnt1;
            } else if (r % 4 == 0) {
                // the node's b children rows are one contiguous block: loaded
                // in 16-byte lines by the whole wave into its tile, then row
                // `lane` read back
                cnt = cn[child];
                const f4_t *blk = reinterpret_cast<const f4_t *>(C + (size_t)u * b * r);
                const int n4 = b * r / 4, q4 = r / 4;
                f4_t t[16];
#pragma unroll
                for (int x = 0; x < 16; ++x) t[x] = blk[min(lane + 64 * x, n4 - 1)];   // (clamped to the block)
#pragma unroll
                for (int x = 0; x < 16; ++x) {
                    const int e = lane + 64 * x;
                    if (e < n4) *reinterpret_cast<f4_t *>(rt + (e / q4) * kInsRS + 4 * (e % q4)) = t[x];
                }
                wave_sync();
#pragma unroll
                for (int x = 0; x < 16; ++x) {
                    const f4_t v = *reinterpret_cast<const f4_t *>(rt + min(lane, b - 1) * kInsRS + 4 * x);
                    row[4 * x] = v.x; row[4 * x + 1] = v.y; row[4 * x + 2] = v.z; row[4 * x + 3] = v.w;
                }
                wave_sync();
            } else {
                ins_child_row(C, child, r, row);
                cnt = cn[child];
            }
            u = u * b + ins_nearest(zr, row, r, lane < b && cnt > 0);
            if (lane == 0) path_s[j][l - 1] = (int32_t)u;
        }
    }
    __syncthreads();
    // the nodes on the paths (the descents all used the centroids as they
    // were before the batch): per level the (node, key) pairs ranked and cut
    // into runs, then every (level, run) updated at once, a wave each
    for (int l = 1; l <= L; ++l) {
        if (tid < m) {
            const uint64_t key = ((uint64_t)(uint32_t)path_s[tid][l - 1] << 32) | (uint32_t)tid;
            int rank = 0;
            for (int e = 0; e < m; ++e) rank += ((((uint64_t)(uint32_t)path_s[e][l - 1] << 32) | (uint32_t)e) < key) ? 1 : 0;
            ks[l - 1][rank] = key;
        }
    }
    __syncthreads();
    if (tid < L) {
        int ns = 0;
        for (int e = 0; e < m; ++e)
            if (e == 0 || (ks[tid][e] >> 32) != (ks[tid][e - 1] >> 32)) seg_s[tid][ns++] = e;
        seg_s[tid][ns] = m;
        nseg_s[tid] = ns;
    }
    __syncthreads();
    int tot_runs = 0;
    for (int l = 0; l < L; ++l) tot_runs += nseg_s[l];
    for (int t = wv; t < tot_runs; t += blockDim.x / kWave) {
        int l = 0, q = t;
        while (q >= nseg_s[l]) { q -= nseg_s[l]; ++l; }
        float *C = (float *)(A.index + A.centroid_off[l + 1]) + (size_t)g * A.nodes[l + 1] * r;
        int32_t *cn = (int32_t *)(A.index + A.count_off[l + 1]) + (size_t)g * A.nodes[l + 1];
        const int e0 = seg_s[l][q], e1 = seg_s[l][q + 1];
        const uint32_t v = (uint32_t)(ks[l][e0] >> 32);
        const int c0 = cn[v];
        const double cd = (double)c0, cnew = (double)(c0 + (e1 - e0));
        if (lane < r) {
            double S = 0.0;
            for (int e = e0; e < e1; ++e) S = S + (double)zl[(uint32_t)ks[l][e]][lane];
            const double num = cd * (double)C[(size_t)v * r + lane] + S;
            C[(size_t)v * r + lane] = (float)(num / cnew);
        }
        wave_sync();
        if (lane == 0) cn[v] = c0 + (e1 - e0);
    }
    if (tid < m) {
        // the sorted new key tid: after its leaf's old members and the new
        // keys before it (the leaf offsets are still the old ones)
        const int32_t *lo = (const int32_t *)(A.index + A.leaf_off_off) + (size_t)g * (A.nleaf + 1);
        const uint64_t key = ks[L - 1][tid];
        const uint32_t leaf = (uint32_t)(key >> 32);
        A.slist[(size_t)g * kInsMax + tid] = key;
        A.qpos[(size_t)g * kInsMax + tid] = lo[leaf + 1] + tid;
        A.qid[(size_t)g * kInsMax + tid] = (int32_t)(A.n + (uint32_t)key);
    }
}

// The leaf offsets and the member array, rewritten in place.  Leaf offset v
// of head g: old + new keys in leaves below v (one thread reads and writes
// each entry; the head's new-key leaves staged in LDS).  Member slot
// J = g (n + m) + j of the new flat array holds the new key placed at j, or
// the old member g n + j - c (c: new keys placed below j), whose index is
// never above J.  So the flat array is cut into chunks of kMvChunk slots,
// one per workgroup, chunk nchunks - 1 - w for workgroup w (the top first): a
// chunk's sources are read into registers, the chunk is marked read, and it
// is written once every chunk above that reads from its range (at most
// D = ceil(h m / kMvChunk) of them) is marked.  The mark is stored after, and
// computed from, every value the chunk read, and a chunk's stores are issued
// only after the loads that saw the marks above it returned, so no store can
// overtake a read of the same slot.  A chunk waits only on lower-numbered
// workgroups, which the dispatcher started first.
constexpr int kMvLo = 12;          // leaf offsets a thread rewrites (up to)
constexpr int kMvLoc = 8;          // new keys of a head inside one chunk held in registers (up to)
__global__ __launch_bounds__(256) void k_ins_move(InsArgs A) {
    __shared__ int32_t q_s[2][kInsMax];          // new-key positions of the chunk's first two heads
    __shared__ uint32_t lf_s[kInsMax];           // new-key leaves of one head
    __shared__ uint32_t chk_s[4];
    __shared__ int cb_s[2], nl_s[2];
    const int tid = threadIdx.x;
    const int m = (int)A.m;
    const int64_t nn = A.n + A.m, total = (int64_t)A.h * nn;
    const int64_t k = A.nchunks - 1 - blockIdx.x;
    const int g0 = (int)((k * kMvChunk) / nn);     // the chunk's first head
    const bool two = (k + 1) * kMvChunk <= (int64_t)(g0 + 2) * nn;   // the chunk spans at most two heads
    for (int e = tid; e < m; e += blockDim.x) {
        q_s[0][e] = A.qpos[(size_t)g0 * kInsMax + e];
        if (g0 + 1 < A.h) q_s[1][e] = A.qpos[(size_t)(g0 + 1) * kInsMax + e];
    }
    __syncthreads();
    // the run [cb, cb + nloc) of each head's sorted positions inside the chunk
    if (two && tid < 2) {
        const int g = g0 + tid;
        const int64_t jlo = max<int64_t>(k * kMvChunk - (int64_t)g * nn, 0);
        const int64_t jhi = min<int64_t>((k + 1) * kMvChunk - (int64_t)g * nn, nn);
        int cb = 0, ce = 0;
        if (g < A.h && jhi > 0) {
            int a = 0, z = m;
            while (a < z) { const int mid = (a + z) >> 1; if ((int64_t)q_s[tid][mid] < jlo) a = mid + 1; else z = mid; }
            cb = a;
            z = m;
            while (a < z) { const int mid = (a + z) >> 1; if ((int64_t)q_s[tid][mid] < jhi) a = mid + 1; else z = mid; }
            ce = a;
        }
        cb_s[tid] = cb;
        nl_s[tid] = ce - cb;
    }
    __syncthreads();
    int32_t *perm = (int32_t *)(A.index + A.perm_off);
    int32_t val[kMvPer];
    // (each path searches one address space and loads each member from one
    // chosen address, so no member load waits for another)
    if (two && nl_s[0] <= kMvLoc && nl_s[1] <= kMvLoc) {
        int32_t pa[kMvLoc], pb[kMvLoc];
#pragma unroll
        for (int u = 0; u < kMvLoc; ++u) {
            pa[u] = u < nl_s[0] ? q_s[0][cb_s[0] + u] : INT32_MAX;
            pb[u] = u < nl_s[1] ? q_s[1][cb_s[1] + u] : INT32_MAX;
        }
#pragma unroll
        for (int x = 0; x < kMvPer; ++x) {
            const int64_t J = min<int64_t>(k * kMvChunk + tid + 256 * x, total - 1);
            const bool second = J >= (int64_t)(g0 + 1) * nn;
            const int g = second ? g0 + 1 : g0;
            const int32_t j = (int32_t)(J - (int64_t)g * nn);
            int c = second ? cb_s[1] : cb_s[0], hit = -1;
#pragma unroll
            for (int u = 0; u < kMvLoc; ++u) {
                const int32_t p = second ? pb[u] : pa[u];
                hit = p == j ? c : hit;
                c += p < j ? 1 : 0;
            }
            const int32_t *src = hit >= 0 ? A.qid + (size_t)g * kInsMax + hit : perm + (size_t)g * A.n + (j - c);
            val[x] = *src;
        }
    } else if (two) {
#pragma unroll
        for (int x = 0; x < kMvPer; ++x) {
            const int64_t J = min<int64_t>(k * kMvChunk + tid + 256 * x, total - 1);
            const int h1 = J >= (int64_t)(g0 + 1) * nn ? 1 : 0, g = g0 + h1;
            const int64_t j = J - (int64_t)g * nn;
            int a = 0, z = m;                // new keys placed below j
            while (a < z) {
                const int mid = (a + z) >> 1;
                if ((int64_t)q_s[h1][mid] < j) a = mid + 1; else z = mid;
            }
            const bool isnew = a < m && q_s[h1][a] == j;
            const int32_t *src = isnew ? A.qid + (size_t)g * kInsMax + a : perm + (size_t)g * A.n + (j - a);
            val[x] = *src;
        }
    } else {
#pragma unroll
        for (int x = 0; x < kMvPer; ++x) {
            const int64_t J = min<int64_t>(k * kMvChunk + tid + 256 * x, total - 1);
            const int g = (int)(J / nn);
            const int64_t j = J - (int64_t)g * nn;
            const int32_t *q = A.qpos + (size_t)g * kInsMax;
            int a = 0, z = m;
            while (a < z) {
                const int mid = (a + z) >> 1;
                if ((int64_t)q[mid] < j) a = mid + 1; else z = mid;
            }
            const bool isnew = a < m && q[a] == j;
            const int32_t *src = isnew ? A.qid + (size_t)g * kInsMax + a : perm + (size_t)g * A.n + (j - a);
            val[x] = *src;
        }
    }
    // mark the chunk read: the mark depends on every value read
    uint32_t chk = 0;
#pragma unroll
    for (int x = 0; x < kMvPer; ++x) chk ^= (uint32_t)val[x];
    if ((tid & (kWave - 1)) == 0) chk_s[tid / kWave] = 0;
    __syncthreads();
    atomicXor(&chk_s[tid / kWave], chk);
    __syncthreads();
    if (tid == 0) {
        const uint32_t all = chk_s[0] ^ chk_s[1] ^ chk_s[2] ^ chk_s[3];
        __hip_atomic_store(A.flags + k, (all == 0x5bd1e995u && total < 0) ? 2 : 1, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    // leaf offsets of this workgroup's share, head by head
    {
        int32_t *lo = (int32_t *)(A.index + A.leaf_off_off);
        const int64_t nl = A.nleaf + 1, per = (nl + gridDim.x - 1) / gridDim.x;
        const int64_t v0 = (int64_t)blockIdx.x * per, v1 = min<int64_t>(nl, v0 + per);
        for (int g = 0; g < A.h; ++g) {
            for (int e = tid; e < m; e += blockDim.x) lf_s[e] = (uint32_t)(A.slist[(size_t)g * kInsMax + e] >> 32);
            __syncthreads();
            int32_t *lg = lo + (size_t)g * nl;
            for (int64_t v = v0 + tid; v < v1; v += blockDim.x) {
                int a = 0, z = m;                // new keys in leaves below v
                while (a < z) {
                    const int mid = (a + z) >> 1;
                    if (lf_s[mid] < (uint32_t)v) a = mid + 1; else z = mid;
                }
                lg[v] = v == A.nleaf ? (int32_t)nn : lg[v] + a;
            }
            __syncthreads();
        }
    }
    // then the chunks above that read from this one's range
    if (tid == 0) {
        const int64_t D = ((int64_t)A.h * A.m + kMvChunk - 1) / kMvChunk;
        for (int64_t k2 = k + 1; k2 <= min(k + D, A.nchunks - 1); ++k2)
            for (int spins = 0; spins < kMvSpin; ++spins)
                if (__hip_atomic_load(A.flags + k2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) break;
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < kMvPer; ++x) {
        const int64_t J = k * kMvChunk + tid + 256 * x;
        if (J < total) perm[J] = val[x];
    }
}

// k_ins_move for batches of at most kMvFew keys (the decode step's case):
// every head's new positions and leaves staged in LDS once, a member's shift
// counted over them in registers (no search), and the leaf offsets' loads
// issued with the members' reads: two rounds of loads a workgroup.
constexpr int kMvFew = 8;
constexpr int kMvFewHeads = 64;
__global__ __launch_bounds__(256) void k_ins_move_few(InsArgs A) {
    __shared__ int32_t pos_s[kMvFewHeads][kMvFew], leaf_s[kMvFewHeads][kMvFew];
    __shared__ uint32_t chk_s[4];
    const int tid = threadIdx.x;
    const int m = (int)A.m, h = A.h;
    const int64_t nn = A.n + A.m, total = (int64_t)h * nn;
    const int64_t k = A.nchunks - 1 - blockIdx.x;
    for (int e = tid; e < h * kMvFew; e += blockDim.x) {
        const int g = e / kMvFew, u = e % kMvFew;
        const bool in = u < m;
        pos_s[g][u] = in ? A.qpos[(size_t)g * kInsMax + u] : INT32_MAX;
        leaf_s[g][u] = in ? (int32_t)(A.slist[(size_t)g * kInsMax + u] >> 32) : INT32_MAX;
    }
    __syncthreads();
    int32_t *perm = (int32_t *)(A.index + A.perm_off);
    // the chunk's (at most two: n + m >= kMvChunk) heads: their new
    // positions in registers
    const int g0 = (int)((k * kMvChunk) / nn);
    const int g1 = min(g0 + 1, h - 1);
    int32_t pa[kMvFew], pb[kMvFew];
#pragma unroll
    for (int u = 0; u < kMvFew; ++u) { pa[u] = pos_s[g0][u]; pb[u] = pos_s[g1][u]; }
    int32_t val[kMvPer];
#pragma unroll
    for (int x = 0; x < kMvPer; ++x) {
        const int64_t J = min<int64_t>(k * kMvChunk + tid + 256 * x, total - 1);
        const bool second = J >= (int64_t)(g0 + 1) * nn;
        const int g = second ? g0 + 1 : g0;
        const int32_t j = (int32_t)(J - (int64_t)g * nn);
        int c = 0, hit = -1;
#pragma unroll
        for (int u = 0; u < kMvFew; ++u) {
            const int32_t p = second ? pb[u] : pa[u];
            c += p < j ? 1 : 0;
            hit = p == j ? u : hit;
        }
        // one load from the chosen address (a select between two loaded
        // values would wait for each load in turn)
        const int32_t *src = hit >= 0 ? A.qid + (size_t)g * kInsMax + hit : perm + (size_t)g * A.n + (j - c);
        val[x] = *src;
    }
    // the leaf offsets of this workgroup's share, loaded with the members
    int32_t *lo = (int32_t *)(A.index + A.leaf_off_off);
    const int64_t nl = A.nleaf + 1, nlt = (int64_t)h * nl, per = (nlt + gridDim.x - 1) / gridDim.x;
    const int64_t e0 = (int64_t)blockIdx.x * per, e1 = min<int64_t>(nlt, e0 + per);
    // (per <= min(kMvLo * 256, nl): registers, and within two heads)
    const int lg0 = (int)(e0 / nl), lg1 = min(lg0 + 1, h - 1);
    int32_t lv[kMvLo];
#pragma unroll
    for (int u = 0; u < kMvLo; ++u) {
        const int64_t e = e0 + tid + 256 * u;
        lv[u] = e < e1 ? lo[e] : 0;
    }
    // mark the chunk read: the mark depends on every member read
    uint32_t chk = 0;
#pragma unroll
    for (int x = 0; x < kMvPer; ++x) chk ^= (uint32_t)val[x];
    if ((tid & (kWave - 1)) == 0) chk_s[tid / kWave] = 0;
    __syncthreads();
    atomicXor(&chk_s[tid / kWave], chk);
    __syncthreads();
    if (tid == 0) {
        const uint32_t all = chk_s[0] ^ chk_s[1] ^ chk_s[2] ^ chk_s[3];
        __hip_atomic_store(A.flags + k, (all == 0x5bd1e995u && total < 0) ? 2 : 1, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    // leaf offset e = (head g, leaf v): old + new keys in leaves below v
    {
        int32_t la[kMvFew], lb[kMvFew];
#pragma unroll
        for (int u = 0; u < kMvFew; ++u) { la[u] = leaf_s[lg0][u]; lb[u] = leaf_s[lg1][u]; }
#pragma unroll
        for (int u = 0; u < kMvLo; ++u) {
            const int64_t e = e0 + tid + 256 * u;
            if (e < e1) {
                const bool second = e >= (int64_t)(lg0 + 1) * nl;
                const int64_t v = e - (int64_t)(second ? lg0 + 1 : lg0) * nl;
                int c = 0;
#pragma unroll
                for (int w = 0; w < kMvFew; ++w) c += (second ? lb[w] : la[w]) < v ? 1 : 0;
                lo[e] = v == A.nleaf ? (int32_t)nn : lv[u] + c;
            }
        }
    }
    // then the chunk above (the only one that reads from this one's range:
    // h m <= kMvChunk)
    if (tid == 0 && k + 1 < A.nchunks)
        for (int spins = 0; spins < kMvSpin; ++spins)
            if (__hip_atomic_load(A.flags + k + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) break;
    __syncthreads();
#pragma unroll
    for (int x = 0; x < kMvPer; ++x) {
        const int64_t J = k * kMvChunk + tid + 256 * x;
        if (J < total) perm[J] = val[x];
    }
}

inline size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

struct InsWs { float *Z; int32_t *path; uint64_t *slist; int32_t *qpos, *qid, *flags; size_t bytes; };

int64_t move_chunks(int64_t m, int64_t n, int h) { return ((int64_t)h * (n + m) + kMvChunk - 1) / kMvChunk; }

InsWs carve_ins_ws(char *base, int64_t m, int64_t n, int h, int r, int L, int64_t nleaf) {
    size_t cur = 0;
    InsWs w{};
    (void)nleaf;
    auto take = [&](size_t b) { char *p = base ? base + cur : nullptr; cur = a256(cur + b); return p; };
    w.Z = (float *)take(sizeof(float) * (size_t)h * m * r);
    w.path = (int32_t *)take(sizeof(int32_t) * (size_t)h * m * L);
    w.slist = (uint64_t *)take(sizeof(uint64_t) * (size_t)h * kInsMax);
    w.qpos = (int32_t *)take(sizeof(int32_t) * (size_t)h * kInsMax);
    w.qid = (int32_t *)take(sizeof(int32_t) * (size_t)h * kInsMax);
    w.flags = (int32_t *)take(sizeof(int32_t) * (size_t)move_chunks(m, n, h));
    w.bytes = cur;
    return w;
}

}  // namespace

int64_t insert_workspace_bytes(int64_t m, int64_t n, int h, int r, int L, int64_t nleaf) {
    return (int64_t)carve_ins_ws(nullptr, m, n, h, r, L, nleaf).bytes;
}

hipError_t index_insert(const void *K_new, int dtype, int64_t m, int d, const float *W, char *index, int64_t n, int h,
                        int r, int b, int L, const int64_t *nodes, const int64_t *centroid_off,
                        const int64_t *count_off, int64_t leaf_off_off, int64_t perm_off, void *ws, hipStream_t st) {
    InsArgs A{};
    A.m = m; A.n = n; A.h = h; A.r = r; A.b = b; A.L = L; A.nleaf = nodes[L]; A.index = index;
    for (int l = 0; l <= L; ++l) { A.nodes[l] = nodes[l]; A.centroid_off[l] = centroid_off[l]; A.count_off[l] = count_off[l]; }
    A.leaf_off_off = leaf_off_off; A.perm_off = perm_off;
    InsWs w = carve_ins_ws((char *)ws, m, n, h, r, L, A.nleaf);
    A.K = K_new; A.d = d; A.dtype = dtype; A.W = W;
    A.Z = w.Z; A.path = w.path; A.slist = w.slist; A.qpos = w.qpos; A.qid = w.qid; A.flags = w.flags;
    A.nchunks = move_chunks(m, n, h);
    if (m <= kInsSmall) {
        // (one workgroup per head; W_g in dynamic LDS, at most 256 x 64 floats:
        // the limit is raised once per device)
        const size_t shm = sizeof(float) * ((((size_t)d * r + 3) & ~(size_t)3) + 4 * 64 * (size_t)kInsRS);
        static std::atomic<int> attr_set[64];
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
        if (!attr_set[dev].load(std::memory_order_acquire)) {
            for (const void *f : {(const void *)k_ins_small<float>, (const void *)k_ins_small<bf16_t>}) {
                hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024);
                if (e != hipSuccess) return e;
            }
            attr_set[dev].store(1, std::memory_order_release);
        }
        if (dtype == 0) hipLaunchKernelGGL(k_ins_small<float>, dim3((unsigned)h), dim3(256), shm, st, A);
        else hipLaunchKernelGGL(k_ins_small<bf16_t>, dim3((unsigned)h), dim3(256), shm, st, A);
    } else {
        if (dtype == 0) hipLaunchKernelGGL(k_ins_descend<float>, dim3((unsigned)((m + 3) / 4), (unsigned)h), dim3(256), 0, st, A);
        else hipLaunchKernelGGL(k_ins_descend<bf16_t>, dim3((unsigned)((m + 3) / 4), (unsigned)h), dim3(256), 0, st, A);
        hipLaunchKernelGGL(k_ins_update, dim3((unsigned)L, (unsigned)h), dim3(256), 0, st, A);
        hipLaunchKernelGGL(k_ins_place, dim3((unsigned)std::max<int64_t>((std::max<int64_t>(m, 256) + 255) / 256, 1), (unsigned)h),
                           dim3(256), 0, st, A);
    }
    const int64_t nlt = (int64_t)h * (A.nleaf + 1), lper = (nlt + A.nchunks - 1) / A.nchunks;
    if (m <= kMvFew && h <= kMvFewHeads && (int64_t)h * m <= kMvChunk && n + m >= kMvChunk &&
        lper <= std::min<int64_t>(A.nleaf + 1, (int64_t)kMvLo * 256))
        hipLaunchKernelGGL(k_ins_move_few, dim3((unsigned)A.nchunks), dim3(256), 0, st, A);
    else
        hipLaunchKernelGGL(k_ins_move, dim3((unsigned)A.nchunks), dim3(256), 0, st, A);
    return hipGetLastError();
}

}  // namespace lsa
