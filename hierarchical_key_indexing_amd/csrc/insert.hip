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
//   k_ins_copy     the member array and leaf offsets to the workspace (16-byte
//                  copies of the contiguous [h][n] and [h][leaves + 1] arrays);
//   k_ins_descend  one wave per new key: its latent (lane c: dimension c,
//                  summed as the build's projection does), then lane c scores
//                  child c of the node at every level;
//   k_ins_update   one workgroup per (level, head): the batch's (node, key)
//                  pairs sorted, each node's run (one wave, a lane per
//                  dimension) summed in key order and its centroid and count
//                  rewritten;
//   k_ins_offsets  one thread per leaf: new offset = old offset + new keys in
//                  earlier leaves (binary search in the sorted leaf run); and
//                  the new position of every sorted new key (the end of its
//                  leaf in the old list plus the new keys before it);
//   k_ins_gather   one thread per slot of the new member list: the new key
//                  placed there, or the old member shifted by the number of
//                  new keys before the slot (binary search over the new keys'
//                  positions in LDS), coalesced reads and writes.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace lsa {

namespace {

constexpr int kInsMax = 4096;      // keys per batch (the update kernel sorts them in LDS)

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
    int32_t *perm_old;             // [h][n]
    int32_t *lo_old;               // [h][nleaf + 1]
    int32_t *qpos, *qid;           // [h][kInsMax] new position and key id of each sorted new key
};

// Flat copy of `count` ints from src to dst (both 16-byte aligned): 16-byte
// moves, then the tail.
LSA_DEV void copy_ints(int32_t *__restrict__ dst, const int32_t *__restrict__ src, int64_t count, int64_t t0,
                       int64_t stride) {
    const int64_t n4 = count / 4;
    const int4 *s4 = reinterpret_cast<const int4 *>(src);
    int4 *d4 = reinterpret_cast<int4 *>(dst);
    for (int64_t e = t0; e < n4; e += stride) d4[e] = s4[e];
    for (int64_t e = 4 * n4 + t0; e < count; e += stride) dst[e] = src[e];
}

__global__ __launch_bounds__(256) void k_ins_copy(InsArgs A) {
    const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x, stride = (int64_t)gridDim.x * blockDim.x;
    copy_ints(A.perm_old, (const int32_t *)(A.index + A.perm_off), (int64_t)A.h * A.n, t0, stride);
    copy_ints(A.lo_old, (const int32_t *)(A.index + A.leaf_off_off), (int64_t)A.h * (A.nleaf + 1), t0, stride);
}

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

template <typename T>
__global__ __launch_bounds__(256) void k_ins_descend(InsArgs A) {
    __shared__ float z_s[4][64];
    __shared__ float k_s[4][256];
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
        const bool ok = lane < b && cnt > 0;
        // distances are >= 0, so their bit patterns order like the values
        uint64_t key = ok ? (uint64_t)__double_as_longlong(sq_dist(z_s[wv], row, r)) : ~0ull;
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
        u = u * b + best;
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

// number of sorted leaf-run entries with leaf < v
LSA_DEV int leaf_lower(const uint64_t *sl, int m, uint32_t v) {
    int lo = 0, hi = m;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if ((uint32_t)(sl[mid] >> 32) < v) lo = mid + 1; else hi = mid;
    }
    return lo;
}

__global__ __launch_bounds__(256) void k_ins_offsets(InsArgs A) {
    const int g = blockIdx.y;
    const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int m = (int)A.m;
    const int64_t nn = A.n + A.m;
    const uint64_t *sl = A.slist + (size_t)g * kInsMax;
    const int32_t *lo = A.lo_old + (size_t)g * (A.nleaf + 1);
    if (v < m) {
        // sorted new key v: after its leaf's old members and the new keys before it
        const uint32_t leaf = (uint32_t)(sl[v] >> 32);
        A.qpos[(size_t)g * kInsMax + v] = lo[leaf + 1] + (int32_t)v;
        A.qid[(size_t)g * kInsMax + v] = (int32_t)(A.n + (uint32_t)sl[v]);
    }
    if (v > A.nleaf) return;
    int32_t *lo_new = (int32_t *)(A.index + A.leaf_off_off) + (size_t)g * (A.nleaf + 1);
    lo_new[v] = v == A.nleaf ? (int32_t)nn : lo[v] + leaf_lower(sl, m, (uint32_t)v);
}

constexpr int kInsStage = 1024;    // new-key positions staged in LDS by every gather workgroup (up to)

__global__ __launch_bounds__(256) void k_ins_gather(InsArgs A) {
    __shared__ int32_t q_s[kInsStage];
    const int g = blockIdx.y;
    const int m = (int)A.m;
    const int64_t nn = A.n + A.m;
    const int32_t *qp = A.qpos + (size_t)g * kInsMax;
    const bool staged = m <= kInsStage;
    if (staged) {
        for (int e = threadIdx.x; e < m; e += blockDim.x) q_s[e] = qp[e];
        __syncthreads();
    }
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= nn) return;
    // c = number of new keys placed before slot j (larger batches search the
    // positions in memory, where they stay cached)
    const int32_t *q = staged ? q_s : qp;
    int lo = 0, hi = m;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (q[mid] < j) lo = mid + 1; else hi = mid;
    }
    int32_t *perm_new = (int32_t *)(A.index + A.perm_off) + (size_t)g * nn;
    perm_new[j] = (lo < m && q[lo] == j) ? A.qid[(size_t)g * kInsMax + lo]
                                           : A.perm_old[(size_t)g * A.n + (j - lo)];
}

inline size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

struct InsWs { float *Z; int32_t *path; uint64_t *slist; int32_t *perm_old, *lo_old, *qpos, *qid; size_t bytes; };

InsWs carve_ins_ws(char *base, int64_t m, int64_t n, int h, int r, int L, int64_t nleaf) {
    size_t cur = 0;
    InsWs w{};
    auto take = [&](size_t b) { char *p = base ? base + cur : nullptr; cur = a256(cur + b); return p; };
    w.Z = (float *)take(sizeof(float) * (size_t)h * m * r);
    w.path = (int32_t *)take(sizeof(int32_t) * (size_t)h * m * L);
    w.slist = (uint64_t *)take(sizeof(uint64_t) * (size_t)h * kInsMax);
    w.perm_old = (int32_t *)take(sizeof(int32_t) * (size_t)h * n);
    w.lo_old = (int32_t *)take(sizeof(int32_t) * (size_t)h * (nleaf + 1));
    w.qpos = (int32_t *)take(sizeof(int32_t) * (size_t)h * kInsMax);
    w.qid = (int32_t *)take(sizeof(int32_t) * (size_t)h * kInsMax);
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
    A.Z = w.Z; A.path = w.path; A.slist = w.slist; A.perm_old = w.perm_old; A.lo_old = w.lo_old;
    A.qpos = w.qpos; A.qid = w.qid;
    const int64_t ncopy4 = ((int64_t)h * (n + A.nleaf + 1) + 3) / 4;
    hipLaunchKernelGGL(k_ins_copy, dim3((unsigned)std::min<int64_t>((ncopy4 + 255) / 256, 8192)), dim3(256), 0, st, A);
    if (dtype == 0) hipLaunchKernelGGL(k_ins_descend<float>, dim3((unsigned)((m + 3) / 4), (unsigned)h), dim3(256), 0, st, A);
    else hipLaunchKernelGGL(k_ins_descend<bf16_t>, dim3((unsigned)((m + 3) / 4), (unsigned)h), dim3(256), 0, st, A);
    hipLaunchKernelGGL(k_ins_update, dim3((unsigned)L, (unsigned)h), dim3(256), 0, st, A);
    const int64_t noff = std::max<int64_t>(A.nleaf + 1, m);
    hipLaunchKernelGGL(k_ins_offsets, dim3((unsigned)((noff + 255) / 256), (unsigned)h), dim3(256), 0, st, A);
    hipLaunchKernelGGL(k_ins_gather, dim3((unsigned)((n + m + 255) / 256), (unsigned)h), dim3(256), 0, st, A);
    return hipGetLastError();
}

}  // namespace lsa
