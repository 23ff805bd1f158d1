// Top-down selection over the cluster tree (gfx950).
//
// A query scores only a few clusters per level, starting at the root, and
// descends the most promising branches to the leaves ("Latent Sparse
// Attention Breaks Through the Million-Token Context Bottleneck",
// kongchang.com, section "How LSA Sidesteps Per-Key Scoring with Hierarchical
// Clustering"); with a fixed budget per level, a fixed number of original keys
// is then retrieved from the chosen clusters ("Latent sparse attention",
// bdtechtalks.com, section "How latent sparse attention works"), and causal
// attention only sees earlier tokens (same page, "The compute bottleneck of
// sparse attention").
//
// One workgroup per (query row, KV head): the group's mean query is projected
// into the latent space, each level's candidates are scored with double
// accumulation, the best `beam` are kept by a bitonic sort of 64-bit
// (score, id) keys in LDS, and at the leaf level the candidate leaves are
// ordered, their eligible members counted and prefix-summed, and each leaf's
// taken members written at its prefix offset (retrieval order).
#include "common.h"
#include "internal.h"

namespace lsa {

struct SelectArgs {
    const void *Q;
    int64_t m;
    int h_q, h_kv, d;
    const int32_t *q_pos;
    const char *index;
    int64_t n;
    int r, b, L;
    int64_t nodes[8];
    int64_t centroid_off[8];
    int64_t count_off[8];
    int64_t leaf_off_off, perm_off;
    const float *W;
    int beam, k;
    int32_t *sel;
    int32_t *sel_count;
    float *sel_cutoff;
};

// u . row in double, ascending index; fp32 x fp32 products are exact in double.
// All loads of a row are issued before the first FMA.
LSA_DEV float score_row(const float *u, const float *__restrict__ row, int r) {
    double s = 0.0;
    if ((r & 3) == 0) {
        const float4 *row4 = reinterpret_cast<const float4 *>(row);
        float4 v[16];
#pragma unroll
        for (int x = 0; x < 16; ++x)
            if (4 * x < r) v[x] = row4[x];
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            if (4 * x < r) {
                s = fma((double)u[4 * x + 0], (double)v[x].x, s);
                s = fma((double)u[4 * x + 1], (double)v[x].y, s);
                s = fma((double)u[4 * x + 2], (double)v[x].z, s);
                s = fma((double)u[4 * x + 3], (double)v[x].w, s);
            }
        }
    } else {
        for (int x = 0; x < r; ++x) s = fma((double)u[x], (double)row[x], s);
    }
    return (float)s;
}

// number of entries <= key in an ascending array
LSA_DEV int count_le(const int32_t *a, int len, int32_t key) {
    int lo = 0, hi = len;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (a[mid] <= key) lo = mid + 1; else hi = mid;
    }
    return lo;
}

template <typename T, int CMAX>
__global__ __launch_bounds__(256) void k_select(SelectArgs A) {
    __shared__ float qbar_s[256];
    __shared__ float u_s[64];
    __shared__ uint64_t keys[CMAX];
    __shared__ int32_t aux[CMAX + 1];
    __shared__ int scratch[8];
    __shared__ int nc_s;
    __shared__ float cut_s;

    const int64_t i = blockIdx.x;
    const int g = blockIdx.y;
    const int G = A.h_q / A.h_kv;
    const int d = A.d, r = A.r, b = A.b, L = A.L;
    const T *Q = (const T *)A.Q;

    // group mean query, then its latent u = fl32(qbar . W_g)
    for (int t = threadIdx.x; t < d; t += blockDim.x) {
        double s = 0.0;
        for (int h = 0; h < G; ++h) s = s + (double)to_float(Q[((size_t)i * A.h_q + (size_t)g * G + h) * d + t]);
        qbar_s[t] = (float)(s / (double)G);
    }
    __syncthreads();
    const float *Wg = A.W + (size_t)g * d * r;
    for (int c = threadIdx.x; c < r; c += blockDim.x) {
        double s = 0.0;
        for (int t = 0; t < d; ++t) s = fma((double)qbar_s[t], (double)Wg[(size_t)t * r + c], s);
        u_s[c] = (float)s;
    }
    // level-1 candidates: the root's non-empty children, in id order
    if (threadIdx.x < kWave) {
        const int32_t *cnt1 = (const int32_t *)(A.index + A.count_off[1]) + (size_t)g * A.nodes[1];
        const bool f = threadIdx.x < b && cnt1[threadIdx.x] > 0;
        const uint64_t msk = __ballot(f);
        if (f) keys[__popcll(msk & lanemask_lt())] = make_key(0.0f, (uint32_t)threadIdx.x);
        if (threadIdx.x == 0) nc_s = __popcll(msk);
    }
    if (threadIdx.x == 0) cut_s = -INFINITY;
    __syncthreads();

    int nc = nc_s;
    for (int l = 1; l <= L; ++l) {
        const float *Cl = (const float *)(A.index + A.centroid_off[l]) + (size_t)g * A.nodes[l] * r;
        for (int idx = threadIdx.x; idx < nc; idx += blockDim.x) {
            const uint32_t v = key_id(keys[idx]);
            keys[idx] = make_key(score_row(u_s, Cl + (size_t)v * r, r), v);
        }
        const int N = next_pow2(nc);
        for (int idx = nc + threadIdx.x; idx < N; idx += blockDim.x) keys[idx] = 0ull;
        __syncthreads();
        block_bitonic_sort<uint64_t, true>(keys, N);
        if (l == L) break;
        // keep the best min(beam, nc); their non-empty children are next
        const int keep = min(A.beam, nc);
        for (int t = threadIdx.x; t < keep; t += blockDim.x) aux[t] = (int32_t)key_id(keys[t]);
        __syncthreads();
        const int32_t *cn = (const int32_t *)(A.index + A.count_off[l + 1]) + (size_t)g * A.nodes[l + 1];
        const int tot = keep * b;
        const int chunk = (tot + blockDim.x - 1) / blockDim.x;
        const int s0 = min(tot, (int)threadIdx.x * chunk), s1 = min(tot, s0 + chunk);
        int local = 0;
        for (int e = s0; e < s1; ++e) local += cn[(int64_t)aux[e / b] * b + (e % b)] > 0;
        int total;
        int w = block_excl_scan(local, scratch, &total);
        for (int e = s0; e < s1; ++e) {
            const int64_t v = (int64_t)aux[e / b] * b + (e % b);
            if (cn[v] > 0) keys[w++] = make_key(0.0f, (uint32_t)v);
        }
        nc = total;
        __syncthreads();
    }

    // fill: leaves in (score desc, id asc) order, eligible members ascending
    const int64_t nleaf = A.nodes[L];
    const int32_t *lo = (const int32_t *)(A.index + A.leaf_off_off) + (size_t)g * (nleaf + 1);
    const int32_t *pm = (const int32_t *)(A.index + A.perm_off) + (size_t)g * A.n;
    const int32_t pos = A.q_pos[i];
    {
        const int chunk = (nc + blockDim.x - 1) / blockDim.x;
        const int s0 = min(nc, (int)threadIdx.x * chunk), s1 = min(nc, s0 + chunk);
        int el[16];
        int local = 0;
        for (int e = s0; e < s1; ++e) {
            const uint32_t v = key_id(keys[e]);
            const int32_t a = lo[v], z = lo[v + 1];
            const int c = count_le(pm + a, z - a, pos);
            el[e - s0] = c;
            local += c;
        }
        int total;
        int run = block_excl_scan(local, scratch, &total);
        for (int e = s0; e < s1; ++e) { aux[e] = run; run += el[e - s0]; }
        if (threadIdx.x == 0) { aux[nc] = total; nc_s = total; }
        __syncthreads();
    }
    const int avail = nc_s;
    const int count = min(A.k, avail);
    int32_t *out = A.sel + ((size_t)i * A.h_kv + g) * A.k;
    for (int e = threadIdx.x; e < nc; e += blockDim.x) {
        const int p0 = aux[e];
        if (p0 >= count) continue;
        const int p1 = aux[e + 1];
        const int take = min(p1 - p0, count - p0);
        const uint32_t v = key_id(keys[e]);
        const int32_t a = lo[v];
        for (int t = 0; t < take; ++t) out[p0 + t] = pm[a + t];
        if (count == A.k && p1 >= A.k) cut_s = key_score(keys[e]);
    }
    for (int t = count + threadIdx.x; t < A.k; t += blockDim.x) out[t] = -1;
    __syncthreads();
    if (threadIdx.x == 0) {
        A.sel_count[(size_t)i * A.h_kv + g] = count;
        if (A.sel_cutoff) A.sel_cutoff[(size_t)i * A.h_kv + g] = cut_s;
    }
}

hipError_t select_keys(const void *Q, int dtype, int64_t m, int h_q, int d, const int32_t *q_pos, const char *index,
                       int64_t n, int h_kv, int r, int b, int L, const int64_t *nodes, const int64_t *centroid_off,
                       const int64_t *count_off, int64_t leaf_off_off, int64_t perm_off, const float *W, int beam,
                       int k, int32_t *sel, int32_t *sel_count, float *sel_cutoff, hipStream_t st) {
    SelectArgs A{};
    A.Q = Q; A.m = m; A.h_q = h_q; A.h_kv = h_kv; A.d = d; A.q_pos = q_pos; A.index = index; A.n = n;
    A.r = r; A.b = b; A.L = L;
    for (int l = 0; l <= L; ++l) { A.nodes[l] = nodes[l]; A.centroid_off[l] = centroid_off[l]; A.count_off[l] = count_off[l]; }
    A.leaf_off_off = leaf_off_off; A.perm_off = perm_off; A.W = W; A.beam = beam; A.k = k;
    A.sel = sel; A.sel_count = sel_count; A.sel_cutoff = sel_cutoff;
    const dim3 grid((unsigned)m, (unsigned)h_kv);
    const int cmax = beam * b > b ? beam * b : b;
    const bool small = cmax <= 1024;
    if (dtype == 0) {
        if (small) hipLaunchKernelGGL((k_select<float, 1024>), grid, dim3(256), 0, st, A);
        else hipLaunchKernelGGL((k_select<float, 4096>), grid, dim3(256), 0, st, A);
    } else {
        if (small) hipLaunchKernelGGL((k_select<bf16_t, 1024>), grid, dim3(256), 0, st, A);
        else hipLaunchKernelGGL((k_select<bf16_t, 4096>), grid, dim3(256), 0, st, A);
    }
    return hipGetLastError();
}

}  // namespace lsa
