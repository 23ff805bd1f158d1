// Flat search over the leaves of the cluster tree (gfx950).
//
// Instead of descending the tree, the query is compared against every cluster
// centroid ("Latent sparse attention", bdtechtalks.com, section "How latent
// sparse attention works": flat search against hierarchical search).  The
// clusters are the tree's leaves: every non-empty leaf is scored, the leaves
// are visited in (score desc, id asc) order and the keys are retrieved exactly
// as in the top-down selection (retrieval range, k, sinks and window).
//
// Three kernels per batch of rows:
//   k_flat_latent  u = fl32(fl32(mean of the group's query heads) . W_g) per
//                  (row, KV head);
//   k_flat_score   1024 leaves x up to 64 rows of one KV head per workgroup:
//                  a leaf's centroid row is loaded once into registers and
//                  scored against every row's u (double accumulation in
//                  ascending index order, two rows at a time), and its members
//                  in each row's retrieval range are counted; writes the
//                  orderable score and min(count, k) of every (row, leaf);
//   k_flat_select  one workgroup per (row, KV head): weighted radix selection
//                  over the 64-bit keys (score, ~leaf), up to 11 bits a round,
//                  narrows the boundary to a bucket that fits in LDS together
//                  with every key above it; those keys are collected, sorted
//                  and filled in order.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace lsa {

namespace {

constexpr int kFlatLeaves = 1024;   // leaves per scoring workgroup
constexpr int kFlatRows = 64;       // rows per scoring workgroup
constexpr int kFlatList = 16384;    // keys collected per (row, KV head) in LDS
constexpr int kFlatBins = 2048;     // radix digits of up to 11 bits
constexpr int64_t kFlatBatch = 256; // rows per batch the workspace query sizes for

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
    uint32_t *sc;               // [mb][h_kv][nleaf] orderable scores
    uint16_t *wt;               // [mb][h_kv][nleaf] min(members in range, k); 0: not a candidate
    int32_t *sel, *sel_count;   // the batch's rows
    float *sel_cutoff;
};

template <typename T>
__global__ __launch_bounds__(256) void k_flat_latent(FlatArgs A) {
    __shared__ float qbar_s[256];
    const int64_t i = blockIdx.x;
    const int g = blockIdx.y;
    const int G = A.h_q / A.h_kv, d = A.d, r = A.r;
    const T *Q = (const T *)A.Q;
    for (int t = threadIdx.x; t < d; t += blockDim.x) {
        double s = 0.0;
        for (int h = 0; h < G; ++h) s = s + (double)to_float(Q[((size_t)i * A.h_q + (size_t)g * G + h) * d + t]);
        qbar_s[t] = (float)(s / (double)G);
    }
    __syncthreads();
    if ((int)threadIdx.x < r) {
        const float *Wg = A.W + (size_t)g * d * r;
        double s = 0.0;
        for (int t = 0; t < d; ++t) s = fma((double)qbar_s[t], (double)Wg[(size_t)t * r + threadIdx.x], s);
        A.U[((size_t)i * A.h_kv + g) * r + threadIdx.x] = (float)s;
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

// members of a leaf (ascending, pm[0..len), first and last given) in [rlo, rhi]
LSA_DEV int members_in(const int32_t *pm, int len, int32_t first, int32_t last, int32_t rlo, int32_t rhi) {
    if (first >= rlo && last <= rhi) return len;
    if (last < rlo || first > rhi) return 0;
    return max(0, count_le(pm, len, rhi) - count_le(pm, len, rlo - 1));
}

template <int RC>
__global__ __launch_bounds__(256) void k_flat_score(FlatArgs A) {
    __shared__ __attribute__((aligned(16))) float u_s[kFlatRows * 64];
    __shared__ int32_t rlo_s[kFlatRows], rhi_s[kFlatRows];
    const int64_t v0 = (int64_t)blockIdx.x * kFlatLeaves;
    const int64_t i0 = (int64_t)blockIdx.y * kFlatRows;
    const int g = blockIdx.z;
    const int r = RC > 0 ? RC : A.r;
    const int nr = (int)min<int64_t>(kFlatRows, A.mb - i0);
    for (int e = threadIdx.x; e < nr * r; e += blockDim.x)
        u_s[(e / r) * 64 + e % r] = A.U[((size_t)(i0 + e / r) * A.h_kv + g) * r + e % r];
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
    for (int j = 0; j < kFlatLeaves / 256; ++j) {
        const int64_t v = v0 + j * 256 + threadIdx.x;
        if (v >= A.nleaf) break;
        const size_t o = ((size_t)i0 * A.h_kv + g) * A.nleaf + v;
        const int c = cn[v];
        if (c <= 0) {
            for (int rr = 0; rr < nr; ++rr) A.wt[o + rr * rs] = 0;
            continue;
        }
        const int32_t a0 = lo[v], a1 = lo[v + 1];
        const int32_t first = pm[a0], last = pm[a1 - 1];
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
            A.sc[o + rr * rs] = e0 > 0 ? orderable((float)s0) : 0u;
            A.wt[o + rr * rs] = (uint16_t)min(e0, A.k);
            if (two) {
                A.sc[o + (rr + 1) * rs] = e1 > 0 ? orderable((float)s1) : 0u;
                A.wt[o + (rr + 1) * rs] = (uint16_t)min(e1, A.k);
            }
        }
    }
}

__global__ __launch_bounds__(256) void k_flat_select(FlatArgs A) {
    extern __shared__ __attribute__((aligned(16))) uint64_t lst[];   // [kFlatList] keys
    int *hw = reinterpret_cast<int *>(lst + kFlatList);               // [kFlatBins] weight per digit
    int *hc = hw + kFlatBins;                                          // [kFlatBins] keys per digit
    __shared__ int scr[8], nlist_s, res_s[4];
    __shared__ float cut_s;
    const int64_t gi = blockIdx.x;                 // row * h_kv + KV head, within the batch
    const int64_t i = gi / A.h_kv;
    const int g = (int)(gi % A.h_kv);
    const int tid = threadIdx.x;
    const uint32_t *sc = A.sc + (size_t)gi * A.nleaf;
    const uint16_t *wt = A.wt + (size_t)gi * A.nleaf;
    auto keyof = [&](int64_t v) -> uint64_t { return ((uint64_t)sc[v] << 32) | (uint64_t)(~(uint32_t)v); };

    // ---- boundary: the top `fixed` bits `prefix` of the key whose inclusion
    // brings the weight of the keys above it to k; refined until the keys above
    // the bucket and the bucket itself fit in LDS (at 64 bits the bucket is
    // one key: the keys are distinct)
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
        // thread t owns the digits nb-1-t*per .. nb-t*per-per (descending): the
        // weight of larger digits is an exclusive scan in thread order
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

    // ---- the keys above the bucket and in it (all candidates when their total
    // weight is below k: fewer than k of them), sorted descending
    if (tid == 0) { nlist_s = 0; cut_s = -INFINITY; }
    __syncthreads();
    for (int64_t v = tid; v < A.nleaf; v += blockDim.x) {
        if (wt[v] == 0) continue;
        const uint64_t key = keyof(v);
        if (!take_all && (key >> (64 - fixed)) < prefix) continue;
        const int at = atomicAdd(&nlist_s, 1);
        if (at < kFlatList) lst[at] = key;
    }
    __syncthreads();
    const int nl = min(nlist_s, kFlatList);
    const int np2 = next_pow2(max(nl, 2));
    for (int e = nl + tid; e < np2; e += blockDim.x) lst[e] = 0ull;
    __syncthreads();
    block_bitonic_sort<uint64_t, true>(lst, np2);

    // ---- fill: leaves in order, each giving its members in the retrieval range
    const AttnSet as = attn_set(A.q_pos[i], A.n, A.n_sink, A.window);
    const int32_t *lo = A.leaf_off + (size_t)g * (A.nleaf + 1);
    const int32_t *pm = A.perm + (size_t)g * A.n;
    const int chunk = (nl + blockDim.x - 1) / blockDim.x;
    const int e0 = min(nl, tid * chunk), e1 = min(nl, e0 + chunk);
    int local = 0;
    for (int e = e0; e < e1; ++e) local += wt[~(uint32_t)lst[e]];
    int total;
    int run = block_excl_scan(local, scr, &total);
    const int count = min(A.k, total);
    int32_t *out = A.sel + (size_t)gi * A.row;
    for (int e = e0; e < e1 && run < count; ++e) {
        const uint32_t v = ~(uint32_t)lst[e];
        const int w = wt[v];
        const int take = min(w, count - run);
        int f, c;
        in_range(as, pm + lo[v], lo[v + 1] - lo[v], f, c);
        const int32_t a = lo[v] + f;
        for (int t = 0; t < take; ++t) out[run + t] = pm[a + t];
        if (count == A.k && run + w >= A.k) cut_s = unorderable((uint32_t)(lst[e] >> 32));
        run += w;
    }
    for (int t = tid; t < as.nloc; t += blockDim.x) out[count + t] = local_key(as, t);
    for (int t = count + as.nloc + tid; t < A.row; t += blockDim.x) out[t] = -1;
    __syncthreads();
    if (tid == 0) {
        A.sel_count[gi] = count + as.nloc;
        if (A.sel_cutoff) A.sel_cutoff[gi] = cut_s;
    }
}

inline size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

struct FlatWs { float *U; uint32_t *sc; uint16_t *wt; size_t bytes; };

FlatWs carve_flat_ws(char *base, int64_t mb, int h_kv, int r, int64_t nleaf) {
    size_t cur = 0;
    FlatWs w{};
    auto take = [&](size_t n) { char *p = base ? base + cur : nullptr; cur = a256(cur + n); return p; };
    w.U = (float *)take(sizeof(float) * (size_t)mb * h_kv * r);
    w.sc = (uint32_t *)take(sizeof(uint32_t) * (size_t)mb * h_kv * nleaf);
    w.wt = (uint16_t *)take(sizeof(uint16_t) * (size_t)mb * h_kv * nleaf);
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
    static int attr_set[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    const size_t shm = sizeof(uint64_t) * kFlatList + sizeof(int) * 2 * kFlatBins;
    if (!attr_set[dev]) {
        hipError_t e = hipFuncSetAttribute((const void *)k_flat_select, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)shm);
        if (e != hipSuccess) return e;
        attr_set[dev] = 1;
    }
    const int row = k + n_sink + window;
    const size_t esz = dtype == 0 ? 4 : 2;
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
        A.U = w.U; A.sc = w.sc; A.wt = w.wt;
        A.sel = sel + (size_t)i0 * h_kv * row;
        A.sel_count = sel_count + (size_t)i0 * h_kv;
        A.sel_cutoff = sel_cutoff ? sel_cutoff + (size_t)i0 * h_kv : nullptr;
        if (dtype == 0) hipLaunchKernelGGL(k_flat_latent<float>, dim3((unsigned)nb, (unsigned)h_kv), dim3(256), 0, st, A);
        else hipLaunchKernelGGL(k_flat_latent<bf16_t>, dim3((unsigned)nb, (unsigned)h_kv), dim3(256), 0, st, A);
        const dim3 sgrid((unsigned)((nleaf + kFlatLeaves - 1) / kFlatLeaves), (unsigned)((nb + kFlatRows - 1) / kFlatRows),
                         (unsigned)h_kv);
        if (r == 64) hipLaunchKernelGGL(k_flat_score<64>, sgrid, dim3(256), 0, st, A);
        else hipLaunchKernelGGL(k_flat_score<0>, sgrid, dim3(256), 0, st, A);
        hipLaunchKernelGGL(k_flat_select, dim3((unsigned)(nb * h_kv)), dim3(256), shm, st, A);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace lsa
