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
    int n_sink, window;
    int row;              // entries per row of sel: k + n_sink + window
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
    const AttnSet as = attn_set(A.q_pos[i], A.n, A.n_sink, A.window);
    {
        const int chunk = (nc + blockDim.x - 1) / blockDim.x;
        const int s0 = min(nc, (int)threadIdx.x * chunk), s1 = min(nc, s0 + chunk);
        int el[16];
        int local = 0;
        for (int e = s0; e < s1; ++e) {
            const uint32_t v = key_id(keys[e]);
            const int32_t a = lo[v], z = lo[v + 1];
            int f, c;
            in_range(as, pm + a, z - a, f, c);
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
    int32_t *out = A.sel + ((size_t)i * A.h_kv + g) * A.row;
    for (int e = threadIdx.x; e < nc; e += blockDim.x) {
        const int p0 = aux[e];
        if (p0 >= count) continue;
        const int p1 = aux[e + 1];
        const int take = min(p1 - p0, count - p0);
        const uint32_t v = key_id(keys[e]);
        int f, c;
        in_range(as, pm + lo[v], lo[v + 1] - lo[v], f, c);
        const int32_t a = lo[v] + f;
        for (int t = 0; t < take; ++t) out[p0 + t] = pm[a + t];
        if (count == A.k && p1 >= A.k) cut_s = key_score(keys[e]);
    }
    for (int t = threadIdx.x; t < as.nloc; t += blockDim.x) out[count + t] = local_key(as, t);
    for (int t = count + as.nloc + threadIdx.x; t < A.row; t += blockDim.x) out[t] = -1;
    __syncthreads();
    if (threadIdx.x == 0) {
        A.sel_count[(size_t)i * A.h_kv + g] = count + as.nloc;
        if (A.sel_cutoff) A.sel_cutoff[(size_t)i * A.h_kv + g] = cut_s;
    }
}

// ---------------------------------------------------------------- throughput path
// Same selection for many rows (prefill, training layers), shaped for
// throughput: r = 64, b <= 64, beam <= 16, L >= 2, leaf ids below 2^22.
//   * W_g is staged in LDS and u = fl32(qbar . W_g) computed from there;
//   * the root's children are scored by one wave and ranked by a wave sort;
//   * at each deeper level wave w scores the children of kept nodes w, w + 4,
//     ... (lane c: child c, its row loaded straight into registers), and the
//     block sorts all beam * b candidates at once (four keys per thread,
//     DPP exchanges inside a wave, LDS only across waves);
//   * a candidate leaf's key also carries its slot (kept node j, child c), so
//     after the sort its eligible count and first member are found in LDS.
// Scores, order and ties are those of k_select.

// (orderable score) << 32 | (~id, 22 bits) << 10 | slot: orders as make_key for ids < 2^22
LSA_DEV uint64_t make_key_slot(float score, uint32_t id, int slot) {
    return ((uint64_t)orderable(score) << 32) | ((uint64_t)(~id & 0x3FFFFFu) << 10) | (uint64_t)slot;
}
LSA_DEV uint32_t slot_key_id(uint64_t k) { return ~(uint32_t)(k >> 10) & 0x3FFFFFu; }

// u . row (64 floats) in double, ascending index; the row comes straight from
// global memory in two halves (each half's 8 loads issued before its FMAs),
// u from LDS.  Halves keep fewer registers live, so more waves stay resident.
LSA_DEV float score_row64(const float *u, const float *__restrict__ row) {
    const f4_t *r4 = reinterpret_cast<const f4_t *>(row);
    const f4_t *u4 = reinterpret_cast<const f4_t *>(u) + opaque(0);   // u read at each use, not kept live
    double s = 0.0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        f4_t v[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) v[x] = r4[8 * h + x];
#pragma unroll
        for (int x = 0; x < 8; ++x) {
            const f4_t a = u4[8 * h + x];
            s = fma((double)a.x, (double)v[x].x, s);
            s = fma((double)a.y, (double)v[x].y, s);
            s = fma((double)a.z, (double)v[x].z, s);
            s = fma((double)a.w, (double)v[x].w, s);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    return (float)s;
}

constexpr int kFastP = 16;          // beam limit of the throughput path
constexpr int kFastR = 64;          // latent dimension of the throughput path
constexpr int kWRows = 64;          // rows of W staged at a time (16 KB)

template <typename T>
__global__ __launch_bounds__(256, 5) void k_select_fast(SelectArgs A) {
    extern __shared__ __attribute__((aligned(16))) float dynf[];   // W_g, then keys and leaf tables
    __shared__ __attribute__((aligned(16))) float qbar_s[256];
    __shared__ __attribute__((aligned(16))) float u_s[kFastR];
    __shared__ int32_t kept_s[kFastP];
    __shared__ int keep_s, ncol_s, scratch[8], hist_s[256], sel_s[4];
    __shared__ uint64_t col_s[kFastP];
    __shared__ float cut_s;
    constexpr int R = kFastR;
    const int64_t i = blockIdx.x;
    const int g = blockIdx.y;
    const int G = A.h_q / A.h_kv, d = A.d, b = A.b, L = A.L, P = A.beam;
    const int tid = threadIdx.x, lane = lane_id(), wv = tid / kWave;
    const T *Q = (const T *)A.Q;
    const AttnSet as = attn_set(A.q_pos[i], A.n, A.n_sink, A.window);

    // ---- group latent query.  W_g is staged in LDS 64 input rows (16 KB) at
    // a time; the sum over the input dimension continues in order across them.
    float *Wl = dynf;                                   // [64][R]
    for (int t = tid; t < d; t += blockDim.x) {
        double s = 0.0;
        for (int h = 0; h < G; ++h) s = s + (double)to_float(Q[((size_t)i * A.h_q + (size_t)g * G + h) * d + t]);
        qbar_s[t] = (float)(s / (double)G);
    }
    if (tid == 0) cut_s = -INFINITY;
    double us = 0.0;
    for (int t0 = 0; t0 < d; t0 += kWRows) {
        const int nt = min(kWRows, d - t0);
        g2s_rows<4>(Wl, nt * R, A.W + ((size_t)g * d + t0) * R, nt * R, nt * R);
        __syncthreads();
        if (tid < R)
            for (int t = 0; t < nt; ++t) us = fma((double)qbar_s[t0 + t], (double)Wl[t * R + tid], us);
        __syncthreads();
    }
    if (tid < R) u_s[tid] = (float)us;
    __syncthreads();

    // ---- level 1: the root's non-empty children, best min(beam, #) kept
    if (wv == 0) {
        const float *C1 = (const float *)(A.index + A.centroid_off[1]) + (size_t)g * A.nodes[1] * R;
        const int32_t *cn1 = (const int32_t *)(A.index + A.count_off[1]) + (size_t)g * A.nodes[1];
        uint64_t key = 0;
        int pay = 0;
        if (lane < b && cn1[lane] > 0) key = make_key(score_row64(u_s, C1 + (size_t)lane * R), (uint32_t)lane);
        const int nz = __popcll(__ballot(key != 0));
        wave_sort_desc(key, pay);
        const int keep = min(P, nz);
        if (lane < keep) kept_s[lane] = (int32_t)key_id(key);
        if (lane == 0) keep_s = keep;
    }
    __syncthreads();

    // ---- levels 2..L
    uint64_t *sk = reinterpret_cast<uint64_t *>(dynf);           // 1024 candidate keys
    int32_t *eli = reinterpret_cast<int32_t *>(sk + 1024);        // [kFastP][64] eligible counts
    int32_t *lof = eli + kFastP * 64;                             // [kFastP][64] first member offsets
    const int64_t nleaf = A.nodes[L];
    const int32_t *lo = (const int32_t *)(A.index + A.leaf_off_off) + (size_t)g * (nleaf + 1);
    const int32_t *pm = (const int32_t *)(A.index + A.perm_off) + (size_t)g * A.n;
    uint64_t k4[4];
    for (int l = 2; l <= L; ++l) {
        const bool leaf = l == L;
        const int keep = keep_s;
        const float *Cl = (const float *)(A.index + A.centroid_off[l]) + (size_t)g * A.nodes[l] * R;
        const int32_t *cn = (const int32_t *)(A.index + A.count_off[l]) + (size_t)g * A.nodes[l];
        for (int j = wv; j < kFastP; j += 4) {
            uint64_t key = 0;
            if (j < keep && lane < b) {
                const int64_t child = (int64_t)kept_s[j] * b + lane;
                if (cn[child] > 0) {
                    int e = 1;
                    if (leaf) {
                        const int32_t a0 = lo[child], a1 = lo[child + 1];
                        int f;
                        in_range(as, pm + a0, a1 - a0, f, e);
                        eli[j * 64 + lane] = e;
                        lof[j * 64 + lane] = a0 + f;
                    }
                    if (e > 0) key = make_key_slot(score_row64(u_s, Cl + (size_t)child * R), (uint32_t)child, j * 64 + lane);
                }
            }
            sk[j * 64 + lane] = key;
        }
        __syncthreads();
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) k4[ii] = sk[4 * tid + ii];
        if (leaf) {
            block_sort_desc<4>(k4, sk);
            break;
        }
        // internal level: the beam-th largest key by radix selection, then the
        // keys at or above it (min(beam, #non-empty) of them) ranked by one wave
        const int one[4] = {1, 1, 1, 1};
        const uint64_t thr = block_radix_select(k4, one, P, hist_s, sel_s);
        if (tid == 0) ncol_s = 0;
        __syncthreads();
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
            if (k4[ii] != 0 && k4[ii] >= thr) col_s[atomicAdd(&ncol_s, 1)] = k4[ii];
        __syncthreads();
        if (wv == 0) {
            const int nk = ncol_s;
            uint64_t key = lane < nk ? col_s[lane] : 0ull;
            int pay = 0;
            wave_sort_desc(key, pay);
            if (lane < nk) kept_s[lane] = (int32_t)slot_key_id(key);
            if (lane == 0) keep_s = nk;
        }
        __syncthreads();
    }

    // ---- fill: leaves in sorted order, each giving its first eligible members
    int e4[4], tot = 0;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
        e4[ii] = (k4[ii] != 0) ? eli[(int)(k4[ii] & 1023u)] : 0;
        tot += e4[ii];
    }
    int total;
    int off = block_excl_scan(tot, scratch, &total);
    const int count = min(A.k, total);
    int32_t *out = A.sel + ((size_t)i * A.h_kv + g) * A.row;
    // the thread's (up to) four leaves: the first 8 members of each are loaded
    // in one round (clamped indices), longer leaves finish in a loop
    constexpr int kC = 4;
    int take[4], a0v[4], offv[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
        offv[ii] = off;
        take[ii] = (e4[ii] > 0 && off < count) ? min(e4[ii], count - off) : 0;
        a0v[ii] = take[ii] > 0 ? lof[(int)(k4[ii] & 1023u)] : 0;
        if (take[ii] > 0 && count == A.k && off + e4[ii] >= A.k) cut_s = key_score(k4[ii]);
        off += e4[ii];
    }
    int32_t mv[4][kC];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
        for (int t = 0; t < kC; ++t) mv[ii][t] = take[ii] > 0 ? pm[a0v[ii] + min(t, take[ii] - 1)] : 0;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
#pragma unroll
        for (int t = 0; t < kC; ++t)
            if (t < take[ii]) out[offv[ii] + t] = mv[ii][t];
        for (int t = kC; t < take[ii]; ++t) out[offv[ii] + t] = pm[a0v[ii] + t];
    }
    for (int t = tid; t < as.nloc; t += blockDim.x) out[count + t] = local_key(as, t);
    for (int t = count + as.nloc + tid; t < A.row; t += blockDim.x) out[t] = -1;
    __syncthreads();
    if (tid == 0) {
        A.sel_count[(size_t)i * A.h_kv + g] = count + as.nloc;
        if (A.sel_cutoff) A.sel_cutoff[(size_t)i * A.h_kv + g] = cut_s;
    }
}

hipError_t select_keys(const void *Q, int dtype, int64_t m, int h_q, int d, const int32_t *q_pos, const char *index,
                       int64_t n, int h_kv, int r, int b, int L, const int64_t *nodes, const int64_t *centroid_off,
                       const int64_t *count_off, int64_t leaf_off_off, int64_t perm_off, const float *W, int beam,
                       int k, int n_sink, int window, int32_t *sel, int32_t *sel_count, float *sel_cutoff,
                       hipStream_t st) {
    SelectArgs A{};
    A.Q = Q; A.m = m; A.h_q = h_q; A.h_kv = h_kv; A.d = d; A.q_pos = q_pos; A.index = index; A.n = n;
    A.r = r; A.b = b; A.L = L;
    for (int l = 0; l <= L; ++l) { A.nodes[l] = nodes[l]; A.centroid_off[l] = centroid_off[l]; A.count_off[l] = count_off[l]; }
    A.leaf_off_off = leaf_off_off; A.perm_off = perm_off; A.W = W; A.beam = beam; A.k = k;
    A.n_sink = n_sink; A.window = window; A.row = k + n_sink + window;
    A.sel = sel; A.sel_count = sel_count; A.sel_cutoff = sel_cutoff;
    const dim3 grid((unsigned)m, (unsigned)h_kv);
    if (r == kFastR && b <= 64 && beam <= kFastP && L >= 2 && d <= 256 && nodes[L] <= (int64_t)1 << 22) {
        const size_t shm = std::max(sizeof(float) * (size_t)kWRows * kFastR, sizeof(uint64_t) * 1024 + sizeof(int32_t) * 2 * kFastP * 64);
        if (dtype == 0) hipLaunchKernelGGL((k_select_fast<float>), grid, dim3(256), shm, st, A);
        else hipLaunchKernelGGL((k_select_fast<bf16_t>), grid, dim3(256), shm, st, A);
        return hipGetLastError();
    }
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
