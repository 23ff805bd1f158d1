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
#include <algorithm>

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

// The members of the thread's leaves to sel: leaf ii's first take[ii]
// members (from pm[a0v[ii]]) go to out[offv[ii] ..].  Rounds of RND members
// per leaf, every load of a round issued before its stores (clamped
// indices): a long leaf costs one round trip per RND members, not one per
// member.
template <int KPT, int RND>
LSA_DEV void fill_members(const int32_t *__restrict__ pm, int32_t *__restrict__ out, const int (&take)[KPT],
                          const int (&a0v)[KPT], const int (&offv)[KPT]) {
    int mx = 0;
#pragma unroll
    for (int ii = 0; ii < KPT; ++ii) mx = max(mx, take[ii]);
    for (int t0 = 0; t0 < mx; t0 += RND) {
        int32_t x[KPT][RND];
#pragma unroll
        for (int ii = 0; ii < KPT; ++ii)
#pragma unroll
            for (int t = 0; t < RND; ++t) x[ii][t] = pm[take[ii] > 0 ? a0v[ii] + min(t0 + t, take[ii] - 1) : 0];
#pragma unroll
        for (int ii = 0; ii < KPT; ++ii)
#pragma unroll
            for (int t = 0; t < RND; ++t)
                if (t0 + t < take[ii]) out[offv[ii] + t0 + t] = x[ii][t];
    }
}

// Positions of sel the block copy below covers (count <= kFlatCap).
constexpr int kFlatCap = 2048;

// The same copy with one retrieval position per lane: position f holds
// member f - off of the last taken leaf whose offset off <= f.  Each taken
// leaf marks its offset with its sorted position (KPT * thread + ii, which
// increases with the offset) in `lead` (kFlatCap ints, LDS), a max scan
// carries the marks forward, and dl[leaf] = a0 - off turns a position into
// its member index.  Consecutive lanes then load and store consecutive
// positions: 8 loads and 8 stores a thread for 2048 keys, where the copy by
// leaves issues 4 x 8 mostly masked ones.  Needs count <= kFlatCap; lead and
// dl (KPT * 256 ints) must not be in use by other threads on entry.
template <int KPT>
LSA_DEV void fill_members_flat(const int32_t *__restrict__ pm, int32_t *__restrict__ out, const int (&take)[KPT],
                               const int (&a0v)[KPT], const int (&offv)[KPT], int count, int *lead, int *dl,
                               int *scratch) {
    constexpr int PER = kFlatCap / 256;
    const int tid = threadIdx.x, lane = lane_id(), wv = tid / kWave;
    int4 *l4 = reinterpret_cast<int4 *>(lead + PER * tid);
#pragma unroll
    for (int j = 0; j < PER / 4; ++j) l4[j] = int4{-1, -1, -1, -1};
    __syncthreads();
#pragma unroll
    for (int ii = 0; ii < KPT; ++ii)
        if (take[ii] > 0) { lead[offv[ii]] = KPT * tid + ii; dl[KPT * tid + ii] = a0v[ii] - offv[ii]; }
    __syncthreads();
    // running maximum over the thread's PER positions, then over the threads
    // before it (lanes of its wave through shifts, earlier waves through LDS)
    int v[PER];
    {
        int m = -1;
#pragma unroll
        for (int j = 0; j < PER / 4; ++j) {
            const int4 q = l4[j];
            m = max(m, q.x); v[4 * j] = m;
            m = max(m, q.y); v[4 * j + 1] = m;
            m = max(m, q.z); v[4 * j + 2] = m;
            m = max(m, q.w); v[4 * j + 3] = m;
        }
        int incl = m;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int t = __shfl_up(incl, o);
            if (lane >= o) incl = max(incl, t);
        }
        if (lane == kWave - 1) scratch[wv] = incl;
        int carry = __shfl_up(incl, 1);
        if (lane == 0) carry = -1;
        __syncthreads();
        for (int q = 0; q < wv; ++q) carry = max(carry, scratch[q]);
#pragma unroll
        for (int j = 0; j < PER / 4; ++j)
            l4[j] = int4{max(carry, v[4 * j]), max(carry, v[4 * j + 1]), max(carry, v[4 * j + 2]), max(carry, v[4 * j + 3])};
    }
    __syncthreads();
    int32_t x[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int f = tid + 256 * j;
        x[j] = (f < count) ? pm[dl[max(lead[f], 0)] + f] : 0;
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int f = tid + 256 * j;
        if (f < count) out[f] = x[j];
    }
}

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

// u = fl32(qbar . W_g) of row i, KV head g, into u_s.  W_g is staged in LDS
// (Wl, kWRows x kFastR floats) 64 input rows at a time; the sum over the
// input dimension continues in order across them.
template <typename T>
LSA_DEV void fast_latent(const SelectArgs &A, int64_t i, int g, float *Wl, float *qbar_s, float *u_s) {
    constexpr int R = kFastR;
    const int tid = threadIdx.x, G = A.h_q / A.h_kv, d = A.d;
    const T *Q = (const T *)A.Q;
    for (int t = tid; t < d; t += blockDim.x) {
        double s = 0.0;
        for (int h = 0; h < G; ++h) s = s + (double)to_float(Q[((size_t)i * A.h_q + (size_t)g * G + h) * d + t]);
        qbar_s[t] = (float)(s / (double)G);
    }
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
}

// Level 1: the root's non-empty children scored and ranked by wave 0; the
// best min(beam, #) go to kept_s, their number to *keep_s.
LSA_DEV void fast_level1(const SelectArgs &A, int g, const float *u_s, int32_t *kept_s, int *keep_s) {
    constexpr int R = kFastR;
    const int lane = lane_id();
    if (threadIdx.x / kWave == 0) {
        const float *C1 = (const float *)(A.index + A.centroid_off[1]) + (size_t)g * A.nodes[1] * R;
        const int32_t *cn1 = (const int32_t *)(A.index + A.count_off[1]) + (size_t)g * A.nodes[1];
        uint64_t key = 0;
        int pay = 0;
        if (lane < A.b && cn1[lane] > 0) key = make_key(score_row64(u_s, C1 + (size_t)lane * R), (uint32_t)lane);
        const int nz = __popcll(__ballot(key != 0));
        wave_sort_desc(key, pay);
        const int keep = min(A.beam, nz);
        if (lane < keep) kept_s[lane] = (int32_t)key_id(key);
        if (lane == 0) *keep_s = keep;
    }
    __syncthreads();
}

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

    // ---- group latent query, then level 1
    float *Wl = dynf;                                   // [64][R]
    if (tid == 0) cut_s = -INFINITY;
    fast_latent<T>(A, i, g, Wl, qbar_s, u_s);
    fast_level1(A, g, u_s, kept_s, &keep_s);

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
    // the thread's (up to) four leaves: the first 4 members of each are loaded
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

// ---------------------------------------------------------------- node-major path
// For many rows the kernel above reads, per (row, KV head), the b children of
// each of its `beam` kept nodes at every level: 256 KB per row at the leaf
// level of the 1M workloads, mostly from HBM, although different rows keep
// the same nodes.  Here levels 2..L are scored node by node: the (row, kept
// node) pairs are grouped by node, and a wave loads a node's children rows
// once into registers and scores them against every row that kept it.  The
// keys (with their slots), eligible counts and first members are those of
// k_select_fast, so the rows it writes are identical.
//   k_nm_top     u and level 1 as k_select_fast, four rows of one KV head per
//                workgroup;
//   k_nm_zero, k_nm_count, k_nm_scan, k_nm_fill: the pairs grouped by node
//                (each entry with its node);
//   k_nm_score_mfma  64 pairs per workgroup, 16 per wave: the wave's pairs
//                times the children of their node on the fp64 matrix cores,
//                each pair's candidate keys written to its slots (64 per
//                kept node; with b <= 32 the first 32 of them, the packed
//                slots of nm_slot), at the leaf level with eligible counts
//                and first members;
//   k_nm_keep_w  internal levels, per (row, KV head): the top `beam` by a
//                wave radix selection and a one-wave sort;
//   k_nm_finish  leaf level, per (row, KV head): block sort (1024 slots, or
//                the 512 packed ones) and fill.

struct NmArgs {
    SelectArgs S;
    int64_t row0;                  // first row of the batch
    int64_t groups;                // rows of the batch x h_kv; group = (row - row0) * h_kv + g
    int level;                     // the level being scored (2..L)
    float *U;                      // [groups][64]
    int32_t *kept;                 // [groups][kFastP] node ids at level - 1
    int32_t *keep;                 // [groups]
    uint64_t *keys;                // [groups][kFastP * 64]
    int32_t *eli, *lof;            // [groups][kFastP * 64] (leaf level)
    int32_t *ncnt, *noff, *fptr;   // [h_kv * nodes(level - 1) + 1]
    int32_t *pairs;                // [groups * kFastP]: group * kFastP + slot, grouped by node
    int32_t *pnode;                // [groups * kFastP]: the node of each entry of pairs
    // for the node-major attention (NULL when none follows):
    int32_t *ppos;                 // [groups * kFastP]: where each leaf-level entry sits in pairs
    uint4 *pinf;                   // [groups * kFastP][2]: the pair records, in the order of pairs: taken
                                   // children mask (low, high), entry, retrieval range low; range high,
                                   // child of the leaf taken in part (-1: none), its last taken key, 0
};

// kTopRows rows of one KV head per workgroup: W_g is staged once for them,
// thread (rr, c) continues u[c] of row rr across the staged chunks (the same
// order as fast_latent), and wave rr scores and ranks row rr's level 1.
constexpr int kTopRows = 4;

template <typename T>
__global__ __launch_bounds__(256) void k_nm_top(NmArgs N) {
    __shared__ __attribute__((aligned(16))) float Wl[kWRows * kFastR];
    __shared__ __attribute__((aligned(16))) float qbar_s[kTopRows][256];
    __shared__ __attribute__((aligned(16))) float u_s[kTopRows][kFastR];
    constexpr int R = kFastR;
    const SelectArgs &A = N.S;
    const int g = blockIdx.y;
    const int64_t rb = (int64_t)blockIdx.x * kTopRows;                 // first row, relative to the batch
    const int nr = (int)min<int64_t>(kTopRows, N.groups / A.h_kv - rb);
    const int tid = threadIdx.x, G = A.h_q / A.h_kv, d = A.d;
    const T *Q = (const T *)A.Q;
    for (int e = tid; e < kTopRows * d; e += blockDim.x) {
        const int rr = e / d, t = e % d;
        float val = 0.0f;
        if (rr < nr) {
            const int64_t i = N.row0 + rb + rr;
            double s = 0.0;
            for (int h = 0; h < G; ++h) s = s + (double)to_float(Q[((size_t)i * A.h_q + (size_t)g * G + h) * d + t]);
            val = (float)(s / (double)G);
        }
        qbar_s[rr][t] = val;
    }
    const int rr = tid / kWave, lane = tid % kWave;
    double us = 0.0;
    for (int t0 = 0; t0 < d; t0 += kWRows) {
        const int nt = min(kWRows, d - t0);
        __syncthreads();                 // qbar_s written / the previous chunk read
        g2s_rows<4>(Wl, nt * R, A.W + ((size_t)g * d + t0) * R, nt * R, nt * R);
        __syncthreads();
        for (int t = 0; t < nt; ++t) us = fma((double)qbar_s[rr][t0 + t], (double)Wl[t * R + lane], us);
    }
    u_s[rr][lane] = (float)us;
    wave_sync();
    if (rr < nr) {
        const int64_t grp = (rb + rr) * A.h_kv + g;
        const float *C1 = (const float *)(A.index + A.centroid_off[1]) + (size_t)g * A.nodes[1] * R;
        const int32_t *cn1 = (const int32_t *)(A.index + A.count_off[1]) + (size_t)g * A.nodes[1];
        uint64_t key = 0;
        int pay = 0;
        if (lane < A.b && cn1[lane] > 0) key = make_key(score_row64(u_s[rr], C1 + (size_t)lane * R), (uint32_t)lane);
        const int nz = __popcll(__ballot(key != 0));
        wave_sort_desc(key, pay);
        const int keep = min(A.beam, nz);
        N.U[grp * R + lane] = u_s[rr][lane];
        if (lane < kFastP) N.kept[grp * kFastP + lane] = lane < keep ? (int32_t)key_id(key) : 0;
        if (lane == 0) N.keep[grp] = keep;
    }
}

// The same step on the fp64 matrix cores (d a multiple of 8, 64 rows of one
// KV head per workgroup).  qbar is staged in LDS transposed ([dim][row]);
// wave w forms latent columns 16 w .. 16 w + 15 of the four 16-row blocks as
// v_mfma_f64_16x16x4_f64 chains over dims 4 blk + k (blk ascending), which is
// fast_latent's sequential double sum bit for bit.  Then wave w scores rows
// 16 w .. 16 w + 15 against the root's children (16 children a product, the
// same chains over the 64 latent dims as score_row64), and ranks each of its
// rows with one wave sort.  u and the kept nodes equal k_nm_top's.  NQ = d / 4
// when fixed at compile time (the lane's W_g column in registers), else 0.
constexpr int kTopMRows = 64;
constexpr int kTopUS = kFastR + 4;    // u row stride in LDS (16-byte rows)
constexpr int kTopSS = kFastR + 1;    // score row stride in LDS

size_t nm_top_mfma_lds(int d) {
    const size_t q = (size_t)d * (kTopMRows + 1), us = (size_t)kTopMRows * (kTopUS + kTopSS);
    return sizeof(float) * (q > us ? q : us);
}

template <typename T, int NQ>
__global__ __launch_bounds__(256) void k_nm_top_mfma(NmArgs N) {
    constexpr int R = kFastR, RB = kTopMRows, ST = RB + 1;
    extern __shared__ __attribute__((aligned(16))) float tsm[];
    float *qt = tsm;                          // [d][ST], then u rows and scores:
    float *u_s = tsm;                         // [RB][kTopUS]
    float *sc_s = tsm + RB * kTopUS;          // [RB][kTopSS]
    const SelectArgs &A = N.S;
    const int g = blockIdx.y;
    const int64_t rb = (int64_t)blockIdx.x * RB;                      // first row, relative to the batch
    const int nr = (int)min<int64_t>(RB, N.groups / A.h_kv - rb);
    const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave, lr = lane % 16, lk = lane / 16;
    const int G = A.h_q / A.h_kv, d = A.d, nq = NQ > 0 ? NQ : d / 4;
    const T *Q = (const T *)A.Q;
    const float *wcol = A.W + (size_t)g * d * R + 16 * w + lr;
    const float *C1 = (const float *)(A.index + A.centroid_off[1]) + (size_t)g * A.nodes[1] * R;
    const int32_t *cn1 = (const int32_t *)(A.index + A.count_off[1]) + (size_t)g * A.nodes[1];
    const int cnt1 = lane < A.b ? cn1[lane] : 0;
    // qbar of row rr, dims 8 x .. 8 x + 7: the G heads summed in double in
    // head order, divided by G, rounded once
    if constexpr (NQ > 0) {
        // (d = 4 NQ: the thread's SL chunks loaded together, two heads a round)
        constexpr int XC = NQ / 2, SL = RB * XC / 256;
        static_assert(RB * XC % 256 == 0, "whole chunks per thread");
        double s[SL][8];
        size_t at[SL];
        bool ok[SL];
#pragma unroll
        for (int sl = 0; sl < SL; ++sl) {
            const int idx = tid + 256 * sl, rr = idx / XC, x = idx % XC;
            ok[sl] = rr < nr;
            at[sl] = ok[sl] ? ((size_t)(N.row0 + rb + rr) * A.h_q + (size_t)g * G) * d + 8 * x : 0;
#pragma unroll
            for (int u = 0; u < 8; ++u) s[sl][u] = 0.0;
        }
        for (int h = 0; h < G; h += 2) {
            const int h1 = h + 1 < G ? h + 1 : h;
            float v[SL][8], v1[SL][8];
#pragma unroll
            for (int sl = 0; sl < SL; ++sl) {
                load8(Q, at[sl] + (size_t)h * d, v[sl]);
                load8(Q, at[sl] + (size_t)h1 * d, v1[sl]);
            }
#pragma unroll
            for (int sl = 0; sl < SL; ++sl)
#pragma unroll
                for (int u = 0; u < 8; ++u) s[sl][u] = s[sl][u] + (double)v[sl][u];
            if (h1 != h) {
#pragma unroll
                for (int sl = 0; sl < SL; ++sl)
#pragma unroll
                    for (int u = 0; u < 8; ++u) s[sl][u] = s[sl][u] + (double)v1[sl][u];
            }
        }
#pragma unroll
        for (int sl = 0; sl < SL; ++sl) {
            const int idx = tid + 256 * sl, rr = idx / XC, x = idx % XC;
#pragma unroll
            for (int u = 0; u < 8; ++u) qt[(8 * x + u) * ST + rr] = ok[sl] ? (float)(s[sl][u] / (double)G) : 0.0f;
        }
    } else {
        for (int idx = tid; idx < RB * (d / 8); idx += blockDim.x) {
            const int rr = idx / (d / 8), x = idx % (d / 8);
            double s[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
            if (rr < nr) {
                const size_t at = ((size_t)(N.row0 + rb + rr) * A.h_q + (size_t)g * G) * d + 8 * x;
                for (int h = 0; h < G; ++h) {
                    float v[8];
                    load8(Q, at + (size_t)h * d, v);
#pragma unroll
                    for (int u = 0; u < 8; ++u) s[u] = s[u] + (double)v[u];
                }
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) qt[(8 * x + u) * ST + rr] = (float)(s[u] / (double)G);
        }
    }
    // the lane's W_g column (dims 4 blk + l / 16), in flight across the barrier
    float wv[NQ > 0 ? NQ : 1];
    if constexpr (NQ > 0) {
#pragma unroll
        for (int blk = 0; blk < NQ; ++blk) wv[blk] = wcol[(size_t)(4 * blk + lk) * R];
    }
    __syncthreads();
    d4_t acc[RB / 16];
#pragma unroll
    for (int kb = 0; kb < RB / 16; ++kb) acc[kb] = d4_t{0.0, 0.0, 0.0, 0.0};
#pragma unroll(NQ > 0 ? NQ : 1)
    for (int blk = 0; blk < nq; ++blk) {
        double bw;
        if constexpr (NQ > 0) bw = (double)wv[blk];
        else bw = (double)wcol[(size_t)(4 * blk + lk) * R];
        const float *qrow = qt + (4 * blk + lk) * ST + lr;
#pragma unroll
        for (int kb = 0; kb < RB / 16; ++kb)
            acc[kb] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)qrow[16 * kb], bw, acc[kb], 0, 0, 0);
    }
    __syncthreads();                     // qt read by every wave: its space now takes u
    // element e of lane l: row 16 kb + l / 16 + 4 e, latent column 16 w + l % 16
#pragma unroll
    for (int kb = 0; kb < RB / 16; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int rr = 16 * kb + lk + 4 * e;
            const float uv = (float)acc[kb][e];
            u_s[rr * kTopUS + 16 * w + lr] = uv;
            if (rr < nr) N.U[((rb + rr) * A.h_kv + g) * R + 16 * w + lr] = uv;
        }
    // level 1: rows 16 w .. 16 w + 15 (this wave's) x children 16 cb .. 16 cb + 15
    const int cbn = (A.b + 15) / 16;
    f4_t crow[4][4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
        if (cb < cbn) load_row_mfma(C1 + (size_t)min(16 * cb + lr, A.b - 1) * R, lk, crow[cb]);
    __syncthreads();                     // every wave's u rows in LDS
    double ua[16];
    {
        f4_t v[4];
        load_row_mfma(u_s + (16 * w + lr) * kTopUS, lk, v);
        widen_row_mfma(v, ua);
    }
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        if (cb >= cbn) continue;
        const d4_t sc = mfma_dot64(ua, crow[cb]);
#pragma unroll
        for (int e = 0; e < 4; ++e) sc_s[(16 * w + lk + 4 * e) * kTopSS + 16 * cb + lr] = (float)sc[e];
    }
    wave_sync();                         // the wave ranks only its own rows
    if (A.b <= 32) {
        // two rows a sort: row 16 w + q in lanes 0..31, row 16 w + q + 1 in 32..63
        const int c = lane & 31, hi = lane >> 5;
        const int cnt1h = __shfl(cnt1, c);
        for (int q = 0; q < 16; q += 2) {
            const int rr = 16 * w + q + hi;
            if (16 * w + q >= nr) break;
            uint64_t key = (c < A.b && cnt1h > 0 && rr < nr) ? make_key(sc_s[rr * kTopSS + c], (uint32_t)c) : 0ull;
            int pay = 0;
            const uint64_t nzm = __ballot(key != 0);
            const int nz = __popcll(hi ? (nzm >> 32) : (nzm & 0xffffffffull));
            half_wave_sort_desc(key, pay);
            const int keep = min(A.beam, nz);
            if (rr < nr) {
                const int64_t grp = (rb + rr) * A.h_kv + g;
                if (c < kFastP) N.kept[grp * kFastP + c] = c < keep ? (int32_t)key_id(key) : 0;
                if (c == 0) N.keep[grp] = keep;
            }
        }
    } else {
        for (int q = 0; q < 16; ++q) {
            const int rr = 16 * w + q;
            if (rr >= nr) break;
            const int64_t grp = (rb + rr) * A.h_kv + g;
            uint64_t key = (lane < A.b && cnt1 > 0) ? make_key(sc_s[rr * kTopSS + lane], (uint32_t)lane) : 0ull;
            int pay = 0;
            const int nz = __popcll(__ballot(key != 0));
            wave_sort_desc(key, pay);
            const int keep = min(A.beam, nz);
            if (lane < kFastP) N.kept[grp * kFastP + lane] = lane < keep ? (int32_t)key_id(key) : 0;
            if (lane == 0) N.keep[grp] = keep;
        }
    }
}

__global__ __launch_bounds__(256) void k_nm_zero(NmArgs N, int64_t count) {
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < count; e += (int64_t)gridDim.x * blockDim.x)
        N.ncnt[e] = 0;
}

constexpr int kNmChunk = 2048;      // pair entries per counting workgroup
constexpr int kNmBins = 16384;      // (head, node) counters held in LDS (larger tables go straight to memory)
constexpr int kNmSparse = 8192;     // from this many bins a fill workgroup reserves runs from its entries

// the (head, node) bin of pair entry e, or -1 when the slot is empty
LSA_DEV int64_t nm_bin(const NmArgs &N, int64_t e) {
    if (e >= N.groups * kFastP) return -1;
    const int64_t grp = e / kFastP;
    const int j = (int)(e % kFastP);
    if (j >= N.keep[grp]) return -1;
    return (int64_t)(grp % N.S.h_kv) * N.S.nodes[N.level - 1] + N.kept[grp * kFastP + j];
}

// counts per (head, node): each workgroup takes kNmChunk entries, counts them
// in LDS and adds its nonzero counters to memory
__global__ __launch_bounds__(256) void k_nm_count(NmArgs N, int64_t nbins) {
    extern __shared__ int h_s[];            // nbins counters when nbins <= kNmBins
    const int64_t e0 = (int64_t)blockIdx.x * kNmChunk;
    if (nbins > kNmBins) {
        for (int u = threadIdx.x; u < kNmChunk; u += blockDim.x) {
            const int64_t bin = nm_bin(N, e0 + u);
            if (bin >= 0) atomicAdd(N.ncnt + bin, 1);
        }
        return;
    }
    for (int u = threadIdx.x; u < nbins; u += blockDim.x) h_s[u] = 0;
    __syncthreads();
    for (int u = threadIdx.x; u < kNmChunk; u += blockDim.x) {
        const int64_t bin = nm_bin(N, e0 + u);
        if (bin >= 0) atomicAdd(&h_s[bin], 1);
    }
    __syncthreads();
    for (int u = threadIdx.x; u < nbins; u += blockDim.x)
        if (h_s[u] > 0) atomicAdd(N.ncnt + u, h_s[u]);
}

// exclusive scan of ncnt[0..count) into noff and fptr, total at noff[count]
constexpr int kNmScanT = 1024, kNmScanV = 16;   // threads, counts a thread (one round covers 16384 bins)
__global__ __launch_bounds__(kNmScanT) void k_nm_scan(NmArgs N, int64_t count) {
    __shared__ int scr[kNmScanT / kWave + 1];
    const bool al = (((uintptr_t)N.ncnt | (uintptr_t)N.noff | (uintptr_t)N.fptr) & 15) == 0;
    int carry = 0;
    for (int64_t base = 0; base < count; base += (int64_t)kNmScanT * kNmScanV) {
        const int64_t e0 = base + (int64_t)threadIdx.x * kNmScanV;
        const bool whole = al && e0 + kNmScanV <= count;
        int v[kNmScanV], s = 0;
        if (whole) {
#pragma unroll
            for (int q = 0; q < kNmScanV / 4; ++q) {
                const int4 x = *reinterpret_cast<const int4 *>(N.ncnt + e0 + 4 * q);
                v[4 * q] = x.x; v[4 * q + 1] = x.y; v[4 * q + 2] = x.z; v[4 * q + 3] = x.w;
            }
        } else {
#pragma unroll
            for (int u = 0; u < kNmScanV; ++u) v[u] = e0 + u < count ? N.ncnt[e0 + u] : 0;
        }
#pragma unroll
        for (int u = 0; u < kNmScanV; ++u) s += v[u];
        int tot;
        int run = carry + block_excl_scan(s, scr, &tot);
        int o[kNmScanV];
#pragma unroll
        for (int u = 0; u < kNmScanV; ++u) { o[u] = run; run += v[u]; }
        if (whole) {
#pragma unroll
            for (int q = 0; q < kNmScanV / 4; ++q) {
                const int4 x = int4{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]};
                *reinterpret_cast<int4 *>(N.noff + e0 + 4 * q) = x;
                *reinterpret_cast<int4 *>(N.fptr + e0 + 4 * q) = x;
            }
        } else {
#pragma unroll
            for (int u = 0; u < kNmScanV; ++u)
                if (e0 + u < count) { N.noff[e0 + u] = o[u]; N.fptr[e0 + u] = o[u]; }
        }
        carry += tot;
    }
    if (threadIdx.x == 0) N.noff[count] = carry;
}

// pair entries grouped by (head, node): each workgroup ranks its entries per
// bin in LDS, reserves one run per nonzero bin, then writes them
__global__ __launch_bounds__(256) void k_nm_fill(NmArgs N, int64_t nbins) {
    extern __shared__ int h_s[];            // nbins run offsets when nbins <= kNmBins
    constexpr int U = kNmChunk / 256;
    const int64_t e0 = (int64_t)blockIdx.x * kNmChunk;
    if (nbins > kNmBins) {
        for (int u = threadIdx.x; u < kNmChunk; u += blockDim.x) {
            const int64_t bin = nm_bin(N, e0 + u);
            if (bin >= 0) {
                const int32_t at = atomicAdd(N.fptr + bin, 1);
                N.pairs[at] = (int32_t)(e0 + u);
                N.pnode[at] = (int32_t)(bin % N.S.nodes[N.level - 1]);
                if (N.ppos && N.level == N.S.L) N.ppos[e0 + u] = at;
            }
        }
        return;
    }
    for (int u = threadIdx.x; u < nbins; u += blockDim.x) h_s[u] = 0;
    __syncthreads();
    int64_t bin[U];
    int rk[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        bin[u] = nm_bin(N, e0 + threadIdx.x + 256 * u);
        rk[u] = bin[u] >= 0 ? atomicAdd(&h_s[bin[u]], 1) : 0;
    }
    __syncthreads();
    // this workgroup's run of each bin
    if (nbins >= kNmSparse) {
        // few entries per bin: reserved by the bin's first entry here, every
        // reservation of a thread in flight together
        int run[U];
#pragma unroll
        for (int u = 0; u < U; ++u) run[u] = (bin[u] >= 0 && rk[u] == 0) ? atomicAdd(N.fptr + bin[u], h_s[bin[u]]) : 0;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (bin[u] >= 0 && rk[u] == 0) h_s[bin[u]] = run[u];
    } else {
        // many: one pass over the bins (consecutive bins a wave)
        for (int u = threadIdx.x; u < nbins; u += blockDim.x)
            if (h_s[u] > 0) h_s[u] = atomicAdd(N.fptr + u, h_s[u]);
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (bin[u] >= 0) {
            const int32_t at = h_s[bin[u]] + rk[u];
            N.pairs[at] = (int32_t)(e0 + threadIdx.x + 256 * u);
            N.pnode[at] = (int32_t)(bin[u] % N.S.nodes[N.level - 1]);
            if (N.ppos && N.level == N.S.L) N.ppos[e0 + threadIdx.x + 256 * u] = at;
        }
}

// Members of a leaf held in registers by the scorer (longer leaves are
// searched in memory).
constexpr int kNmMemReg = 8;

// The wave's 16 pairs are the 16 rows of the product (lane (k, c): u of pair
// c at dims 4 blk + k, widened once), a node's children are its columns, 16
// at a time (lane (k, c): child 16 cb + c).  Runs of pairs that share a
// (head, node) take that node's children; rows outside the run are computed
// and dropped.  Each lane then owns the scores of four pairs (k + 4 e)
// against one child and writes their keys, and at the leaf level eligible
// counts and first members.  At the leaf level a run's member ranges and
// first members are loaded with lane = child and shared through LDS; the
// next block's rows are loaded while a block is multiplied.
__global__ __launch_bounds__(256) void k_nm_score_mfma(NmArgs N) {
    __shared__ int32_t pe_s[4][16], pv_s[4][16], pp_s[4][16];
    constexpr int kInfo = 3 + kNmMemReg;              // a0, len, last, first members
    __shared__ int32_t info_s[4][kInfo][64];
    constexpr int R = kFastR;
    const SelectArgs &A = N.S;
    const int l = N.level, b = A.b;
    const bool leaf = l == A.L;
    const int wv = threadIdx.x / kWave, lane = lane_id();
    const int col = lane & 15, kk = lane >> 4;
    const int ncb = b <= 32 ? 2 : 4;                   // 16-child column blocks written (packed slots when b <= 32)
    const int nvb = (b + 15) / 16;                     // blocks that hold children
    const int64_t nodes_prev = A.nodes[l - 1];
    const int64_t npairs = N.noff[(size_t)A.h_kv * nodes_prev];
    const float *Cl = (const float *)(A.index + A.centroid_off[l]);
    const int32_t *cn = (const int32_t *)(A.index + A.count_off[l]);
    const int32_t *pm = (const int32_t *)(A.index + A.perm_off);
    const int64_t p0 = (int64_t)blockIdx.x * 64 + wv * 16;
    const int np = (int)max<int64_t>(0, min<int64_t>(16, npairs - p0));
    if (np == 0) return;                               // wave-local: the kernel has no block barrier
    if (lane < 16) {
        const int64_t at = p0 + min(lane, np - 1);
        const int e = N.pairs[at];
        pe_s[wv][lane] = e;
        pv_s[wv][lane] = N.pnode[at];
        pp_s[wv][lane] = A.q_pos[N.row0 + (e / kFastP) / A.h_kv];
    }
    wave_sync();
    // runs of one (head, node): pair q starts one when it differs from pair q - 1
    bool head = lane == 0;
    if (lane > 0 && lane < np) {
        const int e1 = pe_s[wv][lane], e0 = pe_s[wv][lane - 1];
        head = pv_s[wv][lane] != pv_s[wv][lane - 1] || (e1 / kFastP) % A.h_kv != (e0 / kFastP) % A.h_kv;
    }
    uint64_t starts = __ballot(head) & ~1ull;          // the first run starts at pair 0
    int s = 0;
    int g = (int)((__builtin_amdgcn_readfirstlane(pe_s[wv][0]) / kFastP) % A.h_kv);
    int64_t v = __builtin_amdgcn_readfirstlane(pv_s[wv][0]);
    // A operand: pair col (rows past np repeat the last pair)
    double ua[16];
    {
        f4_t t[4];
        load_row_mfma(N.U + (size_t)(pe_s[wv][min(col, np - 1)] / kFastP) * R, kk, t);
        widen_row_mfma(t, ua);
    }
    while (true) {
        const int e_end = starts ? __builtin_ctzll(starts) : np;
        const size_t gc0 = (size_t)g * A.nodes[l] + (size_t)v * b;      // the node's first child
        // block 0's children rows and counts (the next block's are loaded while
        // this one is multiplied)
        f4_t cur[4];
        load_row_mfma(Cl + (gc0 + min(col, b - 1)) * R, kk, cur);
        int cnt_cur = col < b ? cn[gc0 + col] : 0;
        if (leaf) {
            // lane c: child c's member range and first members (clamped into the
            // head's member array: an empty leaf may start at n)
            const int32_t *pg = pm + (size_t)g * A.n;
            const int32_t *lg = (const int32_t *)(A.index + A.leaf_off_off) + (size_t)g * (A.nodes[l] + 1) + (size_t)v * b;
            const int c = min(lane, b - 1);
            const int a0 = lg[c], len = lane < b ? lg[c + 1] - a0 : 0;
            int32_t mem[kNmMemReg];
#pragma unroll
            for (int t = 0; t < kNmMemReg; ++t) mem[t] = pg[min<int64_t>(a0 + max(0, min(t, len - 1)), A.n - 1)];
            const int32_t last = len > kNmMemReg ? pg[a0 + len - 1] : mem[kNmMemReg - 1];
            wave_sync();                               // the previous run's readers are done
            info_s[wv][0][lane] = a0;
            info_s[wv][1][lane] = len;
            info_s[wv][2][lane] = last;
#pragma unroll
            for (int t = 0; t < kNmMemReg; ++t) info_s[wv][3 + t][lane] = mem[t];
            wave_sync();
        }
#pragma unroll 1
        for (int cb = 0; cb < ncb; ++cb) {
            const int c = 16 * cb + col;               // child index inside the node
            const bool more = cb + 1 < nvb;
            f4_t nxt[4];
            int cnt_nxt = 0;
            if (more) {
                load_row_mfma(Cl + (gc0 + min(c + 16, b - 1)) * R, kk, nxt);
                cnt_nxt = c + 16 < b ? cn[gc0 + c + 16] : 0;
            }
            const int c_cnt = cb < nvb ? cnt_cur : 0;
            const d4_t acc = cb < nvb ? mfma_dot64(ua, cur) : d4_t{0.0, 0.0, 0.0, 0.0};
            int c_a0 = 0, c_len = 0, c_last = 0;
            int32_t mem[kNmMemReg];
            if (leaf) {
                const int ci = min(c, 63);
                c_a0 = info_s[wv][0][ci];
                c_len = c_cnt > 0 ? info_s[wv][1][ci] : 0;
                c_last = info_s[wv][2][ci];
#pragma unroll
                for (int t = 0; t < kNmMemReg; ++t) mem[t] = info_s[wv][3 + t][ci];
            }
#pragma unroll 1
            for (int e = 0; e < 4; ++e) {
                const int q = kk + 4 * e;
                if (q < s || q >= e_end) continue;
                const double sc = e == 0 ? acc[0] : e == 1 ? acc[1] : e == 2 ? acc[2] : acc[3];
                const int pe_e = pe_s[wv][q];
                int ec = c_len, fc = 0;
                if (leaf && c_len > 0) {
                    const AttnSet as = attn_set(pp_s[wv][q], A.n, A.n_sink, A.window);
                    const int32_t first = mem[0];
                    if (as.all || (first >= as.rlo && c_last <= as.rhi)) {
                    } else if (c_last < as.rlo || first > as.rhi) {
                        ec = 0;
                    } else if (c_len <= kNmMemReg) {
                        int a = 0, z = 0;
#pragma unroll
                        for (int u = 0; u < kNmMemReg; ++u) {
                            a += (u < c_len && mem[u] < as.rlo) ? 1 : 0;
                            z += (u < c_len && mem[u] <= as.rhi) ? 1 : 0;
                        }
                        fc = a;
                        ec = max(0, z - a);
                    } else {
                        in_range(as, pm + (size_t)g * A.n + c_a0, c_len, fc, ec);
                    }
                }
                const bool ok = c_cnt > 0 && (!leaf || ec > 0);
                const int j = pe_e % kFastP;
                const uint64_t key = ok ? make_key_slot((float)sc, (uint32_t)(v * b + c), j * 64 + c) : 0ull;
                const size_t o = (size_t)(pe_e / kFastP) * (kFastP * 64) + j * 64 + c;
                N.keys[o] = key;
                if (leaf) { N.eli[o] = ok ? ec : 0; N.lof[o] = c_a0 + (ok ? fc : 0); }
            }
            if (more) {
#pragma unroll
                for (int h = 0; h < 4; ++h) cur[h] = nxt[h];
                cnt_cur = cnt_nxt;
            }
        }
        if (!starts) break;
        s = __builtin_ctzll(starts);
        starts &= starts - 1;
        g = (int)((__builtin_amdgcn_readfirstlane(pe_s[wv][s]) / kFastP) % A.h_kv);
        v = __builtin_amdgcn_readfirstlane(pv_s[wv][s]);
    }
}

// Candidate e of a group in slot order: slot e, or with b <= 32 (packed) the
// e-th of the slots j * 64 + c, c < 32.
LSA_DEV int nm_slot(int e, bool packed) { return packed ? (e >> 5) * 64 + (e & 31) : e; }

// this group's candidates, KPT per thread (slots beyond keep are empty)
template <int KPT>
LSA_DEV void nm_load_keys(const NmArgs &N, int64_t grp, uint64_t (&k)[KPT], bool packed) {
    const int keep = N.keep[grp];
    const int per = packed ? 32 : 64, tot = kFastP * per;
#pragma unroll
    for (int ii = 0; ii < KPT; ++ii) {
        const int e = KPT * (int)threadIdx.x + ii;
        k[ii] = (e < tot && e / per < keep) ? N.keys[(size_t)grp * (kFastP * 64) + nm_slot(e, packed)] : 0ull;
    }
}

// Internal levels: the top `beam` of each group's candidates, one wave per
// group (four groups a workgroup, no workgroup barrier).  The candidates sit
// KPL a lane (KPL = 8: the 512 packed slots of b <= 32; 16: all 1024); a wave
// radix selection takes eight bits a round from the top and stops once the
// digit holding the boundary is taken whole (as block_radix_select), then a
// one-wave sort orders the kept keys.
template <int KPL>
__global__ __launch_bounds__(256) void k_nm_keep_w(NmArgs N) {
    __shared__ __attribute__((aligned(16))) int hist_s[4][256];
    __shared__ uint64_t col_s[4][kWave];
    const int wv = threadIdx.x / kWave, lane = lane_id();
    const int64_t grp = (int64_t)blockIdx.x * 4 + wv;
    if (grp >= N.groups) return;                            // (uniform in the wave)
    constexpr bool packed = KPL == 8;
    constexpr int per = packed ? 32 : 64, tot = kFastP * per;
    const int keep = N.keep[grp];
    uint64_t k[KPL];
#pragma unroll
    for (int ii = 0; ii < KPL; ++ii) {
        const int e = lane + kWave * ii;
        k[ii] = e / per < keep ? N.keys[(size_t)grp * (kFastP * 64) + nm_slot(e, packed)] : 0ull;
    }
    static_assert(KPL * kWave == tot, "a lane per 1/64 of the slots");
    int *hist = hist_s[wv];
    int want = N.S.beam;
    uint64_t prefix = 0, mask = 0;
    bool none = false;
    for (int shift = 56; shift >= 0; shift -= 8) {
        wave_sync();                                        // the last round's reads done
        *reinterpret_cast<int4 *>(hist + 4 * lane) = int4{0, 0, 0, 0};
        wave_sync();
#pragma unroll
        for (int ii = 0; ii < KPL; ++ii)
            if (k[ii] != 0 && (k[ii] & mask) == prefix) atomicAdd(&hist[(int)((k[ii] >> shift) & 255u)], 1);
        wave_sync();
        // lane l holds digits 255 - 4 l - j (j = 0..3): the count of the
        // larger digits is an exclusive scan in lane order
        const int4 hq = *reinterpret_cast<const int4 *>(hist + 252 - 4 * lane);
        const int h[4] = {hq.w, hq.z, hq.y, hq.x};
        const int lsum = h[0] + h[1] + h[2] + h[3];
        const int incl = wave_incl_scan_add(lsum);
        int before = incl - lsum, dg = -1, rest = 0, hv = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (h[j] > 0 && before < want && before + h[j] >= want) { dg = 255 - 4 * lane - j; rest = want - before; hv = h[j]; }
            before += h[j];
        }
        const uint64_t fm = __ballot(dg >= 0);
        if (fm == 0) { none = true; break; }                // all keys together weigh less than want
        const int fl = __builtin_ctzll(fm);
        dg = __builtin_amdgcn_readlane(dg, fl);
        want = __builtin_amdgcn_readlane(rest, fl);
        hv = __builtin_amdgcn_readlane(hv, fl);
        prefix |= (uint64_t)dg << shift;
        mask |= (uint64_t)255 << shift;
        if (hv == want) break;                              // the whole digit is taken
    }
    const uint64_t thr = none ? 0ull : prefix;
    // the kept keys (min(beam, nonzero) of them) gathered and sorted
    int mine = 0;
#pragma unroll
    for (int ii = 0; ii < KPL; ++ii) mine += (k[ii] != 0 && k[ii] >= thr) ? 1 : 0;
    const int incl = wave_incl_scan_add(mine);
    int at = incl - mine;
    const int nk = __builtin_amdgcn_readlane(incl, kWave - 1);
#pragma unroll
    for (int ii = 0; ii < KPL; ++ii)
        if (k[ii] != 0 && k[ii] >= thr) col_s[wv][at++] = k[ii];
    wave_sync();
    uint64_t key = lane < nk ? col_s[wv][lane] : 0ull;
    int pay = 0;
    wave_sort_desc(key, pay);
    if (lane < kFastP) N.kept[grp * kFastP + lane] = lane < nk ? (int32_t)slot_key_id(key) : 0;
    if (lane == 0) N.keep[grp] = nk;
}

// KPT = 4: 1024 candidate slots; KPT = 2: the 512 packed slots of b <= 32
template <int KPT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(7))) void k_nm_finish(NmArgs N) {
    __shared__ __attribute__((aligned(16))) uint64_t sk[1024];   // the sort's, then the copy's position marks
    __shared__ int dl_s[256 * KPT];
    __shared__ int eli_s[kFastP * 64], lof_s[kFastP * 64];
    static_assert(sizeof(sk) >= kFlatCap * sizeof(int), "the position marks reuse the sort's array");
    __shared__ int scratch[8];
    __shared__ float cut_s;
    __shared__ unsigned long long msk_s[kFastP];
    __shared__ int32_t bnd_s[2];
    const SelectArgs &A = N.S;
    const int64_t grp = blockIdx.x;
    const int64_t i = N.row0 + grp / A.h_kv;
    const int g = (int)(grp % A.h_kv);
    const int tid = threadIdx.x;
    if (tid == 0) { cut_s = -INFINITY; bnd_s[0] = -1; bnd_s[1] = 0; }
    if (tid < kFastP) msk_s[tid] = 0ull;
    // (the attention's: the kept count and where this group's slots sit in
    // pairs, loaded early)
    const int keepv = N.pinf ? N.keep[grp] : 0;
    const int32_t pos = (N.pinf && tid < kFastP) ? N.ppos[grp * kFastP + tid] : 0;
    uint64_t k4[KPT];
    nm_load_keys<KPT>(N, grp, k4, KPT == 2);
    {
        // the eligible counts and first members of the thread's slots, loaded
        // with the keys and kept in LDS by slot for the sorted keys to find
        const int32_t *eli = N.eli + (size_t)grp * (kFastP * 64);
        const int32_t *lof = N.lof + (size_t)grp * (kFastP * 64);
        const int keep = N.keep[grp], per = KPT == 2 ? 32 : 64;
        int ev[KPT], lv[KPT];
#pragma unroll
        for (int ii = 0; ii < KPT; ++ii) {
            const int e = KPT * tid + ii, sl = nm_slot(e, KPT == 2);
            const bool in = e < kFastP * per && e / per < keep;
            ev[ii] = in ? eli[sl] : 0;
            lv[ii] = in ? lof[sl] : 0;
        }
#pragma unroll
        for (int ii = 0; ii < KPT; ++ii) {
            const int sl = nm_slot(KPT * tid + ii, KPT == 2);
            eli_s[sl] = ev[ii];
            lof_s[sl] = lv[ii];
        }
    }
    block_sort_desc<KPT>(k4, sk);
    lds_barrier();                      // eli_s and lof_s written by every thread
    const int32_t *pm = (const int32_t *)(A.index + A.perm_off) + (size_t)g * A.n;
    int e4[KPT], tot = 0;
#pragma unroll
    for (int ii = 0; ii < KPT; ++ii) {
        e4[ii] = (k4[ii] != 0) ? eli_s[(int)(k4[ii] & 1023u)] : 0;
        tot += e4[ii];
    }
    int total;
    int off = block_excl_scan(tot, scratch, &total);
    const int count = min(A.k, total);
    int32_t *out = A.sel + ((size_t)i * A.h_kv + g) * A.row;
    int take[KPT], a0v[KPT], offv[KPT];
#pragma unroll
    for (int ii = 0; ii < KPT; ++ii) {
        offv[ii] = off;
        take[ii] = (e4[ii] > 0 && off < count) ? min(e4[ii], count - off) : 0;
        a0v[ii] = take[ii] > 0 ? lof_s[(int)(k4[ii] & 1023u)] : 0;
        if (take[ii] > 0 && count == A.k && off + e4[ii] >= A.k) cut_s = key_score(k4[ii]);
        off += e4[ii];
    }
    if (N.pinf) {
        // the taken leaves per kept node, and the one leaf (if any) whose
        // eligible members are taken only in part: its last taken key
#pragma unroll
        for (int ii = 0; ii < KPT; ++ii) {
            if (take[ii] <= 0) continue;
            const int slot = (int)(k4[ii] & 1023u);
            atomicOr(&msk_s[slot >> 6], 1ull << (slot & 63));
            if (take[ii] < e4[ii]) { bnd_s[0] = slot; bnd_s[1] = pm[a0v[ii] + take[ii] - 1]; }
        }
    }
    if (count <= kFlatCap) fill_members_flat<KPT>(pm, out, take, a0v, offv, count, reinterpret_cast<int *>(sk), dl_s, scratch);
    else fill_members<KPT, 8>(pm, out, take, a0v, offv);
    const AttnSet as = attn_set(A.q_pos[i], A.n, A.n_sink, A.window);
    for (int t = tid; t < as.nloc; t += blockDim.x) out[count + t] = local_key(as, t);
    for (int t = count + as.nloc + tid; t < A.row; t += blockDim.x) out[t] = -1;
    __syncthreads();
    if (tid == 0) {
        A.sel_count[(size_t)i * A.h_kv + g] = count + as.nloc;
        if (A.sel_cutoff) A.sel_cutoff[(size_t)i * A.h_kv + g] = cut_s;
    }
    if (N.pinf && tid < keepv) {
        // the attention's record of kept slot tid, at its place in pairs
        const uint64_t mask = msk_s[tid];
        const int32_t bs = bnd_s[0];
        const int32_t bc = (bs >= 0 && (bs >> 6) == tid) ? (bs & 63) : -1;
        N.pinf[2 * pos] = uint4{(uint32_t)mask, (uint32_t)(mask >> 32), (uint32_t)(grp * kFastP + tid), (uint32_t)as.rlo};
        N.pinf[2 * pos + 1] = uint4{(uint32_t)as.rhi, (uint32_t)bc, (uint32_t)bnd_s[1], 0u};
    }
}

static inline size_t nm_a256(size_t x) { return (x + 255) & ~(size_t)255; }

struct NmWs { float *U; int32_t *kept, *keep; uint64_t *keys; int32_t *eli, *lof, *ncnt, *noff, *fptr, *pairs, *pnode; size_t bytes; };

// (after the workspace's reserved prefix, which this path never writes)
static NmWs carve_nm_ws(char *base, int64_t groups, int h_kv, int64_t max_nodes) {
    size_t cur = (size_t)ws_reserved_bytes();
    NmWs w{};
    auto take = [&](size_t n) { char *p = base ? base + cur : nullptr; cur = nm_a256(cur + n); return p; };
    w.U = (float *)take(sizeof(float) * groups * kFastR);
    w.kept = (int32_t *)take(sizeof(int32_t) * groups * kFastP);
    w.keep = (int32_t *)take(sizeof(int32_t) * groups);
    w.keys = (uint64_t *)take(sizeof(uint64_t) * groups * kFastP * 64);
    w.eli = (int32_t *)take(sizeof(int32_t) * groups * kFastP * 64);
    w.lof = (int32_t *)take(sizeof(int32_t) * groups * kFastP * 64);
    w.ncnt = (int32_t *)take(sizeof(int32_t) * (h_kv * max_nodes + 1));
    w.noff = (int32_t *)take(sizeof(int32_t) * (h_kv * max_nodes + 1));
    w.fptr = (int32_t *)take(sizeof(int32_t) * (h_kv * max_nodes + 1));
    w.pairs = (int32_t *)take(sizeof(int32_t) * groups * kFastP);
    w.pnode = (int32_t *)take(sizeof(int32_t) * groups * kFastP);
    w.bytes = cur;
    return w;
}

constexpr int64_t kNmRows = 32768;  // rows per batch the workspace query sizes for

// the node-major path applies to the throughput kernel's shapes
bool nm_shape_ok(int r, int b, int L, int beam, int d, const int64_t *nodes) {
    return r == kFastR && b <= 64 && beam <= kFastP && L >= 2 && d <= 256 && nodes[L] <= ((int64_t)1 << 22);
}

// Workspace bytes of one batch: the selection's buffers, then (G > 0) those
// of the node-major attention that follows it.
static int64_t nm_batch_bytes(int64_t groups, int h_kv, int L, const int64_t *nodes, int G) {
    const int64_t sel = (int64_t)carve_nm_ws(nullptr, groups, h_kv, nodes[L - 1]).bytes;
    return G > 0 ? sel + (int64_t)carve_nma_ws(nullptr, groups, G, (int64_t)h_kv * nodes[L - 1]).bytes : sel;
}

int64_t nm_workspace_bytes(int64_t m, int h_kv, int L, const int64_t *nodes) {
    return nm_batch_bytes(std::max<int64_t>(1, std::min(m, kNmRows)) * h_kv, h_kv, L, nodes, 0);
}

int64_t nm_attend_workspace_bytes(int64_t m, int h_q, int h_kv, int L, const int64_t *nodes) {
    return nm_batch_bytes(std::max<int64_t>(1, std::min(m, kNmRows)) * h_kv, h_kv, L, nodes, h_q / h_kv);
}

static int64_t nm_batch_rows(int64_t m, int h_kv, int L, const int64_t *nodes, int64_t ws_bytes, int G = 0) {
    int64_t mb = std::min(m, kNmRows);
    while (mb > 0 && nm_batch_bytes(mb * h_kv, h_kv, L, nodes, G) > ws_bytes) mb >>= 1;
    return mb;
}

// What the node-major attention after each batch needs besides the selection.
struct NmAttendReq { const void *K, *V; float scale; void *out; float *lse; };

static hipError_t select_nm(const SelectArgs &A, int dtype, void *ws, int64_t ws_bytes, hipStream_t st,
                            const NmAttendReq *att = nullptr) {
    const int G = att ? A.h_q / A.h_kv : 0;
    const int64_t mb = nm_batch_rows(A.m, A.h_kv, A.L, A.nodes, ws_bytes, G);
    if (mb < 1) return hipErrorInvalidValue;
    // the matrix-core top step takes 16-byte loads of 8-element query chunks
    const bool top_mfma = A.d % 8 == 0 && ((uintptr_t)A.Q & 15) == 0;
    if (top_mfma && nm_top_mfma_lds(A.d) > 65536) {
        const size_t lds = nm_top_mfma_lds(A.d);
        const hipError_t e = dtype == 0
            ? hipFuncSetAttribute((const void *)k_nm_top_mfma<float, 0>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)
            : hipFuncSetAttribute((const void *)k_nm_top_mfma<bf16_t, 0>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    for (int64_t r0 = 0; r0 < A.m; r0 += mb) {
        const int64_t nb = std::min(mb, A.m - r0);
        const int64_t groups = nb * A.h_kv;
        NmWs w = carve_nm_ws((char *)ws, groups, A.h_kv, A.nodes[A.L - 1]);
        NmArgs N{};
        N.S = A; N.row0 = r0; N.groups = groups;
        N.U = w.U; N.kept = w.kept; N.keep = w.keep; N.keys = w.keys; N.eli = w.eli; N.lof = w.lof;
        N.ncnt = w.ncnt; N.noff = w.noff; N.fptr = w.fptr; N.pairs = w.pairs; N.pnode = w.pnode;
        NmaWs aw{};
        if (att) {
            aw = carve_nma_ws((char *)ws + w.bytes, groups, G, (int64_t)A.h_kv * A.nodes[A.L - 1]);
            N.ppos = aw.ppos;
            N.pinf = (uint4 *)aw.pinf;
        }
        if (top_mfma) {
            const dim3 tg((unsigned)((nb + kTopMRows - 1) / kTopMRows), (unsigned)A.h_kv);
            const size_t lds = nm_top_mfma_lds(A.d);
            if (dtype == 0 && A.d == 128) hipLaunchKernelGGL((k_nm_top_mfma<float, 32>), tg, dim3(256), lds, st, N);
            else if (dtype == 0) hipLaunchKernelGGL((k_nm_top_mfma<float, 0>), tg, dim3(256), lds, st, N);
            else if (A.d == 128) hipLaunchKernelGGL((k_nm_top_mfma<bf16_t, 32>), tg, dim3(256), lds, st, N);
            else hipLaunchKernelGGL((k_nm_top_mfma<bf16_t, 0>), tg, dim3(256), lds, st, N);
        } else {
            const dim3 tg((unsigned)((nb + kTopRows - 1) / kTopRows), (unsigned)A.h_kv);
            if (dtype == 0) hipLaunchKernelGGL(k_nm_top<float>, tg, dim3(256), 0, st, N);
            else hipLaunchKernelGGL(k_nm_top<bf16_t>, tg, dim3(256), 0, st, N);
        }
        for (int l = 2; l <= A.L; ++l) {
            N.level = l;
            const int64_t cnt = (int64_t)A.h_kv * A.nodes[l - 1];
            const unsigned cg = (unsigned)((groups * kFastP + kNmChunk - 1) / kNmChunk);
            hipLaunchKernelGGL(k_nm_zero, dim3((unsigned)std::min<int64_t>((cnt + 255) / 256, 1024)), dim3(256), 0, st, N,
                               cnt);
            const size_t hb = cnt <= kNmBins ? (size_t)cnt * sizeof(int) : 0;
            hipLaunchKernelGGL(k_nm_count, dim3(cg), dim3(256), hb, st, N, cnt);
            hipLaunchKernelGGL(k_nm_scan, dim3(1), dim3(kNmScanT), 0, st, N, cnt);
            hipLaunchKernelGGL(k_nm_fill, dim3(cg), dim3(256), hb, st, N, cnt);
            const bool packed = A.b <= 32;
            hipLaunchKernelGGL(k_nm_score_mfma, dim3((unsigned)((groups * kFastP + 63) / 64)), dim3(256), 0, st, N);
            if (l < A.L && packed) hipLaunchKernelGGL(k_nm_keep_w<8>, dim3((unsigned)((groups + 3) / 4)), dim3(256), 0, st, N);
            else if (l < A.L) hipLaunchKernelGGL(k_nm_keep_w<16>, dim3((unsigned)((groups + 3) / 4)), dim3(256), 0, st, N);
            else if (packed) hipLaunchKernelGGL(k_nm_finish<2>, dim3((unsigned)groups), dim3(256), 0, st, N);
            else hipLaunchKernelGGL(k_nm_finish<4>, dim3((unsigned)groups), dim3(256), 0, st, N);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (att) {
            // the leaf level's pairs (grouped by kept level-(L-1) node) and the
            // records the finish wrote for them drive the attention of this batch
            NmaBatch B{};
            B.Q = A.Q; B.K = att->K; B.V = att->V; B.q_pos = A.q_pos; B.row0 = r0; B.groups = groups;
            B.h_q = A.h_q; B.h_kv = A.h_kv; B.n = A.n; B.b = A.b;
            B.nodes_prev = A.nodes[A.L - 1]; B.nleaf = A.nodes[A.L];
            B.leaf_off = (const int32_t *)(A.index + A.leaf_off_off);
            B.perm = (const int32_t *)(A.index + A.perm_off);
            B.n_sink = A.n_sink; B.window = A.window;
            B.pairs = w.pairs; B.noff = w.noff; B.keep = w.keep;
            B.ws = aw; B.scale = att->scale; B.out = att->out; B.lse = att->lse;
            if ((e = nm_attend_batch(B, st)) != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

hipError_t select_attend_nm(const void *Q, const void *K, const void *V, int dtype, int64_t m, int h_q, int d,
                            const int32_t *q_pos, const char *index, int64_t n, int h_kv, int r, int b, int L,
                            const int64_t *nodes, const int64_t *centroid_off, const int64_t *count_off,
                            int64_t leaf_off_off, int64_t perm_off, const float *W, int beam, int k, int n_sink,
                            int window, int32_t *sel, int32_t *sel_count, float *sel_cutoff, float scale, void *out,
                            float *lse, void *ws, int64_t ws_bytes, hipStream_t st) {
    SelectArgs A{};
    A.Q = Q; A.m = m; A.h_q = h_q; A.h_kv = h_kv; A.d = d; A.q_pos = q_pos; A.index = index; A.n = n;
    A.r = r; A.b = b; A.L = L;
    for (int l = 0; l <= L; ++l) { A.nodes[l] = nodes[l]; A.centroid_off[l] = centroid_off[l]; A.count_off[l] = count_off[l]; }
    A.leaf_off_off = leaf_off_off; A.perm_off = perm_off; A.W = W; A.beam = beam; A.k = k;
    A.n_sink = n_sink; A.window = window; A.row = k + n_sink + window;
    A.sel = sel; A.sel_count = sel_count; A.sel_cutoff = sel_cutoff;
    const NmAttendReq att{K, V, scale, out, lse};
    return select_nm(A, dtype, ws, ws_bytes, st, &att);
}

// The node-major attention runs when the shapes allow and a batch of at least
// one row fits the workspace.
bool nm_attend_fits(int64_t m, int h_q, int h_kv, int L, const int64_t *nodes, int64_t ws_bytes) {
    return nm_batch_rows(m, h_kv, L, nodes, ws_bytes, h_q / h_kv) >= 1;
}

hipError_t select_keys(const void *Q, int dtype, int64_t m, int h_q, int d, const int32_t *q_pos, const char *index,
                       int64_t n, int h_kv, int r, int b, int L, const int64_t *nodes, const int64_t *centroid_off,
                       const int64_t *count_off, int64_t leaf_off_off, int64_t perm_off, const float *W, int beam,
                       int k, int n_sink, int window, int32_t *sel, int32_t *sel_count, float *sel_cutoff,
                       void *ws, int64_t ws_bytes, hipStream_t st) {
    SelectArgs A{};
    A.Q = Q; A.m = m; A.h_q = h_q; A.h_kv = h_kv; A.d = d; A.q_pos = q_pos; A.index = index; A.n = n;
    A.r = r; A.b = b; A.L = L;
    for (int l = 0; l <= L; ++l) { A.nodes[l] = nodes[l]; A.centroid_off[l] = centroid_off[l]; A.count_off[l] = count_off[l]; }
    A.leaf_off_off = leaf_off_off; A.perm_off = perm_off; A.W = W; A.beam = beam; A.k = k;
    A.n_sink = n_sink; A.window = window; A.row = k + n_sink + window;
    A.sel = sel; A.sel_count = sel_count; A.sel_cutoff = sel_cutoff;
    const dim3 grid((unsigned)m, (unsigned)h_kv);
    if (ws && nm_shape_ok(r, b, L, beam, d, nodes) && nm_batch_rows(m, h_kv, L, nodes, ws_bytes) >= 1)
        return select_nm(A, dtype, ws, ws_bytes, st);
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
