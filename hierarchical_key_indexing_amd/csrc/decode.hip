// Multi-workgroup descent (and fused attention) for few query rows (gfx950).
//
// Same method and arithmetic as k_select / k_attend (top-down descent with a
// fixed budget per level, "Latent Sparse Attention Breaks Through the
// Million-Token Context Bottleneck", kongchang.com, section "How LSA Sidesteps
// Per-Key Scoring with Hierarchical Clustering"; retrieval of a fixed number of
// keys from the chosen clusters and attention over them, "Latent sparse
// attention", bdtechtalks.com, section "How latent sparse attention works"),
// laid out for latency when there are only a few (row, KV head) groups, as in
// single-request decode.
//
// Each group gets P = beam workgroups.  Every workgroup computes the group's
// latent query and the level-1 ranking itself (identical results), then at
// each deeper level workgroup p scores the children of the p-th kept node,
// sorts them within one wave and publishes the sorted list.  After a group
// barrier every workgroup derives the global ranks by binary search in the P
// sorted lists (the global top-beam at internal levels; at the leaf level each
// leaf's count of eligible keys retrieved before it), so no workgroup sorts
// more than 64 keys.  Workgroup p then writes its own leaves' keys at their
// retrieval offsets and attends over them; the last workgroup of the group to
// finish merges the P partial softmax states and resets the group's counters.
//
// Group barriers spin on a device-scope counter in the caller's workspace;
// the grid is at most one workgroup per compute unit, and every spin is
// bounded (a flag in the workspace records a timeout).
#include "common.h"
#include "internal.h"

namespace lsa {

constexpr int kTKD = 64;           // keys per attention tile
constexpr int kMaxP = 32;          // beam limit of this path
constexpr int kMemCap = 2048;      // node members staged in LDS
constexpr int kSpinLimit = 1 << 20;

struct DecodeArgs {
    const void *Q, *K, *V;
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
    int32_t *sel, *sel_count;
    float *sel_cutoff;
    float scale_log2;
    void *out;
    float *lse;
    // workspace
    int32_t *ctrl;        // [groups][4]: barrier, arrivals, timeout flag
    uint64_t *lists;      // [L-2][groups][P][beam]
    uint64_t *leaf_keys;  // [groups][P][64]
    int32_t *leaf_pre;    // [groups][P][64]
    float *part;          // [groups][P][G*d + 2*G]
};

// ---------------------------------------------------------------- wave helpers
LSA_DEV uint64_t shfl_xor64(uint64_t v, int m) {
    const uint32_t lo = __shfl_xor((unsigned int)(v & 0xffffffffu), m, kWave);
    const uint32_t hi = __shfl_xor((unsigned int)(v >> 32), m, kWave);
    return ((uint64_t)hi << 32) | lo;
}

// Bitonic sort of one 64-bit key (plus payload) per lane, descending by lane.
LSA_DEV void wave_sort_desc(uint64_t &key, int &pay) {
    const int l = lane_id();
#pragma unroll
    for (int size = 2; size <= kWave; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const uint64_t ok = shfl_xor64(key, stride);
            const int op = __shfl_xor(pay, stride, kWave);
            const bool lower = (l & stride) == 0;
            const bool desc_seg = (l & size) == 0;      // this segment ends descending
            // lower lane keeps the larger key in a descending segment
            const bool take_other = (lower == desc_seg) ? (ok > key) : (ok < key);
            if (take_other) { key = ok; pay = op; }
        }
    }
}

LSA_DEV float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}
LSA_DEV float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// number of entries > x in a list sorted descending
LSA_DEV int count_gt_desc(const uint64_t *a, int len, uint64_t x) {
    int lo = 0, hi = len;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (a[mid] > x) lo = mid + 1; else hi = mid;
    }
    return lo;
}

LSA_DEV int count_le_i32(const int32_t *a, int len, int32_t key) {
    int lo = 0, hi = len;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (a[mid] <= key) lo = mid + 1; else hi = mid;
    }
    return lo;
}

LSA_DEV float score_lds(const float *u, const float *row, int r) {
    double s = 0.0;
    for (int x = 0; x < r; ++x) s = fma((double)u[x], (double)row[x], s);
    return (float)s;
}

// Contiguous global -> LDS copy with U loads in flight per thread.
template <int U, typename E>
LSA_DEV void g2s_flat(E *dst, const E *__restrict__ src, int n) {
    for (int base = 0; base < n; base += U * (int)blockDim.x) {
        E t[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = base + (int)threadIdx.x + u * (int)blockDim.x;
            if (e < n) t[u] = src[e];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = base + (int)threadIdx.x + u * (int)blockDim.x;
            if (e < n) dst[e] = t[u];
        }
    }
}

// b rows of r floats (a node's children) into LDS rows of stride 65.
LSA_DEV void load_rows(float *Cs, const float *__restrict__ src, int b, int r) {
    if ((r & 3) == 0) g2s_rows<4>(Cs, 65, src, b * r, r);
    else g2s_scalar<16, float, float>(Cs, 65, src, b * r, r);
}

// All workgroups of a group wait here until `target` arrivals are counted.
LSA_DEV void group_barrier(int32_t *ctr, int target, int32_t *flag) {
    __syncthreads();
    if (threadIdx.x == 0) {
        __threadfence();
        __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        int spins = 0;
        while (__hip_atomic_load(ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < target) {
            __builtin_amdgcn_s_sleep(1);
            if (++spins > kSpinLimit) {
                __hip_atomic_store(flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
        __threadfence();
    }
    __syncthreads();
}

template <typename T, bool ATTEND>
__global__ __launch_bounds__(256) void k_decode(DecodeArgs A) {
    extern __shared__ float dyn[];                 // W staging, then attention tiles
    __shared__ float qbar_s[256];
    __shared__ float u_s[64];
    __shared__ float Cs[64 * 65];
    __shared__ int32_t ccnt[64];
    __shared__ int32_t clo[65];
    __shared__ int32_t kept_s[kMaxP];
    __shared__ uint64_t lk[kMaxP * 64];
    __shared__ int32_t lp[kMaxP * 64];
    __shared__ int32_t take_s[64], toff_s[65];
    __shared__ int32_t mem_s[kMemCap];
    __shared__ int keep_s, count_s, last_s, nz_s;
    __shared__ float m_run[16], l_run[16], alpha_s[16];
    __shared__ int32_t ids_s[kTKD];

    const int P = A.beam;
    const int p = blockIdx.x;
    const int gi = blockIdx.y;
    const int64_t i = gi / A.h_kv;
    const int g = gi % A.h_kv;
    const int G = A.h_q / A.h_kv;
    const int d = A.d, r = A.r, b = A.b, L = A.L;
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wv = tid / kWave;
    const T *Q = (const T *)A.Q;
    int32_t *ctrl = A.ctrl + (size_t)gi * 4;
    const int32_t pos = A.q_pos[i];
    const int64_t nleaf = A.nodes[L];
    const int32_t *perm = (const int32_t *)(A.index + A.perm_off) + (size_t)g * A.n;
    const int32_t *leaf_off = (const int32_t *)(A.index + A.leaf_off_off) + (size_t)g * (nleaf + 1);
    const bool all_eligible = pos >= A.n - 1;

    // ---- level-1 rows (independent of the query), W, the group's queries
    {
        const float *C1 = (const float *)(A.index + A.centroid_off[1]) + (size_t)g * A.nodes[1] * r;
        const int32_t *cn1 = (const int32_t *)(A.index + A.count_off[1]) + (size_t)g * A.nodes[1];
        if (tid < b) ccnt[tid] = cn1[tid];
        load_rows(Cs, C1, b, r);
        const float *Wg = A.W + (size_t)g * d * r;
        if (((d * r) & 3) == 0) g2s_rows<8>(dyn, d * r, Wg, d * r, d * r);
        else g2s_flat<16>(dyn, Wg, d * r);
        for (int t = tid; t < d; t += blockDim.x) {
            float qv[16];
#pragma unroll
            for (int h = 0; h < 16; ++h)
                qv[h] = (h < G) ? to_float(Q[((size_t)i * A.h_q + (size_t)g * G + h) * d + t]) : 0.0f;
            double s = 0.0;
#pragma unroll
            for (int h = 0; h < 16; ++h)
                if (h < G) s = s + (double)qv[h];
            qbar_s[t] = (float)(s / (double)G);
        }
        if (tid == 0) { count_s = 0; last_s = 0; }
    }
    __syncthreads();
    for (int c = tid; c < r; c += blockDim.x) {
        double s = 0.0;
        for (int t = 0; t < d; ++t) s = fma((double)qbar_s[t], (double)dyn[t * r + c], s);
        u_s[c] = (float)s;
    }
    __syncthreads();
    // ---- level 1 (every workgroup of the group computes the same ranking)
    if (wv == 0) {
        uint64_t key = 0;
        int pay = 0;
        if (lane < b && ccnt[lane] > 0) key = make_key(score_lds(u_s, Cs + lane * 65, r), (uint32_t)lane);
        const int nz = __popcll(__ballot(key != 0));
        wave_sort_desc(key, pay);
        const int keep = min(P, nz);
        if (lane < keep) kept_s[lane] = (int32_t)key_id(key);
        if (lane == 0) keep_s = keep;
    }
    __syncthreads();

    int barriers = 0;
    int64_t v = -1;
    for (int l = 2; l <= L; ++l) {
        const int keep_prev = keep_s;
        v = (p < keep_prev) ? kept_s[p] : -1;
        const bool leaf = (l == L);
        if (v >= 0) {
            const float *Cl = (const float *)(A.index + A.centroid_off[l]) + ((size_t)g * A.nodes[l] + (size_t)v * b) * r;
            const int32_t *cn = (const int32_t *)(A.index + A.count_off[l]) + (size_t)g * A.nodes[l] + (size_t)v * b;
            if (tid < b) ccnt[tid] = cn[tid];
            if (leaf && tid <= b) clo[tid] = leaf_off[(size_t)v * b + tid];
            load_rows(Cs, Cl, b, r);
        }
        __syncthreads();
        if (leaf && v >= 0) {
            // stage the node's members (leaves of one node are contiguous)
            const int m0 = clo[0], mn = clo[b] - clo[0];
            if (mn <= kMemCap) g2s_flat<8>(mem_s, perm + m0, mn);
            __syncthreads();
        }
        if (wv == 0) {
            uint64_t key = 0;
            int e = 0;
            if (v >= 0 && lane < b && ccnt[lane] > 0) {
                key = make_key(score_lds(u_s, Cs + lane * 65, r), (uint32_t)(v * b + lane));
                if (leaf) {
                    const int a0 = clo[lane], a1 = clo[lane + 1];
                    if (all_eligible) e = a1 - a0;
                    else if (clo[b] - clo[0] <= kMemCap) e = count_le_i32(mem_s + (a0 - clo[0]), a1 - a0, pos);
                    else e = count_le_i32(perm + a0, a1 - a0, pos);
                    if (e == 0) key = 0;
                }
            }
            wave_sort_desc(key, e);
            if (!leaf) {
                uint64_t *dst = A.lists + (((size_t)(l - 2) * (A.m * A.h_kv) + gi) * P + p) * P;
                if (lane < P) dst[lane] = key;
            } else {
                const int incl = wave_incl_scan_add(e);
                const size_t o = ((size_t)gi * P + p) * 64 + lane;
                A.leaf_keys[o] = key;
                A.leaf_pre[o] = incl;
            }
        }
        ++barriers;
        group_barrier(ctrl, barriers * P, ctrl + 2);
        if (!leaf) {
            const uint64_t *src = A.lists + ((size_t)(l - 2) * (A.m * A.h_kv) + gi) * P * P;
            g2s_flat<4>(lk, src, P * P);
            if (tid == 0) nz_s = 0;
            __syncthreads();
            for (int e = tid; e < P * P; e += blockDim.x) {
                const uint64_t x = lk[e];
                if (x == 0) continue;
                atomicAdd(&nz_s, 1);
                const int q = e / P, j = e % P;
                int rank = j;
                for (int q2 = 0; q2 < P; ++q2)
                    if (q2 != q) rank += count_gt_desc(lk + q2 * P, P, x);
                if (rank < P) kept_s[rank] = (int32_t)key_id(x);
            }
            __syncthreads();
            if (tid == 0) keep_s = min(P, nz_s);
            __syncthreads();
        }
    }

    // ---- fill: every workgroup places its own leaves' keys
    {
        const uint64_t *srck = A.leaf_keys + (size_t)gi * P * 64;
        const int32_t *srcp = A.leaf_pre + (size_t)gi * P * 64;
        g2s_flat<8>(lk, srck, P * 64);
        g2s_flat<8>(lp, srcp, P * 64);
        if (tid < 64) take_s[tid] = 0;
        __syncthreads();
        if (tid == 0) {
            int tot = 0;
            for (int q = 0; q < P; ++q) tot += lp[q * 64 + 63];
            count_s = min(A.k, tot);
        }
        __syncthreads();
        const int count = count_s;
        int32_t *out = A.sel + (size_t)gi * A.k;
        if (wv == 0 && v >= 0) {
            const uint64_t x = lk[p * 64 + lane];
            if (x != 0) {
                const int before = lane > 0 ? lp[p * 64 + lane - 1] : 0;
                const int e = lp[p * 64 + lane] - before;
                int wex = before;
                for (int q = 0; q < P; ++q) {
                    if (q == p) continue;
                    const int c = count_gt_desc(lk + q * 64, 64, x);
                    if (c > 0) wex += lp[q * 64 + c - 1];
                }
                const int take = max(0, min(e, count - wex));
                const int c = (int)(key_id(x) - (uint32_t)(v * b));
                take_s[c] = take;
                if (take > 0) {
                    const int a0 = clo[c];
                    for (int t = 0; t < take; ++t) out[wex + t] = perm[a0 + t];
                }
                if (count == A.k && wex < A.k && wex + e >= A.k && A.sel_cutoff)
                    A.sel_cutoff[gi] = key_score(x);
            }
        }
        for (int t = count + p * blockDim.x + tid; t < A.k; t += P * blockDim.x) out[t] = -1;
        if (p == 0 && tid == 0) {
            A.sel_count[gi] = count;
            if (count < A.k && A.sel_cutoff) A.sel_cutoff[gi] = -INFINITY;
        }
        __syncthreads();
    }

    if constexpr (ATTEND) {
        // ---- attention over this workgroup's own keys
        const int dp = d + 1;
        float *qs = dyn;                       // [G][d]
        float *Kt = qs + G * d;                // [TK][d + 1]
        float *Vt = Kt + kTKD * dp;            // [TK][d]
        float *S = Vt + kTKD * d;              // [G][TK]
        if (wv == 0) {
            const int tk = take_s[lane];
            const int incl = wave_incl_scan_add(tk);
            toff_s[lane] = incl - tk;
            if (lane == 63) toff_s[64] = incl;
        }
        for (int e = tid; e < G * d; e += blockDim.x)
            qs[e] = to_float(Q[((size_t)i * A.h_q + (size_t)g * G) * d + e]) * A.scale_log2;
        if (tid < 16) { m_run[tid] = -INFINITY; l_run[tid] = 0.0f; }
        __syncthreads();
        const int own = (v >= 0) ? toff_s[64] : 0;
        const int ne = (G * d + blockDim.x - 1) / blockDim.x;
        float acc[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[q] = 0.0f;
        const T *Kg = (const T *)A.K + (size_t)g * A.n * d;
        const T *Vg = (const T *)A.V + (size_t)g * A.n * d;
        const bool staged = v >= 0 && (clo[b] - clo[0]) <= kMemCap;
        for (int f0 = 0; f0 < own; f0 += kTKD) {
            const int nk = min(kTKD, own - f0);
            if (tid < nk) {
                const int f = f0 + tid;
                int lo = 0, hi = 64;                 // last leaf c with toff_s[c] <= f
                while (hi - lo > 1) { const int mid = (lo + hi) >> 1; if (toff_s[mid] <= f) lo = mid; else hi = mid; }
                const int off = clo[lo] + (f - toff_s[lo]);
                ids_s[tid] = staged ? mem_s[off - clo[0]] : perm[off];
            }
            __syncthreads();
            // gather rows, 8 elements per load
            gather_tile<T>(Kg, Vg, ids_s, nk, d, Kt, dp, Vt);
            __syncthreads();
            for (int e = tid; e < G * kTKD; e += blockDim.x) {
                const int h = e / kTKD, kk = e % kTKD;
                float s = -INFINITY;
                if (kk < nk) {
                    const float *qh = qs + h * d;
                    const float *kr = Kt + kk * dp;
                    s = 0.0f;
                    for (int t = 0; t < d; ++t) s = fmaf(qh[t], kr[t], s);
                }
                S[h * kTKD + kk] = s;
            }
            __syncthreads();
            for (int h = wv; h < G; h += blockDim.x / kWave) {
                const float x = S[h * kTKD + lane];
                const float mt = wave_max(x);
                const float mnew = fmaxf(m_run[h], mt);
                const float pr = (lane < nk) ? exp2f(x - mnew) : 0.0f;
                S[h * kTKD + lane] = pr;
                const float ls = wave_sum(pr);
                if (lane == 0) {
                    const float al = exp2f(m_run[h] - mnew);
                    alpha_s[h] = al;
                    l_run[h] = l_run[h] * al + ls;
                    m_run[h] = mnew;
                }
            }
            __syncthreads();
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                if (q >= ne) break;
                const int e = tid + q * blockDim.x;
                if (e >= G * d) break;
                const int h = e / d, t = e % d;
                const float *ph = S + h * kTKD;
                float a = acc[q] * alpha_s[h];
                for (int kk = 0; kk < nk; ++kk) a = fmaf(ph[kk], Vt[kk * d + t], a);
                acc[q] = a;
            }
            __syncthreads();
        }
        // partial state of this workgroup
        float *pp = A.part + ((size_t)gi * P + p) * (G * d + 2 * G);
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            if (q >= ne) break;
            const int e = tid + q * blockDim.x;
            if (e >= G * d) break;
            pp[e] = acc[q];
        }
        if (tid < G) { pp[G * d + tid] = m_run[tid]; pp[G * d + G + tid] = l_run[tid]; }
    }

    // ---- arrival; the last workgroup merges and resets the group's counters
    __syncthreads();
    if (tid == 0) {
        __threadfence();
        const int old = __hip_atomic_fetch_add(ctrl + 1, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        last_s = (old == P - 1);
        __threadfence();
    }
    __syncthreads();
    if (!last_s) return;
    if constexpr (ATTEND) {
        const float *pb = A.part + (size_t)gi * P * (G * d + 2 * G);
        const int stride = G * d + 2 * G;
        // per-(workgroup, head) weights 2^(m_q - M) and the total sums, in LDS
        float *wq = dyn;                       // [P][G]
        float *lq = dyn + kMaxP * 16;          // [P][G]
        float *Ms = lq + kMaxP * 16;           // [G], then L [G]
        for (int e = tid; e < P * G; e += blockDim.x) {
            const int q = e / G, h = e % G;
            wq[e] = pb[(size_t)q * stride + G * d + h];
            lq[e] = pb[(size_t)q * stride + G * d + G + h];
        }
        __syncthreads();
        if (tid < G) {
            float M = -INFINITY;
            for (int q = 0; q < P; ++q) M = fmaxf(M, wq[q * G + tid]);
            float l = 0.0f;
            for (int q = 0; q < P; ++q) {
                const float mq = wq[q * G + tid];
                const float w = (mq > -INFINITY) ? exp2f(mq - M) : 0.0f;
                wq[q * G + tid] = w;
                l += lq[q * G + tid] * w;
            }
            Ms[tid] = M;
            Ms[16 + tid] = l;
        }
        __syncthreads();
        for (int e = tid; e < G * d; e += blockDim.x) {
            const int h = e / d;
            float t[kMaxP];
#pragma unroll
            for (int q = 0; q < kMaxP; ++q) t[q] = (q < P) ? pb[(size_t)q * stride + e] : 0.0f;
            float o = 0.0f;
#pragma unroll
            for (int q = 0; q < kMaxP; ++q) if (q < P) o += t[q] * wq[q * G + h];
            const float l = Ms[16 + h];
            const size_t oh = (size_t)i * A.h_q + (size_t)g * G + h;
            ((T *)A.out)[oh * d + (e % d)] = from_float<T>(l > 0.0f ? o / l : 0.0f);
            if ((e % d) == 0 && A.lse) A.lse[oh] = (l > 0.0f) ? (Ms[h] + log2f(l)) * 0.69314718055994531f : -INFINITY;
        }
    }
    if (tid == 0) {
        __hip_atomic_store(ctrl, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(ctrl + 1, 0, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ---------------------------------------------------------------- host side
static inline size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

struct DecodeWs { int32_t *ctrl; uint64_t *lists, *leaf_keys; int32_t *leaf_pre; float *part; size_t bytes; };

static DecodeWs carve_decode_ws(char *base, int64_t groups, int P, int L, int G, int d) {
    size_t cur = 0;
    DecodeWs w{};
    auto take = [&](size_t n) { char *p = base ? base + cur : nullptr; cur = a256(cur + n); return p; };
    w.ctrl = (int32_t *)take(sizeof(int32_t) * 4 * (size_t)groups);
    w.lists = (uint64_t *)take(sizeof(uint64_t) * (size_t)(L > 2 ? L - 2 : 1) * groups * P * P);
    w.leaf_keys = (uint64_t *)take(sizeof(uint64_t) * (size_t)groups * P * 64);
    w.leaf_pre = (int32_t *)take(sizeof(int32_t) * (size_t)groups * P * 64);
    w.part = (float *)take(sizeof(float) * (size_t)groups * P * ((size_t)G * d + 2 * G));
    w.bytes = cur;
    return w;
}

static int device_cus() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cus[dev] == 0) {
        int c = 0;
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cus[dev] = c;
    }
    return cus[dev];
}

static size_t decode_dyn_bytes(int G, int d, int r) {
    const size_t att = sizeof(float) * ((size_t)G * d + (size_t)kTKD * (d + 1) + (size_t)kTKD * d + (size_t)G * kTKD);
    const size_t w = sizeof(float) * (size_t)d * r;
    return att > w ? att : w;
}

constexpr size_t kStaticLds = 56 * 1024;      // upper bound of k_decode's static LDS
constexpr size_t kLdsPerCu = 160 * 1024;

bool decode_path_ok(int64_t m, int h_q, int h_kv, int d, int r, int b, int L, int beam, int k) {
    const int G = h_q / h_kv;
    if (L < 2 || b > 64 || r > 64 || beam > kMaxP || beam < 1 || G > 16 || d > 256 || d % 8 != 0) return false;
    if (decode_dyn_bytes(G, d, r) + kStaticLds > kLdsPerCu) return false;
    (void)k;
    const int cus = device_cus();
    return cus > 0 && m * h_kv * beam <= cus;
}

int64_t decode_workspace_bytes(int64_t m, int h_q, int h_kv, int d, int L, int beam) {
    return (int64_t)carve_decode_ws(nullptr, m * h_kv, beam, L, h_q / h_kv, d).bytes;
}

hipError_t decode(const void *Q, const void *K, const void *V, int dtype, int64_t m, int h_q, int h_kv, int d,
                  const int32_t *q_pos, const char *index, int64_t n, int r, int b, int L, const int64_t *nodes,
                  const int64_t *centroid_off, const int64_t *count_off, int64_t leaf_off_off, int64_t perm_off,
                  const float *W, int beam, int k, int32_t *sel, int32_t *sel_count, float *sel_cutoff, float scale,
                  void *out, float *lse, void *ws, bool attend, hipStream_t st) {
    DecodeArgs A{};
    A.Q = Q; A.K = K; A.V = V; A.m = m; A.h_q = h_q; A.h_kv = h_kv; A.d = d; A.q_pos = q_pos;
    A.index = index; A.n = n; A.r = r; A.b = b; A.L = L;
    for (int l = 0; l <= L; ++l) { A.nodes[l] = nodes[l]; A.centroid_off[l] = centroid_off[l]; A.count_off[l] = count_off[l]; }
    A.leaf_off_off = leaf_off_off; A.perm_off = perm_off; A.W = W; A.beam = beam; A.k = k;
    A.sel = sel; A.sel_count = sel_count; A.sel_cutoff = sel_cutoff;
    A.scale_log2 = scale * 1.4426950408889634f; A.out = out; A.lse = lse;
    const int G = h_q / h_kv;
    DecodeWs w = carve_decode_ws((char *)ws, m * h_kv, beam, L, G, d);
    A.ctrl = w.ctrl; A.lists = w.lists; A.leaf_keys = w.leaf_keys; A.leaf_pre = w.leaf_pre; A.part = w.part;
    const size_t shm = decode_dyn_bytes(G, d, r);
    const dim3 grid((unsigned)beam, (unsigned)(m * h_kv));
    // allow the largest dynamic LDS this path uses, once per kernel and device
    static int attr_set[64][4] = {{0}};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    const int which = (dtype == 0 ? 0 : 2) + (attend ? 1 : 0);
    if (!attr_set[dev][which]) {
        const void *fn;
        if (dtype == 0) fn = attend ? (const void *)k_decode<float, true> : (const void *)k_decode<float, false>;
        else fn = attend ? (const void *)k_decode<bf16_t, true> : (const void *)k_decode<bf16_t, false>;
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)(kLdsPerCu - kStaticLds));
        if (e != hipSuccess) return e;
        attr_set[dev][which] = 1;
    }
    if (dtype == 0) {
        if (attend) hipLaunchKernelGGL((k_decode<float, true>), grid, dim3(256), shm, st, A);
        else hipLaunchKernelGGL((k_decode<float, false>), grid, dim3(256), shm, st, A);
    } else {
        if (attend) hipLaunchKernelGGL((k_decode<bf16_t, true>), grid, dim3(256), shm, st, A);
        else hipLaunchKernelGGL((k_decode<bf16_t, false>), grid, dim3(256), shm, st, A);
    }
    return hipGetLastError();
}

}  // namespace lsa
