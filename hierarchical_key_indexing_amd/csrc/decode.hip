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
// sorts them within one wave and publishes its top P (its whole sorted list at
// the leaf level, with the running eligible counts).  Every workgroup then
// derives global ranks from the published lists by side-by-side binary
// searches (the global top-beam at internal levels; at the leaf level, how
// many eligible keys are retrieved before each of its leaves), so no
// workgroup sorts more than 64 keys.  Workgroup p writes its own leaves' keys
// at their retrieval offsets, and then attends over an even 1/P slice of the
// retrieval order (matrix cores for bf16).  Each workgroup then sends every
// other one its partial softmax state for that workgroup's slice of the
// outputs, and merges the P states of its own slice.
//
// Workgroups exchange data through the caller's workspace without barriers:
// it starts zeroed, a writer publishes nonzero words with device-scope stores,
// and a reader polls each word it needs until it is nonzero (bounded).  Every
// word is zeroed again before the launch ends: a partial-state word by its
// one reader once read, the exchange words by all workgroups in slices once
// their merge has received every partial state (a workgroup sends its states
// only after its last exchange read).  A wait that gives up sets the status
// word at the start of the workspace, which the host reads
// (lsa_workspace_status, or after every call in debug mode); the workspace
// must then be zero-filled again before its next use.  The grid is at most
// one workgroup per compute unit, so every workgroup of a group is resident
// while the others wait on its words.  No other path of the library writes
// the part of a workspace that these workgroups poll (ws_reserved_bytes), so
// a stale word can only be one this kernel left, and it leaves none.
#include "common.h"
#include "internal.h"
#include "mfma_attn.h"
#include "lsa.h"

#include <atomic>
#include <mutex>

namespace lsa {

constexpr int kMaxP = 32;          // beam limit of this path
constexpr int kMemCap = 2048;      // node members staged in LDS
constexpr int kOwnCap = 2048;      // own (selected) keys listed in LDS
constexpr int kSpinLimit = 1 << 20;
constexpr uint64_t kEmpty = 1;     // published "no key" (real keys are >= 2^32)
constexpr int kTKD = 64;           // keys per tile of the vector attention path

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
    int n_sink, window;
    int row;              // entries per row of sel: k + n_sink + window
    int nx;               // XCDs (accelerator complexes) the grid is spread over
    int32_t *sel, *sel_count;
    float *sel_cutoff;
    float scale_log2;
    void *out;
    float *lse;
    // workspace
    int32_t *status;      // the workspace's status word (kStatusWaitTimeout bit)
    // Exchange buffers: zero before a launch, published with device-scope
    // stores of nonzero values, polled by the readers, zeroed again at the end.
    int32_t *ctrl;        // [groups][4]: -, -, a timeout flag seeded by the host (read and cleared by workgroup 0), -
    uint64_t *lists;      // [L-2][groups][P][P] top P child keys per workgroup (kEmpty: none)
    uint64_t *leaf_keys;  // [groups][P][64] sorted leaf keys (kEmpty: none)
    int32_t *leaf_pre;    // [groups][P][64] 1 + inclusive prefix of eligible counts
    int32_t *keys;        // [groups][k] 1 + key id at each retrieval position
    uint32_t *recs;       // [groups][P writers][P readers][rec_stride]: partial states (done tokens without attention)
};

// Partial-state records.  The G * d outputs of a group are cut into P slices,
// slice p = [slice_lo(p), slice_lo(p + 1)), merged by workgroup p.  Workgroup
// q sends p one record: its unnormalised outputs of slice p (at most
// slice_max words), then the maximum and the sum of each head the slice
// touches (at most slice_heads heads), each word stored as the complement of
// the float's bits, so that a published word is never zero.
// (32-bit: T * p stays below 2^31 for every buffer sliced here)
LSA_HOST_DEV inline int slice_lo(int T, int P, int p) { return (T * p) / P; }
LSA_HOST_DEV inline int slice_max(int T, int P) { return (T + P - 1) / P; }
LSA_HOST_DEV inline int slice_heads(int T, int P, int d) { return slice_max(T, P) / d + 2; }
LSA_HOST_DEV inline int rec_stride(int T, int P, int d, bool attend) {
    return attend ? (slice_max(T, P) + 2 * slice_heads(T, P, d) + 3) & ~3 : 4;
}
LSA_DEV uint32_t enc_word(float x) {
    uint32_t u = __float_as_uint(x);
    if (u == 0xFFFFFFFFu) u = 0x7FC00000u;     // (a NaN; any other float's complement is nonzero)
    return ~u;
}
LSA_DEV float dec_word(uint32_t w) { return __uint_as_float(~w); }

// ---------------------------------------------------------------- helpers
// For key x and the descending key lists a + q * stride (q = q0, q0 + dq, ...
// below nq; len <= LEN entries each): c[i] = number of leading entries of list
// q0 + i * dq greater than x.  Binary lifting, all lists side by side, so the
// dependent LDS reads take log2(LEN) + 1 rounds.
template <int NQ, int LEN>
LSA_DEV void count_gt_lists(const uint64_t *a, int stride, int q0, int dq, int nq, int len, uint64_t x, int (&c)[NQ]) {
#pragma unroll
    for (int i = 0; i < NQ; ++i) c[i] = 0;
#pragma unroll
    for (int s = LEN; s >= 1; s >>= 1) {
        // branch-free step, all reads issued before the first compare (lists
        // q >= nq are read but not counted; the caller's array holds
        // q0 + (NQ - 1) * dq + 1 lists of stride entries)
        uint64_t v[NQ];
#pragma unroll
        for (int i = 0; i < NQ; ++i) v[i] = a[(q0 + i * dq) * stride + min(c[i] + s, len) - 1];
#pragma unroll
        for (int i = 0; i < NQ; ++i) c[i] += (q0 + i * dq < nq && c[i] + s <= len && v[i] > x) ? s : 0;
    }
}

template <int RC>
LSA_DEV float score_lds(const double *u, const float *row, int r) {
    double s = 0.0;
    if constexpr (RC > 0 && RC % 4 == 0) {
        // 16-byte LDS reads (u, already widened, is a broadcast); products
        // summed in dimension order
        const double2 *u2 = reinterpret_cast<const double2 *>(u);
        const f4_t *r4 = reinterpret_cast<const f4_t *>(row);
#pragma unroll
        for (int x = 0; x < RC / 4; ++x) {
            const double2 a = u2[2 * x], b2 = u2[2 * x + 1];
            const f4_t c = r4[x];
            s = fma(a.x, (double)c.x, s);
            s = fma(a.y, (double)c.y, s);
            s = fma(b2.x, (double)c.z, s);
            s = fma(b2.y, (double)c.w, s);
        }
    } else {
        for (int x = 0; x < r; ++x) s = fma(u[x], (double)row[x], s);
    }
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
            t[u] = src[min(e, n - 1)];         // clamped: every load stays in bounds
        }
        __builtin_amdgcn_sched_barrier(0);     // all loads issued before the first store waits
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = base + (int)threadIdx.x + u * (int)blockDim.x;
            if (e < n) dst[e] = t[u];
        }
    }
}

// b <= 64 rows of 64 floats into LDS rows of stride kCS: four 16-byte loads per
// thread, all issued before any store (sources clamped to the b rows; rows at
// and beyond b receive copies that are never read).
LSA_DEV void load_rows64(float *Cs, const float *__restrict__ src, int b);

// LDS row stride of staged centroid rows: a multiple of 4 (16-byte row reads)
// whose eight consecutive rows start in eight different 4-bank groups.
constexpr int kCS = 68;

LSA_DEV void load_rows64(float *Cs, const float *__restrict__ src, int b) {
    const f4_t *s4 = reinterpret_cast<const f4_t *>(src);
    f4_t t[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) t[u] = s4[min((int)threadIdx.x + 256 * u, b * 16 - 1)];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int e = (int)threadIdx.x + 256 * u;
        *reinterpret_cast<f4_t *>(Cs + (e / 16) * kCS + (e % 16) * 4) = t[u];
    }
}

// b rows of r floats (one node's children) into LDS rows of stride kCS.
LSA_DEV void load_rows(float *Cs, const float *__restrict__ src, int b, int r) {
    if ((r & 3) == 0) g2s_rows<4>(Cs, kCS, src, b * r, r);
    else g2s_scalar<16, float, float>(Cs, kCS, src, b * r, r);
}

// Polls the words src[e] (e = threadIdx.x + blockDim.x * u < n) until each is
// nonzero; every round issues all of the thread's outstanding loads at once.
// Bounded: after kSpinLimit rounds `flag` (this workgroup's, in LDS) records a
// timeout and words still zero are returned as zero.
template <int U, typename W>
LSA_DEV void poll_nonzero(const W *src, int n, W (&out)[U], int32_t *flag) {
#pragma unroll
    for (int u = 0; u < U; ++u) out[u] = 0;
    for (int spins = 0;; ++spins) {
        bool missing = false;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = (int)threadIdx.x + (int)blockDim.x * u;
            if (e < n && out[u] == 0)
                out[u] = __hip_atomic_load(src + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) missing |= ((int)threadIdx.x + (int)blockDim.x * u < n) && out[u] == 0;
        if (!missing) break;
        if (spins >= kSpinLimit) {
            *flag = 1;
            break;
        }
    }
}

// Polls the word pairs a[e], c[e] (e = t + nt * u < n; t in [0, nt)) until
// both are nonzero; every round issues the loads of both arrays at once.
// Bounded like poll_nonzero.
template <int U>
LSA_DEV void poll_pair(const uint64_t *a, const int32_t *c, int n, int t, int nt, uint64_t (&oa)[U],
                       int32_t (&oc)[U], int32_t *flag) {
#pragma unroll
    for (int u = 0; u < U; ++u) { oa[u] = 0; oc[u] = 0; }
    for (int spins = 0;; ++spins) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = t + nt * u;
            if (e < n) {
                if (oa[u] == 0) oa[u] = __hip_atomic_load(a + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (oc[u] == 0) oc[u] = __hip_atomic_load(c + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        bool missing = false;
#pragma unroll
        for (int u = 0; u < U; ++u) missing |= (t + nt * u < n) && (oa[u] == 0 || oc[u] == 0);
        if (!missing) break;
        if (spins >= kSpinLimit) {
            *flag = 1;
            break;
        }
    }
}

// A polled key id, kept inside [0, n) so that no gather can leave the cache.
LSA_DEV int32_t clamp_id(int32_t id, int64_t n) { return (int32_t)min<int64_t>(max(id, 0), n - 1); }

template <typename W>
LSA_DEV void publish(W *dst, W v) { __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

// Waits until this wave's global stores have completed (reached the L2): a
// workgroup barrier alone does not wait for other waves' stores, so before one
// thread releases data that every wave wrote, each wave waits here first.
LSA_DEV void wave_stores_done() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xF70);     // vmcnt(0); expcnt, lgkmcnt not waited on
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <typename T, bool ATTEND, int RC, int DC, int PC>
__global__ __launch_bounds__(256) void k_decode(DecodeArgs A) {
    extern __shared__ __attribute__((aligned(16))) float dyn[];
    __shared__ double qbar_s[256];                            // fl32(mean), widened
    __shared__ __attribute__((aligned(16))) double u_s[64];   // fl32(u), widened
    __shared__ __attribute__((aligned(16))) float Cs[64 * kCS];
    __shared__ int32_t ccnt[64];
    __shared__ int32_t clo[65];
    __shared__ int32_t kept_s[kMaxP];
    __shared__ __attribute__((aligned(16))) uint64_t lk[kMaxP * 64];
    __shared__ int32_t lp[kMaxP * 64];
    __shared__ int32_t toff_s[65], a0_s[64], wex_s[64], wpart[4][64], skip_s[64];
    __shared__ __attribute__((aligned(16))) int32_t own_s[kOwnCap + 4 * kMT];
    __shared__ int32_t mem_s[kMemCap];
    __shared__ int keep_s, count_s, flag_s;
    __shared__ float m_run[16], l_run[16], alpha_s[16];

    constexpr bool kMfma = ATTEND && sizeof(T) == 2 && DC > 0 && DC % 32 == 0;
    const int r = RC > 0 ? RC : A.r;
    const int d = DC > 0 ? DC : A.d;
    const int P = PC > 0 ? PC : A.beam;      // workgroups per group (= beam)
    const size_t groups = (size_t)A.m * A.h_kv;
    // Workgroups are dispatched to the XCDs in turn (workgroup w to XCD
    // w mod nx), so every group is given workgroups of one XCD: its
    // exchanges then travel through one L2, and what one of its workgroups
    // loads the others find there.  Correctness does not depend on it (every
    // exchange is device-scope); workgroups past the last group leave at once.
    const int xw = (int)blockIdx.x % A.nx, qw = (int)blockIdx.x / A.nx;
    const int p = qw % P;
    const size_t gsl = (size_t)xw + (size_t)A.nx * (size_t)(qw / P);
    if (gsl >= groups) return;
    const int gi = (int)gsl;
    const int64_t i = gi / A.h_kv;
    const int g = gi % A.h_kv;
    const int G = A.h_q / A.h_kv;
    const int b = A.b, L = A.L;
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wv = tid / kWave;
    const T *Q = (const T *)A.Q;
    int32_t *ctrl = A.ctrl + (size_t)gi * 4;
    int32_t seeded = 0;
    const AttnSet as = attn_set(A.q_pos[i], A.n, A.n_sink, A.window);
    const int64_t nleaf = A.nodes[L];
    const int32_t *perm = (const int32_t *)(A.index + A.perm_off) + (size_t)g * A.n;
    const int32_t *leaf_off = (const int32_t *)(A.index + A.leaf_off_off) + (size_t)g * (nleaf + 1);

    // ---- prologue: level-1 rows and counts, W_g and the group's queries.
    // With r = 64, L >= 3 and b <= 4 P, wave w of workgroup p also owns
    // level-1 node vw = p + P w (every level-1 node has one owner) and loads
    // its children's rows (16 KB, coalesced: lane l holds float4 l + 64 x)
    // and counts (lane c: child c) into registers behind the other loads, so
    // level 2 needs no load after level 1.
    constexpr bool kPreShape = RC == 64 && DC == 128 && sizeof(T) == 2;
    const bool pre = kPreShape && L >= 3 && b <= 4 * P;
    const int vw = p + P * wv;
    f4_t rw[16];
    int32_t rcnt = 0;
    // W_g staged widened to double in the bf16, d = 128, r = 64 kernel (no
    // conversion in the u chain), as float otherwise
    float *Wl = dyn;                                      // [d][r] float
    double *Wd = reinterpret_cast<double *>(dyn);         // [d][r] double (kPreShape)
    float *Ql = kPreShape ? dyn + 2 * d * r : dyn + d * r;   // [G][d]
    {
        const float *C1 = (const float *)(A.index + A.centroid_off[1]) + (size_t)g * A.nodes[1] * r;
        const int32_t *cn1 = (const int32_t *)(A.index + A.count_off[1]) + (size_t)g * A.nodes[1];
        const int32_t cnt_r = cn1[min(tid, b - 1)];       // stored after the other loads are issued
        const float *Wg = A.W + (size_t)g * d * r;
        if constexpr (RC == 64 && DC == 128 && sizeof(T) == 2) {
            // one round of loads: 4 float4 of rows, 8 float4 of W, 1 uint4 of Q per thread
            const f4_t *c4 = reinterpret_cast<const f4_t *>(C1);
            const f4_t *w4 = reinterpret_cast<const f4_t *>(Wg);
            const uint4 *q4 = reinterpret_cast<const uint4 *>(Q + ((size_t)i * A.h_q + (size_t)g * G) * DC);
            f4_t cr[4], wr[8];
            uint4 qr;
#pragma unroll
            for (int u = 0; u < 4; ++u) cr[u] = c4[min(tid + 256 * u, b * 16 - 1)];   // clamped: loads stay in bounds
#pragma unroll
            for (int u = 0; u < 8; ++u) wr[u] = w4[tid + 256 * u];
            qr = q4[min(tid, G * 16 - 1)];
            __builtin_amdgcn_sched_barrier(0);     // all loads issued before the first store waits
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = tid + 256 * u;      // rows at and beyond b get copies that are never read
                *reinterpret_cast<f4_t *>(Cs + (e / 16) * kCS + (e % 16) * 4) = cr[u];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                double2 *w2 = reinterpret_cast<double2 *>(Wd + 4 * (tid + 256 * u));
                w2[0] = double2{(double)wr[u].x, (double)wr[u].y};
                w2[1] = double2{(double)wr[u].z, (double)wr[u].w};
            }
            if (tid < G * 16) {
                const uint32_t qw[4] = {qr.x, qr.y, qr.z, qr.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    Ql[tid * 8 + 2 * j] = __uint_as_float(qw[j] << 16);
                    Ql[tid * 8 + 2 * j + 1] = __uint_as_float(qw[j] & 0xffff0000u);
                }
            }
        } else {
            load_rows(Cs, C1, b, r);
            if (((d * r) & 3) == 0) g2s_rows<8>(Wl, d * r, Wg, d * r, d * r);
            else g2s_flat<16>(Wl, Wg, d * r);
            g2s_scalar<16, T, float>(Ql, G * d, Q + ((size_t)i * A.h_q + (size_t)g * G) * d, G * d, G * d);
        }
        if (tid < b) ccnt[tid] = cnt_r;
        if (tid == 0) { count_s = 0; flag_s = 0; }
        // the group's host-seeded timeout flag (read here, reported and
        // cleared at the end by workgroup 0 alone)
        if (p == 0 && tid == 0) seeded = __hip_atomic_load(ctrl + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // (issued after the stores above, so no wait there covers them: they
        // land while the latent query is computed)
        // Unconditional loads (a wave that owns no node reads the start of
        // the index instead), so that no branch pulls a use of them forward.
        if constexpr (kPreShape) {
            const bool own = pre && vw < b;
            const size_t n0 = own ? (size_t)g * A.nodes[2] + (size_t)vw * b : 0;
            const char *cb = own ? A.index + A.centroid_off[2] : A.index;
            const char *nb = own ? A.index + A.count_off[2] : A.index;
            const f4_t *r4 = reinterpret_cast<const f4_t *>((const float *)cb + n0 * 64);
#pragma unroll
            for (int x = 0; x < 16; ++x) rw[x] = r4[min(lane + 64 * x, b * 16 - 1)];   // (clamped to the b rows)
            rcnt = ((const int32_t *)nb)[n0 + (own ? min(lane, b - 1) : 0)];
        }
    }
    lds_barrier();                 // (the level-2 rows stay in flight)
    for (int t = tid; t < d; t += blockDim.x) {
        double s = 0.0;
        for (int h = 0; h < G; ++h) s = s + (double)Ql[h * d + t];
        qbar_s[t] = (double)(float)(s / (double)G);
    }
    lds_barrier();
    if constexpr (kPreShape) {
        // u_c = fl32 of the sequential double sum over t of qbar_t W[t][c]
        // (each product exact).  The four waves sum dims 32 w .. 32 w + 31
        // and the terms' magnitudes; wave 0 adds the partials.  The sequential
        // sum and this one both lie within 161 u A of the exact sum (u = 2^-53,
        // A the sum of magnitudes), so with B = 256 u A (plus an underflow
        // floor) covering that and the rounding of S +- B: when S - B and
        // S + B round to the same float, so does the sequential sum; any
        // other lane takes the sequential chain itself.
        double *part = reinterpret_cast<double *>(Ql);       // [8][64] (the Q staging, read above)
        double s = 0.0, a = 0.0;
#pragma unroll
        for (int t = 32 * wv; t < 32 * wv + 32; ++t) {
            const double q = qbar_s[t], w = Wd[t * 64 + lane];
            s = fma(q, w, s);
            a = fma(fabs(q), fabs(w), a);
        }
        part[wv * 64 + lane] = s;
        part[(4 + wv) * 64 + lane] = a;
        lds_barrier();
        if (wv == 0) {
            const double S = ((part[lane] + part[64 + lane]) + part[128 + lane]) + part[192 + lane];
            const double A2 = ((part[256 + lane] + part[320 + lane]) + part[384 + lane]) + part[448 + lane];
            const double B = A2 * 0x1p-45 + 0x1p-1060;
            const float lo = (float)(S - B), hi = (float)(S + B);
            float v = lo;
            if (__float_as_uint(lo) != __float_as_uint(hi)) {
                double q = 0.0;
                for (int t = 0; t < DC; ++t) q = fma(qbar_s[t], Wd[t * 64 + lane], q);
                v = (float)q;
            }
            u_s[lane] = (double)v;
        }
    } else {
        for (int c = tid; c < r; c += blockDim.x) {
            double s = 0.0;
            if constexpr (DC > 0) {
#pragma unroll 32
                for (int t = 0; t < DC; ++t) s = fma(qbar_s[t], (double)Wl[t * r + c], s);
            } else {
                for (int t = 0; t < d; ++t) s = fma(qbar_s[t], (double)Wl[t * r + c], s);
            }
            u_s[c] = (double)(float)s;
        }
    }
    lds_barrier();
    // ---- level 1 (every workgroup of the group computes the same ranking)
    if (pre) {
        // every wave scores the level-1 nodes itself; the owner of a kept node
        // (rank below P among the nonzero keys) scores, sorts and publishes its
        // children as list number `rank`, which is the list the workgroup of
        // that rank would publish after loading them; lists from keep to P-1
        // are published empty by the workgroup of that index
        uint64_t k1 = 0;
        if (lane < b && ccnt[lane] > 0) k1 = make_key(score_lds<RC>(u_s, Cs + lane * kCS, r), (uint32_t)lane);
        const int keep = min(P, __popcll(__ballot(k1 != 0)));
        if (vw < b) {
            const uint64_t kw = ((uint64_t)__builtin_amdgcn_readlane((int)(k1 >> 32), vw) << 32) |
                                (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)k1, vw);
            const int rank = __popcll(__ballot(k1 > kw));
            if (kw != 0 && rank < P) {
                // the rows to this wave's LDS slice (the W / Q staging area,
                // free once u is known), row c at stride kCS; lane c scores row c
                float *Rs = dyn + (size_t)wv * 64 * kCS;
#pragma unroll
                for (int x = 0; x < 16; ++x) {
                    const int e = lane + 64 * x;
                    *reinterpret_cast<f4_t *>(Rs + (e / 16) * kCS + (e % 16) * 4) = rw[x];
                }
                wave_sync();
                uint64_t key = 0;
                if (lane < b && rcnt > 0) key = make_key(score_lds<RC>(u_s, Rs + lane * kCS, r), (uint32_t)(vw * b + lane));
                // the top P by rank (the number of larger keys, over all 64
                // in this wave's slice of own_s; empty slots get distinct
                // keys below every real one and stay empty)
                uint64_t *wk = reinterpret_cast<uint64_t *>(own_s + wv * 192), *wt = wk + 64;
                wk[lane] = key ? key : (uint64_t)(63 - lane);
                wave_sync();
                const uint64_t x = wk[lane];
                int above = 0;
#pragma unroll
                for (int j = 0; j < 64; j += 2) {
                    const uint4 kk = *reinterpret_cast<const uint4 *>(wk + j);
                    above += ((((uint64_t)kk.y << 32) | kk.x) > x) ? 1 : 0;
                    above += ((((uint64_t)kk.w << 32) | kk.z) > x) ? 1 : 0;
                }
                if (above < P) wt[above] = x;
                wave_sync();
                if (lane < P) {
                    const uint64_t t = wt[lane];
                    publish(A.lists + ((size_t)gi * P + rank) * P + lane, t >= (1ull << 32) ? t : kEmpty);
                }
            }
        }
        if (wv == 0 && p >= keep && lane < P) publish(A.lists + ((size_t)gi * P + p) * P + lane, kEmpty);
    } else if (wv == 0) {
        uint64_t key = 0;
        int pay = 0;
        if (lane < b && ccnt[lane] > 0) key = make_key(score_lds<RC>(u_s, Cs + lane * kCS, r), (uint32_t)lane);
        const int nz = __popcll(__ballot(key != 0));
        wave_sort_desc(key, pay);
        const int keep = min(P, nz);
        if (lane < keep) kept_s[lane] = (int32_t)key_id(key);
        if (lane == 0) keep_s = keep;
    }
    __syncthreads();

    int64_t v = -1;
    for (int l = 2; l <= L; ++l) {
        const bool leaf = (l == L);
        if (!(pre && l == 2)) {
        v = (p < keep_s) ? kept_s[p] : -1;
        if (v >= 0) {
            const float *Cl = (const float *)(A.index + A.centroid_off[l]) + ((size_t)g * A.nodes[l] + (size_t)v * b) * r;
            const int32_t *cn = (const int32_t *)(A.index + A.count_off[l]) + (size_t)g * A.nodes[l] + (size_t)v * b;
            // counts, leaf offsets and rows in one round of loads (clamped
            // indices; the LDS stores come after every load is issued)
            const int32_t cnt_r = cn[min(tid, b - 1)];
            const int32_t lo_r = leaf ? leaf_off[(size_t)v * b + min(tid, b)] : 0;
            if constexpr (RC == 64) load_rows64(Cs, Cl, b);
            else load_rows(Cs, Cl, b, r);
            if (tid < b) ccnt[tid] = cnt_r;
            if (leaf && tid <= b) clo[tid] = lo_r;
        }
        __syncthreads();
        if (leaf && v >= 0) {
            // the node's members (its leaves are contiguous): causal counts,
            // the keys this workgroup writes and attends over
            const int mn = clo[b] - clo[0];
            if (mn <= kMemCap) g2s_flat<8>(mem_s, perm + clo[0], mn);
            __syncthreads();
        }
        // wave 0 scores the node's children; then all four waves rank them
        // (the rank of a key is the number of larger keys; empty slots get
        // distinct keys below every real one and stay empty), in LDS that is
        // free until the fill (own_s, wpart)
        uint64_t *rk_key = reinterpret_cast<uint64_t *>(own_s), *rk_sk = rk_key + 64;
        int32_t *rk_e = own_s + 256, *rk_se = own_s + 320;
        if (wv == 0) {
            uint64_t key = 0;
            int e = 0;
            if (v >= 0 && lane < b && ccnt[lane] > 0) {
                key = make_key(score_lds<RC>(u_s, Cs + lane * kCS, r), (uint32_t)(v * b + lane));
                if (leaf) {
                    // members in the retrieval range: the first one and their number
                    const int a0 = clo[lane], a1 = clo[lane + 1];
                    int f;
                    if (clo[b] - clo[0] <= kMemCap) in_range(as, mem_s + (a0 - clo[0]), a1 - a0, f, e);
                    else in_range(as, perm + a0, a1 - a0, f, e);
                    skip_s[lane] = f;
                    if (e == 0) key = 0;
                }
            }
            rk_key[lane] = key ? key : (uint64_t)(63 - lane);
            rk_e[lane] = e;
        }
        lds_barrier();
        {
            const uint64_t x = rk_key[lane];
            int c = 0;
#pragma unroll
            for (int j = 0; j < 16; ++j) c += (rk_key[16 * wv + j] > x) ? 1 : 0;
            wpart[wv][lane] = c;
        }
        lds_barrier();
        if (wv == 0) {
            const int rank = wpart[0][lane] + wpart[1][lane] + wpart[2][lane] + wpart[3][lane];
            rk_sk[rank] = rk_key[lane];
            rk_se[rank] = rk_e[lane];
            wave_sync();
            uint64_t key = rk_sk[lane];
            const int e = rk_se[lane];
            if (key < (1ull << 32)) key = 0;      // (an empty slot)
            if (!leaf) {
                if (lane < P) publish(A.lists + (((size_t)(l - 2) * groups + gi) * P + p) * P + lane, key ? key : kEmpty);
            } else {
                const int incl = wave_incl_scan_add(e);
                const size_t o = ((size_t)gi * P + p) * 64 + lane;
                publish(A.leaf_keys + o, key ? key : kEmpty);
                publish(A.leaf_pre + o, incl + 1);
            }
        }
        }   // level l scored by this workgroup
        if (!leaf) {
            // candidates: the first P entries of every list (the global top P
            // lie among them).  Two merge rounds: the top P of each quartet of
            // lists, placed at their ranks within the quartet, then the top P
            // of those merged lists.  A rank is the number of entries above
            // the key in every list of its round (its own list gives its
            // position), found by side-by-side binary searches.
            constexpr int LQ = PC > 0 ? PC : kMaxP;          // list length bound
            const uint64_t *src = A.lists + ((size_t)(l - 2) * groups + gi) * P * P;
            const int nc = P * P;
            const int nm = (P + 3) / 4;                       // merged lists
            uint64_t *m1 = lk + kMaxP * kMaxP;                // [nm][P]
            {
                uint64_t w[kMaxP * kMaxP / 256];
                poll_nonzero(src, nc, w, &flag_s);
#pragma unroll
                for (int u = 0; u < kMaxP * kMaxP / 256; ++u) {
                    const int e = tid + 256 * u;
                    if (e < nc) lk[e] = (w[u] == kEmpty) ? 0ull : w[u];
                }
            }
            for (int e = tid; e < nm * P; e += blockDim.x) m1[e] = 0ull;
            __syncthreads();
            int nonzero = 0;
            for (int e = tid; e < nc; e += blockDim.x) {
                const uint64_t x = lk[e];
                if (x != 0) {
                    const int quad = (e / P) / 4;
                    int c[4];
                    count_gt_lists<4, LQ>(lk, P, 4 * quad, 1, P, P, x, c);
                    const int rank = c[0] + c[1] + c[2] + c[3];
                    if (rank < P) m1[quad * P + rank] = x;
                    ++nonzero;
                }
            }
            const int nz = __syncthreads_count(nonzero);
            for (int e = tid; e < nm * P; e += blockDim.x) {
                const uint64_t x = m1[e];
                if (x != 0) {
                    int c[LQ / 4];
                    count_gt_lists<LQ / 4, LQ>(m1, P, 0, 1, nm, P, x, c);
                    int rank = 0;
#pragma unroll
                    for (int q = 0; q < LQ / 4; ++q) rank += c[q];
                    // (clamped: a node id of this level whatever the buffer held)
                    if (rank < P) kept_s[rank] = (int32_t)min<int64_t>(key_id(x), A.nodes[l] - 1);
                }
            }
            if (tid == 0) keep_s = min(P, nz);
            __syncthreads();
        }
    }

    // ---- fill: every workgroup places its own leaves' keys
    {
        {
            // keys and prefix counts of all P lists, polled as they are
            // published (both arrays in every round)
            constexpr int U = kMaxP * 64 / 256;
            uint64_t tk[U];
            int32_t tp[U];
            poll_pair(A.leaf_keys + (size_t)gi * P * 64, A.leaf_pre + (size_t)gi * P * 64, P * 64, tid, 256, tk, tp,
                      &flag_s);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e = tid + 256 * u;
                // prefixes clamped to [0, k]: exact for published lists (only
                // offsets below k place keys) and bounded sums whatever the
                // buffer held, so every offset below stays in [0, k)
                if (e < P * 64) { lk[e] = (tk[u] == kEmpty) ? 0ull : tk[u]; lp[e] = min(max(tp[u] - 1, 0), A.k); }
            }
        }
        lds_barrier();
        if (wv == 0) {
            int tot = (lane < P) ? lp[lane * 64 + 63] : 0;
            tot = wave_sum_i(tot);
            if (lane == 0) count_s = max(0, min(A.k, tot));
        }
        // eligible keys retrieved before each own leaf: wave w sums, over the
        // lists q = w, w + 4, ..., the eligible counts of the leaves above it
        // (a binary search in list q, then its inclusive prefix); the own list
        // gives the keys before it
        {
            const uint64_t x = lk[p * 64 + lane];
            int part = 0;
            if (x != 0) {
                constexpr int NQ = (PC > 0 ? PC : kMaxP) / 4;
                int c[NQ];
                count_gt_lists<NQ, 64>(lk, 64, wv, 4, P, 64, x, c);
#pragma unroll
                for (int i = 0; i < NQ; ++i) {
                    const int q = wv + 4 * i;
                    part += (q < P && c[i] > 0) ? lp[q * 64 + c[i] - 1] : 0;
                }
            }
            wpart[wv][lane] = part;
        }
        lds_barrier();
        const int count = count_s;
        int32_t *out = A.sel + (size_t)gi * A.row;
        if (wv == 0) {
            // lane j: the j-th own leaf in score order; its first `take` members
            // go to sel from its retrieval offset wex and to own_s (this
            // workgroup's keys, in lane order) from its offset toff
            const uint64_t x = (v >= 0) ? lk[p * 64 + lane] : 0ull;
            int take = 0, wex = 0, e = 0, a0 = 0;
            if (x != 0) {
                e = lp[p * 64 + lane] - (lane > 0 ? lp[p * 64 + lane - 1] : 0);
                wex = wpart[0][lane] + wpart[1][lane] + wpart[2][lane] + wpart[3][lane];
                take = max(0, min(e, count - wex));
                const int c = min(max((int)(key_id(x) - (uint32_t)(v * b)), 0), b - 1);
                a0 = clo[c] + skip_s[c];
            }
            const int incl = wave_incl_scan_add(take);
            toff_s[lane] = incl - take;
            a0_s[lane] = a0;
            wex_s[lane] = wex;
            if (lane == 63) toff_s[64] = incl;
            if (x != 0 && count == A.k && wex < A.k && wex + e >= A.k && A.sel_cutoff)
                A.sel_cutoff[gi] = key_score(x);
        }
        lds_barrier();
        // own key f (all threads): its lane j is the last with toff_s[j] <= f
        const int own = toff_s[64];
        const bool staged = v >= 0 && (clo[b] - clo[0]) <= kMemCap;
        auto own_lane = [&](int f) -> int {
            int j = 0;
#pragma unroll
            for (int step = 32; step >= 1; step >>= 1) j += (j + step < 64 && toff_s[j + step] <= f) ? step : 0;
            return j;
        };
        for (int f = tid; f < own; f += blockDim.x) {
            const int j = own_lane(f), t = f - toff_s[j];
            const int32_t id = staged ? mem_s[a0_s[j] - clo[0] + t] : perm[a0_s[j] + t];
            out[wex_s[j] + t] = id;
            if (ATTEND) publish(A.keys + (size_t)gi * A.k + wex_s[j] + t, id + 1);
        }
        // the sinks and the window follow the retrieved keys
        for (int t = p * blockDim.x + tid; t < as.nloc; t += P * blockDim.x) out[count + t] = local_key(as, t);
        for (int t = count + as.nloc + p * blockDim.x + tid; t < A.row; t += P * blockDim.x) out[t] = -1;
        if (p == 0 && tid == 0) {
            A.sel_count[gi] = count + as.nloc;
            if (count < A.k && A.sel_cutoff) A.sel_cutoff[gi] = -INFINITY;
        }
        // LDS only: no one in this workgroup reads the stores above (the
        // published ids are polled), so they need not complete here
        lds_barrier();
    }

    if constexpr (ATTEND) {
        // ---- attention.  The row's attention set is the retrieved keys
        // (positions [0, count)) followed by the sinks and the window;
        // workgroup p attends over positions [tot * p / P, tot * (p + 1) / P),
        // whichever workgroups placed them, so the gathers are spread evenly
        // whatever the nodes supplied.  Retrieved ids are polled from the
        // published keys, local ones computed, into own_s in chunks of up to
        // kOwnCap, padded with key 0 to whole 4 x 32-key steps.
        const int cnt_all = count_s;
        const int tot = cnt_all + as.nloc;
        const int lo = (int)(((int64_t)tot * p) / P), hi = (int)(((int64_t)tot * (p + 1)) / P);
        // the combined unnormalised outputs [G][d] in LDS (oc), the maxima
        // and sums in m_run, l_run, then sent to the readers below
        float *oc = kMfma ? dyn + 4 * kWave * (DC / 4) + 128 : dyn;
        if constexpr (kMfma) {
            const uint16_t *Kg = (const uint16_t *)A.K + (size_t)g * A.n * DC;
            const uint16_t *Vg = (const uint16_t *)A.V + (size_t)g * A.n * DC;
            const uint16_t *Qb = (const uint16_t *)A.Q + ((size_t)i * A.h_q + (size_t)g * G) * DC;
            uint16_t *vt = reinterpret_cast<uint16_t *>(dyn) + (size_t)wv * DC * kVTS;
            bf16x8_t qf[DC / 32];
            wave_load_q<DC>(qf, Qb, G);
            WaveAttn<DC> st;
            wave_attn_init<DC>(st);
            for (int c0 = lo; c0 < hi; c0 += kOwnCap) {
                const int own = min(kOwnCap, hi - c0);
                const int nr = max(0, min(own, cnt_all - c0));     // retrieved entries of the chunk
                const int nsteps = (own + 4 * kMT - 1) / (4 * kMT);
                for (int f0 = 0; f0 < nr; f0 += 8 * 256) {
                    int32_t w[8];
                    poll_nonzero(A.keys + (size_t)gi * A.k + c0 + f0, nr - f0, w, &flag_s);
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        if (f0 + tid + 256 * u < nr) own_s[f0 + tid + 256 * u] = clamp_id(w[u] - 1, A.n);
                }
                for (int f = nr + tid; f < own; f += blockDim.x) own_s[f] = local_key(as, c0 + f - cnt_all);
                for (int f = own + tid; f < nsteps * 4 * kMT; f += blockDim.x) own_s[f] = 0;
                __syncthreads();
                for (int t = 0; t < nsteps; ++t) {
                    const int fb = (4 * t + wv) * kMT;
                    const int nk = max(0, min(kMT, own - fb));
                    bf16x8_t pf;
                    float alpha;
                    wave_attn_part1<DC>(Kg, Vg, own_s + fb, nk, qf, A.scale_log2, vt, st, pf, alpha);
                    wave_sync();
                    wave_attn_part2<DC>(vt, pf, alpha, st, c0 == lo && t == 0);
                }
                __syncthreads();
            }
            wave_attn_stash<DC>(st, dyn);
            __syncthreads();
            // the four waves' states combined into [G][DC] in LDS, then sent
            // one output a lane, so that each store instruction writes whole
            // lines of a record
            for (int e4 = tid; e4 < G * DC / 4; e4 += blockDim.x) {
                const int h = e4 / (DC / 4), dd = 4 * (e4 % (DC / 4));
                float M, Ls;
                *reinterpret_cast<floatx4_t *>(oc + h * DC + dd) = wave_attn_combine4<DC>(dyn, h, dd, M, Ls);
                if (dd == 0) { m_run[h] = M; l_run[h] = Ls; }
            }
        } else {
            const int dp = d + 1;
            float *qs = dyn;                       // [G][d]
            float *Kt = qs + G * d;                // [TK][d + 1]
            float *Vt = Kt + kTKD * dp;            // [TK][d]
            float *S = Vt + kTKD * d;              // [G][TK]
            int32_t *ids_s = own_s;                // kTKD ids
            for (int e = tid; e < G * d; e += blockDim.x)
                qs[e] = to_float(Q[((size_t)i * A.h_q + (size_t)g * G) * d + e]) * A.scale_log2;
            if (tid < 16) { m_run[tid] = -INFINITY; l_run[tid] = 0.0f; }
            __syncthreads();
            const int ne = (G * d + blockDim.x - 1) / blockDim.x;
            float acc[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[q] = 0.0f;
            const T *Kg = (const T *)A.K + (size_t)g * A.n * d;
            const T *Vg = (const T *)A.V + (size_t)g * A.n * d;
            for (int f0 = lo; f0 < hi; f0 += kTKD) {
                const int nk = min(kTKD, hi - f0);
                const int nr = max(0, min(nk, cnt_all - f0));      // retrieved entries of the tile
                {
                    int32_t w[1];
                    poll_nonzero(A.keys + (size_t)gi * A.k + f0, nr, w, &flag_s);
                    if (tid < nr) ids_s[tid] = clamp_id(w[0] - 1, A.n);
                    else if (tid < nk) ids_s[tid] = local_key(as, f0 + tid - cnt_all);
                }
                __syncthreads();
                gather_tile<T>(Kg, Vg, ids_s, nk, d, Kt, dp, Vt);
                __syncthreads();
                for (int e = tid; e < G * kTKD; e += blockDim.x) {
                    const int h = e / kTKD, kk = e % kTKD;
                    float s = -INFINITY;
                    if (kk < nk) {
                        const float *qh = qs + h * d;
                        const float *kr = Kt + kk * dp;
                        s = 0.0f;
#pragma unroll 8
                        for (int t = 0; t < d; ++t) s = fmaf(qh[t], kr[t], s);
                    }
                    S[h * kTKD + kk] = s;
                }
                __syncthreads();
                for (int h = wv; h < G; h += blockDim.x / kWave) {
                    const float x = S[h * kTKD + lane];
                    const float mt = wave_max_f(x);
                    const float mnew = fmaxf(m_run[h], mt);
                    const float pr = (lane < nk) ? exp2f(x - mnew) : 0.0f;
                    S[h * kTKD + lane] = pr;
                    const float ls = wave_sum_f(pr);
                    if (lane == 0) {
                        const float al = (m_run[h] == -INFINITY) ? 0.0f : exp2f(m_run[h] - mnew);
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
#pragma unroll 8
                    for (int kk = 0; kk < nk; ++kk) a = fmaf(ph[kk], Vt[kk * d + t], a);
                    acc[q] = a;
                }
                __syncthreads();
            }
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                if (q >= ne) break;
                const int e = tid + q * blockDim.x;
                if (e >= G * d) break;
                oc[e] = acc[q];
            }
        }
        lds_barrier();
        // records, one per reader r (wave r % 4 sends it): the outputs of
        // slice r, then the maximum and the sum of each head it touches
        const int NO = G * d, SM = slice_max(NO, P), RS = rec_stride(NO, P, d, true);
        uint32_t *mine = A.recs + ((size_t)gi * P + p) * P * RS;
        for (int r = wv; r < P; r += 4) {
            const int lo_r = slice_lo(NO, P, r), hi_r = slice_lo(NO, P, r + 1), hl = lo_r / d;
            const int nh = hi_r > lo_r ? (hi_r - 1) / d - hl + 1 : 0;
            uint32_t *rec = mine + (size_t)r * RS;
            for (int e = lo_r + lane; e < hi_r; e += kWave) publish(rec + (e - lo_r), enc_word(oc[e]));
            if (lane < 2 * nh) publish(rec + SM + lane, enc_word((lane & 1) ? l_run[hl + lane / 2] : m_run[hl + lane / 2]));
        }
    }

    // ---- merge.  Workgroup p polls the P records of its slice (with
    // attention) or the P done tokens (without); once it has them all, every
    // workgroup of the group is past its last exchange read.
    const int NO = G * d, RS = rec_stride(NO, P, d, ATTEND);
    uint32_t *recs_g = A.recs + (size_t)gi * P * P * RS;     // [writer][reader][RS]
    if constexpr (ATTEND) {
        // the words of this slice, record q's word j at rv[q][j] (j < sp: output
        // lo + j; then the maximum and the sum of each head of the slice),
        // polled by all threads with every load of a round in flight, and
        // cleared once read (each has this one reader)
        const int SM = slice_max(NO, P);
        const int lo = slice_lo(NO, P, p), hi = slice_lo(NO, P, p + 1), hlo = lo / d;
        const int sp = hi - lo, nh = hi > lo ? (hi - 1) / d - hlo + 1 : 0, len = sp + 2 * nh;
        float *rv = (kMfma ? dyn + 4 * kWave * (DC / 4) + 128 : dyn) + G * d;
        const int nw = P * len;
        constexpr int U = 8;
        for (int f0 = 0; f0 < nw; f0 += U * (int)blockDim.x) {
            uint32_t w[U], *src[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int f = f0 + tid + u * (int)blockDim.x, fc = min(f, nw - 1);
                const int q = fc / len, j = fc - q * len;
                src[u] = recs_g + ((size_t)q * P + p) * RS + (j < sp ? j : SM + (j - sp));
                w[u] = f < nw ? 0u : 1u;          // (words past the slice: nothing to wait for)
            }
            for (int spins = 0;; ++spins) {
                bool missing = false;
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (w[u] == 0) w[u] = __hip_atomic_load(src[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
                for (int u = 0; u < U; ++u) missing |= w[u] == 0;
                if (!missing) break;
                if (spins >= kSpinLimit) { flag_s = 1; break; }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int f = f0 + tid + u * (int)blockDim.x;
                if (f < nw) {
                    rv[f] = dec_word(w[u]);
                    publish(src[u], 0u);
                }
            }
        }
        lds_barrier();
        for (int e = lo + tid; e < hi; e += blockDim.x) {
            const int h = e / d, jm = sp + 2 * (h - hlo);
            float M = -INFINITY;
            for (int q = 0; q < P; ++q) M = fmaxf(M, rv[q * len + jm]);
            float l = 0.0f, acc = 0.0f;
            for (int q = 0; q < P; ++q) {
                const float mq = rv[q * len + jm];
                if (mq > -INFINITY) {
                    const float w = exp2f(mq - M);
                    l += rv[q * len + jm + 1] * w;
                    acc += rv[q * len + (e - lo)] * w;
                }
            }
            const size_t oh = (size_t)i * A.h_q + (size_t)g * G + h;
            ((T *)A.out)[oh * d + (e % d)] = from_float<T>(l > 0.0f ? acc / l : 0.0f);
            if ((e % d) == 0 && A.lse) A.lse[oh] = (l > 0.0f) ? (M + log2f(l)) * 0.69314718055994531f : -INFINITY;
        }
    } else {
        // done tokens: this workgroup's to every reader, then the P addressed to it
        if (tid < P) {
            publish(recs_g + ((size_t)p * P + tid) * RS, 1u);
            const uint32_t *tok = recs_g + ((size_t)tid * P + p) * RS;     // writer tid's token to this workgroup
            for (int spins = 0;; ++spins) {
                if (__hip_atomic_load(tok, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) break;
                if (spins >= kSpinLimit) { flag_s = 1; break; }
            }
        }
    }
    // every workgroup of the group is past its exchange reads: clear the
    // exchange words, each workgroup one slice of every buffer
    {
        auto clear32 = [&](int32_t *base, int n) {
            for (int e = slice_lo(n, P, p) + tid; e < slice_lo(n, P, p + 1); e += blockDim.x) publish(base + e, 0);
        };
        auto clear64 = [&](uint64_t *base, int n) {
            for (int e = slice_lo(n, P, p) + tid; e < slice_lo(n, P, p + 1); e += blockDim.x) publish(base + e, (uint64_t)0);
        };
        for (int l = 0; l < L - 2; ++l) clear64(A.lists + ((size_t)l * groups + gi) * P * P, P * P);
        clear64(A.leaf_keys + (size_t)gi * P * 64, P * 64);
        clear32(A.leaf_pre + (size_t)gi * P * 64, P * 64);
        if (ATTEND) clear32(A.keys + (size_t)gi * A.k, count_s);
    }
    if (!ATTEND && tid < P) publish(recs_g + ((size_t)tid * P + p) * RS, 0u);
    lds_barrier();
    if (tid == 0) {
        // a bounded wait of this workgroup gave up (results may be wrong), or
        // workgroup 0 found the group's seeded flag: report it in the status
        // word, which stays set until the host reads it
        if (flag_s != 0 || seeded != 0)
            __hip_atomic_fetch_or(A.status, kStatusWaitTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (seeded != 0) publish(ctrl + 2, 0);
    }
}

// ---------------------------------------------------------------- host side
static inline size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

struct DecodeWs {
    int32_t *status, *ctrl; uint64_t *lists, *leaf_keys; int32_t *leaf_pre, *keys; uint32_t *recs; size_t bytes;
};

// Workspace layout: the status word (kWsHeader bytes), then the exchange
// buffers and the partial-state records, all polled.
static DecodeWs carve_decode_ws(char *base, int64_t groups, int P, int L, int G, int d, int k) {
    size_t cur = 0;
    DecodeWs w{};
    auto take = [&](size_t n) { char *p = base ? base + cur : nullptr; cur = a256(cur + n); return p; };
    w.status = (int32_t *)take(kWsHeader);
    w.ctrl = (int32_t *)take(sizeof(int32_t) * 4 * (size_t)groups);
    w.lists = (uint64_t *)take(sizeof(uint64_t) * (size_t)(L > 2 ? L - 2 : 1) * groups * P * P);
    w.leaf_keys = (uint64_t *)take(sizeof(uint64_t) * (size_t)groups * P * 64);
    w.leaf_pre = (int32_t *)take(sizeof(int32_t) * (size_t)groups * P * 64);
    w.keys = (int32_t *)take(sizeof(int32_t) * (size_t)groups * k);
    w.recs = (uint32_t *)take(sizeof(uint32_t) * (size_t)groups * P * P * (size_t)rec_stride(G * d, P, d, true));
    w.bytes = cur;
    return w;
}

int device_cus() {
    // per device, filled on first use (concurrent first uses store the same value)
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int c = cus[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cus[dev].store(c, std::memory_order_relaxed);
    }
    return c;
}

// XCDs of the current device (1 when the runtime cannot say): the decode grid
// gives each group workgroups of one XCD.
int device_xccs() {
    static std::atomic<int> xcc[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
    int c = xcc[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || c < 1) c = 1;
        xcc[dev].store(c, std::memory_order_relaxed);
    }
    return c;
}

// Workgroups of the decode grid: nx XCDs x (groups per XCD, rounded up) x beam.
static int64_t decode_grid(int64_t groups, int beam, int nx) { return (int64_t)nx * ((groups + nx - 1) / nx) * beam; }

static bool fast_shape(int dtype, int d, int r) { return dtype == 1 && d == 128 && r == 64; }

static size_t decode_dyn_bytes(int dtype, int G, int d, int r, int P) {
    // W (double in the fast shape), Q staging
    const size_t stage = (fast_shape(dtype, d, r) ? sizeof(double) : sizeof(float)) * (size_t)d * r +
                         sizeof(float) * (size_t)G * d;
    // attention, then the combined outputs and the polled records of the merge
    const size_t merge_words = (size_t)G * d + (size_t)P * rec_stride(G * d, P, d, true);
    size_t att;
    if (fast_shape(dtype, d, r))
        att = std::max(sizeof(uint16_t) * 4 * (size_t)d * kVTS, sizeof(float) * (4 * (size_t)d * 16 + 128 + merge_words));
    else
        att = sizeof(float) * std::max((size_t)G * d + (size_t)kTKD * (d + 1) + (size_t)kTKD * d + (size_t)G * kTKD,
                                       merge_words);
    // fast shape: four waves' level-2 node blocks (64 rows at stride kCS)
    const size_t pre = fast_shape(dtype, d, r) ? sizeof(float) * 4 * 64 * (size_t)kCS : 0;
    return std::max(std::max(stage, pre), att);
}

constexpr size_t kStaticLds = 64 * 1024;      // upper bound of k_decode's static LDS
constexpr size_t kLdsPerCu = 160 * 1024;

bool decode_path_ok(int64_t m, int h_q, int h_kv, int d, int r, int b, int L, int beam, int k) {
    const int G = h_q / h_kv;
    if (L < 2 || b > 64 || r > 64 || beam > kMaxP || beam < 1 || G > 16 || d > 256 || d % 8 != 0) return false;
    if (decode_dyn_bytes(0, G, d, r, beam) + kStaticLds > kLdsPerCu) return false;
    (void)k;
    // every workgroup of a group must be resident at once: the whole grid,
    // one workgroup per compute unit at this kernel's LDS size
    const int cus = device_cus();
    return cus > 0 && decode_grid(m * h_kv, beam, device_xccs()) <= cus;
}

int64_t decode_workspace_bytes(int64_t m, int h_q, int h_kv, int d, int L, int beam, int k) {
    return (int64_t)carve_decode_ws(nullptr, m * h_kv, beam, L, h_q / h_kv, d, k).bytes;
}

// An upper bound on the bytes from the start of a workspace that this path
// polls (all of its workspace), over every batch it accepts:
// groups * beam <= compute units, beam <= kMaxP, L <= LSA_MAX_LEVELS,
// k <= 8192, G * d <= 16 * 256.  A group's records take
// beam * beam * rec_stride <= beam * (G * d + 2 G + 13 beam) words.
int64_t decode_polled_bytes_bound() {
    const int64_t c = std::max(device_cus(), 1);
    const int64_t ctrl = sizeof(int32_t) * 4 * c, lists = sizeof(uint64_t) * (LSA_MAX_LEVELS - 2) * c * kMaxP;
    const int64_t leaf = (sizeof(uint64_t) + sizeof(int32_t)) * c * 64, keys = sizeof(int32_t) * c * 8192;
    const int64_t recs = sizeof(uint32_t) * c * (16 * 256 + 2 * 16 + 13 * kMaxP);
    return kWsHeader + ctrl + lists + leaf + keys + recs + 6 * 256;
}

// The other paths place their buffers after this many bytes of a workspace,
// so that they never write a word the decode kernel polls.
int64_t ws_reserved_bytes() { return (int64_t)a256((size_t)decode_polled_bytes_bound()); }

template <typename T, bool ATT, int RC, int DC, int PC>
static hipError_t launch_decode(const DecodeArgs &A, dim3 grid, size_t shm, hipStream_t st) {
    // the attribute is set once per device (setting it twice is harmless)
    static std::atomic<int> attr_set[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    if (!attr_set[dev].load(std::memory_order_acquire)) {
        hipError_t e = hipFuncSetAttribute((const void *)k_decode<T, ATT, RC, DC, PC>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)(kLdsPerCu - kStaticLds));
        if (e != hipSuccess) return e;
        attr_set[dev].store(1, std::memory_order_release);
    }
    hipLaunchKernelGGL((k_decode<T, ATT, RC, DC, PC>), grid, dim3(256), shm, st, A);
    return hipGetLastError();
}

// ---------------------------------------------------------------- fixed scratch
// The workspace of lsa_select_attend_noalloc, for callers that cannot
// allocate: one copy per device, held until the process ends.  In host code
// `scratch` names a host-side stand-in, not device memory, so host code only
// ever uses the address hipGetSymbolAddress returns for the current device.
constexpr int64_t kScratchBytes = (int64_t)4 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

__global__ __launch_bounds__(256) void k_scratch_clear(int4 *p, int64_t count) {
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < count; e += (int64_t)gridDim.x * blockDim.x)
        p[e] = int4{0, 0, 0, 0};
}

int64_t scratch_bytes() { return kScratchBytes; }

// This device's copy of the scratch.  Set up once per device, with that
// device current: its address is taken, and it is cleared on `st` (the decode
// kernel needs the words it polls zero on entry, and leaves them zero).
hipError_t scratch_ptr(void **out, hipStream_t st) {
    static std::mutex mu;
    static void *dev_ptr[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!dev_ptr[dev]) {
        void *ptr = nullptr;
        hipError_t e = hipGetSymbolAddress((void **)&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        hipLaunchKernelGGL(k_scratch_clear, dim3(256), dim3(256), 0, st, (int4 *)ptr, kScratchBytes / 16);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        dev_ptr[dev] = ptr;
    }
    *out = dev_ptr[dev];
    return hipSuccess;
}

hipError_t decode(const void *Q, const void *K, const void *V, int dtype, int64_t m, int h_q, int h_kv, int d,
                  const int32_t *q_pos, const char *index, int64_t n, int r, int b, int L, const int64_t *nodes,
                  const int64_t *centroid_off, const int64_t *count_off, int64_t leaf_off_off, int64_t perm_off,
                  const float *W, int beam, int k, int n_sink, int window, int32_t *sel, int32_t *sel_count,
                  float *sel_cutoff, float scale, void *out, float *lse, void *ws, bool attend, hipStream_t st) {
    DecodeArgs A{};
    A.Q = Q; A.K = K; A.V = V; A.m = m; A.h_q = h_q; A.h_kv = h_kv; A.d = d; A.q_pos = q_pos;
    A.index = index; A.n = n; A.r = r; A.b = b; A.L = L;
    for (int l = 0; l <= L; ++l) { A.nodes[l] = nodes[l]; A.centroid_off[l] = centroid_off[l]; A.count_off[l] = count_off[l]; }
    A.leaf_off_off = leaf_off_off; A.perm_off = perm_off; A.W = W; A.beam = beam; A.k = k;
    A.n_sink = n_sink; A.window = window; A.row = k + n_sink + window;
    A.sel = sel; A.sel_count = sel_count; A.sel_cutoff = sel_cutoff;
    A.scale_log2 = scale * 1.4426950408889634f; A.out = out; A.lse = lse;
    A.nx = device_xccs();
    const int G = h_q / h_kv;
    DecodeWs w = carve_decode_ws((char *)ws, m * h_kv, beam, L, G, d, k);
    A.status = w.status; A.ctrl = w.ctrl; A.lists = w.lists; A.leaf_keys = w.leaf_keys; A.leaf_pre = w.leaf_pre; A.keys = w.keys;
    A.recs = w.recs;
    const size_t shm = decode_dyn_bytes(dtype, G, d, r, beam);
    const dim3 grid((unsigned)decode_grid(m * h_kv, beam, A.nx));
    if (fast_shape(dtype, d, r) && beam == 16) {
        return attend ? launch_decode<bf16_t, true, 64, 128, 16>(A, grid, shm, st)
                      : launch_decode<bf16_t, false, 64, 128, 16>(A, grid, shm, st);
    }
    if (fast_shape(dtype, d, r)) {
        return attend ? launch_decode<bf16_t, true, 64, 128, 0>(A, grid, shm, st)
                      : launch_decode<bf16_t, false, 64, 128, 0>(A, grid, shm, st);
    }
    if (dtype == 0)
        return attend ? launch_decode<float, true, 0, 0, 0>(A, grid, shm, st)
                      : launch_decode<float, false, 0, 0, 0>(A, grid, shm, st);
    return attend ? launch_decode<bf16_t, true, 0, 0, 0>(A, grid, shm, st)
                  : launch_decode<bf16_t, false, 0, 0, 0>(A, grid, shm, st);
}

}  // namespace lsa
