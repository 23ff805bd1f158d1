// Sparse attention over the selected keys (gfx950).
//
// Each query attends to k selected keys instead of all n ("Latent Sparse
// Attention Breaks Through the Million-Token Context Bottleneck",
// kongchang.com, section "The Accuracy-Efficiency Dilemma of Sparse
// Attention"); attention is computed over the retrieved keys ("Latent sparse
// attention", bdtechtalks.com, section "How latent sparse attention works").
//
// The G query heads that share a KV head share one selected set, so one
// workgroup serves all G heads of a (row, KV head) pair and reads each
// gathered K/V row once.  The set is cut into `nsplit` slices (split-K) to
// fill the chip when there are few rows; slices keep a running max and sum
// (online softmax, base 2) and a merge kernel combines them by log-sum-exp.
// In the matrix-core kernel each wave keeps the next 32-key step's gathers in
// flight while it computes the current one.
#include "common.h"
#include "internal.h"
#include "mfma_attn.h"

namespace lsa {

constexpr int kTK = 32;   // keys per tile

struct AttendArgs {
    const void *Q, *K, *V;
    int64_t m;
    int h_q, h_kv;
    int64_t n;
    int d;
    const int32_t *sel, *sel_count;
    int k;
    float scale_log2;     // scale * log2(e)
    int nsplit;
    void *out;
    float *lse;
    float *part;          // [m][h_q][nsplit][d + 2] when nsplit > 1
};

// The (row, KV head) group of head-major index y (all rows of KV head 0,
// then head 1, ...): the workgroups resident at one time then gather from
// one head's K/V region, and the shared last-level cache holds a larger part
// of it than when the heads of every row are interleaved.
LSA_DEV int64_t attend_row(const AttendArgs &A, int64_t y) { return (y % A.m) * A.h_kv + y / A.m; }

// A group's count and its selected ids as read from the caller's arrays, kept
// in range ([0, row length] and [0, n)) so that no gather leaves the cache
// whatever those arrays hold; in-range inputs pass unchanged.
LSA_DEV int attend_count(const AttendArgs &A, int64_t row) { return min(max(A.sel_count[row], 0), A.k); }
LSA_DEV int32_t attend_id(const AttendArgs &A, int32_t id) { return (int32_t)min<int64_t>(max(id, 0), A.n - 1); }


template <typename T>
__global__ __launch_bounds__(256) void k_attend(AttendArgs A) {
    extern __shared__ float smem[];
    const int d = A.d;
    const int G = A.h_q / A.h_kv;
    const int dp = d + 1;
    float *qs = smem;                    // [G][d]
    float *Ks = qs + G * d;              // [kTK][d + 1]
    float *Vs = Ks + kTK * dp;           // [kTK][d]
    float *Sc = Vs + kTK * d;            // [G][kTK]
    __shared__ int32_t ids[kTK];

    const int64_t row = attend_row(A, blockIdx.y);     // i * h_kv + g
    const int64_t i = row / A.h_kv;
    const int g = (int)(row % A.h_kv);
    const int split = blockIdx.x;
    const int cnt = attend_count(A, row);
    const int per = (cnt + A.nsplit - 1) / A.nsplit;
    const int s0 = min(cnt, split * per), s1 = min(cnt, s0 + per);
    const T *Q = (const T *)A.Q;
    const T *Kg = (const T *)A.K + (size_t)g * A.n * d;
    const T *Vg = (const T *)A.V + (size_t)g * A.n * d;
    const int32_t *S = A.sel + (size_t)row * A.k;

    for (int e = threadIdx.x; e < G * d; e += blockDim.x)
        qs[e] = to_float(Q[((size_t)i * A.h_q + (size_t)g * G) * d + e]) * A.scale_log2;

    constexpr int MAXE = 16;             // G * d <= 4096 elements over 256 threads
    const int ne = (G * d + blockDim.x - 1) / blockDim.x;
    float acc[MAXE], mrun[MAXE], lrun[MAXE];
#pragma unroll
    for (int q = 0; q < MAXE; ++q) { acc[q] = 0.0f; mrun[q] = -INFINITY; lrun[q] = 0.0f; }

    for (int kb = s0; kb < s1; kb += kTK) {
        const int nk = min(kTK, s1 - kb);
        __syncthreads();
        if (threadIdx.x < nk) ids[threadIdx.x] = attend_id(A, S[kb + threadIdx.x]);
        __syncthreads();
        gather_tile<T>(Kg, Vg, ids, nk, d, Ks, dp, Vs);
        __syncthreads();
        for (int e = threadIdx.x; e < G * nk; e += blockDim.x) {
            const int h = e / nk, kk = e % nk;
            const float *qh = qs + h * d;
            const float *kr = Ks + kk * dp;
            float s = 0.0f;
            for (int t = 0; t < d; ++t) s = fmaf(qh[t], kr[t], s);
            Sc[h * kTK + kk] = s;
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < MAXE; ++q) {
            if (q >= ne) break;
            const int e = threadIdx.x + q * blockDim.x;
            if (e >= G * d) break;
            const int h = e / d, t = e % d;
            const float *sc = Sc + h * kTK;
            float mt = -INFINITY;
            for (int kk = 0; kk < nk; ++kk) mt = fmaxf(mt, sc[kk]);
            const float mnew = fmaxf(mrun[q], mt);
            const float alpha = exp2f(mrun[q] - mnew);
            float a = acc[q] * alpha, ls = 0.0f;
            for (int kk = 0; kk < nk; ++kk) {
                const float p = exp2f(sc[kk] - mnew);
                ls += p;
                a = fmaf(p, Vs[kk * d + t], a);
            }
            acc[q] = a;
            lrun[q] = lrun[q] * alpha + ls;
            mrun[q] = mnew;
        }
    }
    const float ln2 = 0.69314718055994531f;
#pragma unroll
    for (int q = 0; q < MAXE; ++q) {
        if (q >= ne) break;
        const int e = threadIdx.x + q * blockDim.x;
        if (e >= G * d) break;
        const int h = e / d, t = e % d;
        const size_t oh = (size_t)i * A.h_q + (size_t)g * G + h;
        if (A.nsplit == 1) {
            const float o = (lrun[q] > 0.0f) ? acc[q] / lrun[q] : 0.0f;
            ((T *)A.out)[oh * d + t] = from_float<T>(o);
            if (t == 0 && A.lse) A.lse[oh] = (lrun[q] > 0.0f) ? (mrun[q] + log2f(lrun[q])) * ln2 : -INFINITY;
        } else {
            float *pp = A.part + (oh * A.nsplit + split) * (size_t)(d + 2);
            pp[t] = acc[q];
            if (t == 0) { pp[d] = mrun[q]; pp[d + 1] = lrun[q]; }
        }
    }
}

// ---------------------------------------------------------------- MFMA path (bf16)
// Each of the four waves walks its own 32-key steps of the workgroup's slice
// with the matrix-core step of mfma_attn.h and keeps its own softmax state;
// the four states are combined at the end.
constexpr int kIdsCap = 2048;       // selected ids of a slice staged in LDS at a time
constexpr int kWaveMax = 1024;      // sets this short are attended by one wave each
constexpr int kIdsW = kIdsCap / 4;  // ids staged per wave in that mode


// Output of one group from a normalised-later state: o / l in the input
// dtype (or the partial state of split `split`), lse on request.
LSA_DEV void attend_write(const AttendArgs &A, int64_t i, int g, int h, int dd, const floatx4_t &o, float M, float Ls,
                          int split, int D) {
    const size_t oh = (size_t)i * A.h_q + (size_t)g * (A.h_q / A.h_kv) + h;
    if (A.nsplit == 1) {
        const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
        bf16_t *op = (bf16_t *)A.out + oh * D + dd;
#pragma unroll
        for (int j = 0; j < 4; ++j) op[j] = from_float<bf16_t>(o[j] * inv);
        if (dd == 0 && A.lse) A.lse[oh] = (Ls > 0.0f) ? (M + log2f(Ls)) * 0.69314718055994531f : -INFINITY;
    } else {
        float *pp = A.part + (oh * A.nsplit + split) * (size_t)(D + 2);
#pragma unroll
        for (int j = 0; j < 4; ++j) pp[dd + j] = o[j];
        if (dd == 0) { pp[D] = M; pp[D + 1] = Ls; }
    }
}

// One wave's steps over ids[0, own) (LDS), the next step's gathers in flight
// while the current one is computed; steps step0, step0 + stride, ...
template <int D>
LSA_DEV void attend_steps(const uint16_t *Kg, const uint16_t *Vg, const int32_t *ids, int own, int step0, int stride,
                          const bf16x8_t (&qf)[D / 32], float scale_log2, uint16_t *vt, WaveAttn<D> &st,
                          bool &first) {
    const int nsteps = (own + kMT - 1) / kMT;
    if (step0 >= nsteps) return;
    WaveRows<D> ra, rb;
    int t = step0;
    wave_attn_load<D>(Kg, Vg, ids + t * kMT, ra);
    while (t < nsteps) {
        // step t in ra, the next one loading into rb (then the roles swap)
        if (t + stride < nsteps) wave_attn_load<D>(Kg, Vg, ids + (t + stride) * kMT, rb);
        {
            bf16x8_t pf;
            float alpha;
            wave_attn_compute<D>(ra, max(0, min(kMT, own - t * kMT)), qf, scale_log2, vt, st, pf, alpha);
            wave_sync();
            wave_attn_part2<D>(vt, pf, alpha, st, first);
            wave_sync();
            first = false;
        }
        t += stride;
        if (t >= nsteps) break;
        if (t + stride < nsteps) wave_attn_load<D>(Kg, Vg, ids + (t + stride) * kMT, ra);
        {
            bf16x8_t pf;
            float alpha;
            wave_attn_compute<D>(rb, max(0, min(kMT, own - t * kMT)), qf, scale_log2, vt, st, pf, alpha);
            wave_sync();
            wave_attn_part2<D>(vt, pf, alpha, st, first);
            wave_sync();
            first = false;
        }
        t += stride;
    }
}

// All four waves on one group's slice `split`: ids staged kIdsCap at a time,
// wave w takes steps w, w + 4, ...; the four states are combined in LDS.
template <int D>
LSA_DEV void attend_group_coop(const AttendArgs &A, int64_t row, int split, uint16_t (*vt)[D * kVTS],
                               int32_t *ids_s) {
    const int64_t i = row / A.h_kv;
    const int g = (int)(row % A.h_kv);
    const int G = A.h_q / A.h_kv;
    const int cnt = attend_count(A, row);
    const int per = (cnt + A.nsplit - 1) / A.nsplit;
    const int s0 = min(cnt, split * per), s1 = min(cnt, s0 + per);
    const int w = threadIdx.x / kWave;
    const uint16_t *Kg = (const uint16_t *)A.K + (size_t)g * A.n * D;
    const uint16_t *Vg = (const uint16_t *)A.V + (size_t)g * A.n * D;
    const uint16_t *Qb = (const uint16_t *)A.Q + ((size_t)i * A.h_q + (size_t)g * G) * D;
    const int32_t *S = A.sel + (size_t)row * A.k;
    bf16x8_t qf[D / 32];
    wave_load_q<D>(qf, Qb, G);
    WaveAttn<D> st;
    wave_attn_init<D>(st);
    bool first = true;
    // (ids padded with the chunk's first id to whole 4 x 32-key steps)
    for (int c0 = s0; c0 < s1; c0 += kIdsCap) {
        const int own = min(kIdsCap, s1 - c0);
        const int nsteps = (own + 4 * kMT - 1) / (4 * kMT);
        for (int f = threadIdx.x; f < nsteps * 4 * kMT; f += blockDim.x) ids_s[f] = attend_id(A, S[c0 + (f < own ? f : 0)]);
        __syncthreads();
        attend_steps<D>(Kg, Vg, ids_s, own, w, 4, qf, A.scale_log2, vt[w], st, first);
        __syncthreads();                 // ids_s is rewritten by the next chunk
    }
    __syncthreads();
    float *scratch = reinterpret_cast<float *>(&vt[0][0]);
    wave_attn_stash<D>(st, scratch);
    __syncthreads();
    for (int e4 = threadIdx.x; e4 < G * D / 4; e4 += blockDim.x) {
        const int h = e4 / (D / 4), dd = 4 * (e4 % (D / 4));
        float M, Ls;
        const floatx4_t o = wave_attn_combine4<D>(scratch, h, dd, M, Ls);
        attend_write(A, i, g, h, dd, o, M, Ls, split, D);
    }
}

// One wave on one whole group (nsplit == 1), ids staged kIdsW at a time in
// the wave's own part of ids_s; the wave writes the outputs itself.
template <int D>
LSA_DEV void attend_group_wave(const AttendArgs &A, int64_t row, uint16_t *vt, int32_t *ids_w) {
    const int l = lane_id();
    const int64_t i = row / A.h_kv;
    const int g = (int)(row % A.h_kv);
    const int G = A.h_q / A.h_kv;
    const int cnt = attend_count(A, row);
    const uint16_t *Kg = (const uint16_t *)A.K + (size_t)g * A.n * D;
    const uint16_t *Vg = (const uint16_t *)A.V + (size_t)g * A.n * D;
    const uint16_t *Qb = (const uint16_t *)A.Q + ((size_t)i * A.h_q + (size_t)g * G) * D;
    const int32_t *S = A.sel + (size_t)row * A.k;
    bf16x8_t qf[D / 32];
    wave_load_q<D>(qf, Qb, G);
    WaveAttn<D> st;
    wave_attn_init<D>(st);
    bool first = true;
    for (int c0 = 0; c0 < cnt; c0 += kIdsW) {
        const int own = min(kIdsW, cnt - c0);
        const int nsteps = (own + kMT - 1) / kMT;
        for (int f = l; f < nsteps * kMT; f += kWave) ids_w[f] = attend_id(A, S[c0 + (f < own ? f : 0)]);
        wave_sync();
        attend_steps<D>(Kg, Vg, ids_w, own, 0, 1, qf, A.scale_log2, vt, st, first);
        wave_sync();
    }
    // lane l holds head l % 16, dimensions 16 nb + 4 (l / 16) + j
    const int h = l % 16, q = l / 16;
    if (h < G) {
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb) attend_write(A, i, g, h, 16 * nb + 4 * q, st.acc[nb], st.m, st.l, 0, D);
    }
}

// nsplit > 1: one group's slice per workgroup (grid nsplit x groups).
// nsplit == 1: four consecutive head-major groups per workgroup; when all
// four sets are short (<= kWaveMax keys) each wave attends one of them alone,
// otherwise the four waves take the groups one after another together.
template <int D>
__global__ __launch_bounds__(256, 2) void k_attend_mfma(AttendArgs A) {
    __shared__ __attribute__((aligned(16))) uint16_t vt[4][D * kVTS];
    __shared__ int32_t ids_s[kIdsCap];
    if (A.nsplit > 1) {
        attend_group_coop<D>(A, attend_row(A, blockIdx.y), blockIdx.x, vt, ids_s);
        return;
    }
    const int64_t y0 = (int64_t)blockIdx.x * 4;
    const int ny = (int)min<int64_t>(4, A.m * A.h_kv - y0);
    int cmax = 0;
    for (int q = 0; q < ny; ++q) cmax = max(cmax, attend_count(A, attend_row(A, y0 + q)));
    if (cmax <= kWaveMax) {
        const int w = threadIdx.x / kWave;
        if (w < ny) attend_group_wave<D>(A, attend_row(A, y0 + w), vt[w], ids_s + w * kIdsW);
        return;
    }
    for (int q = 0; q < ny; ++q) {
        attend_group_coop<D>(A, attend_row(A, y0 + q), 0, vt, ids_s);
        __syncthreads();                 // vt (the combine scratch) and ids_s are reused by the next group
    }
}

// Combine split-K slices: M = max m_s, l = sum l_s 2^(m_s - M),
// o = sum o_s 2^(m_s - M) / l.
template <typename T>
__global__ __launch_bounds__(256) void k_attend_merge(AttendArgs A) {
    const int d = A.d;
    const int64_t oh = blockIdx.x;                  // i * h_q + h
    const float *pp = A.part + (size_t)oh * A.nsplit * (d + 2);
    float M = -INFINITY;
    for (int s = 0; s < A.nsplit; ++s) M = fmaxf(M, pp[(size_t)s * (d + 2) + d]);
    float l = 0.0f;
    for (int s = 0; s < A.nsplit; ++s) {
        const float ms = pp[(size_t)s * (d + 2) + d];
        if (ms > -INFINITY) l += pp[(size_t)s * (d + 2) + d + 1] * exp2f(ms - M);
    }
    for (int t = threadIdx.x; t < d; t += blockDim.x) {
        float o = 0.0f;
        for (int s = 0; s < A.nsplit; ++s) {
            const float ms = pp[(size_t)s * (d + 2) + d];
            if (ms > -INFINITY) o += pp[(size_t)s * (d + 2) + t] * exp2f(ms - M);
        }
        ((T *)A.out)[(size_t)oh * d + t] = from_float<T>(l > 0.0f ? o / l : 0.0f);
    }
    if (threadIdx.x == 0 && A.lse) A.lse[oh] = (l > 0.0f) ? (M + log2f(l)) * 0.69314718055994531f : -INFINITY;
}

int attend_nsplit(int64_t m, int h_kv, int k) {
    const int64_t groups = m * h_kv;
    int64_t want = (512 + groups - 1) / groups;
    const int64_t cap = (k + 127) / 128;
    if (want > cap) want = cap;
    if (want < 1) want = 1;
    if (want > 64) want = 64;
    return (int)want;
}

// Split partial states sit after the workspace's reserved prefix, which this
// path never writes.
int64_t attend_workspace_bytes(int64_t m, int h_q, int h_kv, int d, int k) {
    const int ns = attend_nsplit(m, h_kv, k);
    if (ns == 1) return 0;
    return ws_reserved_bytes() + (int64_t)m * h_q * ns * (d + 2) * (int64_t)sizeof(float);
}

hipError_t attend(const void *Q, const void *K, const void *V, int dtype, int64_t m, int h_q, int h_kv, int64_t n,
                  int d, const int32_t *sel, const int32_t *sel_count, int k, float scale, void *out, float *lse,
                  void *ws, hipStream_t st) {
    AttendArgs A{};
    A.Q = Q; A.K = K; A.V = V; A.m = m; A.h_q = h_q; A.h_kv = h_kv; A.n = n; A.d = d;
    A.sel = sel; A.sel_count = sel_count; A.k = k;
    A.scale_log2 = scale * 1.4426950408889634f;
    A.nsplit = attend_nsplit(m, h_kv, k);
    A.out = out; A.lse = lse;
    A.part = A.nsplit > 1 ? (float *)((char *)ws + ws_reserved_bytes()) : nullptr;
    const int G = h_q / h_kv;
    const size_t shm = sizeof(float) * ((size_t)G * d + (size_t)kTK * (d + 1) + (size_t)kTK * d + (size_t)G * kTK);
    const dim3 grid((unsigned)A.nsplit, (unsigned)(m * h_kv));
    if (shm > 65536) {
        hipError_t e = dtype == 0
            ? hipFuncSetAttribute((const void *)k_attend<float>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm)
            : hipFuncSetAttribute((const void *)k_attend<bf16_t>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
        if (e != hipSuccess) return e;
    }
    if (dtype == 0) {
        hipLaunchKernelGGL(k_attend<float>, grid, dim3(256), shm, st, A);
        if (A.nsplit > 1) hipLaunchKernelGGL(k_attend_merge<float>, dim3((unsigned)(m * h_q)), dim3(128), 0, st, A);
    } else {
        const dim3 mgrid = A.nsplit > 1 ? grid : dim3((unsigned)((m * h_kv + 3) / 4));
        if (d == 128) hipLaunchKernelGGL(k_attend_mfma<128>, mgrid, dim3(256), 0, st, A);
        else if (d == 64) hipLaunchKernelGGL(k_attend_mfma<64>, mgrid, dim3(256), 0, st, A);
        else if (d == 256) hipLaunchKernelGGL(k_attend_mfma<256>, mgrid, dim3(256), 0, st, A);
        else hipLaunchKernelGGL(k_attend<bf16_t>, grid, dim3(256), shm, st, A);
        if (A.nsplit > 1) hipLaunchKernelGGL(k_attend_merge<bf16_t>, dim3((unsigned)(m * h_q)), dim3(128), 0, st, A);
    }
    return hipGetLastError();
}

}  // namespace lsa
