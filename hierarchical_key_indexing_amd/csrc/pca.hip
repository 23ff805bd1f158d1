// Training-free latent projection by principal component analysis (gfx950).
//
// Instead of trained projection matrices, the indexing space can be built
// with principal component analysis of the keys ("Latent sparse attention",
// bdtechtalks.com, section "How latent sparse attention works", the
// training-free version of distilled LSA).  Per KV head the projection's r
// columns are the eigenvectors of the key covariance with the r largest
// eigenvalues, largest first, each signed so that its entry of largest
// magnitude (the first such) is positive.
//
// Four kernels, one grid dimension per KV head:
//   k_pca_mean    column sums of 8192-key chunks in double (each column's
//                 even keys, then its odd keys, ascending);
//   k_pca_gram    the centred Gram matrix of one chunk per workgroup: the
//                 chunk's mean-free keys staged in LDS as doubles 32 at a
//                 time, thread t accumulating an 8 x 8 block (64 FMAs per key);
//   k_pca_reduce  chunk partials summed in chunk order, divided by n;
//   k_pca_jacobi  the symmetric eigenproblem by cyclic Jacobi rotations in one
//                 workgroup: the matrix in LDS, the rotations' product V in
//                 the workspace, each step a round of disjoint pairs
//                 (round-robin order) rotated at once; sweeps until every
//                 off-diagonal entry is below 1e-14 of the largest diagonal
//                 one (at most 40), then the r leading eigenvectors are
//                 ranked, signed and rounded to fp32.
#include <algorithm>
#include <atomic>

#include "common.h"
#include "internal.h"

namespace lsa {

namespace {

constexpr int kPcaChunk = 8192;    // keys per chunk
constexpr int kPcaTile = 32;       // keys staged per step of k_pca_gram
constexpr int kPcaD = 128;         // largest d (the Jacobi matrix fills 128 KB of LDS)
constexpr int kPcaSweeps = 40;

struct PcaArgs {
    const void *K;                 // [h][n][d]
    int64_t n;
    int h, d, r, nchunk;
    double *mean_part;             // [h][nchunk][kPcaD]
    double *gram_part;             // [h][nchunk][kPcaD][kPcaD]
    double *cov;                   // [h][kPcaD][kPcaD]
    double *V;                     // [h][kPcaD][kPcaD], transposed: V[g][col][row]
    float *W;                      // [h][d][r]
    double *evals;                 // [h][r] or null
};

// A tile of kPcaTile keys x kPcaD dimensions: thread t holds elements
// t + 256 u (u < kPer), i.e. dimension t % 128 of keys 2u + t / 128 (zero
// beyond the chunk or beyond d).  All loads are issued before any is used.
constexpr int kPer = kPcaTile * kPcaD / 256;
template <typename T>
LSA_DEV void load_tile(const T *K, int d, int64_t j0, int nt, float (&v)[kPer]) {
    const int col = threadIdx.x % kPcaD, half = threadIdx.x / kPcaD;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int jj = 2 * u + half;
        const bool in = jj < nt && col < d;
        v[u] = to_float(K[(size_t)(j0 + (in ? jj : 0)) * d + (in ? col : 0)]);   // clamped
        if (!in) v[u] = 0.0f;
    }
}

template <typename T>
__global__ __launch_bounds__(256) void k_pca_mean(PcaArgs A) {
    __shared__ double half_s[kPcaD];
    const int c = blockIdx.x, g = blockIdx.y, t = threadIdx.x;
    const int64_t r0 = (int64_t)c * kPcaChunk, r1 = min<int64_t>(A.n, r0 + kPcaChunk);
    const T *K = (const T *)A.K + (size_t)g * A.n * A.d;
    // thread t: dimension t % 128 over the keys of parity t / 128, ascending
    double s = 0.0;
    float v[kPer], nv[kPer];
    load_tile(K, A.d, r0, (int)min<int64_t>(kPcaTile, r1 - r0), v);
    for (int64_t j0 = r0; j0 < r1; j0 += kPcaTile) {
        const int64_t j1 = j0 + kPcaTile;
        if (j1 < r1) load_tile(K, A.d, j1, (int)min<int64_t>(kPcaTile, r1 - j1), nv);
#pragma unroll
        for (int u = 0; u < kPer; ++u) s += (double)v[u];
#pragma unroll
        for (int u = 0; u < kPer; ++u) v[u] = nv[u];
    }
    if (t >= kPcaD) half_s[t - kPcaD] = s;
    __syncthreads();
    if (t < kPcaD && t < A.d) A.mean_part[((size_t)g * A.nchunk + c) * kPcaD + t] = s + half_s[t];
}

template <typename T>
__global__ __launch_bounds__(256) void k_pca_gram(PcaArgs A) {
    __shared__ double mu_s[kPcaD];
    __shared__ __attribute__((aligned(16))) double x_s[kPcaTile][kPcaD];
    const int c = blockIdx.x, g = blockIdx.y, t = threadIdx.x;
    const int d = A.d;
    const int64_t r0 = (int64_t)c * kPcaChunk, r1 = min<int64_t>(A.n, r0 + kPcaChunk);
    // the mean: chunk partials summed in chunk order
    if (t < kPcaD) {
        double s = 0.0;
        if (t < d)
            for (int q = 0; q < A.nchunk; ++q) s += A.mean_part[((size_t)g * A.nchunk + q) * kPcaD + t];
        mu_s[t] = s / (double)A.n;
    }
    const T *K = (const T *)A.K + (size_t)g * A.n * d;
    const int bi = 8 * (t / 16), bj = 8 * (t % 16);      // this thread's 8 x 8 block
    const int col = t % kPcaD, half = t / kPcaD;
    double acc[8][8];
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) acc[a][b] = 0.0;
    float v[kPer], nv[kPer];
    load_tile(K, d, r0, (int)min<int64_t>(kPcaTile, r1 - r0), v);
    __syncthreads();                                         // mean ready
    const double mu = mu_s[col];
    for (int64_t j0 = r0; j0 < r1; j0 += kPcaTile) {
        const int nt = (int)min<int64_t>(kPcaTile, r1 - j0);
        // mean-free keys of this tile (zero rows beyond the chunk add nothing)
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int jj = 2 * u + half;
            x_s[jj][col] = (jj < nt && col < d) ? (double)v[u] - mu : 0.0;
        }
        __syncthreads();
        const int64_t j1 = j0 + kPcaTile;
        if (j1 < r1) load_tile(K, d, j1, (int)min<int64_t>(kPcaTile, r1 - j1), nv);    // next tile in flight
        for (int jj = 0; jj < nt; ++jj) {
            double xa[8], xb[8];
#pragma unroll
            for (int a = 0; a < 8; a += 2) {
                const double2 va = *reinterpret_cast<const double2 *>(&x_s[jj][bi + a]);
                const double2 vb = *reinterpret_cast<const double2 *>(&x_s[jj][bj + a]);
                xa[a] = va.x; xa[a + 1] = va.y;
                xb[a] = vb.x; xb[a + 1] = vb.y;
            }
#pragma unroll
            for (int a = 0; a < 8; ++a)
#pragma unroll
                for (int b = 0; b < 8; ++b) acc[a][b] = fma(xa[a], xb[b], acc[a][b]);
        }
        __syncthreads();                                     // tile consumed
#pragma unroll
        for (int u = 0; u < kPer; ++u) v[u] = nv[u];
    }
    double *out = A.gram_part + ((size_t)g * A.nchunk + c) * kPcaD * kPcaD;
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) out[(size_t)(bi + a) * kPcaD + bj + b] = acc[a][b];
}

__global__ __launch_bounds__(256) void k_pca_reduce(PcaArgs A) {
    const int g = blockIdx.y;
    const int e = blockIdx.x * blockDim.x + threadIdx.x;     // entry of the 128 x 128 matrix
    if (e >= kPcaD * kPcaD) return;
    double s = 0.0;
    for (int q = 0; q < A.nchunk; ++q) s += A.gram_part[((size_t)g * A.nchunk + q) * kPcaD * kPcaD + e];
    A.cov[(size_t)g * kPcaD * kPcaD + e] = s / (double)A.n;
}

// Round-robin pairing of m (even) indices: round k's pairs are (L[i],
// L[m-1-i]) with L[0] = 0 and L[j] = 1 + (j - 1 + k) % (m - 1); over m - 1
// rounds every pair meets once.
LSA_DEV int rr_index(int j, int k, int m) { return j == 0 ? 0 : 1 + (j - 1 + k) % (m - 1); }

__global__ __launch_bounds__(256) void k_pca_jacobi(PcaArgs A) {
    extern __shared__ __attribute__((aligned(16))) double a_s[];    // [m][m + 1] (padded rows)
    __shared__ double cs_s[kPcaD / 2][2];
    __shared__ int pq_s[kPcaD / 2][2];
    __shared__ double red_s[2];
    __shared__ int rank_s[kPcaD], arg_s[kPcaD];
    const int g = blockIdx.x, t = threadIdx.x;
    const int d = A.d, m = d + (d & 1), np = m / 2;
    double *Vt = A.V + (size_t)g * kPcaD * kPcaD;              // Vt[col][row], row stride kPcaD
    // padded row stride: a column's entries (consecutive rows) fall in distinct banks
    auto at = [&](int i, int j) -> double & { return a_s[i * (m + 1) + j]; };
    for (int e = t; e < m * m; e += blockDim.x) {
        const int i = e / m, j = e % m;
        at(i, j) = (i < d && j < d) ? A.cov[(size_t)g * kPcaD * kPcaD + (size_t)i * kPcaD + j] : 0.0;
        Vt[(size_t)i * kPcaD + j] = (i == j) ? 1.0 : 0.0;
    }
    __syncthreads();
    for (int sweep = 0; sweep < kPcaSweeps; ++sweep) {
        // converged when every off-diagonal entry is below 1e-14 of the largest diagonal one
        if (t < 2) red_s[t] = 0.0;
        __syncthreads();
        double off = 0.0, dia = 0.0;
        for (int e = t; e < d * d; e += blockDim.x) {
            const int i = e / d, j = e % d;
            const double v = fabs(at(i, j));
            if (i == j) dia = fmax(dia, v); else off = fmax(off, v);
        }
        off = wave_max_d(off);
        dia = wave_max_d(dia);
        if (lane_id() == 0) {
            atomicMax(reinterpret_cast<unsigned long long *>(&red_s[0]), (unsigned long long)__double_as_longlong(off));
            atomicMax(reinterpret_cast<unsigned long long *>(&red_s[1]), (unsigned long long)__double_as_longlong(dia));
        }
        __syncthreads();
        const bool done = red_s[0] <= 1e-14 * red_s[1];
        __syncthreads();
        if (done) break;
        for (int k = 0; k < m - 1; ++k) {
            if (t < np) {
                const int p = rr_index(t, k, m), q = rr_index(m - 1 - t, k, m);
                double c = 1.0, s = 0.0;
                if (p < d && q < d) {
                    const double apq = at(p, q);
                    if (apq != 0.0) {
                        const double th = (at(q, q) - at(p, p)) / (2.0 * apq);
                        const double tt = (fabs(th) > 1e150) ? 0.5 / th : copysign(1.0, th) / (fabs(th) + sqrt(th * th + 1.0));
                        c = 1.0 / sqrt(tt * tt + 1.0);
                        s = tt * c;
                    }
                }
                cs_s[t][0] = c; cs_s[t][1] = s;
                pq_s[t][0] = p; pq_s[t][1] = q;
            }
            __syncthreads();
            // columns: A <- A J, V <- V J.  Thread t takes entries t + 256 u
            // (pair e / m, row e % m); its V entries are all loaded first.
            {
                constexpr int U = kPcaD / 2 * kPcaD / 256;
                double vp[U], vq[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int e = min(t + 256 * u, np * m - 1);               // clamped: in bounds
                    const int pr = e / m, row = e % m;
                    vp[u] = Vt[(size_t)pq_s[pr][0] * kPcaD + row];
                    vq[u] = Vt[(size_t)pq_s[pr][1] * kPcaD + row];
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int e = t + 256 * u;
                    if (e >= np * m) break;
                    const int pr = e / m, row = e % m;
                    const double c = cs_s[pr][0], s = cs_s[pr][1];
                    if (s == 0.0) continue;
                    const int p = pq_s[pr][0], q = pq_s[pr][1];
                    const double ap = at(row, p), aq = at(row, q);
                    at(row, p) = c * ap - s * aq;
                    at(row, q) = s * ap + c * aq;
                    Vt[(size_t)p * kPcaD + row] = c * vp[u] - s * vq[u];
                    Vt[(size_t)q * kPcaD + row] = s * vp[u] + c * vq[u];
                }
            }
            __syncthreads();
            // rows: A <- J^T A
            for (int e = t; e < np * m; e += blockDim.x) {
                const int pr = e / m, col = e % m;
                const double c = cs_s[pr][0], s = cs_s[pr][1];
                if (s == 0.0) continue;
                const int p = pq_s[pr][0], q = pq_s[pr][1];
                const double bp = at(p, col), bq = at(q, col);
                at(p, col) = c * bp - s * bq;
                at(q, col) = s * bp + c * bq;
            }
            __syncthreads();
        }
    }
    // rank of eigenvalue i: the larger ones, then equal ones of lower index
    if (t < d) {
        const double li = at(t, t);
        int rk = 0;
        for (int j = 0; j < d; ++j) {
            const double lj = at(j, j);
            rk += (lj > li || (lj == li && j < t)) ? 1 : 0;
        }
        rank_s[t] = rk;
        arg_s[rk] = t;
    }
    __syncthreads();
    // column c of W: eigenvector arg_s[c], signed by its largest entry
    if (t < A.r) {
        const int i = arg_s[t];
        int jm = 0;
        double vm = -1.0;
        const double *vi = Vt + (size_t)i * kPcaD;
        for (int x = 0; x < d; ++x) {
            const double v = fabs(vi[x]);
            if (v > vm) { vm = v; jm = x; }
        }
        const double sg = vi[jm] < 0.0 ? -1.0 : 1.0;
        for (int x = 0; x < d; ++x) A.W[((size_t)g * d + x) * A.r + t] = (float)(sg * vi[x]);
        if (A.evals) A.evals[(size_t)g * A.r + t] = at(i, i);
    }
}

inline size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

struct PcaWs { double *mean_part, *gram_part, *cov, *V; size_t bytes; };

PcaWs carve_pca_ws(char *base, int64_t n, int h) {
    size_t cur = 0;
    PcaWs w{};
    auto take = [&](size_t b) { char *p = base ? base + cur : nullptr; cur = a256(cur + b); return p; };
    const size_t nchunk = (size_t)((n + kPcaChunk - 1) / kPcaChunk);
    w.mean_part = (double *)take(sizeof(double) * h * nchunk * kPcaD);
    w.gram_part = (double *)take(sizeof(double) * h * nchunk * kPcaD * kPcaD);
    w.cov = (double *)take(sizeof(double) * h * kPcaD * kPcaD);
    w.V = (double *)take(sizeof(double) * h * kPcaD * kPcaD);
    w.bytes = cur;
    return w;
}

}  // namespace

int64_t pca_workspace_bytes(int64_t n, int h) { return (int64_t)carve_pca_ws(nullptr, n, h).bytes; }

hipError_t pca_projection(const void *K, int dtype, int64_t n, int h, int d, int r, float *W, double *evals, void *ws,
                          hipStream_t st) {
    PcaWs w = carve_pca_ws((char *)ws, n, h);
    PcaArgs A{};
    A.K = K; A.n = n; A.h = h; A.d = d; A.r = r;
    A.nchunk = (int)((n + kPcaChunk - 1) / kPcaChunk);
    A.mean_part = w.mean_part; A.gram_part = w.gram_part; A.cov = w.cov; A.V = w.V; A.W = W; A.evals = evals;
    const dim3 cg((unsigned)A.nchunk, (unsigned)h);
    if (dtype == 0) {
        hipLaunchKernelGGL(k_pca_mean<float>, cg, dim3(256), 0, st, A);
        hipLaunchKernelGGL(k_pca_gram<float>, cg, dim3(256), 0, st, A);
    } else {
        hipLaunchKernelGGL(k_pca_mean<bf16_t>, cg, dim3(256), 0, st, A);
        hipLaunchKernelGGL(k_pca_gram<bf16_t>, cg, dim3(256), 0, st, A);
    }
    hipLaunchKernelGGL(k_pca_reduce, dim3(kPcaD * kPcaD / 256, (unsigned)h), dim3(256), 0, st, A);
    const int m = d + (d & 1);
    const size_t shm = sizeof(double) * (size_t)m * (m + 1);
    // the attribute is set once per device (setting it twice is harmless)
    static std::atomic<int> attr_set[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    if (!attr_set[dev].load(std::memory_order_acquire)) {
        hipError_t e = hipFuncSetAttribute((const void *)k_pca_jacobi, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)(sizeof(double) * kPcaD * (kPcaD + 1)));
        if (e != hipSuccess) return e;
        attr_set[dev].store(1, std::memory_order_release);
    }
    hipLaunchKernelGGL(k_pca_jacobi, dim3((unsigned)h), dim3(256), shm, st, A);
    return hipGetLastError();
}

}  // namespace lsa
