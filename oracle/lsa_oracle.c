/*
 * CPU oracle for the latent-sparse-attention (LSA) layer: index build, top-down
 * selection and sparse attention, written plainly for checking, not for speed.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
 * baseline may call this library. It shares no code with the HIP library.
 *
 * Source of the method: "Latent Sparse Attention Breaks Through the
 * Million-Token Context Bottleneck" (kongchang.com), section "How LSA Sidesteps
 * Per-Key Scoring with Hierarchical Clustering"; "Latent sparse attention"
 * (bdtechtalks.com), sections "The compute bottleneck of sparse attention" and
 * "How latent sparse attention works".  Readings of points the pages leave open
 * are stated at each function.
 *
 * Arithmetic: every sum is accumulated in double, in the index order written
 * in the loop, and rounded once to float where a float value is defined.  The
 * file is compiled with -ffp-contract=off so that a*b+c is two roundings.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#else
static int omp_in_parallel(void) { return 0; }
#endif

int oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Latent projection (kongchang.com, "How LSA Sidesteps ...": keys are mapped
 * into a learned low-dimensional latent space; bdtechtalks.com, "How latent
 * sparse attention works": keys are represented in a latent space).
 * One KV head: z[j][c] = fl32( sum_i K[j][i] * W[i][c] ), i ascending.
 * K: [n][d] float (bf16 inputs are widened exactly), W: [d][r], Z: [n][r]. */
void oracle_project(const float *K, int64_t n, int d, const float *W, int r, float *Z)
{
#pragma omp parallel for schedule(static) if (n > 4096)
    for (int64_t j = 0; j < n; ++j) {
        for (int c = 0; c < r; ++c) {
            double s = 0.0;
            for (int i = 0; i < d; ++i)
                s += (double)K[j * d + i] * (double)W[(int64_t)i * r + c];
            Z[j * r + c] = (float)s;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* One node of the top-down clustering: k-means (Lloyd) on the node's members
 * in latent space, squared Euclidean distance (kongchang.com: divisions become
 * finer toward the leaves, "similar to hierarchical k-means"; bdtechtalks.com:
 * each cluster is represented by a centroid stored with references to its keys).
 *
 * Readings (the pages are silent on these):
 *   - a = min(b, m) children are active; child c < a starts at the member of
 *     rank floor(c*m/a) in ascending key order; children c >= a stay empty;
 *   - T rounds of: assign every member to the nearest active child (ties to
 *     the smaller child index), then replace each child that received members
 *     by fl32(mean of their latents); a child with no members keeps its
 *     centroid;
 *   - the node's final partition is the T-th assignment.
 *
 * S: members (ascending key ids), m of them.  C: [b][r] out (inactive rows 0).
 * assign: [m] out.  cnt: [b] out. */
void oracle_lloyd_node(const float *Z, int r, const int32_t *S, int64_t m, int b, int T,
                       float *C, int32_t *assign, int64_t *cnt)
{
    int a = (m < b) ? (int)m : b;
    memset(C, 0, sizeof(float) * (size_t)b * (size_t)r);
    for (int c = 0; c < b; ++c) cnt[c] = 0;
    if (m == 0) return;
    for (int c = 0; c < a; ++c) {
        int64_t rank = ((int64_t)c * m) / a;
        memcpy(C + (size_t)c * r, Z + (int64_t)S[rank] * r, sizeof(float) * (size_t)r);
    }
    double *sum = (double *)malloc(sizeof(double) * (size_t)r);
    for (int t = 0; t < T; ++t) {
        /* assignment step */
#pragma omp parallel for schedule(static) if (m > 8192 && !omp_in_parallel())
        for (int64_t p = 0; p < m; ++p) {
            const float *z = Z + (int64_t)S[p] * r;
            int best = 0;
            double bestd = 0.0;
            for (int c = 0; c < a; ++c) {
                const float *cc = C + (size_t)c * r;
                double dist = 0.0;
                for (int i = 0; i < r; ++i) {
                    double diff = (double)z[i] - (double)cc[i];
                    dist += diff * diff;
                }
                if (c == 0 || dist < bestd) { bestd = dist; best = c; }
            }
            assign[p] = best;
        }
        /* update step */
        for (int c = 0; c < a; ++c) {
            int64_t k = 0;
            for (int i = 0; i < r; ++i) sum[i] = 0.0;
            for (int64_t p = 0; p < m; ++p) {
                if (assign[p] != c) continue;
                const float *z = Z + (int64_t)S[p] * r;
                for (int i = 0; i < r; ++i) sum[i] += (double)z[i];
                ++k;
            }
            if (k > 0)
                for (int i = 0; i < r; ++i) C[(size_t)c * r + i] = (float)(sum[i] / (double)k);
        }
    }
    for (int64_t p = 0; p < m; ++p) cnt[assign[p]]++;
    free(sum);
}

static int64_t ipow(int64_t b, int e) { int64_t v = 1; while (e-- > 0) v *= b; return v; }

/* Offset (in elements) of level l (1..L) inside the concatenated per-level
 * arrays: level l of head g starts at h_kv * sum_{l' < l} b^l' + g * b^l. */
int64_t oracle_level_base(int h_kv, int b, int l)
{
    int64_t s = 0;
    for (int q = 1; q < l; ++q) s += ipow(b, q);
    return s * h_kv;
}

/* ------------------------------------------------------------------------ */
/* Index build, every KV head independently (kongchang.com, "How LSA Sidesteps
 * ...": the root represents all keys; each level divides further; the tree is
 * precomputed).  Reading: a complete b-ary tree with L levels below the root,
 * children of node v are v*b + c; empty nodes are allowed.
 *
 * K: [h][n][d], W: [h][d][r].
 * C_all: concatenation over l = 1..L of [h][b^l][r] floats.
 * cnt_all: concatenation over l = 1..L of [h][b^l] int64.
 * leaf_off: [h][b^L + 1]; perm: [h][n] (keys grouped by leaf, ascending
 * within a leaf).  Returns 0. */
int oracle_build(const float *K, int64_t n, int h_kv, int d, const float *W, int r,
                 int b, int L, int T, float *C_all, int64_t *cnt_all, int64_t *leaf_off,
                 int32_t *perm)
{
    float *Z = (float *)malloc(sizeof(float) * (size_t)n * (size_t)r);
    int32_t *cur = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
    int32_t *nxt = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
    int64_t nleaf = ipow(b, L);
    int64_t *off = (int64_t *)malloc(sizeof(int64_t) * (size_t)(nleaf + 1));
    int64_t *noff = (int64_t *)malloc(sizeof(int64_t) * (size_t)(nleaf + 1));
    for (int g = 0; g < h_kv; ++g) {
        oracle_project(K + (int64_t)g * n * d, n, d, W + (int64_t)g * d * r, r, Z);
        for (int64_t j = 0; j < n; ++j) cur[j] = (int32_t)j;
        off[0] = 0; off[1] = n;
        for (int l = 1; l <= L; ++l) {
            int64_t nparent = ipow(b, l - 1);
            int64_t nodes = nparent * b;
            float *C = C_all + (oracle_level_base(h_kv, b, l) + (int64_t)g * nodes) * r;
            int64_t *cnt = cnt_all + oracle_level_base(h_kv, b, l) + (int64_t)g * nodes;
#pragma omp parallel for schedule(dynamic, 16) if (nparent >= 8)
            for (int64_t u = 0; u < nparent; ++u) {
                int64_t s = off[u], m = off[u + 1] - off[u];
                int32_t *asg = (int32_t *)malloc(sizeof(int32_t) * (size_t)(m > 0 ? m : 1));
                oracle_lloyd_node(Z, r, cur + s, m, b, T, C + u * b * r, asg, cnt + u * b);
                /* children's member lists, each in ascending key order */
                int64_t w = s;
                for (int c = 0; c < b; ++c) {
                    noff[u * b + c] = w;
                    for (int64_t p = 0; p < m; ++p)
                        if (asg[p] == c) nxt[w++] = cur[s + p];
                }
                free(asg);
            }
            noff[nodes] = n;
            int32_t *tp = cur; cur = nxt; nxt = tp;
            int64_t *to = off; off = noff; noff = to;
        }
        memcpy(leaf_off + (int64_t)g * (nleaf + 1), off, sizeof(int64_t) * (size_t)(nleaf + 1));
        memcpy(perm + (int64_t)g * n, cur, sizeof(int32_t) * (size_t)n);
    }
    free(Z); free(cur); free(nxt); free(off); free(noff);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Selection (kongchang.com, "How LSA Sidesteps ...": the query starts at the
 * root, scores a few candidate clusters per level and descends the chosen
 * branches to the leaves; bdtechtalks.com, "How latent sparse attention
 * works": a fixed search budget per level, then a fixed number of original
 * keys is retrieved from the chosen clusters; causal attention sees only
 * earlier tokens, "The compute bottleneck of sparse attention").
 *
 * Readings:
 *   - query heads sharing a KV head score with their mean qbar, projected by
 *     the same W as the keys: u = fl32(qbar . W);
 *   - score(v) = fl32(u . C[v]) (plain inner product);
 *   - level 1 candidates are the non-empty children of the root; at levels
 *     1..L-1 the first min(beam, |F|) candidates in (score desc, id asc) order
 *     are kept and their non-empty children become the next candidates; every
 *     candidate at level L is a candidate leaf;
 *   - leaves are visited in (score desc, id asc) order, each emitting its
 *     members in ascending position; keys at positions > pos are skipped
 *     (a key at the query's own position is visible); the first k are taken;
 *   - sel lists the taken keys in the order they were retrieved (leaf order,
 *     then ascending position inside a leaf); cutoff is the score of the leaf
 *     holding the k-th taken key, -inf when fewer than k keys were available.
 *
 * Sinks and window (bdtechtalks.com, "How latent sparse attention works": the
 * retrieved keys are joined by a window of recent tokens and a few initial
 * sink tokens).  Readings: with hi = min(pos, n - 1) the latest key the query
 * sees, the sinks are the keys [0, min(n_sink, hi + 1)) and the window is the
 * `window` latest visible keys that are not sinks, [max(n_sink, hi - window +
 * 1), hi]; retrieval skips both, so it only takes keys in [n_sink, hi -
 * window] and still takes up to k of them.  The three parts are disjoint and
 * their union is the attention set.  A row of sel holds k + n_sink + window
 * entries: the retrieved keys, then the sinks ascending, then the window
 * ascending, padded with -1; count is the number of entries before the
 * padding.  n_sink = window = 0 is the plain retrieval above.
 * Optional outputs (may be NULL): kept [m][h_kv][L-1][beam] (ids, -1 padded, in
 * rank order), nscored [m][h_kv] (number of centroids scored). */
typedef struct { float s; int64_t id; } cand_t;

static int cand_cmp(const void *pa, const void *pb)
{
    const cand_t *a = (const cand_t *)pa, *b = (const cand_t *)pb;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return (a->id < b->id) ? -1 : (a->id > b->id);
}

static float score_row(const float *u, const float *c, int r)
{
    double s = 0.0;
    for (int i = 0; i < r; ++i) s += (double)u[i] * (double)c[i];
    return (float)s;
}

int oracle_select(const float *Q, int64_t m, int h_q, int d, const int32_t *pos,
                  int64_t n, int h_kv, int r, int b, int L,
                  const float *C_all, const int64_t *cnt_all, const int64_t *leaf_off,
                  const int32_t *perm, const float *W, int beam, int k, int n_sink, int window,
                  int32_t *sel, int32_t *sel_count, float *cutoff,
                  int32_t *kept, int64_t *nscored)
{
    int G = h_q / h_kv;
    int64_t nleaf = ipow(b, L);
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t i = 0; i < m; ++i) {
        for (int g = 0; g < h_kv; ++g) {
            float *qbar = (float *)malloc(sizeof(float) * (size_t)d);
            float *u = (float *)malloc(sizeof(float) * (size_t)r);
            for (int t = 0; t < d; ++t) {
                double s = 0.0;
                for (int h = 0; h < G; ++h) s += (double)Q[(i * h_q + (int64_t)g * G + h) * d + t];
                qbar[t] = (float)(s / (double)G);
            }
            const float *Wg = W + (int64_t)g * d * r;
            for (int c = 0; c < r; ++c) {
                double s = 0.0;
                for (int t = 0; t < d; ++t) s += (double)qbar[t] * (double)Wg[(int64_t)t * r + c];
                u[c] = (float)s;
            }
            /* candidates at level 1: non-empty children of the root */
            int64_t cap = (int64_t)b * (beam > 1 ? beam : 1);
            if (cap < b) cap = b;
            cand_t *F = (cand_t *)malloc(sizeof(cand_t) * (size_t)cap);
            int64_t nf = 0, scored = 0;
            {
                const int64_t *cnt1 = cnt_all + oracle_level_base(h_kv, b, 1) + (int64_t)g * b;
                for (int c = 0; c < b; ++c)
                    if (cnt1[c] > 0) { F[nf].id = c; nf++; }
            }
            for (int l = 1; l <= L; ++l) {
                int64_t nodes = ipow(b, l);
                const float *C = C_all + (oracle_level_base(h_kv, b, l) + (int64_t)g * nodes) * r;
                for (int64_t t = 0; t < nf; ++t) F[t].s = score_row(u, C + F[t].id * r, r);
                scored += nf;
                qsort(F, (size_t)nf, sizeof(cand_t), cand_cmp);
                if (l == L) break;
                int64_t keep = nf < beam ? nf : beam;
                if (kept) {
                    int32_t *kp = kept + ((i * h_kv + g) * (int64_t)(L - 1) + (l - 1)) * beam;
                    for (int t = 0; t < beam; ++t) kp[t] = (t < keep) ? (int32_t)F[t].id : -1;
                }
                const int64_t *cn = cnt_all + oracle_level_base(h_kv, b, l + 1) + (int64_t)g * nodes * b;
                cand_t *nx = (cand_t *)malloc(sizeof(cand_t) * (size_t)cap);
                int64_t nn = 0;
                for (int64_t t = 0; t < keep; ++t)
                    for (int c = 0; c < b; ++c) {
                        int64_t v = F[t].id * b + c;
                        if (cn[v] > 0) { nx[nn].id = v; nn++; }
                    }
                free(F);
                F = nx;
                nf = nn;
            }
            /* fill: leaves in (score desc, id asc) order, members ascending,
             * only keys in [n_sink, hi - window] */
            const int64_t row = (int64_t)k + n_sink + window;
            int32_t *out = sel + (i * h_kv + g) * row;
            const int64_t *lo = leaf_off + (int64_t)g * (nleaf + 1);
            const int32_t *pm = perm + (int64_t)g * n;
            const int64_t hi = (int64_t)pos[i] < n - 1 ? (int64_t)pos[i] : n - 1;
            int64_t taken = 0;
            float cut = -INFINITY;
            for (int64_t t = 0; t < nf && taken < k; ++t) {
                for (int64_t p = lo[F[t].id]; p < lo[F[t].id + 1] && taken < k; ++p) {
                    if (pm[p] < n_sink || pm[p] > hi - window) continue;
                    out[taken++] = pm[p];
                    if (taken == k) cut = F[t].s;
                }
            }
            int64_t filled = taken;
            /* sinks, then the window */
            for (int64_t j = 0; j < n_sink && j <= hi; ++j) out[filled++] = (int32_t)j;
            for (int64_t j = (hi - window + 1 > n_sink ? hi - window + 1 : n_sink); j <= hi; ++j)
                out[filled++] = (int32_t)j;
            for (int64_t t = filled; t < row; ++t) out[t] = -1;
            sel_count[i * h_kv + g] = (int32_t)filled;
            if (cutoff) cutoff[i * h_kv + g] = cut;
            if (nscored) nscored[i * h_kv + g] = scored;
            free(F); free(qbar); free(u);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Flat search (bdtechtalks.com, "How latent sparse attention works": the
 * query is compared against all cluster centroids; the hierarchical search is
 * the alternative that follows a few branches per level).  Reading: the
 * clusters are the leaves of the tree; every non-empty leaf is scored with
 * score(v) = fl32(u . C_L[v]), the leaves are visited in (score desc, id asc)
 * order and filled exactly as in oracle_select (retrieval range, k, sinks,
 * window, cutoff).  No level above the leaves is consulted.  Outputs as in
 * oracle_select; nscored [m][h_kv] may be NULL. */
int oracle_select_flat(const float *Q, int64_t m, int h_q, int d, const int32_t *pos,
                       int64_t n, int h_kv, int r, int b, int L,
                       const float *C_all, const int64_t *cnt_all, const int64_t *leaf_off,
                       const int32_t *perm, const float *W, int k, int n_sink, int window,
                       int32_t *sel, int32_t *sel_count, float *cutoff, int64_t *nscored)
{
    int G = h_q / h_kv;
    int64_t nleaf = ipow(b, L);
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t i = 0; i < m; ++i) {
        for (int g = 0; g < h_kv; ++g) {
            float *qbar = (float *)malloc(sizeof(float) * (size_t)d);
            float *u = (float *)malloc(sizeof(float) * (size_t)r);
            for (int t = 0; t < d; ++t) {
                double s = 0.0;
                for (int h = 0; h < G; ++h) s += (double)Q[(i * h_q + (int64_t)g * G + h) * d + t];
                qbar[t] = (float)(s / (double)G);
            }
            const float *Wg = W + (int64_t)g * d * r;
            for (int c = 0; c < r; ++c) {
                double s = 0.0;
                for (int t = 0; t < d; ++t) s += (double)qbar[t] * (double)Wg[(int64_t)t * r + c];
                u[c] = (float)s;
            }
            const int64_t *cn = cnt_all + oracle_level_base(h_kv, b, L) + (int64_t)g * nleaf;
            const float *C = C_all + (oracle_level_base(h_kv, b, L) + (int64_t)g * nleaf) * r;
            cand_t *F = (cand_t *)malloc(sizeof(cand_t) * (size_t)(nleaf > 0 ? nleaf : 1));
            int64_t nf = 0;
            for (int64_t v = 0; v < nleaf; ++v)
                if (cn[v] > 0) { F[nf].id = v; F[nf].s = score_row(u, C + v * r, r); nf++; }
            qsort(F, (size_t)nf, sizeof(cand_t), cand_cmp);
            const int64_t row = (int64_t)k + n_sink + window;
            int32_t *out = sel + (i * h_kv + g) * row;
            const int64_t *lo = leaf_off + (int64_t)g * (nleaf + 1);
            const int32_t *pm = perm + (int64_t)g * n;
            const int64_t hi = (int64_t)pos[i] < n - 1 ? (int64_t)pos[i] : n - 1;
            int64_t taken = 0;
            float cut = -INFINITY;
            for (int64_t t = 0; t < nf && taken < k; ++t) {
                for (int64_t p = lo[F[t].id]; p < lo[F[t].id + 1] && taken < k; ++p) {
                    if (pm[p] < n_sink || pm[p] > hi - window) continue;
                    out[taken++] = pm[p];
                    if (taken == k) cut = F[t].s;
                }
            }
            int64_t filled = taken;
            for (int64_t j = 0; j < n_sink && j <= hi; ++j) out[filled++] = (int32_t)j;
            for (int64_t j = (hi - window + 1 > n_sink ? hi - window + 1 : n_sink); j <= hi; ++j)
                out[filled++] = (int32_t)j;
            for (int64_t t = filled; t < row; ++t) out[t] = -1;
            sel_count[i * h_kv + g] = (int32_t)filled;
            if (cutoff) cutoff[i * h_kv + g] = cut;
            if (nscored) nscored[i * h_kv + g] = nf;
            free(F); free(qbar); free(u);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Sparse attention over the selected keys (kongchang.com, "The
 * Accuracy-Efficiency Dilemma ...": each query interacts with k keys instead
 * of all n; bdtechtalks.com, "How latent sparse attention works": attention is
 * computed over the retrieved keys).  Query head h uses KV head h / G.
 * o = sum_j softmax(scale * q.K_j) V_j over the selected j; an empty set gives
 * o = 0 and lse = -inf.  Outputs in double: out [m][h_q][d], lse [m][h_q]. */
int oracle_attend(const float *Q, const float *K, const float *V, int64_t m, int h_q,
                  int h_kv, int64_t n, int d, const int32_t *sel, const int32_t *sel_count,
                  int k, double scale, double *out, double *lse)
{
    int G = h_q / h_kv;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t i = 0; i < m; ++i) {
        for (int h = 0; h < h_q; ++h) {
            int g = h / G;
            int cntv = sel_count[i * h_kv + g];
            const int32_t *S = sel + (i * h_kv + g) * (int64_t)k;
            const float *q = Q + (i * h_q + h) * (int64_t)d;
            double *o = out + (i * h_q + h) * (int64_t)d;
            for (int t = 0; t < d; ++t) o[t] = 0.0;
            if (cntv == 0) { lse[i * h_q + h] = -INFINITY; continue; }
            double *s = (double *)malloc(sizeof(double) * (size_t)cntv);
            double mx = -INFINITY;
            for (int j = 0; j < cntv; ++j) {
                const float *kr = K + ((int64_t)g * n + S[j]) * d;
                double acc = 0.0;
                for (int t = 0; t < d; ++t) acc += (double)q[t] * (double)kr[t];
                s[j] = acc * scale;
                if (s[j] > mx) mx = s[j];
            }
            double l = 0.0;
            for (int j = 0; j < cntv; ++j) {
                double p = exp(s[j] - mx);
                l += p;
                const float *vr = V + ((int64_t)g * n + S[j]) * d;
                for (int t = 0; t < d; ++t) o[t] += p * (double)vr[t];
            }
            for (int t = 0; t < d; ++t) o[t] /= l;
            lse[i * h_q + h] = mx + log(l);
            free(s);
        }
    }
    return 0;
}
