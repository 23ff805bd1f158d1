// C ABI of the LSA layer: argument checks, index layout, dispatch.
#include <math.h>
#include <string.h>

#include "lsa.h"
#include "internal.h"

namespace {

inline int64_t ipow_checked(int64_t b, int e, int64_t cap) {
    int64_t v = 1;
    for (int i = 0; i < e; ++i) {
        if (v > cap / b) return -1;
        v *= b;
    }
    return v;
}

inline int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

inline int check_desc(const lsa_index_desc *desc) {
    if (!desc) return LSA_EINVAL;
    lsa_index_desc ref;
    int rc = lsa_index_layout(desc->n, desc->h_kv, desc->r, desc->b, desc->L, &ref);
    if (rc != LSA_OK) return rc;
    if (memcmp(&ref, desc, sizeof(ref)) != 0) return LSA_EINVAL;
    return LSA_OK;
}

inline bool dtype_ok(int dtype) { return dtype == LSA_F32 || dtype == LSA_BF16; }

constexpr int kMaxRow = 1 << 24;     // longest row of sel (attention set of one row and KV head)

// sinks and window: EINVAL when negative, EUNSUPPORTED when a row would exceed kMaxRow
inline int check_local(int k, int n_sink, int window) {
    if (n_sink < 0 || window < 0) return LSA_EINVAL;
    if ((int64_t)k + n_sink + window > kMaxRow) return LSA_EUNSUPPORTED;
    return LSA_OK;
}

}  // namespace

extern "C" {

int lsa_abi_version(void) { return LSA_ABI_VERSION; }

const char *lsa_strerror(int code) {
    switch (code) {
        case LSA_OK: return "ok";
        case LSA_EINVAL: return "invalid argument";
        case LSA_EUNSUPPORTED: return "unsupported shape or type";
        case LSA_ENOSPC: return "buffer too small";
        case LSA_EHIP: return "HIP launch error";
        default: return "unknown error";
    }
}

int lsa_index_layout(int64_t n, int h_kv, int r, int b, int L, lsa_index_desc *desc) {
    if (!desc) return LSA_EINVAL;
    if (n < 1 || n > INT32_MAX || h_kv < 1 || r < 1 || b < 2 || L < 1) return LSA_EINVAL;
    if (r > 64 || b > 64 || L > LSA_MAX_LEVELS) return LSA_EUNSUPPORTED;
    const int64_t leaves = ipow_checked(b, L, (int64_t)INT32_MAX - 1);
    if (leaves < 0) return LSA_EUNSUPPORTED;
    lsa_index_desc D;
    memset(&D, 0, sizeof(D));
    D.n = n; D.h_kv = h_kv; D.r = r; D.b = b; D.L = L;
    int64_t cur = 0;
    D.nodes[0] = 1;
    for (int l = 1; l <= L; ++l) {
        D.nodes[l] = D.nodes[l - 1] * b;
        D.centroid_off[l] = cur;
        cur = align256(cur + (int64_t)h_kv * D.nodes[l] * r * 4);
    }
    for (int l = 1; l <= L; ++l) {
        D.count_off[l] = cur;
        cur = align256(cur + (int64_t)h_kv * D.nodes[l] * 4);
    }
    D.leaf_off_off = cur;
    cur = align256(cur + (int64_t)h_kv * (leaves + 1) * 4);
    D.perm_off = cur;
    cur = align256(cur + (int64_t)h_kv * n * 4);
    D.bytes = cur;
    *desc = D;
    return LSA_OK;
}

int lsa_build_workspace_bytes(int64_t n, int h_kv, int d, int r, int b, int L, int64_t *bytes) {
    lsa_index_desc D;
    int rc = lsa_index_layout(n, h_kv, r, b, L, &D);
    if (rc != LSA_OK) return rc;
    if (d < 1) return LSA_EINVAL;
    if (d > 256) return LSA_EUNSUPPORTED;
    if (!bytes) return LSA_EINVAL;
    *bytes = lsa::build_workspace_bytes(n, h_kv, r, b, L);
    return LSA_OK;
}

int lsa_build_index(const void *K, int dtype, int64_t n, int h_kv, int d, const float *W, int r, int b, int L,
                    int iters, void *index, int64_t index_bytes, void *ws, int64_t ws_bytes, lsa_index_desc *desc,
                    void *stream) {
    lsa_index_desc D;
    int rc = lsa_index_layout(n, h_kv, r, b, L, &D);
    if (rc != LSA_OK) return rc;
    if (!K || !W || !index || !desc || iters < 1 || d < 1) return LSA_EINVAL;
    if (!dtype_ok(dtype)) return LSA_EUNSUPPORTED;
    if (d > 256) return LSA_EUNSUPPORTED;
    if (index_bytes < D.bytes) return LSA_ENOSPC;
    const int64_t need = lsa::build_workspace_bytes(n, h_kv, r, b, L);
    if (ws_bytes < need || (!ws && need > 0)) return LSA_ENOSPC;
    *desc = D;
    hipError_t e = lsa::build_index(K, dtype, n, h_kv, d, W, r, b, L, iters, (char *)index, D.centroid_off,
                                    D.count_off, D.leaf_off_off, D.perm_off, ws, (hipStream_t)stream);
    return e == hipSuccess ? LSA_OK : LSA_EHIP;
}

int lsa_index_insert_workspace_bytes(int64_t m, const lsa_index_desc *desc, int64_t *bytes) {
    int rc = check_desc(desc);
    if (rc != LSA_OK) return rc;
    if (m < 1 || !bytes) return LSA_EINVAL;
    if (m > 4096) return LSA_EUNSUPPORTED;
    *bytes = lsa::insert_workspace_bytes(m, desc->n, desc->h_kv, desc->r, desc->L, desc->nodes[desc->L]);
    return LSA_OK;
}

int lsa_index_insert(const void *K_new, int dtype, int64_t m, int d, const float *W, lsa_index_desc *desc,
                     void *index, int64_t index_bytes, void *ws, int64_t ws_bytes, void *stream) {
    int rc = check_desc(desc);
    if (rc != LSA_OK) return rc;
    if (m < 1 || d < 1) return LSA_EINVAL;
    if (!dtype_ok(dtype)) return LSA_EUNSUPPORTED;
    if (m > 4096 || d > 256) return LSA_EUNSUPPORTED;
    if (desc->n + m > INT32_MAX) return LSA_EUNSUPPORTED;
    if (!K_new || !W || !index) return LSA_EINVAL;
    lsa_index_desc grown;
    rc = lsa_index_layout(desc->n + m, desc->h_kv, desc->r, desc->b, desc->L, &grown);
    if (rc != LSA_OK) return rc;
    if (grown.perm_off != desc->perm_off || grown.leaf_off_off != desc->leaf_off_off) return LSA_EINVAL;
    if (index_bytes < grown.bytes) return LSA_ENOSPC;
    const int64_t need = lsa::insert_workspace_bytes(m, desc->n, desc->h_kv, desc->r, desc->L, desc->nodes[desc->L]);
    if (!ws || ws_bytes < need) return LSA_ENOSPC;
    hipError_t e = lsa::index_insert(K_new, dtype, m, d, W, (char *)index, desc->n, desc->h_kv, desc->r, desc->b,
                                     desc->L, desc->nodes, desc->centroid_off, desc->count_off, desc->leaf_off_off,
                                     desc->perm_off, ws, (hipStream_t)stream);
    if (e != hipSuccess) return LSA_EHIP;
    *desc = grown;
    return LSA_OK;
}

int lsa_select_workspace_bytes(int64_t m, int h_q, int d, const lsa_index_desc *desc, int beam, int k,
                               int n_sink, int window, int64_t *bytes) {
    int rc = check_desc(desc);
    if (rc != LSA_OK) return rc;
    if (m < 0 || h_q < 1 || d < 1 || beam < 1 || k < 1 || !bytes) return LSA_EINVAL;
    if (h_q % desc->h_kv != 0) return LSA_EINVAL;
    if ((rc = check_local(k, n_sink, window)) != LSA_OK) return rc;
    if (lsa::decode_path_ok(m, h_q, desc->h_kv, d, desc->r, desc->b, desc->L, beam, k))
        *bytes = lsa::decode_workspace_bytes(m, h_q, desc->h_kv, d, desc->L, beam, k);
    else if (lsa::nm_shape_ok(desc->r, desc->b, desc->L, beam, d, desc->nodes))
        *bytes = lsa::nm_workspace_bytes(m, desc->h_kv, desc->L, desc->nodes);
    else
        *bytes = 0;
    return LSA_OK;
}

int lsa_select(const void *Q, int dtype, int64_t m, int h_q, int d, const int32_t *q_pos,
               const lsa_index_desc *desc, const void *index, const float *W, int beam, int k, int n_sink,
               int window, int32_t *sel, int32_t *sel_count, float *sel_cutoff, void *ws, int64_t ws_bytes,
               void *stream) {
    int rc = check_desc(desc);
    if (rc != LSA_OK) return rc;
    if (m < 0 || h_q < 1 || d < 1 || beam < 1 || k < 1) return LSA_EINVAL;
    if (h_q % desc->h_kv != 0) return LSA_EINVAL;
    if ((rc = check_local(k, n_sink, window)) != LSA_OK) return rc;
    if (!dtype_ok(dtype)) return LSA_EUNSUPPORTED;
    if (d > 256 || (int64_t)beam * desc->b > 4096 || k > 8192) return LSA_EUNSUPPORTED;
    if (m > INT32_MAX) return LSA_EUNSUPPORTED;
    if (m == 0) return LSA_OK;
    if (!Q || !q_pos || !index || !W || !sel || !sel_count) return LSA_EINVAL;
    if (ws && lsa::decode_path_ok(m, h_q, desc->h_kv, d, desc->r, desc->b, desc->L, beam, k) &&
        ws_bytes >= lsa::decode_workspace_bytes(m, h_q, desc->h_kv, d, desc->L, beam, k)) {
        hipError_t e = lsa::decode(Q, nullptr, nullptr, dtype, m, h_q, desc->h_kv, d, q_pos, (const char *)index,
                                   desc->n, desc->r, desc->b, desc->L, desc->nodes, desc->centroid_off,
                                   desc->count_off, desc->leaf_off_off, desc->perm_off, W, beam, k, n_sink, window,
                                   sel, sel_count, sel_cutoff, 0.0f, nullptr, nullptr, ws, false,
                                   (hipStream_t)stream);
        return e == hipSuccess ? LSA_OK : LSA_EHIP;
    }
    hipError_t e = lsa::select_keys(Q, dtype, m, h_q, d, q_pos, (const char *)index, desc->n, desc->h_kv, desc->r,
                                    desc->b, desc->L, desc->nodes, desc->centroid_off, desc->count_off,
                                    desc->leaf_off_off, desc->perm_off, W, beam, k, n_sink, window, sel, sel_count,
                                    sel_cutoff, ws, ws ? ws_bytes : 0, (hipStream_t)stream);
    return e == hipSuccess ? LSA_OK : LSA_EHIP;
}

int lsa_select_flat_workspace_bytes(int64_t m, int h_q, const lsa_index_desc *desc, int64_t *bytes) {
    int rc = check_desc(desc);
    if (rc != LSA_OK) return rc;
    if (m < 0 || h_q < 1 || !bytes) return LSA_EINVAL;
    if (h_q % desc->h_kv != 0) return LSA_EINVAL;
    *bytes = lsa::flat_workspace_bytes(m, desc->h_kv, desc->r, desc->nodes[desc->L]);
    return LSA_OK;
}

int lsa_select_flat(const void *Q, int dtype, int64_t m, int h_q, int d, const int32_t *q_pos,
                    const lsa_index_desc *desc, const void *index, const float *W, int k, int n_sink, int window,
                    int32_t *sel, int32_t *sel_count, float *sel_cutoff, void *ws, int64_t ws_bytes, void *stream) {
    int rc = check_desc(desc);
    if (rc != LSA_OK) return rc;
    if (m < 0 || h_q < 1 || d < 1 || k < 1) return LSA_EINVAL;
    if (h_q % desc->h_kv != 0) return LSA_EINVAL;
    if ((rc = check_local(k, n_sink, window)) != LSA_OK) return rc;
    if (!dtype_ok(dtype)) return LSA_EUNSUPPORTED;
    if (d > 256 || k > 8192 || m > INT32_MAX) return LSA_EUNSUPPORTED;
    if (m == 0) return LSA_OK;
    if (!Q || !q_pos || !index || !W || !sel || !sel_count) return LSA_EINVAL;
    const int64_t nleaf = desc->nodes[desc->L];
    if (!ws || lsa::flat_batch_rows(m, desc->h_kv, desc->r, nleaf, ws_bytes) < 1) return LSA_ENOSPC;
    hipError_t e = lsa::select_flat(Q, dtype, m, h_q, d, q_pos, (const char *)index, desc->n, desc->h_kv, desc->r,
                                    nleaf, desc->centroid_off[desc->L], desc->count_off[desc->L],
                                    desc->leaf_off_off, desc->perm_off, W, k, n_sink, window, sel, sel_count,
                                    sel_cutoff, ws, ws_bytes, (hipStream_t)stream);
    if (e == hipSuccess) e = lsa::ws_clear_polled(ws, ws_bytes, (hipStream_t)stream);
    return e == hipSuccess ? LSA_OK : LSA_EHIP;
}

int lsa_pca_workspace_bytes(int64_t n, int h_kv, int d, int64_t *bytes) {
    if (n < 1 || h_kv < 1 || d < 2 || !bytes) return LSA_EINVAL;
    if (d > 128) return LSA_EUNSUPPORTED;
    *bytes = lsa::pca_workspace_bytes(n, h_kv);
    return LSA_OK;
}

int lsa_pca_projection(const void *K, int dtype, int64_t n, int h_kv, int d, int r, float *W, double *eigenvalues,
                       void *ws, int64_t ws_bytes, void *stream) {
    if (n < 1 || n > INT32_MAX || h_kv < 1 || d < 2 || r < 1 || r > d) return LSA_EINVAL;
    if (!dtype_ok(dtype)) return LSA_EUNSUPPORTED;
    if (d > 128) return LSA_EUNSUPPORTED;
    if (!K || !W) return LSA_EINVAL;
    if (!ws || ws_bytes < lsa::pca_workspace_bytes(n, h_kv)) return LSA_ENOSPC;
    hipError_t e = lsa::pca_projection(K, dtype, n, h_kv, d, r, W, eigenvalues, ws, (hipStream_t)stream);
    return e == hipSuccess ? LSA_OK : LSA_EHIP;
}

int lsa_attend_workspace_bytes(int64_t m, int h_q, int h_kv, int d, int k, int64_t *bytes) {
    if (m < 0 || h_q < 1 || h_kv < 1 || d < 1 || k < 1 || !bytes) return LSA_EINVAL;
    if (h_q % h_kv != 0) return LSA_EINVAL;
    *bytes = lsa::attend_workspace_bytes(m, h_q, h_kv, d, k);
    return LSA_OK;
}

int lsa_attend(const void *Q, const void *K, const void *V, int dtype, int64_t m, int h_q, int h_kv, int64_t n, int d,
               const int32_t *sel, const int32_t *sel_count, int k, float scale, void *out, float *lse, void *ws,
               int64_t ws_bytes, void *stream) {
    if (m < 0 || h_q < 1 || h_kv < 1 || n < 1 || n > INT32_MAX || d < 1 || k < 1) return LSA_EINVAL;
    if (h_q % h_kv != 0) return LSA_EINVAL;
    if (!dtype_ok(dtype)) return LSA_EUNSUPPORTED;
    if (h_q / h_kv > 16 || d < 8 || d > 256 || d % 8 != 0 || k > kMaxRow) return LSA_EUNSUPPORTED;
    if (!(scale >= 0.0f) || isinf(scale)) return LSA_EINVAL;
    if (m == 0) return LSA_OK;
    if (!Q || !K || !V || !sel || !sel_count || !out) return LSA_EINVAL;
    const int64_t need = lsa::attend_workspace_bytes(m, h_q, h_kv, d, k);
    if (ws_bytes < need || (!ws && need > 0)) return LSA_ENOSPC;
    if (scale == 0.0f) scale = 1.0f / sqrtf((float)d);
    hipError_t e = lsa::attend(Q, K, V, dtype, m, h_q, h_kv, n, d, sel, sel_count, k, scale, out, lse, ws,
                               (hipStream_t)stream);
    if (e == hipSuccess && need > 0) e = lsa::ws_clear_polled(ws, ws_bytes, (hipStream_t)stream);
    return e == hipSuccess ? LSA_OK : LSA_EHIP;
}

int lsa_select_attend_workspace_bytes(int64_t m, int h_q, int d, const lsa_index_desc *desc, int beam, int k,
                                      int n_sink, int window, int64_t *bytes) {
    int rc = check_desc(desc);
    if (rc != LSA_OK) return rc;
    if (m < 0 || h_q < 1 || d < 1 || beam < 1 || k < 1 || !bytes) return LSA_EINVAL;
    if (h_q % desc->h_kv != 0) return LSA_EINVAL;
    if ((rc = check_local(k, n_sink, window)) != LSA_OK) return rc;
    if (lsa::decode_path_ok(m, h_q, desc->h_kv, d, desc->r, desc->b, desc->L, beam, k))
        *bytes = lsa::decode_workspace_bytes(m, h_q, desc->h_kv, d, desc->L, beam, k);
    else
        *bytes = lsa::attend_workspace_bytes(m, h_q, desc->h_kv, d, k + n_sink + window);
    return LSA_OK;
}

int lsa_select_attend(const void *Q, const void *K, const void *V, int dtype, int64_t m, int h_q, int d,
                      const int32_t *q_pos, const lsa_index_desc *desc, const void *index, const float *W, int beam,
                      int k, int n_sink, int window, float scale, int32_t *sel, int32_t *sel_count, float *sel_cutoff,
                      void *out, float *lse, void *ws, int64_t ws_bytes, void *stream) {
    int rc = check_desc(desc);
    if (rc != LSA_OK) return rc;
    if (m < 0 || h_q < 1 || d < 1 || beam < 1 || k < 1) return LSA_EINVAL;
    if (h_q % desc->h_kv != 0) return LSA_EINVAL;
    if ((rc = check_local(k, n_sink, window)) != LSA_OK) return rc;
    if (!dtype_ok(dtype)) return LSA_EUNSUPPORTED;
    if (d > 256 || (int64_t)beam * desc->b > 4096 || k > 8192) return LSA_EUNSUPPORTED;
    if (h_q / desc->h_kv > 16 || d < 8 || d % 8 != 0) return LSA_EUNSUPPORTED;
    if (!(scale >= 0.0f) || isinf(scale)) return LSA_EINVAL;
    if (m > INT32_MAX) return LSA_EUNSUPPORTED;
    if (m == 0) return LSA_OK;
    if (!Q || !K || !V || !q_pos || !index || !W || !sel || !sel_count || !out) return LSA_EINVAL;
    int64_t need = 0;
    rc = lsa_select_attend_workspace_bytes(m, h_q, d, desc, beam, k, n_sink, window, &need);
    if (rc != LSA_OK) return rc;
    if (ws_bytes < need || (!ws && need > 0)) return LSA_ENOSPC;
    if (scale == 0.0f) scale = 1.0f / sqrtf((float)d);
    hipError_t e;
    if (lsa::decode_path_ok(m, h_q, desc->h_kv, d, desc->r, desc->b, desc->L, beam, k)) {
        e = lsa::decode(Q, K, V, dtype, m, h_q, desc->h_kv, d, q_pos, (const char *)index, desc->n, desc->r,
                        desc->b, desc->L, desc->nodes, desc->centroid_off, desc->count_off, desc->leaf_off_off,
                        desc->perm_off, W, beam, k, n_sink, window, sel, sel_count, sel_cutoff, scale, out, lse,
                        ws, true, (hipStream_t)stream);
    } else {
        e = lsa::select_keys(Q, dtype, m, h_q, d, q_pos, (const char *)index, desc->n, desc->h_kv, desc->r,
                             desc->b, desc->L, desc->nodes, desc->centroid_off, desc->count_off, desc->leaf_off_off,
                             desc->perm_off, W, beam, k, n_sink, window, sel, sel_count, sel_cutoff, nullptr, 0,
                             (hipStream_t)stream);
        if (e == hipSuccess)
            e = lsa::attend(Q, K, V, dtype, m, h_q, desc->h_kv, desc->n, d, sel, sel_count, k + n_sink + window,
                            scale, out, lse, ws, (hipStream_t)stream);
        // the attention's partial states sit where a later one-launch call polls
        if (e == hipSuccess) e = lsa::ws_clear_polled(ws, ws_bytes, (hipStream_t)stream);
    }
    return e == hipSuccess ? LSA_OK : LSA_EHIP;
}

}  // extern "C"
