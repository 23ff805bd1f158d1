// C ABI of the LSA layer: argument checks, index layout, dispatch, index
// export / import with a host-side check of the tree, and debug mode.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <vector>

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

// lsa_select_attend's node-major form (selection grouped by kept node, each
// node's keys attended once per tile of rows) applies to these shapes with
// bf16 inputs
inline bool nm_attend_shape(int d, int h_q, const lsa_index_desc *desc, int beam, int n_sink, int window) {
    return lsa::nm_shape_ok(desc->r, desc->b, desc->L, beam, d, desc->nodes) &&
           lsa::nma_shape_ok(LSA_BF16, d, h_q / desc->h_kv, n_sink, window);
}

// ---------------------------------------------------------------- index check
// The tree held in host memory `h` in the layout D: the properties every
// select kernel relies on to stay inside its buffers ("How LSA Sidesteps
// Per-Key Scoring with Hierarchical Clustering", kongchang.com: the root
// holds every key and each level splits its parent's keys among children).
int check_index_host(const lsa_index_desc &D, const char *h) {
    const int64_t n = D.n;
    const int H = D.h_kv, r = D.r, b = D.b, L = D.L;
    const int64_t nleaf = D.nodes[L];
    std::vector<uint8_t> seen((size_t)n);
    for (int g = 0; g < H; ++g) {
        const int32_t *lo = (const int32_t *)(h + D.leaf_off_off) + (size_t)g * (nleaf + 1);
        const int32_t *perm = (const int32_t *)(h + D.perm_off) + (size_t)g * n;
        if (lo[0] != 0 || lo[nleaf] != n) return LSA_EINVAL;
        const int32_t *cl = (const int32_t *)(h + D.count_off[L]) + (size_t)g * nleaf;
        for (int64_t v = 0; v < nleaf; ++v)
            if (lo[v + 1] < lo[v] || cl[v] != lo[v + 1] - lo[v]) return LSA_EINVAL;
        for (int l = L - 1; l >= 1; --l) {
            const int32_t *c = (const int32_t *)(h + D.count_off[l]) + (size_t)g * D.nodes[l];
            const int32_t *ch = (const int32_t *)(h + D.count_off[l + 1]) + (size_t)g * D.nodes[l + 1];
            for (int64_t v = 0; v < D.nodes[l]; ++v) {
                int64_t s = 0;
                for (int c2 = 0; c2 < b; ++c2) s += ch[v * b + c2];
                if (s != c[v]) return LSA_EINVAL;
            }
        }
        memset(seen.data(), 0, (size_t)n);
        for (int64_t v = 0; v < nleaf; ++v)
            for (int64_t j = lo[v]; j < lo[v + 1]; ++j) {
                const int32_t key = perm[j];
                if (key < 0 || key >= n || seen[(size_t)key]) return LSA_EINVAL;
                if (j > lo[v] && key <= perm[j - 1]) return LSA_EINVAL;
                seen[(size_t)key] = 1;
            }
        for (int l = 1; l <= L; ++l) {
            const int32_t *c = (const int32_t *)(h + D.count_off[l]) + (size_t)g * D.nodes[l];
            const float *C = (const float *)(h + D.centroid_off[l]) + (size_t)g * D.nodes[l] * r;
            for (int64_t v = 0; v < D.nodes[l]; ++v) {
                if (c[v] == 0) continue;
                for (int x = 0; x < r; ++x)
                    if (!isfinite(C[v * r + x])) return LSA_EINVAL;
            }
        }
    }
    return LSA_OK;
}

// ---------------------------------------------------------------- debug mode
bool debug_mode() {
    static const bool on = [] {
        const char *e = getenv("LSA_DEBUG");
        return e && *e && strcmp(e, "0") != 0;
    }();
    return on;
}

// Debug mode, before a select call: the index it reads passes the import check.
int debug_check_index(const lsa_index_desc *desc, const void *index, hipStream_t st) {
    std::vector<char> h((size_t)desc->bytes);
    if (hipMemcpyAsync(h.data(), index, (size_t)desc->bytes, hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return LSA_EHIP;
    return check_index_host(*desc, h.data());
}

// Debug mode: counts in [0, row] and the counted entries of sel in [0, n);
// with `padded`, the entries after the count are -1.
int debug_check_sel(const int32_t *sel, const int32_t *sel_count, int64_t groups, int row, int64_t n, bool padded,
                    hipStream_t st) {
    std::vector<int32_t> s((size_t)groups * row), c((size_t)groups);
    if (hipMemcpyAsync(s.data(), sel, sizeof(int32_t) * s.size(), hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipMemcpyAsync(c.data(), sel_count, sizeof(int32_t) * c.size(), hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return LSA_EHIP;
    for (int64_t q = 0; q < groups; ++q) {
        if (c[q] < 0 || c[q] > row) return LSA_EINVAL;
        for (int t = 0; t < row; ++t) {
            const int32_t v = s[(size_t)q * row + t];
            if (t < c[q] ? (v < 0 || v >= n) : (padded && v != -1)) return LSA_EINVAL;
        }
    }
    return LSA_OK;
}

// Reads and clears the status word at ws (synchronous).
int read_status(void *ws, int32_t *status, hipStream_t st) {
    int32_t v = 0;
    if (hipMemcpyAsync(&v, ws, sizeof(v), hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return LSA_EHIP;
    if (v != 0) {
        const int32_t zero = 0;
        if (hipMemcpyAsync(ws, &zero, sizeof(zero), hipMemcpyHostToDevice, st) != hipSuccess ||
            hipStreamSynchronize(st) != hipSuccess)
            return LSA_EHIP;
    }
    *status = v;
    return LSA_OK;
}

// After a call's launches: the launch status, and in debug mode the kernels'
// completion and, when the call ran the multi-workgroup select (the only
// kernels that set it), the workspace's status word (else status_ws = NULL).
int finish(hipError_t e, void *status_ws, hipStream_t st) {
    if (e != hipSuccess) return LSA_EHIP;
    if (!debug_mode()) return LSA_OK;
    if (hipStreamSynchronize(st) != hipSuccess) return LSA_EHIP;
    if (status_ws) {
        int32_t status = 0;
        const int rc = read_status(status_ws, &status, st);
        if (rc != LSA_OK) return rc;
        if (status != 0) return LSA_EDEVICE;
    }
    return LSA_OK;
}

// Debug mode, after a select call: finish(), then its outputs are in range.
int finish_select(hipError_t e, void *status_ws, const int32_t *sel, const int32_t *sel_count, int64_t groups,
                  int row, int64_t n, hipStream_t st) {
    int rc = finish(e, status_ws, st);
    if (rc != LSA_OK || !debug_mode()) return rc;
    rc = debug_check_sel(sel, sel_count, groups, row, n, true, st);
    return rc == LSA_EINVAL ? LSA_EDEVICE : rc;
}

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
        case LSA_EDEVICE: return "a kernel reported a failure on the device";
        case LSA_ESCRATCH: return "the call needs more than the library's fixed scratch";
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

int lsa_index_export(const lsa_index_desc *desc, const void *index, void *host_dst, int64_t dst_bytes,
                     void *stream) {
    int rc = check_desc(desc);
    if (rc != LSA_OK) return rc;
    if (!index || !host_dst) return LSA_EINVAL;
    if (dst_bytes < desc->bytes) return LSA_ENOSPC;
    hipStream_t st = (hipStream_t)stream;
    if (hipMemcpyAsync(host_dst, index, (size_t)desc->bytes, hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return LSA_EHIP;
    return LSA_OK;
}

int lsa_index_import(const lsa_index_desc *desc, const void *host_src, int64_t src_bytes, void *index,
                     int64_t index_bytes, void *stream) {
    int rc = check_desc(desc);
    if (rc != LSA_OK) return rc;
    if (!index || !host_src) return LSA_EINVAL;
    if (src_bytes < desc->bytes || index_bytes < desc->bytes) return LSA_ENOSPC;
    if ((rc = check_index_host(*desc, (const char *)host_src)) != LSA_OK) return rc;
    hipStream_t st = (hipStream_t)stream;
    if (hipMemcpyAsync(index, host_src, (size_t)desc->bytes, hipMemcpyHostToDevice, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return LSA_EHIP;
    return LSA_OK;
}

int lsa_workspace_status(void *ws, int64_t ws_bytes, int32_t *status, void *stream) {
    if (!status) return LSA_EINVAL;
    hipStream_t st = (hipStream_t)stream;
    if (!ws) {
        // the scratch of lsa_select_attend_noalloc on the current device
        if (lsa::scratch_ptr(&ws, st) != hipSuccess) return LSA_EHIP;
    } else if (ws_bytes < lsa::kWsHeader) {
        return LSA_EINVAL;
    }
    return read_status(ws, status, st);
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
    return finish(e, nullptr, (hipStream_t)stream);
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
    if ((rc = finish(e, nullptr, (hipStream_t)stream)) != LSA_OK) return rc;
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
    hipStream_t st = (hipStream_t)stream;
    if (debug_mode() && (rc = debug_check_index(desc, index, st)) != LSA_OK) return rc;
    const int row = k + n_sink + window;
    if (ws && lsa::decode_path_ok(m, h_q, desc->h_kv, d, desc->r, desc->b, desc->L, beam, k) &&
        ws_bytes >= lsa::decode_workspace_bytes(m, h_q, desc->h_kv, d, desc->L, beam, k)) {
        hipError_t e = lsa::decode(Q, nullptr, nullptr, dtype, m, h_q, desc->h_kv, d, q_pos, (const char *)index,
                                   desc->n, desc->r, desc->b, desc->L, desc->nodes, desc->centroid_off,
                                   desc->count_off, desc->leaf_off_off, desc->perm_off, W, beam, k, n_sink, window,
                                   sel, sel_count, sel_cutoff, 0.0f, nullptr, nullptr, ws, false, st);
        return finish_select(e, ws, sel, sel_count, m * desc->h_kv, row, desc->n, st);
    }
    hipError_t e = lsa::select_keys(Q, dtype, m, h_q, d, q_pos, (const char *)index, desc->n, desc->h_kv, desc->r,
                                    desc->b, desc->L, desc->nodes, desc->centroid_off, desc->count_off,
                                    desc->leaf_off_off, desc->perm_off, W, beam, k, n_sink, window, sel, sel_count,
                                    sel_cutoff, ws, ws ? ws_bytes : 0, st);
    return finish_select(e, nullptr, sel, sel_count, m * desc->h_kv, row, desc->n, st);
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
    hipStream_t st = (hipStream_t)stream;
    if (debug_mode() && (rc = debug_check_index(desc, index, st)) != LSA_OK) return rc;
    hipError_t e = lsa::select_flat(Q, dtype, m, h_q, d, q_pos, (const char *)index, desc->n, desc->h_kv, desc->r,
                                    nleaf, desc->centroid_off[desc->L], desc->count_off[desc->L],
                                    desc->leaf_off_off, desc->perm_off, W, k, n_sink, window, sel, sel_count,
                                    sel_cutoff, ws, ws_bytes, st);
    return finish_select(e, nullptr, sel, sel_count, m * desc->h_kv, k + n_sink + window, desc->n, st);
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
    return finish(e, nullptr, (hipStream_t)stream);
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
    int rc;
    const int64_t need = lsa::attend_workspace_bytes(m, h_q, h_kv, d, k);
    if (ws_bytes < need || (!ws && need > 0)) return LSA_ENOSPC;
    if (scale == 0.0f) scale = 1.0f / sqrtf((float)d);
    hipStream_t st = (hipStream_t)stream;
    if (debug_mode() && (rc = debug_check_sel(sel, sel_count, m * h_kv, k, n, false, st)) != LSA_OK) return rc;
    hipError_t e = lsa::attend(Q, K, V, dtype, m, h_q, h_kv, n, d, sel, sel_count, k, scale, out, lse, ws, st);
    return finish(e, nullptr, st);
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
    else if (nm_attend_shape(d, h_q, desc, beam, n_sink, window))
        // sized for the node-major form (bf16 inputs); fp32 inputs need less
        *bytes = std::max(lsa::nm_attend_workspace_bytes(m, h_q, desc->h_kv, desc->L, desc->nodes),
                          lsa::attend_workspace_bytes(m, h_q, desc->h_kv, d, k + n_sink + window));
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
    // (the node-major form runs when its batches fit ws; below that size the
    // two-step form needs only the attention's workspace)
    const int64_t need = lsa::decode_path_ok(m, h_q, desc->h_kv, d, desc->r, desc->b, desc->L, beam, k)
                             ? lsa::decode_workspace_bytes(m, h_q, desc->h_kv, d, desc->L, beam, k)
                             : lsa::attend_workspace_bytes(m, h_q, desc->h_kv, d, k + n_sink + window);
    if (ws_bytes < need || (!ws && need > 0)) return LSA_ENOSPC;
    if (scale == 0.0f) scale = 1.0f / sqrtf((float)d);
    hipStream_t st = (hipStream_t)stream;
    if (debug_mode() && (rc = debug_check_index(desc, index, st)) != LSA_OK) return rc;
    hipError_t e;
    const bool one_launch = lsa::decode_path_ok(m, h_q, desc->h_kv, d, desc->r, desc->b, desc->L, beam, k);
    if (one_launch) {
        e = lsa::decode(Q, K, V, dtype, m, h_q, desc->h_kv, d, q_pos, (const char *)index, desc->n, desc->r,
                        desc->b, desc->L, desc->nodes, desc->centroid_off, desc->count_off, desc->leaf_off_off,
                        desc->perm_off, W, beam, k, n_sink, window, sel, sel_count, sel_cutoff, scale, out, lse,
                        ws, true, st);
    } else if (ws && lsa::nma_shape_ok(dtype, d, h_q / desc->h_kv, n_sink, window) &&
               lsa::nm_shape_ok(desc->r, desc->b, desc->L, beam, d, desc->nodes) &&
               lsa::nm_attend_fits(m, h_q, desc->h_kv, desc->L, desc->nodes, ws_bytes)) {
        e = lsa::select_attend_nm(Q, K, V, dtype, m, h_q, d, q_pos, (const char *)index, desc->n, desc->h_kv,
                                  desc->r, desc->b, desc->L, desc->nodes, desc->centroid_off, desc->count_off,
                                  desc->leaf_off_off, desc->perm_off, W, beam, k, n_sink, window, sel, sel_count,
                                  sel_cutoff, scale, out, lse, ws, ws_bytes, st);
    } else {
        e = lsa::select_keys(Q, dtype, m, h_q, d, q_pos, (const char *)index, desc->n, desc->h_kv, desc->r,
                             desc->b, desc->L, desc->nodes, desc->centroid_off, desc->count_off, desc->leaf_off_off,
                             desc->perm_off, W, beam, k, n_sink, window, sel, sel_count, sel_cutoff, nullptr, 0, st);
        if (e == hipSuccess)
            e = lsa::attend(Q, K, V, dtype, m, h_q, desc->h_kv, desc->n, d, sel, sel_count, k + n_sink + window,
                            scale, out, lse, ws, st);
    }
    return finish_select(e, one_launch ? ws : nullptr, sel, sel_count, m * desc->h_kv, k + n_sink + window, desc->n,
                         st);
}

int lsa_select_attend_noalloc(const void *Q, const void *K, const void *V, int dtype, int64_t m, int h_q, int d,
                              const int32_t *q_pos, const lsa_index_desc *desc, const void *index, const float *W,
                              int beam, int k, int n_sink, int window, float scale, int32_t *sel, int32_t *sel_count,
                              float *sel_cutoff, void *out, float *lse, void *stream) {
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
    if (!lsa::decode_path_ok(m, h_q, desc->h_kv, d, desc->r, desc->b, desc->L, beam, k)) return LSA_EUNSUPPORTED;
    if (lsa::decode_workspace_bytes(m, h_q, desc->h_kv, d, desc->L, beam, k) > lsa::scratch_bytes())
        return LSA_ESCRATCH;
    if (scale == 0.0f) scale = 1.0f / sqrtf((float)d);
    hipStream_t st = (hipStream_t)stream;
    void *ws = nullptr;
    hipError_t e = lsa::scratch_ptr(&ws, st);
    if (e == hipSuccess)
        e = lsa::decode(Q, K, V, dtype, m, h_q, desc->h_kv, d, q_pos, (const char *)index, desc->n, desc->r,
                        desc->b, desc->L, desc->nodes, desc->centroid_off, desc->count_off, desc->leaf_off_off,
                        desc->perm_off, W, beam, k, n_sink, window, sel, sel_count, sel_cutoff, scale, out, lse,
                        ws, true, st);
    // (debug mode: the stream is synchronised and the status word read, with
    // no host-side copies of the index or of sel)
    return finish(e, ws, st);
}

}  // extern "C"
