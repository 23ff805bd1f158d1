// Host-side entry points of the kernel files, used by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lsa.h"

namespace lsa {

// Every workspace starts with a header whose first int32 is the status word
// (LSA_STATUS_* bits set by kernels, read and cleared by the host).
constexpr int kWsHeader = 256;
constexpr int32_t kStatusWaitTimeout = LSA_STATUS_WAIT_TIMEOUT;

int device_cus();

int64_t build_workspace_bytes(int64_t n, int h, int r, int b, int L);
hipError_t build_index(const void *K, int dtype, int64_t n, int h, int d, const float *W, int r, int b, int L,
                       int iters, char *index, const int64_t *centroid_off, const int64_t *count_off,
                       int64_t leaf_off_off, int64_t perm_off, void *ws, hipStream_t st);

int64_t insert_workspace_bytes(int64_t m, int64_t n, int h, int r, int L, int64_t nleaf);
hipError_t index_insert(const void *K_new, int dtype, int64_t m, int d, const float *W, char *index, int64_t n, int h,
                        int r, int b, int L, const int64_t *nodes, const int64_t *centroid_off,
                        const int64_t *count_off, int64_t leaf_off_off, int64_t perm_off, void *ws, hipStream_t st);

hipError_t select_keys(const void *Q, int dtype, int64_t m, int h_q, int d, const int32_t *q_pos, const char *index,
                       int64_t n, int h_kv, int r, int b, int L, const int64_t *nodes, const int64_t *centroid_off,
                       const int64_t *count_off, int64_t leaf_off_off, int64_t perm_off, const float *W, int beam,
                       int k, int n_sink, int window, int32_t *sel, int32_t *sel_count, float *sel_cutoff,
                       void *ws, int64_t ws_bytes, hipStream_t st);
bool nm_shape_ok(int r, int b, int L, int beam, int d, const int64_t *nodes);
int64_t nm_workspace_bytes(int64_t m, int h_kv, int L, const int64_t *nodes);

// node-major attention (nm_attend.hip), run after each batch of node-major
// selection when select and attention are called together
struct NmaWs { int32_t *ppos, *toff, *coff, *wr, *tdesc; char *pinf, *po; float *pml; size_t bytes; };
struct NmaBatch {
    const void *Q, *K, *V;
    const int32_t *q_pos;
    int64_t row0, groups;
    int h_q, h_kv;
    int64_t n;
    int b;
    int64_t nodes_prev, nleaf;
    const int32_t *leaf_off, *perm;
    int n_sink, window;
    const int32_t *pairs, *noff, *keep;
    NmaWs ws;
    float scale;
    void *out;
    float *lse;
};
bool nma_shape_ok(int dtype, int d, int G, int n_sink, int window);
NmaWs carve_nma_ws(char *base, int64_t groups, int G, int64_t nbins);
hipError_t nm_attend_batch(const NmaBatch &B, hipStream_t st);
int64_t nm_attend_workspace_bytes(int64_t m, int h_q, int h_kv, int L, const int64_t *nodes);
bool nm_attend_fits(int64_t m, int h_q, int h_kv, int L, const int64_t *nodes, int64_t ws_bytes);
hipError_t select_attend_nm(const void *Q, const void *K, const void *V, int dtype, int64_t m, int h_q, int d,
                            const int32_t *q_pos, const char *index, int64_t n, int h_kv, int r, int b, int L,
                            const int64_t *nodes, const int64_t *centroid_off, const int64_t *count_off,
                            int64_t leaf_off_off, int64_t perm_off, const float *W, int beam, int k, int n_sink,
                            int window, int32_t *sel, int32_t *sel_count, float *sel_cutoff, float scale, void *out,
                            float *lse, void *ws, int64_t ws_bytes, hipStream_t st);

int attend_nsplit(int64_t m, int h_kv, int k);
int64_t attend_workspace_bytes(int64_t m, int h_q, int h_kv, int d, int k);
hipError_t attend(const void *Q, const void *K, const void *V, int dtype, int64_t m, int h_q, int h_kv, int64_t n,
                  int d, const int32_t *sel, const int32_t *sel_count, int k, float scale, void *out, float *lse,
                  void *ws, hipStream_t st);

int64_t flat_workspace_bytes(int64_t m, int h_kv, int r, int64_t nleaf);
int64_t flat_batch_rows(int64_t m, int h_kv, int r, int64_t nleaf, int64_t ws_bytes);
hipError_t select_flat(const void *Q, int dtype, int64_t m, int h_q, int d, const int32_t *q_pos, const char *index,
                       int64_t n, int h_kv, int r, int64_t nleaf, int64_t leaf_c_off, int64_t leaf_cnt_off,
                       int64_t leaf_off_off, int64_t perm_off, const float *W, int k, int n_sink, int window,
                       int32_t *sel, int32_t *sel_count, float *sel_cutoff, void *ws, int64_t ws_bytes,
                       hipStream_t st);

int64_t pca_workspace_bytes(int64_t n, int h);
hipError_t pca_projection(const void *K, int dtype, int64_t n, int h, int d, int r, float *W, double *evals, void *ws,
                          hipStream_t st);

bool decode_path_ok(int64_t m, int h_q, int h_kv, int d, int r, int b, int L, int beam, int k);
int64_t decode_workspace_bytes(int64_t m, int h_q, int h_kv, int d, int L, int beam, int k);
int64_t decode_polled_bytes_bound();
int64_t ws_reserved_bytes();
int64_t scratch_bytes();
hipError_t scratch_ptr(void **out, hipStream_t st);
hipError_t decode(const void *Q, const void *K, const void *V, int dtype, int64_t m, int h_q, int h_kv, int d,
                  const int32_t *q_pos, const char *index, int64_t n, int r, int b, int L, const int64_t *nodes,
                  const int64_t *centroid_off, const int64_t *count_off, int64_t leaf_off_off, int64_t perm_off,
                  const float *W, int beam, int k, int n_sink, int window, int32_t *sel, int32_t *sel_count,
                  float *sel_cutoff, float scale, void *out, float *lse, void *ws, bool attend, hipStream_t st);

}  // namespace lsa
