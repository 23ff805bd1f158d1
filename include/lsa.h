/*
 * lsa.h - C ABI of the latent-sparse-attention (LSA) layer for AMD Instinct
 * MI355X (gfx950).
 *
 * The layer follows the pages that describe the method:
 *   - "Latent Sparse Attention Breaks Through the Million-Token Context
 *     Bottleneck" (kongchang.com), section "How LSA Sidesteps Per-Key Scoring
 *     with Hierarchical Clustering": keys are mapped into a learned latent
 *     space and clustered top-down into a tree; a query scores a few clusters
 *     per level from the root and descends the best branches to the leaves.
 *   - "Latent sparse attention" (bdtechtalks.com), section "How latent sparse
 *     attention works": each cluster keeps a centroid and references to its
 *     keys; a fixed search budget per level; a fixed number of original keys
 *     is retrieved from the chosen clusters and attention runs over them.
 *   - kongchang.com, section "The Accuracy-Efficiency Dilemma of Sparse
 *     Attention": sparse attention lets each query interact with k keys.
 *
 * Conventions shared by every entry point
 *   - All pointers named as device buffers are device memory on the current
 *     HIP device; the caller owns every buffer.  The library allocates no
 *     memory and keeps no state between calls, except the fixed scratch of
 *     lsa_select_attend_noalloc (4 MiB per device that calls it, kept until
 *     the process ends).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every call only enqueues work on that stream and returns; results are
 *     ready once the stream reaches that point.
 *   - Arguments are checked on the host before anything is enqueued.  A call
 *     that returns an error has enqueued nothing, except LSA_EHIP, which
 *     reports a failed launch (the stream's earlier work is unaffected).
 *   - Layout: row-major, innermost dimension last, no padding.  "bf16" is
 *     IEEE-754 binary32 truncated to its upper 16 bits (bfloat16).
 *   - Positions are int32: n <= 2^31 - 1 keys.
 *   - Results are deterministic: the same inputs give the same bytes.
 *   - Failures on the device.  The only kernels that wait on other
 *     workgroups (the multi-workgroup select of lsa_select and
 *     lsa_select_attend) bound every wait; a wait that gives up sets
 *     LSA_STATUS_WAIT_TIMEOUT in the status word of the call's workspace
 *     (its results may then be wrong, and the workspace must be zero-filled
 *     again before its next use), which lsa_workspace_status reads.
 *   - Debug mode: with the environment variable LSA_DEBUG set to a value
 *     other than "0" when the library is first used, every entry point also
 *     checks on the host, before enqueueing, the index it reads (as
 *     lsa_index_import does) and the sel / sel_count it reads (entries in
 *     range); and after enqueueing it waits for the stream, returns LSA_EHIP
 *     for a failed kernel, LSA_EDEVICE when a multi-workgroup select set the
 *     workspace's status word (it is cleared) or when a select call wrote an
 *     entry out of range.
 *     Debug mode synchronises and copies to the host: it is for finding
 *     faults, not for timing, and not for use under stream capture.
 */
#ifndef LSA_H
#define LSA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define LSA_OK 0
#define LSA_EINVAL (-1)       /* a shape, size or pointer argument is invalid       */
#define LSA_EUNSUPPORTED (-2) /* valid, but outside what the kernels implement      */
#define LSA_ENOSPC (-3)       /* a caller-provided buffer is too small              */
#define LSA_EHIP (-4)         /* the HIP runtime reported an error on launch        */
#define LSA_EDEVICE (-5)      /* a kernel reported a failure (debug mode, lsa_workspace_status) */
#define LSA_ESCRATCH (-6)     /* the call needs more than the fixed scratch of lsa_select_attend_noalloc */

/* Bits of a workspace's status word (lsa_workspace_status). */
#define LSA_STATUS_WAIT_TIMEOUT 1 /* a bounded wait between workgroups gave up */

/* Element types of Q, K, V and the attention output. */
#define LSA_F32 0
#define LSA_BF16 1

#define LSA_MAX_LEVELS 6

/*
 * Index descriptor: where each array of the tree lives inside one caller-owned
 * device buffer ("index memory").  Plain data; filled by lsa_index_layout.
 *
 * The tree is a complete b-ary tree with L levels below the root (the root
 * holds all keys; level l has b^l nodes; the children of node v are
 * v*b + c, c = 0..b-1; nodes may be empty).  For each KV head g:
 *   centroids of level l : float [h_kv][b^l][r]   at byte offset centroid_off[l]
 *   member counts level l: int32 [h_kv][b^l]      at byte offset count_off[l]
 *   leaf CSR offsets     : int32 [h_kv][b^L + 1]  at byte offset leaf_off_off
 *   leaf members (keys)  : int32 [h_kv][n]        at byte offset perm_off
 * Leaf v of head g holds keys perm[g][leaf_off[g][v] .. leaf_off[g][v+1]) in
 * ascending position.  A node with count 0 is empty.  Entries at index 0 of
 * centroid_off/count_off are unused.
 */
typedef struct lsa_index_desc {
    int64_t n;
    int32_t h_kv, r, b, L;
    int64_t nodes[LSA_MAX_LEVELS + 1];
    int64_t centroid_off[LSA_MAX_LEVELS + 1];
    int64_t count_off[LSA_MAX_LEVELS + 1];
    int64_t leaf_off_off;
    int64_t perm_off;
    int64_t bytes;
} lsa_index_desc;

/* Version of this ABI (the value of LSA_ABI_VERSION). */
#define LSA_ABI_VERSION 2
int lsa_abi_version(void);

/* Message for a return code (static storage, never NULL). */
const char *lsa_strerror(int code);

/*
 * Fill *desc with the layout of an index for n keys, h_kv KV heads, latent
 * dimension r, branching b and L levels.  Host only; touches no device.
 * Limits: 1 <= n <= 2^31-1, 1 <= h_kv, 1 <= r <= 64, 2 <= b <= 64,
 * 1 <= L <= LSA_MAX_LEVELS, b^L <= 2^31 - 2.  Arrays start on 256-byte
 * boundaries.
 */
int lsa_index_layout(int64_t n, int h_kv, int r, int b, int L, lsa_index_desc *desc);

/*
 * Copy an index to host memory (kongchang.com, "How LSA Sidesteps Per-Key
 * Scoring with Hierarchical Clustering": the tree over the keys is
 * precomputed, so it can be stored and loaded like the KV cache).
 *
 *   desc      the index's descriptor (as lsa_index_layout returns it)
 *   index     device, desc->bytes bytes
 *   host_dst  host, dst_bytes >= desc->bytes: receives the index memory byte
 *             for byte, in the layout *desc describes (bytes between arrays
 *             are unspecified)
 * Synchronous: the copy is enqueued on `stream` after its earlier work and
 * the call returns once it is complete.  Errors: LSA_EINVAL (descriptor,
 * NULL pointer), LSA_ENOSPC (dst_bytes too small), LSA_EHIP (copy failed).
 */
int lsa_index_export(const lsa_index_desc *desc, const void *index, void *host_dst, int64_t dst_bytes,
                     void *stream);

/*
 * Load an index from host memory into index memory (the inverse of
 * lsa_index_export).  host_src holds src_bytes >= desc->bytes bytes in the
 * layout *desc describes: written by lsa_index_export, or assembled by any
 * other implementation of the same tree (same arrays, same meaning).  Before
 * anything is copied the contents are checked on the host, and an index that
 * fails a check returns LSA_EINVAL with `index` untouched.  Per KV head:
 *   - leaf offsets start at 0, never decrease and end at n;
 *   - a leaf's count equals its offset difference, an internal node's count
 *     the sum of its children's counts;
 *   - the members are a permutation of 0..n-1, strictly ascending inside
 *     each leaf;
 *   - the centroid of every non-empty node is finite.
 * These are what the select kernels rely on to stay inside their buffers.
 *   index     device, index_bytes >= desc->bytes
 * Synchronous, like lsa_index_export.  Errors: LSA_EINVAL, LSA_ENOSPC,
 * LSA_EHIP.
 */
int lsa_index_import(const lsa_index_desc *desc, const void *host_src, int64_t src_bytes, void *index,
                     int64_t index_bytes, void *stream);

/*
 * Read and clear the status word of a zero-filled workspace used by
 * lsa_select or lsa_select_attend (*status: the LSA_STATUS_* bits that every
 * call since the last read set, 0 when all went well; only their
 * multi-workgroup form sets any).  With ws = NULL it reads the scratch of
 * lsa_select_attend_noalloc on the current device.  Synchronous: waits for
 * `stream` first, so it sees every call enqueued on that stream before it.
 * Errors: LSA_EINVAL (NULL status, ws_bytes < 256 with ws non-NULL), LSA_EHIP.
 */
int lsa_workspace_status(void *ws, int64_t ws_bytes, int32_t *status, void *stream);

/*
 * Bytes of device workspace lsa_build_index needs for these sizes (*bytes).
 */
int lsa_build_workspace_bytes(int64_t n, int h_kv, int d, int r, int b, int L, int64_t *bytes);

/*
 * Build the cluster tree of every KV head (kongchang.com, "How LSA Sidesteps
 * ...": the tree over latent keys is precomputed; bdtechtalks.com, "How latent
 * sparse attention works": centroid plus key references per cluster).
 *
 *   K        device, [h_kv][n][d] of `dtype` (LSA_F32 or LSA_BF16)
 *   W        device, float [h_kv][d][r]: the latent projection of each KV head
 *   iters    Lloyd rounds per level (>= 1)
 *   index    device, desc->bytes bytes, written completely
 *   ws       device workspace of lsa_build_workspace_bytes bytes
 *   desc     out (host): the layout, as lsa_index_layout returns it
 *
 * Per head: z_j = fl32(K_j . W) (latent keys); for l = 1..L, every node of
 * level l-1 splits its members into b children by `iters` rounds of k-means:
 * a = min(b, m) children are seeded with the members of rank floor(c*m/a) in
 * ascending key order, each round assigns every member to the nearest seeded
 * child by squared Euclidean distance (ties to the lower child) and replaces
 * each child's centroid by fl32(mean of its members) (a child without members
 * keeps its centroid).  The last round's assignment is the partition.
 * Distances, sums and means are accumulated in double, in ascending dimension
 * and ascending key order, so the tree is bit-identical across runs.
 * Limits as lsa_index_layout, plus 1 <= d <= 256.
 */
int lsa_build_index(const void *K, int dtype, int64_t n, int h_kv, int d, const float *W, int r,
                    int b, int L, int iters, void *index, int64_t index_bytes, void *ws,
                    int64_t ws_bytes, lsa_index_desc *desc, void *stream);

/*
 * Bytes of device workspace lsa_index_insert needs to insert m keys into the
 * index described by *desc (*bytes).
 */
int lsa_index_insert_workspace_bytes(int64_t m, const lsa_index_desc *desc, int64_t *bytes);

/*
 * Insert m keys appended to the cache into a built index, in place
 * (kongchang.com, "How LSA Sidesteps Per-Key Scoring with Hierarchical
 * Clustering": the key index is precomputed and updated).
 *
 *   K_new     device, [h_kv][m][d] of `dtype`: the keys at positions
 *             desc->n .. desc->n + m - 1
 *   W         device, float [h_kv][d][r]: the index's projection
 *   desc      in: the index over n keys; out (on success): over n + m keys
 *   index     device, the index; index_bytes must hold the layout for n + m
 *             keys (lsa_index_layout(n + m, ...).bytes: only the member array
 *             grows, every other array keeps its offset)
 *   ws        device workspace of lsa_index_insert_workspace_bytes bytes
 * The batch is inserted at once: each new key's latent fl32(k . W_g)
 * descends from the root to the nearest non-empty child at every level
 * (squared distance in double, ties to the smaller child) against the
 * centroids as they were before the batch; then every node on a path, with c
 * its old count and S the double sum of its new keys' latents (keys
 * ascending), gets centroid fl32((c * centroid + S) / (c + #new)) and count
 * c + #new; each leaf lists its old members, then its new keys.  One key per
 * batch is the online k-means update.  Results are deterministic.
 * Limits: 1 <= m <= 4096 (insert longer appends in several batches),
 * n + m <= 2^31 - 1, d <= 256.
 */
int lsa_index_insert(const void *K_new, int dtype, int64_t m, int d, const float *W,
                     lsa_index_desc *desc, void *index, int64_t index_bytes, void *ws, int64_t ws_bytes,
                     void *stream);

/*
 * Bytes of device workspace that let lsa_select run its multi-workgroup
 * paths for this batch (*bytes): the decode kernel for small batches; for
 * larger ones with r = 64, b <= 64, beam <= 16, L >= 2 and leaf ids below
 * 2^22, the node-major path, sized for batches of up to 32768 rows; 0 when
 * neither applies (then every (row, KV head) pair runs in one workgroup).
 */
int lsa_select_workspace_bytes(int64_t m, int h_q, int d, const lsa_index_desc *desc, int beam, int k,
                               int n_sink, int window, int64_t *bytes);

/*
 * Select keys for every (query row, KV head) by top-down descent of the tree
 * (kongchang.com, "How LSA Sidesteps ...": score a few candidate clusters per
 * level and descend; bdtechtalks.com, "How latent sparse attention works":
 * fixed budget per level, a fixed number of original keys retrieved;
 * "The compute bottleneck of sparse attention": causal attention sees only
 * earlier tokens).
 *
 *   Q        device, [m][h_q][d] of `dtype`; query head h uses KV head h / (h_q/h_kv)
 *   q_pos    device, int32 [m]: position of each query row (decode: n)
 *   index    device, built by lsa_build_index with *desc
 *   W        device, float [h_kv][d][r]: the same projection as the keys
 *   beam     nodes kept per level at levels 1..L-1 (>= 1)
 *   k        keys retrieved per row and KV head (>= 1)
 *   n_sink   initial sink tokens joined to the retrieved keys (>= 0)
 *   window   recent tokens joined to the retrieved keys (>= 0)
 *   sel      device out, int32 [m][h_kv][k + n_sink + window]: the attention
 *            set of each row and KV head: the retrieved keys in the order
 *            they are retrieved (leaf by leaf, ascending position inside a
 *            leaf), then the sinks and the window in ascending position,
 *            padded with -1
 *   sel_count device out, int32 [m][h_kv]: number of entries before the padding
 *   sel_cutoff device out or NULL, float [m][h_kv]: score of the leaf that
 *            supplied the k-th retrieved key, -inf when fewer than k keys
 *            could be retrieved
 *
 * The G = h_q/h_kv query heads of a KV head share one selection, scored with
 * their mean qbar projected by W: u = fl32(qbar . W_g); a node's score is
 * fl32(u . centroid).  Level-1 candidates are the root's non-empty children;
 * at levels 1..L-1 the best min(beam, #candidates) in (score desc, id asc)
 * order are kept and their non-empty children become the next candidates; all
 * level-L candidates are candidate leaves.  Leaves are visited in (score desc,
 * id asc) order, each giving its members in ascending position; keys at
 * positions > q_pos are skipped; the first k are taken.  Dot products are
 * accumulated in double in ascending index order.
 *
 * Sinks and window ("Latent sparse attention", bdtechtalks.com, "How latent
 * sparse attention works": the retrieved keys are joined by a window of recent
 * tokens and a few initial sink tokens).  With hi = min(q_pos, n - 1), the
 * latest key the row sees, the sinks are keys [0, min(n_sink, hi + 1)) and the
 * window is [max(n_sink, hi - window + 1), hi]; retrieval skips both (it takes
 * only keys in [n_sink, hi - window], still up to k of them), so the three
 * parts are disjoint.  n_sink = window = 0 gives the retrieved keys alone.
 * Limits: h_q % h_kv == 0, 1 <= d <= 256, beam * b <= 4096, k <= 8192,
 * k + n_sink + window <= 2^24.
 *
 * Workspace: ws may be NULL.  When ws holds at least
 * lsa_select_workspace_bytes bytes (> 0), small batches run on beam
 * workgroups per (row, KV head) group, all of one group on one XCD (L >= 2,
 * beam <= 32, and XCDs * ceil(m * h_kv / XCDs) * beam at most the number of
 * compute units), that exchange their partial rankings through ws (words
 * published into zeroed memory and polled by the readers).  The
 * caller zero-fills ws once before its first use.  Those workgroups poll only
 * a prefix of ws that no other path of lsa_select, lsa_select_attend,
 * lsa_select_flat or lsa_attend writes (their buffers start after it), and
 * they leave it zeroed, so one ws serves any number of calls of these
 * functions, of any sizes that fit it.  The first int32 of ws is its status
 * word (lsa_workspace_status).  Calls that share one ws must not run
 * concurrently (they would read each other's words).  Larger batches of the shapes named at lsa_select_workspace_bytes
 * score levels 2..L node by node: the (row, kept node) pairs are grouped by
 * node in ws, and each kept node's children are read once per group of rows
 * that kept it instead of once per row; rows run in batches that fit ws.
 * Every path gives identical results.
 */
int lsa_select(const void *Q, int dtype, int64_t m, int h_q, int d, const int32_t *q_pos,
               const lsa_index_desc *desc, const void *index, const float *W, int beam, int k,
               int n_sink, int window, int32_t *sel, int32_t *sel_count, float *sel_cutoff, void *ws,
               int64_t ws_bytes, void *stream);

/*
 * Bytes of device workspace lsa_select_flat needs to run m rows in batches of
 * up to 512 rows (*bytes).  Any workspace of at least the one-row size works;
 * a smaller one runs the rows in smaller batches.
 */
int lsa_select_flat_workspace_bytes(int64_t m, int h_q, const lsa_index_desc *desc, int64_t *bytes);

/*
 * Flat search ("Latent sparse attention", bdtechtalks.com, "How latent sparse
 * attention works": the query is compared against all cluster centroids,
 * the alternative to the hierarchical search that follows a few branches per
 * level).  The clusters are the leaves of the tree built by lsa_build_index:
 * every non-empty leaf v is scored with fl32(u . centroid_L[v]) (u as in
 * lsa_select); the leaves are visited in (score desc, id asc) order and the
 * keys retrieved from them exactly as lsa_select retrieves keys from its
 * candidate leaves (retrieval range, k, sinks and window, cutoff).  No level
 * above the leaves is read.  On a tree with L = 1 both searches coincide.
 *
 * Arguments as in lsa_select (no beam).  ws (device, required) holds per row
 * and KV head the score and eligible count of every leaf, 6 bytes a leaf;
 * rows run in batches that fit ws_bytes (LSA_ENOSPC below the one-row size).
 * The work per row is linear in the number of leaves, as the page notes for
 * flat search.  Limits as lsa_select (beam excepted).
 */
int lsa_select_flat(const void *Q, int dtype, int64_t m, int h_q, int d, const int32_t *q_pos,
                    const lsa_index_desc *desc, const void *index, const float *W, int k, int n_sink,
                    int window, int32_t *sel, int32_t *sel_count, float *sel_cutoff, void *ws,
                    int64_t ws_bytes, void *stream);

/*
 * Bytes of device workspace lsa_pca_projection needs for n keys of h_kv KV
 * heads (*bytes): about 128 KB per 8192 keys and head.
 */
int lsa_pca_workspace_bytes(int64_t n, int h_kv, int d, int64_t *bytes);

/*
 * Training-free latent projection ("Latent sparse attention", bdtechtalks.com,
 * "How latent sparse attention works": principal component analysis builds
 * the indexing space without trained projection matrices).  Per KV head g:
 *   mu = mean of the n keys, C = (1/n) sum_j (k_j - mu)(k_j - mu)^T (double),
 *   W[g] = the eigenvectors of C with the r largest eigenvalues, largest
 *   first, each signed so that its entry of largest magnitude (the first such)
 *   is positive, rounded to fp32.
 * The result is a W for lsa_build_index / lsa_select (centring does not
 * change which clusters a query selects: it shifts every centroid's score by
 * the same amount).
 *
 *   K         device, [h_kv][n][d] of `dtype`
 *   W         device out, float [h_kv][d][r]
 *   eigenvalues device out or NULL, double [h_kv][r]
 *   ws        device workspace of lsa_pca_workspace_bytes bytes
 * Sums are taken in a fixed order (results are deterministic); the
 * eigenvectors come from cyclic Jacobi rotations run to convergence, so they
 * agree with any other symmetric eigensolver to within the conditioning of
 * the eigenproblem (close eigenvalues give ill-determined eigenvectors).
 * Limits: 2 <= d <= 128, 1 <= r <= d, 1 <= n <= 2^31 - 1.
 */
int lsa_pca_projection(const void *K, int dtype, int64_t n, int h_kv, int d, int r, float *W,
                       double *eigenvalues, void *ws, int64_t ws_bytes, void *stream);

/*
 * Bytes of device workspace lsa_attend needs (*bytes).
 */
int lsa_attend_workspace_bytes(int64_t m, int h_q, int h_kv, int d, int k, int64_t *bytes);

/*
 * Softmax attention of every query head over its KV head's selected keys
 * (kongchang.com, "The Accuracy-Efficiency Dilemma of Sparse Attention": each
 * query interacts with only k keys).
 *
 *   Q        device, [m][h_q][d] of `dtype`
 *   K, V     device, [h_kv][n][d] of `dtype`
 *   sel, sel_count  as written by lsa_select (k = row length of sel, which
 *            is k + n_sink + window of the lsa_select call)
 *   scale    score scale; 0 means 1/sqrt(d)
 *   out      device out, [m][h_q][d] of `dtype` (fp32 accumulation, rounded
 *            to nearest even for bf16)
 *   lse      device out or NULL, float [m][h_q]: natural-log sum of exp of the
 *            scaled scores; -inf for an empty selection (whose out row is 0)
 *   ws       device workspace of lsa_attend_workspace_bytes bytes
 * Entries of sel must lie in [0, n).  Limits: h_q % h_kv == 0, h_q/h_kv <= 16,
 * 8 <= d <= 256 with d % 8 == 0, k <= 2^24.
 */
int lsa_attend(const void *Q, const void *K, const void *V, int dtype, int64_t m, int h_q,
               int h_kv, int64_t n, int d, const int32_t *sel, const int32_t *sel_count, int k,
               float scale, void *out, float *lse, void *ws, int64_t ws_bytes, void *stream);

/*
 * Bytes of device workspace lsa_select_attend needs (*bytes).
 */
int lsa_select_attend_workspace_bytes(int64_t m, int h_q, int d, const lsa_index_desc *desc, int beam,
                                      int k, int n_sink, int window, int64_t *bytes);

/*
 * lsa_select followed by lsa_attend on the same rows, in one of three forms:
 *   - one launch when the batch is small (the decode case: the beam
 *     workgroups of each (row, KV head) pair also attend over the keys they
 *     retrieved, split evenly over the attention set, and the last one
 *     merges the partial softmax states);
 *   - node-major selection and attention for many rows (bf16, d = 128,
 *     h_q/h_kv <= 16, n_sink = window = 0, the node-major selection's shapes,
 *     and ws of lsa_select_attend_workspace_bytes): the rows are grouped by
 *     the kept clusters they descend into ("Latent Sparse Attention Breaks
 *     Through the Million-Token Context Bottleneck", section "How LSA
 *     Sidesteps Per-Key Scoring with Hierarchical Clustering"), each
 *     cluster's keys are staged once for a tile of (row, head) columns that
 *     attend over the keys they retrieved from it, and the per-cluster
 *     partial states (output / sum as 16-bit fixed point under a power-of-two
 *     scale per column, maximum and sum in fp32) are merged by log-sum-exp;
 *   - otherwise the two calls in sequence.
 * Arguments as in lsa_select and lsa_attend; K and V are the cache the index
 * was built from, [h_kv][n][d].  ws (lsa_select_attend_workspace_bytes
 * bytes) must be zero-filled before its first use; the one-launch form
 * leaves the part it polls zeroed and no other path writes it (see
 * lsa_select), so ws serves any number of calls of any sizes that fit it;
 * calls sharing one ws must not run concurrently.
 * sel, sel_count and sel_cutoff equal those of lsa_select bit for bit; out
 * and lse equal lsa_attend's within fp32 rounding of the accumulation order
 * (plus, in the node-major form, at most 2^-16 of the power of two above
 * each partial output's largest magnitude).
 * Limits: those of lsa_select and of lsa_attend.
 */
int lsa_select_attend(const void *Q, const void *K, const void *V, int dtype, int64_t m, int h_q, int d,
                      const int32_t *q_pos, const lsa_index_desc *desc, const void *index, const float *W,
                      int beam, int k, int n_sink, int window, float scale, int32_t *sel, int32_t *sel_count,
                      float *sel_cutoff, void *out, float *lse, void *ws, int64_t ws_bytes, void *stream);

/*
 * lsa_select_attend in its one-launch form with no workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  It allocates nothing
 * and calls no allocating routine: its workspace is a fixed 4 MiB array of
 * device memory inside the library (one copy per device, set up and cleared
 * on the first call on that device, held until the process ends).
 *
 * Arguments, results and limits as lsa_select_attend, minus ws and ws_bytes.
 * Errors as lsa_select_attend, plus: LSA_EUNSUPPORTED when the batch does not
 * take the one-launch form (m * h_kv * beam above the number of compute
 * units, L < 2, beam > 32, h_q/h_kv > 16); LSA_ESCRATCH when its workspace
 * (lsa_select_attend_workspace_bytes for the same arguments) exceeds 4 MiB.
 * The array is shared by every call on a device and keeps the last call's
 * contents (the call leaves every word it polls zero): calls that overlap on
 * one device, from any stream or thread, race and give wrong results.  Its
 * status word is read with lsa_workspace_status(NULL, ...).
 */
int lsa_select_attend_noalloc(const void *Q, const void *K, const void *V, int dtype, int64_t m, int h_q, int d,
                              const int32_t *q_pos, const lsa_index_desc *desc, const void *index, const float *W,
                              int beam, int k, int n_sink, int window, float scale, int32_t *sel, int32_t *sel_count,
                              float *sel_cutoff, void *out, float *lse, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LSA_H */
