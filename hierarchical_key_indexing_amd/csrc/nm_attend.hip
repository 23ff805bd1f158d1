// Node-major sparse attention for many query rows (gfx950, bf16 K/V, d = 128).
//
// Attention runs over the keys each query retrieved ("Latent sparse
// attention", bdtechtalks.com, section "How latent sparse attention works"),
// and those keys come from the leaves of a few kept clusters ("Latent Sparse
// Attention Breaks Through the Million-Token Context Bottleneck",
// kongchang.com, section "How LSA Sidesteps Per-Key Scoring with Hierarchical
// Clustering").  Many rows keep the same cluster, so instead of gathering each
// (row, KV head) group's keys on its own, the work is taken cluster by
// cluster: the (row, kept level-(L-1) node) pairs that node-major selection
// grouped by node are cut into tiles of up to 128 / G pairs; a workgroup
// stages the node's keys and values in LDS once, 64 keys at a time, and its
// four waves compute the scores and the P V products of every (pair, query
// head) column of the tile on the matrix cores (v_mfma_f32_16x16x32_bf16, 32
// columns per wave).  A column only sees the keys its row retrieved from that
// node: the children whose leaves it took (a 64-bit mask from the selection's
// finish), inside its retrieval range, and for the one leaf taken in part,
// up to the last key taken.  Each column writes a partial state (its output
// divided by its sum as 16-bit fixed point under a power-of-two scale of its
// own, and the base-2 max and sum in fp32); a merge kernel combines a group's
// states by log-sum-exp.  Prefill, which computes in bulk, is where this pays (same
// page, section "The Accuracy-Efficiency Dilemma of Sparse Attention").
#include <algorithm>

#include "common.h"
#include "internal.h"
#include "mfma_attn.h"

namespace lsa {

constexpr int kNmaP = 16;       // kept-node slots per group (the throughput path's beam limit)
constexpr int kNmaD = 128;      // head dimension of this path
constexpr int kNmaKC = 64;      // keys staged per step
constexpr int kNmaCols = 128;   // (pair, head) columns per tile: 32 per wave
constexpr int kNmaMaxWg = 4096;  // attention workgroups at most
constexpr int kNmaThreads = 256;
constexpr int kNmaTd = 512;      // tile descriptors staged in LDS at a time// threads of the attention workgroup (four waves)
constexpr int kKst = kNmaD + 8; // K tile row stride (bf16)
constexpr int kVst = kNmaKC + 8;// V^T tile row stride (bf16)
constexpr float kLazy = 8.0f;   // log2 headroom of the lazily moved running max


typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));   // 16 bytes held in registers

struct NmaArgs {
    const uint16_t *Q, *K, *V;  // bf16: Q [m][h_q][128], K/V [h_kv][n][128]
    const int32_t *q_pos;
    int64_t row0, groups;       // the batch: rows row0.., groups = rows x h_kv
    int h_q, h_kv, G;
    int64_t n;
    int b;
    int64_t nodes_prev, nleaf;  // nodes at level L-1 and L
    const int32_t *leaf_off;    // [h_kv][nleaf + 1]
    const int32_t *perm;        // [h_kv][n]
    int n_sink, window;
    const int32_t *pairs;       // group * kNmaP + slot, grouped by (head, node) bin
    const int32_t *noff;        // [nbins + 1]: the bins' runs in pairs
    const int32_t *keep;        // [groups]
    uint16_t *out;              // bf16 [m][h_q][128]
    float *lse;                 // [m][h_q] or NULL
    int64_t nbins;
    int T;                      // pairs per tile (128 / G)
    int32_t *toff;              // [nbins + 1]: tiles before each bin
    int32_t *coff;              // [nbins + 1]: estimated cost before each bin
    int32_t *wr;                // [nwg + 1]: first tile of each workgroup's share
    int64_t nwg;                // attention workgroups (a multiple of 8)
    int4 *tdesc;                // [tiles]: bin, first pair, pairs of each tile
    const u32x4_t *pinf;        // [pairs][2]: pair records in bin order (written by the selection's leaf finish)
    int16_t *po;                // [groups][kNmaP][G][128]: o / l in units of u, rounded
    floatx4_t *pml;             // [groups][kNmaP][G]: {m (base 2), l, u, 0}
    float scale_log2;
};

// Estimated cost of one tile of bin e: the tile itself plus one unit per
// step of 64 of the node's members.
LSA_DEV int nma_tile_cost(const NmaArgs &A, int64_t e) {
    const int g = (int)(e / A.nodes_prev);
    const int64_t v = e % A.nodes_prev;
    const int32_t *lof = A.leaf_off + (size_t)g * (A.nleaf + 1) + (size_t)v * A.b;
    return 1 + (lof[A.b] - lof[0] + kNmaKC - 1) / kNmaKC;
}

// Per bin, in parallel: its tiles and their estimated cost (two units more
// a bin, for staging its node), into toff and coff before their scan.
__global__ __launch_bounds__(256) void k_nma_count(NmaArgs A) {
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < A.nbins; e += (int64_t)gridDim.x * blockDim.x) {
        const int v = (A.noff[e + 1] - A.noff[e] + A.T - 1) / A.T;
        A.toff[e] = v;
        A.coff[e] = v > 0 ? v * nma_tile_cost(A, e) + 2 : 0;
    }
}

// One workgroup of 1024 threads, 16 bins a thread per round: exclusive
// scans of toff and coff in place (totals at [nbins]).
constexpr int kNmaScanT = 1024, kNmaScanV = 16;
__global__ __launch_bounds__(kNmaScanT) void k_nma_scan(NmaArgs A) {
    __shared__ int scr[kNmaScanT / kWave + 1];
    const bool al = (((uintptr_t)A.toff | (uintptr_t)A.coff) & 15) == 0;
    int carry = 0, ccarry = 0;
    for (int64_t base = 0; base < A.nbins; base += (int64_t)kNmaScanT * kNmaScanV) {
        const int64_t e0 = base + (int64_t)threadIdx.x * kNmaScanV;
        const bool whole = al && e0 + kNmaScanV <= A.nbins;     // 16-byte loads and stores
        int v[kNmaScanV], c[kNmaScanV], s = 0, cs = 0;
        if (whole) {
#pragma unroll
            for (int q4 = 0; q4 < kNmaScanV / 4; ++q4) {
                const int4 x = *reinterpret_cast<const int4 *>(A.toff + e0 + 4 * q4);
                const int4 y = *reinterpret_cast<const int4 *>(A.coff + e0 + 4 * q4);
                v[4 * q4] = x.x; v[4 * q4 + 1] = x.y; v[4 * q4 + 2] = x.z; v[4 * q4 + 3] = x.w;
                c[4 * q4] = y.x; c[4 * q4 + 1] = y.y; c[4 * q4 + 2] = y.z; c[4 * q4 + 3] = y.w;
            }
        } else {
#pragma unroll
            for (int u = 0; u < kNmaScanV; ++u) {
                v[u] = e0 + u < A.nbins ? A.toff[e0 + u] : 0;
                c[u] = e0 + u < A.nbins ? A.coff[e0 + u] : 0;
            }
        }
#pragma unroll
        for (int u = 0; u < kNmaScanV; ++u) { s += v[u]; cs += c[u]; }
        int tot, ctot;
        int run = carry + block_excl_scan(s, scr, &tot);
        int crun = ccarry + block_excl_scan(cs, scr, &ctot);
        int ov[kNmaScanV], oc[kNmaScanV];
#pragma unroll
        for (int u = 0; u < kNmaScanV; ++u) { ov[u] = run; oc[u] = crun; run += v[u]; crun += c[u]; }
        if (whole) {
#pragma unroll
            for (int q4 = 0; q4 < kNmaScanV / 4; ++q4) {
                *reinterpret_cast<int4 *>(A.toff + e0 + 4 * q4) = int4{ov[4 * q4], ov[4 * q4 + 1], ov[4 * q4 + 2], ov[4 * q4 + 3]};
                *reinterpret_cast<int4 *>(A.coff + e0 + 4 * q4) = int4{oc[4 * q4], oc[4 * q4 + 1], oc[4 * q4 + 2], oc[4 * q4 + 3]};
            }
        } else {
#pragma unroll
            for (int u = 0; u < kNmaScanV; ++u)
                if (e0 + u < A.nbins) { A.toff[e0 + u] = ov[u]; A.coff[e0 + u] = oc[u]; }
        }
        carry += tot;
        ccarry += ctot;
    }
    if (threadIdx.x == 0) { A.toff[A.nbins] = carry; A.coff[A.nbins] = ccarry; }
    // the end of the last share; with no tile every share is empty
    for (int64_t r = threadIdx.x; r <= A.nwg; r += blockDim.x)
        if (r == A.nwg || ccarry == 0) A.wr[r] = r == A.nwg ? carry : 0;
}

// Tile descriptors: the bin of each tile, its first pair and its pairs.
// The tile list is cut into nwg shares of equal estimated cost: share r
// starts at cost floor(r C / nwg), C the total, and the bin whose cost range
// holds that point writes wr[r], the first tile of the share.
__global__ __launch_bounds__(256) void k_nma_map(NmaArgs A) {
    const int64_t C = A.coff[A.nbins];
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < A.nbins; e += (int64_t)gridDim.x * blockDim.x) {
        const int32_t p0 = A.noff[e], p1 = A.noff[e + 1];
        const int32_t tb = A.toff[e], tiles = A.toff[e + 1] - tb;
        for (int t = 0; t < tiles; ++t) {
            const int32_t pb = p0 + t * A.T;
            A.tdesc[tb + t] = int4{(int32_t)e, pb, min(A.T, p1 - pb), 0};
        }
        const int64_t c0 = A.coff[e], c1 = A.coff[e + 1];
        if (c1 == c0) continue;
        const int64_t r0 = (c0 * A.nwg + C - 1) / C, r1 = min<int64_t>(A.nwg - 1, (c1 * A.nwg + C - 1) / C - 1);
        const int pc = nma_tile_cost(A, e);
        for (int64_t r = r0; r <= r1; ++r) {
            const int64_t target = r * C / A.nwg;
            A.wr[r] = tb + (int32_t)min<int64_t>(max<int64_t>(0, target - c0 - 2) / pc, tiles);
        }
    }
}

// Tiles [t0, t1) of workgroup `bid`: share r of the tile list, ordered by
// node, where neighbouring shares run on one XCD (workgroup i runs on XCD
// i % 8, nwg a multiple of 8), so the tiles of one node that follow each
// other are served by that XCD's L2.
LSA_DEV void nma_range(const NmaArgs &A, int64_t bid, int64_t &t0, int64_t &t1) {
    const int64_t r = (bid % 8) * (A.nwg / 8) + bid / 8;
    t0 = A.wr[r];
    t1 = A.wr[r + 1];
}

// The child of the node whose leaf holds member position `at` (lof: the
// node's b + 1 leaf offsets; empty leaves share the next leaf's offset).
LSA_DEV int nma_child(const int32_t *lof, int b, int64_t at) {
    int c = 0;
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1)
        if (c + s < b && lof[c + s] <= at) c += s;
    return c;
}

// A large node's members, one step at a time: threads < 64 read the members
// at positions t0.. and their children (64 past the node's end, whose id
// repeats the last member so that every gather stays inside the cache).
LSA_DEV void nma_load_ids(const int32_t *pm, const int32_t *lof_s, int b, int64_t t0, int64_t hi, int32_t *ids,
                          int32_t *cid) {
    const int tid = opaque((int)threadIdx.x);
    if (tid < kNmaKC) {
        const int64_t at = t0 + tid;
        const bool in = at < hi;
        ids[tid] = pm[in ? at : hi - 1];
        cid[tid] = in ? nma_child(lof_s, b, at) : 64;
    }
}

// K: thread = (key tid / 4, 32-dim part tid % 4), four 16-byte loads into
// registers; stored as rows of kKst bf16.
LSA_DEV void nma_load_k(const uint16_t *__restrict__ Kg, const int32_t *ids, u32x4_t (&kr)[4]) {
    const int tid = threadIdx.x;
    const size_t kb = (size_t)ids[tid / 4] * kNmaD + 32 * (tid % 4);
#pragma unroll
    for (int u = 0; u < 4; ++u) kr[u] = *reinterpret_cast<const u32x4_t *>(Kg + kb + 8 * u);
}

LSA_DEV void nma_store_k(uint16_t *Ks, const u32x4_t (&kr)[4]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < 4; ++u) *reinterpret_cast<u32x4_t *>(Ks + (tid / 4) * kKst + 32 * (tid % 4) + 8 * u) = kr[u];
}

// V: thread = (4-key block tid % 16, 8-dim chunk tid / 16), four 16-byte
// loads into registers.
LSA_DEV void nma_load_v(const uint16_t *__restrict__ Vg, const int32_t *ids, u32x4_t (&vr)[4]) {
    const int tid = threadIdx.x;
    const int vkq = tid % 16, vcg = tid / 16;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        vr[j] = *reinterpret_cast<const u32x4_t *>(Vg + (size_t)ids[4 * vkq + j] * kNmaD + 8 * vcg);
}

// V transposed into V^T: a thread's 4 keys x 8 dims become rows 8 vcg + dd
// over keys 4 vkq .. + 3 (8 bytes a row; one byte permute per pair of keys).
LSA_DEV void nma_store_v(uint16_t *Vt, const u32x4_t (&vr)[4]) {
    const int tid = threadIdx.x;
    const int vkq = tid % 16, vcg = tid / 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // dword i of each key holds dims 8 vcg + 2 i (low half) and + 2 i + 1 (high half)
        const uint32_t a0 = __builtin_amdgcn_perm(vr[1][i], vr[0][i], 0x05040100u);
        const uint32_t a1 = __builtin_amdgcn_perm(vr[3][i], vr[2][i], 0x05040100u);
        const uint32_t b0 = __builtin_amdgcn_perm(vr[1][i], vr[0][i], 0x07060302u);
        const uint32_t b1 = __builtin_amdgcn_perm(vr[3][i], vr[2][i], 0x07060302u);
        *reinterpret_cast<uint2 *>(Vt + (8 * vcg + 2 * i) * kVst + 4 * vkq) = uint2{a0, a1};
        *reinterpret_cast<uint2 *>(Vt + (8 * vcg + 2 * i + 1) * kVst + 4 * vkq) = uint2{b0, b1};
    }
}

constexpr int kNmaIds = 1024;   // members of a node staged in LDS (larger nodes: step by step)

// The keys of the current step that each pair of the tile attends: one
// ballot per pair (lane = key), wave w taking pairs w, w + 4, ...
LSA_DEV void nma_pair_masks(int np, const int32_t *ids, const int32_t *chs, const u32x4_t (*pi)[2], uint64_t *pch) {
    const int lane = lane_id();
    const int id = ids[lane], c = chs[lane];
    for (int p = threadIdx.x / kWave; p < np; p += 4) {
        const u32x4_t r0 = pi[p][0], r1 = pi[p][1];
        const uint64_t mask = (uint64_t)r0.x | ((uint64_t)r0.y << 32);
        const int rlo = (int)r0.w, rhi = (int)r1.x, bc = (int)r1.y, plast = (int)r1.z;
        const bool inc = c < 64 && ((mask >> (c & 63)) & 1ull) && id >= rlo && id <= rhi && !(c == bc && id > plast);
        const uint64_t word = __ballot(inc);
        if (lane == 0) pch[p] = word;
    }
}

// Sort the node's cnt staged members (and their children) by key id; the
// padding entries after them stay in place.  Up to one member a thread:
// each counts the smaller ids and moves to that rank.  Larger nodes: a
// bitonic network over the power of two above `span`, padding (child 64)
// sorting last.
LSA_DEV void nma_sort_members(int cnt, int span, int32_t pad_id, int32_t *mid_s, int32_t *mch_s) {
    const int tid = opaque((int)threadIdx.x);
    if (cnt <= kNmaThreads) {
        const int32_t my = tid < cnt ? mid_s[tid] : 0, mc = tid < cnt ? mch_s[tid] : 0;
        int rank = 0;
        if (tid < cnt) {
            const int4 *m4 = reinterpret_cast<const int4 *>(mid_s);
            for (int j = 0; j < cnt; j += 4) {
                const int4 v = m4[j / 4];
                rank += (v.x < my) + (j + 1 < cnt && v.y < my) + (j + 2 < cnt && v.z < my) + (j + 3 < cnt && v.w < my);
            }
        }
        __syncthreads();
        if (tid < cnt) { mid_s[rank] = my; mch_s[rank] = mc; }
        __syncthreads();
        return;
    }
    int N = kNmaKC;
    while (N < span) N <<= 1;
    for (int x = span + tid; x < N; x += kNmaThreads) { mid_s[x] = pad_id; mch_s[x] = 64; }
    __syncthreads();
    for (int k = 2; k <= N; k <<= 1)
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = tid; i < N; i += kNmaThreads) {
                const int o = i ^ j;
                if (o > i) {
                    const int32_t ci = mch_s[i], co = mch_s[o];
                    const int32_t ki = ci == 64 ? INT32_MAX : mid_s[i], ko = co == 64 ? INT32_MAX : mid_s[o];
                    if ((ki > ko) == ((i & k) == 0)) {
                        const int32_t t = mid_s[i];
                        mid_s[i] = mid_s[o];
                        mid_s[o] = t;
                        mch_s[i] = co;
                        mch_s[o] = ci;
                    }
                }
            }
            __syncthreads();
        }
}

// Stage node `bin`: its leaf offsets, then (when they fit) its members and
// their children, padded to whole steps; returns the member range.  When
// the first pair of the tile it is staged for (`frhi`: that pair's last
// visible key) sees at least a whole step less than the node holds (causal
// rows early in the sequence), the members are sorted by id, so that every
// tile can stop after the last key its rows reach (`srt`).  Ends with the
// members visible to the workgroup.
LSA_DEV void nma_stage_node(const NmaArgs &A, int32_t bin, int32_t frhi, int32_t *lof_s, int32_t *mid_s,
                            int32_t *mch_s, int32_t &lo, int32_t &hi, bool &fits, bool &srt, int *late_s) {
    const int tid = opaque((int)threadIdx.x), b = A.b;
    const int g = (int)(bin / A.nodes_prev);
    const int64_t v = bin % A.nodes_prev;
    if (tid <= b) lof_s[tid] = A.leaf_off[(size_t)g * (A.nleaf + 1) + (size_t)v * b + tid];
    if (tid == 0) *late_s = 0;
    __syncthreads();
    lo = lof_s[0];
    hi = lof_s[b];
    const int span = (int)min<int64_t>((int64_t)(hi - lo + kNmaKC - 1) / kNmaKC * kNmaKC, (int64_t)kNmaIds + 1);
    fits = span <= kNmaIds;
    srt = false;
    if (fits && hi > lo) {
        const int32_t *pm = A.perm + (size_t)g * A.n;
        for (int x = tid; x < span; x += kNmaThreads) {    // (span is a multiple of the wave: whole waves take part)
            const int64_t at = (int64_t)lo + x;
            const int32_t id = pm[at < hi ? at : hi - 1];
            mid_s[x] = id;
            mch_s[x] = at < hi ? nma_child(lof_s, b, at) : 64;
            const uint64_t late = __ballot(at < hi && id > frhi);
            if (lane_id() == 0 && late) atomicAdd(late_s, __popcll(late));
        }
        __syncthreads();
        srt = *late_s >= kNmaKC;
        if (srt) nma_sort_members(hi - lo, span, pm[hi - 1], mid_s, mch_s);
    }
    __syncthreads();
}

// The end of the members a tile's pairs can see in a sorted node: past the
// last id at or below the largest retrieval bound among the pairs (the same
// in every wave).
LSA_DEV int32_t nma_tile_end(const u32x4_t (*pi)[2], int np, const int32_t *mid_s, int32_t lo, int32_t hi) {
    const int lane = lane_id();
    int32_t r = INT32_MIN;
    for (int p = lane; p < np; p += kWave) r = max(r, (int32_t)pi[p][1].x);
    r = max(r, xor_lane_i<1>(r));
    r = max(r, xor_lane_i<2>(r));
    r = max(r, xor_lane_i<4>(r));
    r = max(r, xor_lane_i<8>(r));
    r = max(r, xor_lane_i<16>(r));
    r = max(r, xor_lane_i<32>(r));
    // count the sorted ids <= r (at most kNmaIds = 64 x 16): whole blocks of
    // 16 by one ballot, then the members of the block the count ends in
    const int cnt = hi - lo;
    const int full = __popcll(__ballot(16 * lane + 15 < cnt && mid_s[16 * lane + 15] <= r));
    const int base = 16 * full;
    const int part = __popcll(__ballot(lane < 16 && base + lane < cnt && mid_s[base + lane] <= r));
    return lo + base + part;
}

__global__ __launch_bounds__(kNmaThreads, 2) void k_nma_attend(NmaArgs A) {
    __shared__ __attribute__((aligned(16))) uint16_t Ks[kNmaKC * kKst];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[kNmaD * kVst];
    __shared__ __attribute__((aligned(16))) int32_t mid_s[kNmaIds];    // the node's members (padded to whole steps)
    __shared__ __attribute__((aligned(16))) int32_t mch_s[kNmaIds];    // and their children
    __shared__ __attribute__((aligned(16))) int32_t win_s[2][kNmaKC];  // a large node's step members
    __shared__ __attribute__((aligned(16))) int32_t wch_s[2][kNmaKC];
    __shared__ int32_t lof_s[65];
    __shared__ u32x4_t pi_s[2][kNmaCols][2];                           // pair records: this tile's, the next one's
    __shared__ uint64_t pch_s[kNmaCols];
    __shared__ int late_s;
    __shared__ int4 td_s[kNmaTd];                                      // tile descriptors tw .. tw + kNmaTd - 1
    const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
    const int c16 = lane % 16, q = lane / 16;
    const int G = A.G, b = A.b;
    int64_t t0, t1;
    nma_range(A, blockIdx.x, t0, t1);
    if (t0 >= t1) return;                         // (uniform in the workgroup)

    // this workgroup's tile descriptors, kNmaTd at a time, in LDS
    int64_t tw = t0;
    for (int x = opaque(tid); x < kNmaTd && tw + x < t1; x += kNmaThreads) td_s[x] = A.tdesc[tw + x];
    __syncthreads();
    // the first tile: its pair records, its node and its first step's rows
    int32_t bin = td_s[0].x;
    int64_t pb = td_s[0].y;
    int np = td_s[0].z;
    if (tid < np) { pi_s[0][tid][0] = A.pinf[2 * (pb + tid)]; pi_s[0][tid][1] = A.pinf[2 * (pb + tid) + 1]; }
    int32_t lo, hi;
    bool fits, srt;
    nma_stage_node(A, bin, (int32_t)A.pinf[2 * pb + 1].x, lof_s, mid_s, mch_s, lo, hi, fits, srt, &late_s);
    u32x4_t kr[4], vr[4];
    {
        const int g = (int)(bin / A.nodes_prev);
        const uint16_t *Kg = A.K + (size_t)g * A.n * kNmaD, *Vg = A.V + (size_t)g * A.n * kNmaD;
        if (!fits && hi > lo) {
            nma_load_ids(A.perm + (size_t)g * A.n, lof_s, b, lo, hi, win_s[0], wch_s[0]);
            __syncthreads();
        }
        if (hi > lo) {
            nma_load_k(Kg, fits ? mid_s : win_s[0], kr);
            nma_load_v(Vg, fits ? mid_s : win_s[0], vr);
        }
    }
    int pbuf = 0;
    for (int64_t t = t0; t < t1; ++t) {
        // here: pi_s[pbuf] holds this tile's records, node `bin` is staged and
        // kr / vr hold (or are loading) this tile's first step
        const int g = (int)(bin / A.nodes_prev);
        const int32_t *pm = A.perm + (size_t)g * A.n;
        const uint16_t *Kg = A.K + (size_t)g * A.n * kNmaD, *Vg = A.V + (size_t)g * A.n * kNmaD;
        const bool has_next = t + 1 < t1;
        int32_t nbin = 0;
        int64_t npb = 0;
        int nnp = 0;
        if (has_next) {
            if (t + 1 - tw == kNmaTd) {           // the next window (every wave is past the last read)
                tw = t + 1;
                for (int x = opaque(tid); x < kNmaTd && tw + x < t1; x += kNmaThreads) td_s[x] = A.tdesc[tw + x];
                __syncthreads();
            }
            const int4 d = td_s[t + 1 - tw];
            nbin = d.x;
            npb = d.y;
            nnp = d.z;
        }
        const bool next_same = has_next && nbin == bin && fits;
        // this lane's two columns (32 w + 16 cb + c16): (pair, head) and the
        // query fragments (zero past the tile)
        bf16x8_t qf[2][4];
        int pcol[2], hh[2];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            const int col = 32 * w + 16 * cb + c16;
            const bool ok = col < np * G;
            pcol[cb] = ok ? col / G : 0;
            hh[cb] = ok ? col % G : 0;
            const int32_t e = (int32_t)pi_s[pbuf][pcol[cb]][0].z;
            const int64_t i = A.row0 + (e / kNmaP) / A.h_kv;
            const uint16_t *Qr = A.Q + ((size_t)i * A.h_q + (size_t)g * G + hh[cb]) * kNmaD;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                qf[cb][ks] = ok ? *reinterpret_cast<const bf16x8_t *>(Qr + 32 * ks + 8 * q) : bf16x8_t{};
        }
        const bool wave_on = 32 * w < np * G;     // (uniform in the wave)
        const int32_t hi_t = srt ? nma_tile_end(pi_s[pbuf], np, mid_s, lo, hi) : hi;
        floatx4_t acc[2][8];
        float m_run[2], l_run[2];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) acc[cb][nb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
            m_run[cb] = -INFINITY;
            l_run[cb] = 0.0f;
        }
        int wb = 0;
        for (int64_t c0 = lo; c0 < hi_t; c0 += kNmaKC, wb ^= 1) {
            const int32_t *ids = fits ? mid_s + (c0 - lo) : win_s[wb];
            const int32_t *chs = fits ? mch_s + (c0 - lo) : wch_s[wb];
            __syncthreads();                      // the previous step's tiles are read
            nma_store_k(Ks, kr);
            nma_store_v(Vt, vr);
            nma_pair_masks(np, ids, chs, pi_s[pbuf], pch_s);
            const bool more = c0 + kNmaKC < hi_t;
            if (more && !fits) nma_load_ids(pm, lof_s, b, c0 + kNmaKC, hi, win_s[wb ^ 1], wch_s[wb ^ 1]);
            __syncthreads();
            // rows in flight while this step is computed: the next step's, or
            // after the last one the next tile's first (same node); otherwise
            // this step's again, unused (one unconditional load site, so the
            // loads stay in flight across the compute)
            const int32_t *nids = more ? (fits ? mid_s + (c0 + kNmaKC - lo) : win_s[wb ^ 1]) : next_same ? mid_s : ids;
            nma_load_k(Kg, nids, kr);
            nma_load_v(Vg, nids, vr);
            if (!wave_on) continue;
            // S^T = K Q^T for 64 keys (4 blocks of 16) x 2 column blocks
            floatx4_t sacc[2][4];
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                bf16x8_t kf[4];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    kf[ks] = *reinterpret_cast<const bf16x8_t *>(Ks + (16 * mb + c16) * kKst + 32 * ks + 8 * q);
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) {
                    sacc[cb][mb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        sacc[cb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks], qf[cb][ks], sacc[cb][mb], 0, 0, 0);
                }
            }
            // Online softmax in base 2 over raw scores (scale folded into the
            // exponent).  The running max moves only when a column's step max
            // exceeds it by more than kLazy, so probabilities stay below
            // 2^kLazy and most steps rescale nothing.
            bf16x8_t pf[2][2];
            float alpha[2];
            bool grow = false;
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
                // keys 16 mb + 4 q + j of this lane that the column's pair attends
                const uint64_t word = pch_s[pcol[cb]] >> (4 * q);
                float sv[16];
                float mt = -INFINITY;
#pragma unroll
                for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float x = ((word >> (16 * mb + j)) & 1ull) ? sacc[cb][mb][j] : -INFINITY;
                        sv[4 * mb + j] = x;
                        mt = fmaxf(mt, x);
                    }
                mt = fmaxf(mt, xor_lane_f<16>(mt));
                mt = fmaxf(mt, xor_lane_f<32>(mt));
                const float ms = mt * A.scale_log2;                 // (scale > 0: order kept)
                const bool up = ms > m_run[cb] + kLazy;             // (false while the column is empty)
                const float m_new = up ? ms : m_run[cb];
                alpha[cb] = up ? __builtin_amdgcn_exp2f(m_run[cb] - m_new) : 1.0f;   // (0 when m_run = -inf)
                grow |= up;
                const float mb_ = m_new == -INFINITY ? 0.0f : m_new;   // exp2(-inf - mb_) = 0 for masked keys
                float ls = 0.0f;
                // P fragments of the two 32-key PV steps: step s, slot e < 4 is key
                // 32 s + 4 q + e, slot e >= 4 is key 32 s + 16 + 4 q + e - 4
#pragma unroll
                for (int s = 0; s < 2; ++s)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float x = sv[4 * (2 * s + e / 4) + e % 4];
                        const float pr = __builtin_amdgcn_exp2f(fmaf(x, A.scale_log2, -mb_));
                        ls += pr;
                        pf[cb][s][e] = (__bf16)pr;
                    }
                ls += xor_lane_f<16>(ls);
                ls += xor_lane_f<32>(ls);
                l_run[cb] = l_run[cb] * alpha[cb] + ls;
                m_run[cb] = m_new;
            }
            // O^T += V^T P^T (V^T fragments shared by both column blocks); the
            // accumulators are rescaled only when some column's max moved
            if (__any(grow)) {
#pragma unroll
                for (int nb = 0; nb < 8; ++nb)
#pragma unroll
                    for (int cb = 0; cb < 2; ++cb) acc[cb][nb] = acc[cb][nb] * alpha[cb];
            }
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const uint16_t *vrow = Vt + (16 * nb + c16) * kVst + 32 * s;
                    const uint2 vlo = *reinterpret_cast<const uint2 *>(vrow + 4 * q);
                    const uint2 vhi = *reinterpret_cast<const uint2 *>(vrow + 16 + 4 * q);
                    const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, uint4{vlo.x, vlo.y, vhi.x, vhi.y});
#pragma unroll
                    for (int cb = 0; cb < 2; ++cb)
                        acc[cb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[cb][s], acc[cb][nb], 0, 0, 0);
                }
            }
        }
        // the next tile's records, in flight during the partial states
        u32x4_t pn0 = {0u, 0u, 0u, 0u}, pn1 = {0u, 0u, 0u, 0u};
        const int tp = opaque(tid);
        if (has_next && tp < nnp) { pn0 = A.pinf[2 * (npb + tp)]; pn1 = A.pinf[2 * (npb + tp) + 1]; }
        // partial states.  A column's output o / l is stored as 16-bit
        // integers in units of 2^ex / 32767, 2^ex the power of two above its
        // largest magnitude: an absolute error of at most 2^ex / 65534,
        // whatever V holds.  A column with no key stores m = -inf, l = 0 and
        // no output.
        float amax[2] = {0.0f, 0.0f};
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
            for (int nb = 0; nb < 8; ++nb)
#pragma unroll
                for (int x = 0; x < 4; ++x) amax[cb] = fmaxf(amax[cb], fabsf(acc[cb][nb][x]));
            amax[cb] = fmaxf(amax[cb], xor_lane_f<16>(amax[cb]));
            amax[cb] = fmaxf(amax[cb], xor_lane_f<32>(amax[cb]));
        }
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            const int col = 32 * w + 16 * cb + c16;
            if (col >= np * G) continue;
            const int32_t e = (int32_t)pi_s[pbuf][pcol[cb]][0].z;
            const size_t slot = (size_t)e * G + hh[cb];
            const float l = l_run[cb];
            if (!(l > 0.0f)) {
                if (q == 0) A.pml[slot] = floatx4_t{-INFINITY, 0.0f, 0.0f, 0.0f};
                continue;
            }
            // l >= 1: the largest kept score contributes 2^(its lag behind m) >= 1.
            // (o / l) 2^-ex lies in (-1, 1); v_cvt_pknorm_i16_f32 stores it
            // times 32767, rounded and clamped, two values an instruction.
            const float inv_l = 1.0f / l;
            const int ex = __builtin_amdgcn_frexp_expf(amax[cb] * inv_l);
            const float sc = __builtin_ldexpf(inv_l, -ex);
            int16_t *pp = A.po + slot * kNmaD + 4 * q;
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                const auto h01 = __builtin_amdgcn_cvt_pknorm_i16(acc[cb][nb][0] * sc, acc[cb][nb][1] * sc);
                const auto h23 = __builtin_amdgcn_cvt_pknorm_i16(acc[cb][nb][2] * sc, acc[cb][nb][3] * sc);
                *reinterpret_cast<uint2 *>(pp + 16 * nb) =
                    uint2{__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23)};
            }
            if (q == 0) A.pml[slot] = floatx4_t{m_run[cb], l, __builtin_ldexpf(1.0f, ex) * (1.0f / 32767.0f), 0.0f};
        }
        if (!has_next) break;
        // the next tile: its records into the other buffer; a new node is
        // staged (and its first step loaded) once every wave is past this one
        if (tp < nnp) { pi_s[pbuf ^ 1][tp][0] = pn0; pi_s[pbuf ^ 1][tp][1] = pn1; }
        __syncthreads();
        if (!next_same) {
            nma_stage_node(A, nbin, (int32_t)pi_s[pbuf ^ 1][0][1].x, lof_s, mid_s, mch_s, lo, hi, fits, srt,
                           &late_s);
            const int gn = (int)(nbin / A.nodes_prev);
            const uint16_t *Kn = A.K + (size_t)gn * A.n * kNmaD, *Vn = A.V + (size_t)gn * A.n * kNmaD;
            if (!fits && hi > lo) {
                nma_load_ids(A.perm + (size_t)gn * A.n, lof_s, b, lo, hi, win_s[0], wch_s[0]);
                __syncthreads();
            }
            if (hi > lo) {
                nma_load_k(Kn, fits ? mid_s : win_s[0], kr);
                nma_load_v(Vn, fits ? mid_s : win_s[0], vr);
            }
        }
        bin = nbin;
        pb = npb;
        np = nnp;
        pbuf ^= 1;
    }
}

// Merge: M = max m_j, l = sum l_j 2^(m_j - M), o = sum (o_j / l_j) l_j
// 2^(m_j - M) / l over the group's kept nodes j.  Thread = (group, head,
// 8-dim chunk): 16 threads a head, 256 / (16 G) groups a workgroup.
__global__ __launch_bounds__(256) void k_nma_merge(NmaArgs A) {
    const int G = A.G, per = 16 * G, gpw = 256 / per;
    const int tid = threadIdx.x;
    const int64_t grp = (int64_t)blockIdx.x * gpw + tid / per;
    if (tid >= gpw * per || grp >= A.groups) return;
    const int h = (tid % per) / 16, dd = 8 * (tid % 16);
    const floatx4_t *rec = A.pml + (size_t)grp * kNmaP * G + h;
    const int16_t *po = A.po + ((size_t)grp * kNmaP * G + h) * kNmaD + dd;
    typedef int16_t h8_t __attribute__((ext_vector_type(8)));
    typedef float f3_t __attribute__((ext_vector_type(3)));
    // the kept count and every slot's {m, l, unit} in one round (records of
    // slots at or past the kept count are stale and masked below), then the
    // kept states' outputs in the next, all sixteen loads in flight (slots
    // past the count reload slot 0, unused)
    const int P = A.keep[grp];
    f3_t r[kNmaP];
#pragma unroll
    for (int j = 0; j < kNmaP; ++j) r[j] = *reinterpret_cast<const f3_t *>(rec + (size_t)j * G);
    h8_t v[kNmaP];
#pragma unroll
    for (int j = 0; j < kNmaP; ++j) v[j] = *reinterpret_cast<const h8_t *>(po + (size_t)(j < P ? j : 0) * G * kNmaD);
    // the states' maxima and sums, then each output's weight l_j 2^(m_j - M)
    // times the unit of its 16-bit values (0 for an empty state)
    float M = -INFINITY;
#pragma unroll
    for (int j = 0; j < kNmaP; ++j) M = fmaxf(M, j < P ? r[j][0] : -INFINITY);
    float l = 0.0f, wo[kNmaP];
#pragma unroll
    for (int j = 0; j < kNmaP; ++j) {
        const float wl = (j >= P || r[j][0] == -INFINITY) ? 0.0f : r[j][1] * __builtin_amdgcn_exp2f(r[j][0] - M);
        l += wl;
        wo[j] = wl == 0.0f ? 0.0f : wl * r[j][2];      // (a stale record never reaches the product)
    }
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kNmaP; ++j)
        if (wo[j] != 0.0f)
#pragma unroll
            for (int x = 0; x < 8; ++x) o[x] = fmaf((float)v[j][x], wo[j], o[x]);
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    const size_t oh = (size_t)(A.row0 + grp / A.h_kv) * A.h_q + (size_t)(grp % A.h_kv) * G + h;
    uint32_t pk[4];
#pragma unroll
    for (int x = 0; x < 4; ++x)
        pk[x] = (uint32_t)from_float<bf16_t>(o[2 * x] * inv).bits |
                ((uint32_t)from_float<bf16_t>(o[2 * x + 1] * inv).bits << 16);
    *reinterpret_cast<uint4 *>(A.out + oh * kNmaD + dd) = uint4{pk[0], pk[1], pk[2], pk[3]};
    if (dd == 0 && A.lse) A.lse[oh] = (l > 0.0f) ? (M + log2f(l)) * 0.69314718055994531f : -INFINITY;
}

// ---------------------------------------------------------------- host side
bool nma_shape_ok(int dtype, int d, int G, int n_sink, int window) {
    return dtype == 1 && d == kNmaD && G >= 1 && G <= 16 && n_sink == 0 && window == 0;
}

static inline size_t nma_a256(size_t x) { return (x + 255) & ~(size_t)255; }

static int64_t nma_tiles_bound(int64_t groups, int G, int64_t nbins) {
    const int T = kNmaCols / G;
    const int64_t pairs = groups * kNmaP;
    return ((pairs / T + std::min(nbins, pairs) + 8) + 7) / 8 * 8;
}

// Buffers of the node-major attention for one batch, carved from `base`
// (NULL: sizes only): taken-leaf masks, boundaries, tile offsets and map,
// partial states.
NmaWs carve_nma_ws(char *base, int64_t groups, int G, int64_t nbins) {
    size_t cur = 0;
    NmaWs w{};
    auto take = [&](size_t n) { char *p = base ? base + cur : nullptr; cur = nma_a256(cur + n); return p; };
    w.ppos = (int32_t *)take(sizeof(int32_t) * groups * kNmaP);
    w.toff = (int32_t *)take(sizeof(int32_t) * (nbins + 1));
    w.coff = (int32_t *)take(sizeof(int32_t) * (nbins + 1));
    w.wr = (int32_t *)take(sizeof(int32_t) * (kNmaMaxWg + 1));
    w.tdesc = (int32_t *)take(sizeof(int4) * nma_tiles_bound(groups, G, nbins));
    w.pinf = take(32 * (size_t)groups * kNmaP);
    w.po = take(sizeof(int16_t) * groups * kNmaP * G * kNmaD);
    w.pml = (float *)take(sizeof(floatx4_t) * groups * kNmaP * G);
    w.bytes = cur;
    return w;
}

hipError_t nm_attend_batch(const NmaBatch &B, hipStream_t st) {
    NmaArgs A{};
    A.Q = (const uint16_t *)B.Q; A.K = (const uint16_t *)B.K; A.V = (const uint16_t *)B.V; A.q_pos = B.q_pos;
    A.row0 = B.row0; A.groups = B.groups; A.h_q = B.h_q; A.h_kv = B.h_kv; A.G = B.h_q / B.h_kv;
    A.n = B.n; A.b = B.b; A.nodes_prev = B.nodes_prev; A.nleaf = B.nleaf;
    A.leaf_off = B.leaf_off; A.perm = B.perm; A.n_sink = B.n_sink; A.window = B.window;
    A.pairs = B.pairs; A.noff = B.noff; A.keep = B.keep;
    A.nbins = (int64_t)B.h_kv * B.nodes_prev;
    A.T = kNmaCols / A.G;
    A.toff = B.ws.toff; A.coff = B.ws.coff; A.wr = B.ws.wr; A.tdesc = (int4 *)B.ws.tdesc; A.pinf = (u32x4_t *)B.ws.pinf;
    A.po = (int16_t *)B.ws.po; A.pml = (floatx4_t *)B.ws.pml;
    A.scale_log2 = B.scale * 1.4426950408889634f;
    A.out = (uint16_t *)B.out; A.lse = B.lse;
    // two resident workgroups per compute unit, each walking its range of tiles
    const int cus = std::max(device_cus(), 8);
    const int64_t nwg = std::min<int64_t>({nma_tiles_bound(B.groups, A.G, A.nbins), (int64_t)(cus * 2 + 7) / 8 * 8,
                                           (int64_t)kNmaMaxWg});
    A.nwg = nwg;
    const unsigned bin_blocks = (unsigned)std::min<int64_t>((A.nbins + 255) / 256, 4096);
    hipLaunchKernelGGL(k_nma_count, dim3(bin_blocks), dim3(256), 0, st, A);
    hipLaunchKernelGGL(k_nma_scan, dim3(1), dim3(kNmaScanT), 0, st, A);
    hipLaunchKernelGGL(k_nma_map, dim3(bin_blocks), dim3(256), 0, st, A);
    hipLaunchKernelGGL(k_nma_attend, dim3((unsigned)nwg), dim3(kNmaThreads), 0, st, A);
    const int64_t gpw = 256 / (16 * A.G);
    hipLaunchKernelGGL(k_nma_merge, dim3((unsigned)((B.groups + gpw - 1) / gpw)), dim3(256), 0, st, A);
    return hipGetLastError();
}

}  // namespace lsa
