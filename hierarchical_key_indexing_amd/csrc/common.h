// Device helpers shared by the LSA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#define LSA_DEV __device__ __forceinline__
#define LSA_HOST_DEV __host__ __device__

namespace lsa {

constexpr int kWave = 64;

// Native 4-float vector: whole-vector loads and stores keep arrays of these in
// registers (HIP's float4 struct, copied whole, can push an array to scratch).
typedef float f4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- element types
struct bf16_t {
    uint16_t bits;
    LSA_DEV explicit operator float() const { return __uint_as_float(((uint32_t)bits) << 16); }
};

LSA_DEV float to_float(float x) { return x; }
LSA_DEV float to_float(bf16_t x) { return __uint_as_float(((uint32_t)x.bits) << 16); }

template <typename T> LSA_DEV T from_float(float x);
template <> LSA_DEV float from_float<float>(float x) { return x; }
template <> LSA_DEV bf16_t from_float<bf16_t>(float x) {
    // round to nearest even; NaN stays a quiet NaN
    uint32_t u = __float_as_uint(x);
    bf16_t r;
    if ((u & 0x7fffffffu) > 0x7f800000u) { r.bits = 0x7fc0; return r; }
    u += 0x7fffu + ((u >> 16) & 1u);
    r.bits = (uint16_t)(u >> 16);
    return r;
}

// ---------------------------------------------------------------- ordering keys
// 64-bit key whose unsigned order is (score descending -> larger key, then id
// ascending -> larger key).  -0.0 is folded onto +0.0 so that equal scores
// compare equal, as a float comparison would.
LSA_DEV uint32_t orderable(float f) {
    if (f == 0.0f) f = 0.0f;
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
LSA_DEV float unorderable(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(u);
}
LSA_DEV uint64_t make_key(float score, uint32_t id) {
    return ((uint64_t)orderable(score) << 32) | (uint64_t)(~id);
}
LSA_DEV uint32_t key_id(uint64_t key) { return ~(uint32_t)key; }
LSA_DEV float key_score(uint64_t key) { return unorderable((uint32_t)(key >> 32)); }

// ---------------------------------------------------------------- wave helpers
LSA_DEV int lane_id() { return __lane_id(); }

// Orders one wave's LDS accesses across this point (for LDS regions only this
// wave reads and writes): the lanes of a wave run in lockstep and the LDS
// serves one wave's operations in issue order, so no workgroup barrier is needed.
// Workgroup barrier that orders LDS traffic only: each wave waits for its own
// LDS operations, then for the other waves; its global loads may stay in
// flight (a __syncthreads fence would wait for them too).  The memory clobber
// keeps the compiler from moving memory accesses across it.
LSA_DEV void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

LSA_DEV void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

LSA_DEV uint64_t lanemask_lt() {
    int l = lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Value of lane (l ^ M) for every lane l, without a trip through LDS: DPP quad
// permutes for M = 1, 2; DPP row shifts (both directions, then a per-lane
// select) for M = 4; a DPP row rotate by 8 for M = 8; the gfx950 row-swap
// instructions for M = 16, 32.
template <int M>
LSA_DEV uint32_t xor_lane(uint32_t x) {
    static_assert(M == 1 || M == 2 || M == 4 || M == 8 || M == 16 || M == 32, "lane mask");
    if constexpr (M == 1) {
        return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    } else if constexpr (M == 2) {
        return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    } else if constexpr (M == 4) {
        const uint32_t from_below = (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4
        const uint32_t from_above = (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x104, 0xF, 0xF, false);  // row_shl:4
        return (lane_id() & M) ? from_below : from_above;
    } else if constexpr (M == 8) {
        return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x128, 0xF, 0xF, false);   // row_ror:8
    } else if constexpr (M == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        return (lane_id() & 16) ? r[0] : r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        return (lane_id() & 32) ? r[0] : r[1];
    }
}
template <int M>
LSA_DEV uint64_t xor_lane64(uint64_t v) {
    return ((uint64_t)xor_lane<M>((uint32_t)(v >> 32)) << 32) | xor_lane<M>((uint32_t)v);
}
template <int M>
LSA_DEV float xor_lane_f(float v) { return __uint_as_float(xor_lane<M>(__float_as_uint(v))); }
template <int M>
LSA_DEV int xor_lane_i(int v) { return (int)xor_lane<M>((uint32_t)v); }

LSA_DEV float wave_max_f(float v) {
    v = fmaxf(v, xor_lane_f<32>(v)); v = fmaxf(v, xor_lane_f<16>(v)); v = fmaxf(v, xor_lane_f<8>(v));
    v = fmaxf(v, xor_lane_f<4>(v)); v = fmaxf(v, xor_lane_f<2>(v)); v = fmaxf(v, xor_lane_f<1>(v));
    return v;
}
LSA_DEV double wave_max_d(double v) {
    v = fmax(v, __longlong_as_double((long long)xor_lane64<1>((uint64_t)__double_as_longlong(v))));
    v = fmax(v, __longlong_as_double((long long)xor_lane64<2>((uint64_t)__double_as_longlong(v))));
    v = fmax(v, __longlong_as_double((long long)xor_lane64<4>((uint64_t)__double_as_longlong(v))));
    v = fmax(v, __longlong_as_double((long long)xor_lane64<8>((uint64_t)__double_as_longlong(v))));
    v = fmax(v, __longlong_as_double((long long)xor_lane64<16>((uint64_t)__double_as_longlong(v))));
    v = fmax(v, __longlong_as_double((long long)xor_lane64<32>((uint64_t)__double_as_longlong(v))));
    return v;
}
LSA_DEV float wave_sum_f(float v) {
    v += xor_lane_f<32>(v); v += xor_lane_f<16>(v); v += xor_lane_f<8>(v);
    v += xor_lane_f<4>(v); v += xor_lane_f<2>(v); v += xor_lane_f<1>(v);
    return v;
}
LSA_DEV int wave_sum_i(int v) {
    v += xor_lane_i<32>(v); v += xor_lane_i<16>(v); v += xor_lane_i<8>(v);
    v += xor_lane_i<4>(v); v += xor_lane_i<2>(v); v += xor_lane_i<1>(v);
    return v;
}

// An opaque copy of v: values derived from it are recomputed where they are
// used instead of being hoisted and kept live in registers.
LSA_DEV int opaque(int v) {
    asm volatile("" : "+v"(v));
    return v;
}

// Value of lane (l ^ M) for the masks of the wave sort network: M = 2^k (see
// xor_lane) or M = 2^k - 1, a reversal inside blocks of 2^k lanes (DPP quad
// permute, half-row and row mirrors, then row swaps for 31 and 63).
template <int M>
LSA_DEV uint32_t partner_lane(uint32_t x) {
    if constexpr (M == 3) {
        return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x1B, 0xF, 0xF, false);   // quad_perm [3,2,1,0]
    } else if constexpr (M == 7) {
        return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x141, 0xF, 0xF, false);  // row_half_mirror
    } else if constexpr (M == 15) {
        return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x140, 0xF, 0xF, false);  // row_mirror
    } else if constexpr (M == 31) {
        return xor_lane<16>(partner_lane<15>(x));
    } else if constexpr (M == 63) {
        return xor_lane<32>(xor_lane<16>(partner_lane<15>(x)));
    } else {
        return xor_lane<M>(x);
    }
}

// Bitonic sort of one 64-bit key (plus payload) per lane, descending by lane.
// Each merge phase of block size SIZE starts by comparing lane l with lane
// l ^ (SIZE - 1) (the two sorted halves read against each other in reverse)
// and continues with half-cleaners l ^ S, S = SIZE/4 .. 1; in every step the
// lane whose H bit is clear keeps the larger key, so the direction of each
// step is a fixed lane mask.  Every partner value comes through DPP / row
// swaps, never through LDS.
// lanes whose bit H is set (H a power of two below 64)
template <int H>
constexpr uint64_t upper_lanes() {
    uint64_t m = 0;
    for (int l = 0; l < 64; ++l)
        if (l & H) m |= (uint64_t)1 << l;
    return m;
}
template <int M, int H>
LSA_DEV void sort_cx(uint64_t &key, int &pay, int lane) {
    (void)lane;
    const uint64_t o = ((uint64_t)partner_lane<M>((uint32_t)(key >> 32)) << 32) | partner_lane<M>((uint32_t)key);
    const int op = (int)partner_lane<M>((uint32_t)pay);
    // the exchange decision as lane masks: lower lanes take a larger partner,
    // upper lanes a smaller one (the whole wave is active here)
    constexpr uint64_t up = upper_lanes<H>();
    const uint64_t gt = __builtin_amdgcn_ballot_w64(o > key);
    const uint64_t lt = __builtin_amdgcn_ballot_w64(o < key);
    const bool take = __builtin_amdgcn_inverse_ballot_w64((gt & ~up) | (lt & up));
    key = take ? o : key;
    pay = take ? op : pay;
}
template <int S>
LSA_DEV void sort_half_cleaners(uint64_t &key, int &pay, int lane) {
    sort_cx<S, S>(key, pay, lane);
    if constexpr (S > 1) sort_half_cleaners<S / 2>(key, pay, lane);
}
template <int SIZE, int TOP = kWave>
LSA_DEV void sort_phase(uint64_t &key, int &pay, int lane) {
    sort_cx<SIZE - 1, SIZE / 2>(key, pay, lane);
    if constexpr (SIZE >= 4) sort_half_cleaners<SIZE / 4>(key, pay, lane);
    if constexpr (SIZE < TOP) sort_phase<SIZE * 2, TOP>(key, pay, lane);
}
LSA_DEV void wave_sort_desc(uint64_t &key, int &pay) { sort_phase<2>(key, pay, lane_id()); }
// The same network stopped at blocks of 32 lanes: lanes 0..31 and 32..63
// are two independent sorts.
LSA_DEV void half_wave_sort_desc(uint64_t &key, int &pay) { sort_phase<2, 32>(key, pay, lane_id()); }

// Bitonic sort, descending, of the 256 * KPT 64-bit keys of a 256-thread
// block, KPT (1, 2 or 4) per thread: thread t holds elements KPT t ..
// KPT t + KPT - 1 before and after.  Exchanges between a thread's own elements
// stay in registers, between the lanes of a wave they go through DPP / row
// swaps, and only strides that cross waves go through LDS (`sk`, 256 * KPT keys).
// Lanes of this wave whose element e = KPT t + i lies in an ascending block
// of the merge of size SIZE ((e & SIZE) != 0), as a lane mask: a fixed mask
// while SIZE / KPT < 64, else one bit of the wave index (the same for every
// lane), and none at the last merge.
template <int KPT, int SIZE>
LSA_DEV uint64_t bsort_ascending_lanes(int t0) {
    if constexpr (SIZE / KPT < 64) {
        return upper_lanes<SIZE / KPT>();
    } else if constexpr (SIZE < 256 * KPT) {
        const int w = __builtin_amdgcn_readfirstlane(t0 >> 6);
        return (w & (SIZE / KPT / 64)) ? ~0ull : 0ull;
    } else {
        return 0ull;
    }
}

template <int KPT, int SIZE, int S>
LSA_DEV void bsort_stage(uint64_t (&k)[KPT], int t0, uint64_t *sk) {
    if constexpr (S < KPT) {
        // partners inside the thread: element i against i + S; the lower
        // element keeps the larger key in a descending block
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            if ((i & S) == 0) {
                const uint64_t a = k[i], b = k[i + S];
                bool sw;
                if constexpr (SIZE < KPT) {
                    sw = ((i & SIZE) == 0) ? (b > a) : (a > b);
                } else {
                    const uint64_t asc = bsort_ascending_lanes<KPT, SIZE>(t0);
                    const uint64_t gt = __builtin_amdgcn_ballot_w64(b > a);
                    const uint64_t lt = __builtin_amdgcn_ballot_w64(a > b);
                    sw = __builtin_amdgcn_inverse_ballot_w64((gt & ~asc) | (lt & asc));
                }
                k[i] = sw ? b : a;
                k[i + S] = sw ? a : b;
            }
        }
    } else if constexpr (S < 64 * KPT) {
        // partners in other lanes of the wave (DPP / row swaps): a lane keeps
        // the larger key when it is the lower of the pair in a descending
        // block or the upper one in an ascending block
        constexpr uint64_t upper = upper_lanes<S / KPT>();
        const uint64_t want_gt = ~(upper ^ bsort_ascending_lanes<KPT, SIZE>(t0));
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const uint64_t o = xor_lane64<S / KPT>(k[i]);
            const uint64_t gt = __builtin_amdgcn_ballot_w64(o > k[i]);
            const uint64_t lt = __builtin_amdgcn_ballot_w64(o < k[i]);
            const bool take = __builtin_amdgcn_inverse_ballot_w64((gt & want_gt) | (lt & ~want_gt));
            k[i] = take ? o : k[i];
        }
    } else {
        const int t = opaque(t0);
        __syncthreads();                 // earlier readers of sk are done
#pragma unroll
        for (int i = 0; i < KPT; ++i) sk[KPT * t + i] = k[i];
        __syncthreads();
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int e = KPT * t + i;
            const uint64_t o = sk[e ^ S];
            const bool want_gt = ((e & S) == 0) == ((e & SIZE) == 0);
            k[i] = (want_gt ? (o > k[i]) : (o < k[i])) ? o : k[i];
        }
    }
}
template <int KPT, int SIZE, int S>
LSA_DEV void bsort_stages(uint64_t (&k)[KPT], int t, uint64_t *sk) {
    bsort_stage<KPT, SIZE, S>(k, t, sk);
    if constexpr (S > 1) bsort_stages<KPT, SIZE, S / 2>(k, t, sk);
    else if constexpr (SIZE < 256 * KPT) bsort_stages<KPT, SIZE * 2, SIZE>(k, t, sk);
}
template <int KPT>
LSA_DEV void block_sort_desc(uint64_t (&k)[KPT], uint64_t *sk) { bsort_stages<KPT, 2, 1>(k, (int)threadIdx.x, sk); }

// Inclusive prefix sum over the 64 lanes: scans of the four 16-lane rows with
// DPP row shifts (a lane with no source adds 0), then each row adds the
// totals of the rows below it, read from lanes 15, 31 and 47.
LSA_DEV int wave_incl_scan_add(int v) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
        int t;
        switch (o) {
            case 1: t = __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false); break;
            case 2: t = __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false); break;
            case 4: t = __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false); break;
            default: t = __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false); break;
        }
        v += t;
    }
    const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
              r2 = __builtin_amdgcn_readlane(v, 47);
    const int row = lane_id() >> 4;
    return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// Weighted radix selection over the 1024 64-bit keys of a 256-thread block
// (four per thread, zero keys ignored), eight bits per round from the top:
// returns a T such that the keys >= T weigh at least `want` and, without the
// smallest of them, less than `want` (0 when all keys together weigh less).
// The rounds stop once the digit that holds the boundary is taken whole; T
// is then that digit's lower bound rather than the boundary key, and the keys
// >= T are the same.  `hist` holds 256 ints, `sel` 4.  Every thread gets the
// result.
LSA_DEV uint64_t block_radix_select(const uint64_t (&k)[4], const int (&w)[4], int want, int *hist, int *sel) {
    const int tid = threadIdx.x;
    uint64_t prefix = 0, mask = 0;
    for (int shift = 56; shift >= 0; shift -= 8) {
        hist[tid] = 0;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (k[i] != 0 && (k[i] & mask) == prefix && w[i] > 0) atomicAdd(&hist[(int)((k[i] >> shift) & 255u)], w[i]);
        __syncthreads();
        // thread t owns digit 255 - t: the weight of the larger digits is an
        // exclusive scan in thread order
        const int hv = hist[255 - tid];
        const int wvv = tid / kWave;
        const int incl = wave_incl_scan_add(hv);
        if (lane_id() == kWave - 1) sel[wvv] = incl;
        __syncthreads();
        int before = incl - hv;
        for (int q = 0; q < wvv; ++q) before += sel[q];
        __syncthreads();
        if (hv > 0 && before < want && before + hv >= want) { sel[0] = 255 - tid; sel[1] = want - before; sel[2] = hv; }
        if (tid == 255 && before + hv < want) { sel[0] = -1; }        // all keys weigh less than want
        __syncthreads();
        const int dg = sel[0];
        if (dg < 0) return 0;
        want = sel[1];
        prefix |= (uint64_t)dg << shift;
        mask |= (uint64_t)255 << shift;
        // the whole digit is taken: its lower bound already separates the
        // same set of keys as the boundary key would
        const bool whole = sel[2] == want;
        __syncthreads();
        if (whole) break;
    }
    return prefix;
}


// Exclusive prefix sum over a block; returns the thread's exclusive prefix and
// writes the block total to *total.  `scratch` holds >= blockDim/64 + 1 ints.
LSA_DEV int block_excl_scan(int v, int *scratch, int *total) {
    const int nw = blockDim.x / kWave;
    const int w = threadIdx.x / kWave;
    int incl = wave_incl_scan_add(v);
    if (lane_id() == kWave - 1) scratch[w] = incl;
    __syncthreads();
    if (threadIdx.x == 0) {
        int run = 0;
        for (int i = 0; i < nw; ++i) { int t = scratch[i]; scratch[i] = run; run += t; }
        scratch[nw] = run;
    }
    __syncthreads();
    int res = incl - v + scratch[w];
    *total = scratch[nw];
    __syncthreads();
    return res;
}

// Bitonic sort of keys[0..N) in shared memory, N a power of two, by the whole
// block.  Descending when DESC, else ascending.
template <typename K, bool DESC>
LSA_DEV void block_bitonic_sort(K *keys, int N) {
    for (int size = 2; size <= N; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int t = threadIdx.x; t < (N >> 1); t += blockDim.x) {
                int lo = 2 * t - (t & (stride - 1));
                int hi = lo + stride;
                bool up = ((lo & size) == 0) != DESC;   // ascending segment?
                K a = keys[lo], b = keys[hi];
                bool swap = up ? (a > b) : (a < b);
                if (swap) { keys[lo] = b; keys[hi] = a; }
            }
            __syncthreads();
        }
    }
}

// Copy n floats (n % 4 == 0, src 16-byte aligned) from global memory into LDS
// rows of `cols` floats (cols % 4 == 0) with row stride `ld` (ld % 4 == 0, dst
// 16-byte aligned).  Every thread
// issues up to U 16-byte loads before it stores any of them, so one copy costs
// about one memory round trip per U * blockDim float4s.
template <int U>
LSA_DEV void g2s_rows(float *dst, int ld, const float *__restrict__ src, int n, int cols) {
    const f4_t *s4 = reinterpret_cast<const f4_t *>(src);
    const int n4 = n >> 2;
    for (int base = 0; base < n4; base += U * (int)blockDim.x) {
        f4_t t[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = base + (int)threadIdx.x + u * (int)blockDim.x;
            t[u] = s4[min(e, n4 - 1)];        // clamped: every load stays in bounds
        }
        __builtin_amdgcn_sched_barrier(0);     // all loads issued before the first store waits
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = base + (int)threadIdx.x + u * (int)blockDim.x;
            if (e < n4) {
                const int f = e * 4, row = f / cols, col = f % cols;
                *reinterpret_cast<f4_t *>(dst + row * ld + col) = t[u];
            }
        }
    }
}

// Same for arbitrary n and cols (scalar loads, U in flight per thread).
template <int U, typename S, typename D>
LSA_DEV void g2s_scalar(D *dst, int ld, const S *__restrict__ src, int n, int cols) {
    for (int base = 0; base < n; base += U * (int)blockDim.x) {
        S t[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = base + (int)threadIdx.x + u * (int)blockDim.x;
            t[u] = src[min(e, n - 1)];         // clamped: every load stays in bounds
        }
        __builtin_amdgcn_sched_barrier(0);     // all loads issued before the first store waits
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = base + (int)threadIdx.x + u * (int)blockDim.x;
            if (e < n) dst[(e / cols) * ld + (e % cols)] = (D)t[u];
        }
    }
}

// Gather nk rows of K and V (row ids in LDS) into float LDS tiles, 8 elements
// per load, every load of a thread issued before the first use.
template <typename T>
LSA_DEV void gather_tile(const T *__restrict__ Kg, const T *__restrict__ Vg, const int32_t *ids, int nk, int d,
                         float *Kt, int dp, float *Vt) {
    constexpr int U = 4;
    const int cpr = d / 8;
    const int nch = nk * cpr;
    for (int base = 0; base < nch; base += U * (int)blockDim.x) {
        uint4 kr[U][sizeof(T) == 2 ? 1 : 2], vr[U][sizeof(T) == 2 ? 1 : 2];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = base + (int)threadIdx.x + u * (int)blockDim.x;
            if (e < nch) {
                const size_t off = (size_t)ids[e / cpr] * d + (e % cpr) * 8;
                const uint4 *kp = reinterpret_cast<const uint4 *>(Kg + off);
                const uint4 *vp = reinterpret_cast<const uint4 *>(Vg + off);
#pragma unroll
                for (int h = 0; h < (sizeof(T) == 2 ? 1 : 2); ++h) { kr[u][h] = kp[h]; vr[u][h] = vp[h]; }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = base + (int)threadIdx.x + u * (int)blockDim.x;
            if (e < nch) {
                const int kk = e / cpr, c8 = (e % cpr) * 8;
                float kv[8], vv[8];
                if constexpr (sizeof(T) == 2) {
                    const uint32_t kw[4] = {kr[u][0].x, kr[u][0].y, kr[u][0].z, kr[u][0].w};
                    const uint32_t vw[4] = {vr[u][0].x, vr[u][0].y, vr[u][0].z, vr[u][0].w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        kv[2 * q] = __uint_as_float(kw[q] << 16); kv[2 * q + 1] = __uint_as_float(kw[q] & 0xffff0000u);
                        vv[2 * q] = __uint_as_float(vw[q] << 16); vv[2 * q + 1] = __uint_as_float(vw[q] & 0xffff0000u);
                    }
                } else {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        kv[4 * h + 0] = __uint_as_float(kr[u][h].x); kv[4 * h + 1] = __uint_as_float(kr[u][h].y);
                        kv[4 * h + 2] = __uint_as_float(kr[u][h].z); kv[4 * h + 3] = __uint_as_float(kr[u][h].w);
                        vv[4 * h + 0] = __uint_as_float(vr[u][h].x); vv[4 * h + 1] = __uint_as_float(vr[u][h].y);
                        vv[4 * h + 2] = __uint_as_float(vr[u][h].z); vv[4 * h + 3] = __uint_as_float(vr[u][h].w);
                    }
                }
#pragma unroll
                for (int q = 0; q < 8; ++q) { Kt[kk * dp + c8 + q] = kv[q]; Vt[kk * d + c8 + q] = vv[q]; }
            }
        }
    }
}

LSA_DEV int next_pow2(int x) {
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

// Squared Euclidean distance in double, dimensions ascending (r <= 64); the
// difference of two floats and its square are each rounded once, then added.
LSA_DEV double sq_dist(const float *z, const float *cs, int r) {
#pragma clang fp contract(off)
    double dist = 0.0;
#pragma unroll
    for (int x = 0; x < 64; ++x) {
        if (x < r) {
            const double diff = (double)z[x] - (double)cs[x];
            const double sq = diff * diff;
            dist = dist + sq;
        }
    }
    return dist;
}

// number of entries <= key in an ascending array
LSA_DEV int count_le(const int32_t *a, int len, int32_t key) {
    int lo = 0, hi = len;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (a[mid] <= key) lo = mid + 1; else hi = mid;
    }
    return lo;
}

// ---------------------------------------------------------------- attention set
// The retrieved keys are joined by a few initial sink tokens and a window of
// recent tokens ("Latent sparse attention", bdtechtalks.com, section "How
// latent sparse attention works").  With hi = min(pos, n - 1) the latest key a
// row sees: sinks are [0, ns), ns = min(n_sink, hi + 1); the window is
// [wlo, hi], wlo = max(n_sink, hi - window + 1); retrieval only takes keys in
// [rlo, rhi] = [n_sink, hi - window].  The three parts are disjoint.  A row of
// sel lists the retrieved keys, then the nloc sinks and window keys ascending.
struct AttnSet {
    int32_t rlo, rhi;   // retrieval range (empty when rhi < rlo)
    int32_t ns, wlo;    // sinks [0, ns); window from wlo
    int32_t nloc;       // number of sink and window keys
    bool all;           // every key of the cache is in the retrieval range
};
LSA_DEV AttnSet attn_set(int32_t pos, int64_t n, int n_sink, int window) {
    const int64_t hi = min<int64_t>((int64_t)pos, n - 1);
    const int64_t wlo = max<int64_t>((int64_t)n_sink, hi - window + 1);
    AttnSet s;
    s.rlo = n_sink;
    s.rhi = (int32_t)max<int64_t>(hi - window, -1);
    s.ns = (int32_t)max<int64_t>(0, min<int64_t>((int64_t)n_sink, hi + 1));
    s.wlo = (int32_t)wlo;
    s.nloc = s.ns + (int32_t)max<int64_t>(0, hi - wlo + 1);
    s.all = n_sink == 0 && (int64_t)s.rhi >= n - 1;
    return s;
}
// the t-th local key (t < nloc)
LSA_DEV int32_t local_key(const AttnSet &s, int t) { return t < s.ns ? t : s.wlo + (t - s.ns); }
// members of an ascending list that lie in the retrieval range: the first of
// them and their number
LSA_DEV void in_range(const AttnSet &s, const int32_t *mem, int len, int &first, int &cnt) {
    if (s.all || len <= 0) { first = 0; cnt = max(len, 0); return; }
    const int a = (mem[0] >= s.rlo) ? 0 : count_le(mem, len, s.rlo - 1);
    const int z = (mem[len - 1] <= s.rhi) ? len : count_le(mem, len, s.rhi);
    first = a;
    cnt = max(0, z - a);
}

// Eight consecutive elements (16-byte aligned) widened to float.
LSA_DEV void load8(const bf16_t *src, size_t at, float (&v)[8]) {
    const uint4 u = *reinterpret_cast<const uint4 *>(src + at);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[2 * i] = __uint_as_float(w[i] << 16); v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u); }
}
LSA_DEV void load8(const float *src, size_t at, float (&v)[8]) {
    const f4_t a = *reinterpret_cast<const f4_t *>(src + at), b = *reinterpret_cast<const f4_t *>(src + at + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// fp64 MFMA: v_mfma_f64_16x16x4_f64 accumulates D[i][j] += A[i][k] * B[k][j]
// over k = 0..3 in order, each step rounded as a separate fma would be, so a
// chain over dims 4 * blk + k (blk ascending) gives the sequential double sum
// of the exact float products bit for bit.  Lane l supplies A[l % 16][l / 16]
// and B[l / 16][l % 16]; element e of lane l is D[l / 16 + 4 e][l % 16].
typedef double d4_t __attribute__((ext_vector_type(4)));

// 4 x 4 transpose across the four 16-lane rows of a wave: on return lane
// (row r, column c) holds in x[t] what lane (row t, column c) held in x[r].
LSA_DEV void transpose_rows4(f4_t &v) {
    int x0 = __float_as_int(v.x), x1 = __float_as_int(v.y), x2 = __float_as_int(v.z), x3 = __float_as_int(v.w);
    const auto p = __builtin_amdgcn_permlane32_swap(x0, x2, false, false);
    const auto q = __builtin_amdgcn_permlane32_swap(x1, x3, false, false);
    x0 = p[0]; x2 = p[1]; x1 = q[0]; x3 = q[1];
    const auto r = __builtin_amdgcn_permlane16_swap(x0, x1, false, false);
    const auto t = __builtin_amdgcn_permlane16_swap(x2, x3, false, false);
    v.x = __int_as_float(r[0]); v.y = __int_as_float(r[1]); v.z = __int_as_float(t[0]); v.w = __int_as_float(t[1]);
}

// A 64-float row spread over the 16-lane column c: lane (row k, column c)
// loads the quads q0 + k (q0 = 0, 4, 8, 12: four 16-byte loads, the four
// lanes of a column reading 64 contiguous bytes), and after the transposes
// element t of load q0 / 4 is dim 4 (q0 + t) + k, the MFMA operand for block
// q0 + t.
LSA_DEV void load_row_mfma(const float *row, int k, f4_t (&v)[4]) {
#pragma unroll
    for (int h = 0; h < 4; ++h) v[h] = *reinterpret_cast<const f4_t *>(row + 16 * h + 4 * k);
}


// The A operand of a 64-dim row (load_row_mfma layout) widened once: ua[blk]
// is dim 4 blk + k of the lane's row.
LSA_DEV void widen_row_mfma(f4_t (&v)[4], double (&ua)[16]) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        transpose_rows4(v[h]);
        ua[4 * h] = (double)v[h].x; ua[4 * h + 1] = (double)v[h].y;
        ua[4 * h + 2] = (double)v[h].z; ua[4 * h + 3] = (double)v[h].w;
    }
}

// D = A B over 64 dims: A the rows' operand (widen_row_mfma), B the columns'
// rows in load_row_mfma layout (transposed here, widened per use).
LSA_DEV d4_t mfma_dot64(const double (&ua)[16], const f4_t (&rows)[4]) {
    d4_t acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        f4_t t = rows[h];
        transpose_rows4(t);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(ua[4 * h], (double)t.x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(ua[4 * h + 1], (double)t.y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(ua[4 * h + 2], (double)t.z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(ua[4 * h + 3], (double)t.w, acc, 0, 0, 0);
    }
    return acc;
}

}  // namespace lsa
