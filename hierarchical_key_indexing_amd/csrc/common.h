// Device helpers shared by the LSA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define LSA_DEV __device__ __forceinline__

namespace lsa {

constexpr int kWave = 64;

// ---------------------------------------------------------------- element types
struct bf16_t { uint16_t bits; };

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

LSA_DEV uint64_t lanemask_lt() {
    int l = lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

template <typename T>
LSA_DEV T wave_incl_scan_add(T v) {
    int l = lane_id();
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        T t = __shfl_up(v, o, kWave);
        if (l >= o) v += t;
    }
    return v;
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

LSA_DEV int next_pow2(int x) {
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

}  // namespace lsa
