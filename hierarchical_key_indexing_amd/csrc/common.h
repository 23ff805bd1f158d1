// Device helpers shared by the LSA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#define LSA_DEV __device__ __forceinline__
#define LSA_HOST_DEV __host__ __device__

namespace lsa {

constexpr int kWave = 64;

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

// Copy n floats (n % 4 == 0, src 16-byte aligned) from global memory into LDS
// rows of `cols` floats (cols % 4 == 0) with row stride `ld`.  Every thread
// issues up to U 16-byte loads before it stores any of them, so one copy costs
// about one memory round trip per U * blockDim float4s.
template <int U>
LSA_DEV void g2s_rows(float *dst, int ld, const float *__restrict__ src, int n, int cols) {
    const float4 *s4 = reinterpret_cast<const float4 *>(src);
    const int n4 = n >> 2;
    for (int base = 0; base < n4; base += U * (int)blockDim.x) {
        float4 t[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = base + (int)threadIdx.x + u * (int)blockDim.x;
            if (e < n4) t[u] = s4[e];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = base + (int)threadIdx.x + u * (int)blockDim.x;
            if (e < n4) {
                const int f = e * 4, row = f / cols, col = f % cols;
                float *q = dst + row * ld + col;
                q[0] = t[u].x; q[1] = t[u].y; q[2] = t[u].z; q[3] = t[u].w;
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
            if (e < n) t[u] = src[e];
        }
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

}  // namespace lsa
