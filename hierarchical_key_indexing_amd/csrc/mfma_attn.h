// Wave-level sparse attention step on the matrix cores (gfx950, bf16 K/V).
//
// One wave handles 32 selected keys per step for up to 16 query heads that
// share them.  Scores come out transposed, S^T[key][head] = K Q^T, from
// v_mfma_f32_16x16x32_bf16 (A: 16 keys x 32 dims, B: 32 dims x 16 heads, each
// lane holding 8 consecutive bf16 of one row; D: lane l holds head l % 16 and
// keys 4*(l/16)..+3).  K fragments come straight from the gathered rows.  The
// online softmax runs per head column in registers (base 2); the running sum
// uses the fp32 probabilities, the P V product their bf16 rounding.  The output is
// accumulated transposed, O^T[dim][head] += V^T P^T, with the 32 keys of the
// contraction placed in the order each lane already holds its probabilities
// (slot s < 4: key 4*(l/16) + s, slot s >= 4: key 16 + 4*(l/16) + s - 4), so the
// B fragment is the lane's own P values; V^T is staged per wave in LDS: a lane
// loads one 8-dim chunk of 8 keys' V rows, transposes the 8 x 8 block in
// registers and writes it as eight 16-byte rows of V^T.
#pragma once

#include "common.h"

namespace lsa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kMT = 32;        // keys per wave step
constexpr int kVTS = kMT + 8;  // V^T row stride in LDS (bf16 elements; 16-byte aligned rows)

template <int D>
struct WaveAttn {
    floatx4_t acc[D / 16];   // O^T blocks: lane holds head l%16, dims 16*nb + 4*(l/16) + j
    float m, l;              // running max (base 2) and sum for head l % 16
};

template <int D>
LSA_DEV void wave_attn_init(WaveAttn<D> &st) {
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) st.acc[nb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    st.m = -INFINITY;
    st.l = 0.0f;
}

// Q fragments (B operand of S^T): head l % 16 (zero beyond G), dims 8*(l/16) + 32*ks.
template <int D>
LSA_DEV void wave_load_q(bf16x8_t (&qf)[D / 32], const uint16_t *Qg, int G) {
    const int l = lane_id(), q = l / 16, c16 = l % 16;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
        if (c16 < G) qf[ks] = *reinterpret_cast<const bf16x8_t *>(Qg + (size_t)c16 * D + 32 * ks + 8 * q);
        else qf[ks] = bf16x8_t{};
    }
}

// The gathered rows of one step: K fragments (A operand of S^T) and the V
// units this lane transposes.
template <int D>
struct WaveRows {
    static constexpr int KS = D / 32, NU = D / 2, UPL = (NU + kWave - 1) / kWave;
    bf16x8_t kf[2][KS];
    uint4 vv[UPL][8];
};

// Issue the loads of one step.  ids: the wave's 32 key ids (LDS).
template <int D>
LSA_DEV void wave_attn_load(const uint16_t *__restrict__ Kg, const uint16_t *__restrict__ Vg, const int32_t *ids,
                            WaveRows<D> &rw) {
    constexpr int KS = WaveRows<D>::KS, NU = WaveRows<D>::NU, UPL = WaveRows<D>::UPL;
    const int l = lane_id(), q = l / 16, c16 = l % 16;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        const size_t base = (size_t)ids[16 * mb + c16] * D + 8 * q;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) rw.kf[mb][ks] = *reinterpret_cast<const bf16x8_t *>(Kg + base + 32 * ks);
    }
    // V: unit un = (key block kb = un % 4: keys 8 kb..8 kb + 7, chunk cg = un / 4:
    // dims 8 cg..8 cg + 7), D / 2 units over the 64 lanes
#pragma unroll
    for (int t = 0; t < UPL; ++t) {
        const int un = l + kWave * t;
        if (NU % kWave == 0 || un < NU) {
            const int kb = un % 4, cg = un / 4;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                rw.vv[t][j] = *reinterpret_cast<const uint4 *>(Vg + (size_t)ids[8 * kb + j] * D + 8 * cg);
        }
    }
}

// First half of a step on loaded rows: V^T staging, scores and the softmax
// update; keys >= nk are masked.  Returns the P fragment and the rescale
// factor; the caller orders the wave's LDS accesses before part 2.
template <int D>
LSA_DEV void wave_attn_compute(const WaveRows<D> &rw, int nk, const bf16x8_t (&qf)[D / 32], float scale_log2,
                               uint16_t *vt, WaveAttn<D> &st, bf16x8_t &pf, float &alpha) {
    constexpr int KS = WaveRows<D>::KS, NU = WaveRows<D>::NU, UPL = WaveRows<D>::UPL;
    const int l = lane_id(), q = l / 16;
    const auto &kf = rw.kf;
    const auto &vv = rw.vv;
#pragma unroll
    for (int t = 0; t < UPL; ++t) {
        const int un = l + kWave * t;
        if (NU % kWave == 0 || un < NU) {
            const int kb = un % 4, cg = un / 4;
            uint32_t w[8][4];
#pragma unroll
            for (int j = 0; j < 8; ++j) { w[j][0] = vv[t][j].x; w[j][1] = vv[t][j].y; w[j][2] = vv[t][j].z; w[j][3] = vv[t][j].w; }
            // row dd = 2 i + h of V^T: dim 8 cg + dd of keys 8 kb + 2 m, 8 kb + 2 m + 1
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t pl[4], ph[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    // low halves / high halves of keys 2m, 2m + 1 (one byte permute each)
                    pl[m] = __builtin_amdgcn_perm(w[2 * m + 1][i], w[2 * m][i], 0x05040100u);
                    ph[m] = __builtin_amdgcn_perm(w[2 * m + 1][i], w[2 * m][i], 0x07060302u);
                }
                *reinterpret_cast<uint4 *>(vt + (8 * cg + 2 * i) * kVTS + 8 * kb) = uint4{pl[0], pl[1], pl[2], pl[3]};
                *reinterpret_cast<uint4 *>(vt + (8 * cg + 2 * i + 1) * kVTS + 8 * kb) = uint4{ph[0], ph[1], ph[2], ph[3]};
            }
        }
    }
    floatx4_t sacc[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        sacc[mb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            sacc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[mb][ks], qf[ks], sacc[mb], 0, 0, 0);
    }
    float sv[8];
    float mt = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int key = 16 * mb + 4 * q + j;
            const float x = (key < nk) ? sacc[mb][j] * scale_log2 : -INFINITY;
            sv[4 * mb + j] = x;
            mt = fmaxf(mt, x);
        }
    mt = fmaxf(mt, xor_lane_f<16>(mt));
    mt = fmaxf(mt, xor_lane_f<32>(mt));
    const float m_new = fmaxf(st.m, mt);
    alpha = (st.m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(st.m - m_new);
    float ls = 0.0f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const float pr = (sv[s] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(sv[s] - m_new);
        ls += pr;
        pf[s] = (__bf16)pr;                      // round to nearest even
    }
    ls += xor_lane_f<16>(ls);
    ls += xor_lane_f<32>(ls);
    st.l = st.l * alpha + ls;
    st.m = m_new;
}

// Loads and first half of a step together (every K and V load is in flight
// before the first use of any of them).
template <int D>
LSA_DEV void wave_attn_part1(const uint16_t *__restrict__ Kg, const uint16_t *__restrict__ Vg, const int32_t *ids,
                             int nk, const bf16x8_t (&qf)[D / 32], float scale_log2, uint16_t *vt, WaveAttn<D> &st,
                             bf16x8_t &pf, float &alpha) {
    WaveRows<D> rw;
    wave_attn_load<D>(Kg, Vg, ids, rw);
    __builtin_amdgcn_sched_barrier(0);
    wave_attn_compute<D>(rw, nk, qf, scale_log2, vt, st, pf, alpha);
}

// Second half: O^T = alpha * O^T + V^T P^T (V^T from this wave's LDS tile).
template <int D>
LSA_DEV void wave_attn_part2(const uint16_t *vt, const bf16x8_t &pf, float alpha, WaveAttn<D> &st,
                             bool first = false) {
    const int l = lane_id(), q = l / 16, c16 = l % 16;
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) {
        const uint16_t *vr = vt + (16 * nb + c16) * kVTS;
        const uint2 lo = *reinterpret_cast<const uint2 *>(vr + 4 * q);
        const uint2 hi = *reinterpret_cast<const uint2 *>(vr + 16 + 4 * q);
        const uint4 vv = {lo.x, lo.y, hi.x, hi.y};
        const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, vv);
        if (!first) st.acc[nb] = st.acc[nb] * alpha;   // first step: the accumulators are still 0
        st.acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, st.acc[nb], 0, 0, 0);
    }
}

// Write the four waves' states to LDS (scratch: >= 4 * 64 * D / 4 + 128
// floats) so that the workgroup can combine them: lane l of wave w stores its
// D / 4 accumulator values contiguously (16-byte writes) at mo[w][l], then the
// maxima mm[w][head] and sums ll[w][head].
template <int D>
LSA_DEV void wave_attn_stash(const WaveAttn<D> &st, float *scratch) {
    const int w = threadIdx.x / kWave, l = lane_id(), q = l / 16, c16 = l % 16;
    float *mo = scratch + ((size_t)w * kWave + l) * (D / 4);
    float *mm = scratch + 4 * kWave * (D / 4), *ll = mm + 64;
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) *reinterpret_cast<floatx4_t *>(mo + 4 * nb) = st.acc[nb];
    if (q == 0) { mm[w * 16 + c16] = st.m; ll[w * 16 + c16] = st.l; }
}

// Combined state of head h over the four waves for dimensions dd..dd + 3
// (dd % 4 == 0): returns the unnormalised outputs and, through M and Lsum, the
// max and the sum.  Dimension dd of head h sits in lane 16 * ((dd % 16) / 4) + h,
// accumulator block dd / 16.
template <int D>
LSA_DEV floatx4_t wave_attn_combine4(const float *scratch, int h, int dd, float &M, float &Lsum) {
    const float *mm = scratch + 4 * kWave * (D / 4), *ll = mm + 64;
    const int lane = 16 * ((dd % 16) / 4) + h, nb = dd / 16;
    M = -INFINITY;
#pragma unroll
    for (int x = 0; x < 4; ++x) M = fmaxf(M, mm[x * 16 + h]);
    floatx4_t o = {0.f, 0.f, 0.f, 0.f};
    Lsum = 0.0f;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        const float mx = mm[x * 16 + h];
        const floatx4_t v = *reinterpret_cast<const floatx4_t *>(scratch + ((size_t)x * kWave + lane) * (D / 4) + 4 * nb);
        if (mx > -INFINITY) {
            const float wgt = __builtin_amdgcn_exp2f(mx - M);
            Lsum += ll[x * 16 + h] * wgt;
            o += v * wgt;
        }
    }
    return o;
}

}  // namespace lsa
