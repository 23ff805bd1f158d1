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
// B fragment is the lane's own P values; V^T is staged per wave in LDS.
#pragma once

#include "common.h"

namespace lsa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kMT = 32;        // keys per wave step
constexpr int kVTS = kMT + 4;  // V^T row stride in LDS (bf16 elements)

LSA_DEV uint16_t bf16_bits_rne(float x) {
    uint32_t u = __float_as_uint(x);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

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

// First half of a step: loads, V^T staging, scores and the softmax update.
// ids: the wave's 32 key ids (LDS); keys >= nk are masked.  Returns the P
// fragment and the rescale factor; the caller synchronises LDS before part 2.
template <int D>
LSA_DEV void wave_attn_part1(const uint16_t *__restrict__ Kg, const uint16_t *__restrict__ Vg, const int32_t *ids,
                             int nk, const bf16x8_t (&qf)[D / 32], float scale_log2, uint16_t *vt, WaveAttn<D> &st,
                             bf16x8_t &pf, float &alpha) {
    constexpr int KS = D / 32, VCH = D / 16;
    const int l = lane_id(), q = l / 16, c16 = l % 16;
    bf16x8_t kf[2][KS];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        const size_t base = (size_t)ids[16 * mb + c16] * D + 8 * q;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kf[mb][ks] = *reinterpret_cast<const bf16x8_t *>(Kg + base + 32 * ks);
    }
    const int kap = l % kMT;
    uint4 vch[VCH];
    {
        const size_t vb = (size_t)ids[kap] * D;
#pragma unroll
        for (int u = 0; u < VCH; ++u) vch[u] = *reinterpret_cast<const uint4 *>(Vg + vb + 8 * (l / kMT + 2 * u));
    }
#pragma unroll
    for (int u = 0; u < VCH; ++u) {
        const int c = l / kMT + 2 * u;
        const uint32_t w4[4] = {vch[u].x, vch[u].y, vch[u].z, vch[u].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            vt[(8 * c + 2 * j) * kVTS + kap] = (uint16_t)(w4[j] & 0xffffu);
            vt[(8 * c + 2 * j + 1) * kVTS + kap] = (uint16_t)(w4[j] >> 16);
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
    alpha = (st.m == -INFINITY) ? 0.0f : exp2f(st.m - m_new);
    float ls = 0.0f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const float pr = (sv[s] == -INFINITY) ? 0.0f : exp2f(sv[s] - m_new);
        ls += pr;
        pf[s] = __builtin_bit_cast(__bf16, bf16_bits_rne(pr));
    }
    ls += xor_lane_f<16>(ls);
    ls += xor_lane_f<32>(ls);
    st.l = st.l * alpha + ls;
    st.m = m_new;
}

// Second half: O^T = alpha * O^T + V^T P^T (V^T from this wave's LDS tile).
template <int D>
LSA_DEV void wave_attn_part2(const uint16_t *vt, const bf16x8_t &pf, float alpha, WaveAttn<D> &st) {
    const int l = lane_id(), q = l / 16, c16 = l % 16;
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) {
        const uint16_t *vr = vt + (16 * nb + c16) * kVTS;
        const uint2 lo = *reinterpret_cast<const uint2 *>(vr + 4 * q);
        const uint2 hi = *reinterpret_cast<const uint2 *>(vr + 16 + 4 * q);
        const uint4 vv = {lo.x, lo.y, hi.x, hi.y};
        const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, vv);
        st.acc[nb] = st.acc[nb] * alpha;
        st.acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, st.acc[nb], 0, 0, 0);
    }
}

// Write the four waves' states to LDS (scratch: >= 4*D*16 + 128 floats) so
// that the workgroup can combine them: mo[w][dim][head], mm[w][head], ll[w][head].
template <int D>
LSA_DEV void wave_attn_stash(const WaveAttn<D> &st, float *scratch) {
    const int w = threadIdx.x / kWave, l = lane_id(), q = l / 16, c16 = l % 16;
    float *mo = scratch, *mm = scratch + 4 * D * 16, *ll = mm + 64;
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb)
#pragma unroll
        for (int j = 0; j < 4; ++j) mo[((size_t)w * D + 16 * nb + 4 * q + j) * 16 + c16] = st.acc[nb][j];
    if (q == 0) { mm[w * 16 + c16] = st.m; ll[w * 16 + c16] = st.l; }
}

// Combined state of head h over the four waves: returns the unnormalised
// output for dimension dd and, through M and Lsum, the max and the sum.
template <int D>
LSA_DEV float wave_attn_combine(const float *scratch, int h, int dd, float &M, float &Lsum) {
    const float *mo = scratch, *mm = scratch + 4 * D * 16, *ll = mm + 64;
    M = -INFINITY;
#pragma unroll
    for (int x = 0; x < 4; ++x) M = fmaxf(M, mm[x * 16 + h]);
    float o = 0.0f;
    Lsum = 0.0f;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        const float mx = mm[x * 16 + h];
        if (mx > -INFINITY) {
            const float wgt = exp2f(mx - M);
            Lsum += ll[x * 16 + h] * wgt;
            o += mo[((size_t)x * D + dd) * 16 + h] * wgt;
        }
    }
    return o;
}

}  // namespace lsa
