// Host side of the expert quantizer: quantize fp32 expert matrices by the format
// rules of qmoe.h and lay the codes out in the device block layout described in
// qmoe_internal.h.
//
// Source: "Quantized Mixture of Experts (Q-MoE)" page, section 3 components
// table ("Expert Quantizer": per-expert precision INT8 / FP8 / mixed) and
// section 4 (INT4/INT8 quantization); IT Donga DREAM-MoE / SRA-MoE article,
// DREAM-MoE section (4-bit and 3-bit expert weights). The pages fix no rounding
// rule, group size or scale type; the rules implemented here are the ones
// documented in qmoe.h (fp32 arithmetic, round half to even, stored scale used
// for the codes, zero-scale groups get scale 1 and zero codes).
//
// This file must stay free of fused multiply-add contraction and fast-math so
// that every code decision is the plain fp32 IEEE result.
#include <math.h>
#include <string.h>

#include <algorithm>

#include "qmoe_internal.h"

namespace qmoe {
namespace {

// Nearest binary16 (ties to even) of v as a float, saturated at 65504.
float stored_half(float v) {
    _Float16 h = (_Float16)v;
    float r = (float)h;
    if (isinf(r)) r = r > 0 ? 65504.0f : -65504.0f;
    return r;
}

uint16_t half_bits(float exactly_representable) {
    _Float16 h = (_Float16)exactly_representable;
    uint16_t b;
    memcpy(&b, &h, 2);
    return b;
}

float half_from_bits(uint16_t b) {
    _Float16 h;
    memcpy(&h, &b, 2);
    return (float)h;
}

// OCP e4m3fn encoding of v by manipulating its binary32 fields: 3 mantissa bits
// kept with round half to even, exponent re-biased from 127 to 7, values below
// 2^-6 encoded as subnormal multiples of 2^-9, magnitudes above 448 saturated.
uint8_t e4m3_bits(float v) {
    uint32_t b;
    memcpy(&b, &v, 4);
    const uint8_t sign = (uint8_t)((b >> 24) & 0x80u);
    const uint32_t a = b & 0x7FFFFFFFu;
    if (a == 0) return sign;
    int e = (int)(a >> 23) - 127;
    if (e >= -6) {
        uint32_t mant = a & 0x7FFFFFu;
        uint32_t m = mant >> 20, rem = mant & 0xFFFFFu;
        if (rem > 0x80000u || (rem == 0x80000u && (m & 1u))) m++;
        if (m == 8) {
            m = 0;
            e++;
        }
        if (e > 8 || (e == 8 && m == 7)) return (uint8_t)(sign | 0x7E);
        return (uint8_t)(sign | ((e + 7) << 3) | m);
    }
    const float t = rintf(fabsf(v) * 512.0f);   // units of 2^-9; exact scaling
    return (uint8_t)(sign | (uint8_t)t);        // t == 8 encodes 2^-6 as 0x08
}

inline float clampf(float v, float lo, float hi) { return std::min(std::max(v, lo), hi); }

// bf16 bits of a finite float, round to nearest even.
uint16_t bf16_rne_bits(float v) {
    uint32_t u;
    memcpy(&u, &v, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
float bf16_value(uint16_t b) {
    const uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

// Value of an OCP e4m3fn code (finite codes only: the saturating encoder never
// emits NaN): sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0
// holds the subnormal multiples of 2^-9.
float e4m3_value(uint8_t c) {
    const int e = (c >> 3) & 15, m = c & 7;
    const float mag = e == 0 ? ldexpf((float)m, -9) : ldexpf(1.0f + (float)m / 8.0f, e - 7);
    return (c & 0x80) ? -mag : mag;
}

}  // namespace

int quantize_router(int router_quant, int E, int d, const float *w, std::vector<uint16_t> &codes_bf16,
                    std::vector<float> &scale) {
    const int fmt = router_quant == QMOE_RQ_INT8_CH ? QMOE_W_INT8_SYM_CH : QMOE_W_FP8E4M3_CH;
    CanonMatrix m;
    const int rc = quantize_matrix(fmt, E, d, w, m);
    if (rc != QMOE_OK) return rc;
    codes_bf16.resize((size_t)E * d);
    for (size_t i = 0; i < codes_bf16.size(); i++) {
        // int8 codes and e4m3 values are exact in bf16
        const float v = fmt == QMOE_W_INT8_SYM_CH ? (float)m.q[i] : e4m3_value((uint8_t)m.q[i]);
        codes_bf16[i] = bf16_rne_bits(v);
    }
    scale = m.scale;   // [E]: one per expert row
    return QMOE_OK;
}

int quantize_matrix(int wformat, int N, int K, const float *w, CanonMatrix &out) {
    out.N = N;
    out.K = K;
    out.q.assign((size_t)N * K, 0);
    const bool grouped = is_group_wformat(wformat);
    if (grouped && K % kBlockK != 0) return QMOE_EUNSUPPORTED;
    const int G = grouped ? K / kBlockK : 1;
    const int len = grouped ? kBlockK : K;
    out.scale.assign((size_t)N * G, 0.0f);
    out.zero.assign((size_t)N * G, 0.0f);
    for (int n = 0; n < N; n++) {
        for (int g = 0; g < G; g++) {
            const float *src = w + (size_t)n * K + (size_t)g * len;
            int8_t *dst = out.q.data() + (size_t)n * K + (size_t)g * len;
            float s = 1.0f, z = 0.0f;
            bool zero_codes = false;
            switch (wformat) {
            case QMOE_W_INT8_SYM_CH:
            case QMOE_W_FP8E4M3_CH: {
                float amax = 0.0f;
                for (int i = 0; i < len; i++) amax = std::max(amax, fabsf(src[i]));
                s = amax / (wformat == QMOE_W_INT8_SYM_CH ? 127.0f : 448.0f);
                break;
            }
            case QMOE_W_INT4_SYM_G128:
            case QMOE_W_INT3_SYM_G128_IN4: {
                float amax = 0.0f;
                for (int i = 0; i < len; i++) amax = std::max(amax, fabsf(src[i]));
                s = stored_half(amax / (wformat == QMOE_W_INT4_SYM_G128 ? 7.0f : 3.0f));
                break;
            }
            case QMOE_W_INT4_ASYM_G128: {
                float lo = 0.0f, hi = 0.0f;
                for (int i = 0; i < len; i++) {
                    lo = std::min(lo, src[i]);
                    hi = std::max(hi, src[i]);
                }
                s = stored_half((hi - lo) / 15.0f);
                if (s != 0.0f) z = clampf(rintf(-lo / s), 0.0f, 15.0f) + 0.0f;
                break;
            }
            default:
                return QMOE_EINVAL;
            }
            if (s == 0.0f) {
                s = 1.0f;
                z = 0.0f;
                zero_codes = true;
            }
            for (int i = 0; i < len; i++) {
                if (zero_codes) {
                    dst[i] = 0;
                    continue;
                }
                const float t = src[i] / s;
                switch (wformat) {
                case QMOE_W_INT8_SYM_CH: dst[i] = (int8_t)clampf(rintf(t), -127.0f, 127.0f); break;
                case QMOE_W_INT4_SYM_G128: dst[i] = (int8_t)clampf(rintf(t), -8.0f, 7.0f); break;
                case QMOE_W_INT3_SYM_G128_IN4: dst[i] = (int8_t)clampf(rintf(t), -4.0f, 3.0f); break;
                case QMOE_W_INT4_ASYM_G128: dst[i] = (int8_t)clampf(rintf(t) + z, 0.0f, 15.0f); break;
                case QMOE_W_FP8E4M3_CH: dst[i] = (int8_t)e4m3_bits(t); break;
                }
            }
            out.scale[(size_t)n * G + g] = s;
            out.zero[(size_t)n * G + g] = z;
        }
    }
    return QMOE_OK;
}

void interleave_gate_up(const CanonMatrix &gate, const CanonMatrix &up, CanonMatrix &w13, bool group_format) {
    const int F = gate.N, K = gate.K;
    const int G = group_format ? K / kBlockK : 1;
    w13.N = 2 * F;
    w13.K = K;
    w13.q.resize((size_t)2 * F * K);
    w13.scale.resize((size_t)2 * F * G);
    w13.zero.resize((size_t)2 * F * G);
    for (int r = 0; r < 2 * F; r++) {
        const int b = r / kBlockRows, i = r % kBlockRows;
        const CanonMatrix &src = (b % 2 == 0) ? gate : up;
        const int sr = (b / 2) * kBlockRows + i;
        memcpy(&w13.q[(size_t)r * K], &src.q[(size_t)sr * K], (size_t)K);
        for (int g = 0; g < G; g++) {
            w13.scale[(size_t)r * G + g] = src.scale[(size_t)sr * G + g];
            w13.zero[(size_t)r * G + g] = src.zero[(size_t)sr * G + g];
        }
    }
}

void layout_matrix(int wformat, const CanonMatrix &m, PackedMatrix &out) {
    const int df = dev_format(wformat);
    const int bb = block_bytes(df);
    const int NB = m.N / kBlockRows, KB = m.K / kBlockK;
    const bool four_bit = bb == 1024;
    out.codes.assign((size_t)NB * KB * bb, 0);
    for (int rb = 0; rb < NB; rb++) {
        for (int kb = 0; kb < KB; kb++) {
            uint8_t *blk = &out.codes[((size_t)rb * KB + kb) * bb];
            for (int lane = 0; lane < 64; lane++) {
                const int r = rb * kBlockRows + lane % 16;
                for (int s = 0; s < 4; s++) {
                    for (int j = 0; j < 8; j++) {
                        const int k = kb * kBlockK + 32 * s + 8 * (lane / 16) + j;
                        const int8_t code = m.q[(size_t)r * m.K + k];
                        if (four_bit) {
                            const uint32_t u = (uint32_t)(df == DF_I4ASYM ? code : code + 8) & 0xFu;
                            const int pos = (j % 2 == 0) ? 4 * (j / 2) : 16 + 4 * (j / 2);
                            uint32_t *dw = reinterpret_cast<uint32_t *>(blk + lane * 16 + s * 4);
                            *dw |= u << pos;
                        } else {
                            blk[lane * 32 + s * 8 + j] = (uint8_t)code;
                        }
                    }
                }
            }
        }
    }
    out.gscale.clear();
    out.gzero.clear();
    out.pscale.clear();
    if (is_group_wformat(wformat)) {
        out.gscale.resize((size_t)NB * KB * kBlockRows);
        if (df == DF_I4ASYM) out.gzero.resize((size_t)NB * KB * kBlockRows);
        for (int rb = 0; rb < NB; rb++)
            for (int kb = 0; kb < KB; kb++)
                for (int i = 0; i < kBlockRows; i++) {
                    const size_t src = (size_t)(rb * kBlockRows + i) * KB + kb;
                    const size_t dst = ((size_t)rb * KB + kb) * kBlockRows + i;
                    out.gscale[dst] = half_bits(m.scale[src]);
                    if (df == DF_I4ASYM) out.gzero[dst] = half_bits(m.zero[src]);
                }
    } else {
        out.pscale.assign(m.scale.begin(), m.scale.end());
    }
    out.zc.clear();
    if (df == DF_I4ASYM) {
        // s * z / 128 is exact in fp32 (11-bit scale times a 4-bit zero); its
        // bf16 remainder after the rounded high part fits a bf16 exactly.
        const int GS = (KB + 31) / 32;
        out.zc.assign((size_t)NB * GS * 1024, 0);
        for (int rb = 0; rb < NB; rb++)
            for (int gs = 0; gs < GS; gs++) {
                uint16_t *blk = &out.zc[((size_t)rb * GS + gs) * 1024];
                for (int lane = 0; lane < 64; lane++)
                    for (int j = 0; j < 8; j++) {
                        const int n = rb * kBlockRows + lane % 16;
                        const int g = gs * 32 + 8 * (lane / 16) + j;
                        const float v = g < KB ? m.scale[(size_t)n * KB + g] * m.zero[(size_t)n * KB + g] / 128.0f : 0.0f;
                        const uint16_t hi = bf16_rne_bits(v);
                        const uint16_t lo = bf16_rne_bits(v - bf16_value(hi));
                        blk[lane * 8 + j] = hi;
                        blk[512 + lane * 8 + j] = lo;
                    }
            }
    }
}

PackSizes pack_sizes(int wformat, int N, int K) {
    const int df = dev_format(wformat);
    const size_t NB = (size_t)N / kBlockRows, KB = (size_t)K / kBlockK;
    PackSizes z;
    z.codes = NB * KB * (size_t)block_bytes(df);
    if (is_group_wformat(wformat)) {
        z.gscale = NB * KB * kBlockRows;
        if (df == DF_I4ASYM) {
            z.gzero = z.gscale;
            z.zc = NB * ((KB + 31) / 32) * 1024;
        }
    } else {
        z.pscale = (size_t)N;
    }
    return z;
}

void unlayout_matrix(int wformat, const PackedMatrix &p, CanonMatrix &m) {
    const int df = dev_format(wformat);
    const int bb = block_bytes(df);
    const int NB = m.N / kBlockRows, KB = m.K / kBlockK;
    const bool four_bit = bb == 1024;
    m.q.assign((size_t)m.N * m.K, 0);
    for (int rb = 0; rb < NB; rb++)
        for (int kb = 0; kb < KB; kb++) {
            const uint8_t *blk = &p.codes[((size_t)rb * KB + kb) * bb];
            for (int lane = 0; lane < 64; lane++) {
                const int r = rb * kBlockRows + lane % 16;
                for (int s = 0; s < 4; s++)
                    for (int j = 0; j < 8; j++) {
                        const int k = kb * kBlockK + 32 * s + 8 * (lane / 16) + j;
                        int8_t code;
                        if (four_bit) {
                            const uint32_t dw = *reinterpret_cast<const uint32_t *>(blk + lane * 16 + s * 4);
                            const int pos = (j % 2 == 0) ? 4 * (j / 2) : 16 + 4 * (j / 2);
                            const int u = (int)((dw >> pos) & 0xFu);
                            code = (int8_t)(df == DF_I4ASYM ? u : u - 8);
                        } else {
                            code = (int8_t)blk[lane * 32 + s * 8 + j];
                        }
                        m.q[(size_t)r * m.K + k] = code;
                    }
            }
        }
    if (is_group_wformat(wformat)) {
        m.scale.assign((size_t)m.N * KB, 0.0f);
        m.zero.assign((size_t)m.N * KB, 0.0f);
        for (int rb = 0; rb < NB; rb++)
            for (int kb = 0; kb < KB; kb++)
                for (int i = 0; i < kBlockRows; i++) {
                    const size_t dst = (size_t)(rb * kBlockRows + i) * KB + kb;
                    const size_t src = ((size_t)rb * KB + kb) * kBlockRows + i;
                    m.scale[dst] = half_from_bits(p.gscale[src]);
                    if (df == DF_I4ASYM) m.zero[dst] = half_from_bits(p.gzero[src]);
                }
    } else {
        m.scale.assign(p.pscale.begin(), p.pscale.end());
        m.zero.assign(m.scale.size(), 0.0f);
    }
}

}  // namespace qmoe
