// On-device expert quantizer: bf16 expert matrices in device memory become
// the packed arena layout that the host packer (qmoe_pack.cpp) writes, with
// the same rules (fp32 arithmetic, round half to even, the stored scale used
// for the codes, all-zero groups or rows with scale 1 and zero codes) and the
// same bytes. The expert quantizer of the Q-MoE page (section 3 components
// table), run where the weights already are.
//
// Layout reminder: a block holds 16 output rows x 128 input positions; lane l
// of a wave owns row l % 16 and positions 32 s + 8 (l / 16) + j (s < 4, j < 8)
// of the block: 4-bit formats 16 bytes (dword s, nibble j at bit 4 (j / 2) for
// even j, 16 + 4 (j / 2) for odd j), 8-bit formats 32 bytes. So one wave per
// block quantizes exactly the bytes each lane then stores.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "qmoe_internal.h"

// bit-exact with the host quantizer: no contraction of multiplies into adds
#pragma clang fp contract(off)

namespace qmoe {
namespace {

__device__ __forceinline__ float bf16_value_d(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// bf16 bits of a finite float, nearest even
__device__ __forceinline__ uint16_t bf16_rne_d(float v) {
    uint32_t u = __float_as_uint(v);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// nearest binary16 (ties to even) of v as a float, saturated at 65504
__device__ __forceinline__ float stored_half_d(float v) {
    const float r = (float)(_Float16)v;
    return isinf(r) ? (r > 0.0f ? 65504.0f : -65504.0f) : r;
}

__device__ __forceinline__ uint16_t half_bits_d(float exactly_representable) {
    return __builtin_bit_cast(uint16_t, (_Float16)exactly_representable);
}

// OCP e4m3fn code of v: 3 mantissa bits with round half to even, exponent bias
// 7, subnormal multiples of 2^-9 below 2^-6, magnitudes above 448 saturated
__device__ __forceinline__ uint8_t e4m3_code_d(float v) {
    const uint32_t b = __float_as_uint(v);
    const uint32_t sign = (b >> 24) & 0x80u;
    const uint32_t a = b & 0x7FFFFFFFu;
    if (a == 0) return (uint8_t)sign;
    int e = (int)(a >> 23) - 127;
    if (e >= -6) {
        const uint32_t mant = a & 0x7FFFFFu;
        uint32_t m = mant >> 20;
        const uint32_t rem = mant & 0xFFFFFu;
        if (rem > 0x80000u || (rem == 0x80000u && (m & 1u))) m++;
        if (m == 8) {
            m = 0;
            e++;
        }
        if (e > 8 || (e == 8 && m == 7)) return (uint8_t)(sign | 0x7Eu);
        return (uint8_t)(sign | ((uint32_t)(e + 7) << 3) | m);
    }
    const float t = rintf(fabsf(v) * 512.0f);   // units of 2^-9, exact scaling
    return (uint8_t)(sign | (uint32_t)t);
}

__device__ __forceinline__ float clamp_d(float v, float lo, float hi) { return fminf(fmaxf(v, lo), hi); }

// Source row of row r of the matrix being packed: W13 interleaves gate (even
// 16-row blocks) and up (odd); other matrices read `a` directly.
__device__ __forceinline__ const uint16_t *src_row(const uint16_t *a, const uint16_t *b, int interleave, int r,
                                                   int K) {
    if (!interleave) return a + (size_t)r * K;
    const int blk = r >> 4;
    return ((blk & 1) ? b : a) + ((size_t)(blk >> 1) * 16 + (r & 15)) * K;
}

// The 32 values lane `lane` owns in block (rb, kb).
__device__ __forceinline__ void load_lane(const uint16_t *row, int kb, int lane, float (&w)[32]) {
#pragma unroll
    for (int s = 0; s < 4; s++) {
        const uint4 v = *reinterpret_cast<const uint4 *>(row + kb * 128 + 32 * s + 8 * (lane >> 4));
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int h = 0; h < 4; h++) {
            w[8 * s + 2 * h] = bf16_value_d(u[h] & 0xFFFFu);
            w[8 * s + 2 * h + 1] = bf16_value_d(u[h] >> 16);
        }
    }
}

// Group formats: one wave per 16 x 128 block; the 128 values of a row's group
// sit in lanes i, i + 16, i + 32, i + 48.
template <int WF>
__global__ __launch_bounds__(256) void k_quant_group(const uint16_t *__restrict__ a, const uint16_t *__restrict__ b,
                                                     int interleave, int NB, int K, uint8_t *__restrict__ codes,
                                                     uint16_t *__restrict__ gscale, uint16_t *__restrict__ gzero,
                                                     uint16_t *__restrict__ zc) {
    // four waves per workgroup, one 16-row block each
    const int rb = blockIdx.x * 4 + (threadIdx.x >> 6), kb = blockIdx.y, KB = gridDim.y;
    if (rb >= NB) return;
    const int lane = threadIdx.x & 63, i = lane & 15;
    float w[32];
    load_lane(src_row(a, b, interleave, rb * 16 + i, K), kb, lane, w);
    // statistics in the host quantizer's comparison semantics (std::max /
    // std::min with the accumulator first; lo and hi start at +0)
    float amax = 0.0f, lo = 0.0f, hi = 0.0f;
#pragma unroll
    for (int t = 0; t < 32; t++) {
        const float x = w[t], ax = fabsf(x);
        amax = amax < ax ? ax : amax;
        lo = x < lo ? x : lo;
        hi = hi < x ? x : hi;
    }
#pragma unroll
    for (int off = 16; off < 64; off <<= 1) {
        const float oa = __shfl_xor(amax, off), ol = __shfl_xor(lo, off), oh = __shfl_xor(hi, off);
        amax = amax < oa ? oa : amax;
        lo = ol < lo ? ol : lo;
        hi = hi < oh ? oh : hi;
    }
    float s, z = 0.0f;
    if (WF == QMOE_W_INT4_ASYM_G128) {
        s = stored_half_d((hi - lo) / 15.0f);
        if (s != 0.0f) z = clamp_d(rintf(-lo / s), 0.0f, 15.0f) + 0.0f;
    } else {
        s = stored_half_d(amax / (WF == QMOE_W_INT4_SYM_G128 ? 7.0f : 3.0f));
    }
    const bool zero_codes = s == 0.0f;
    if (zero_codes) {
        s = 1.0f;
        z = 0.0f;
    }
    uint32_t dw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int t = 0; t < 32; t++) {
        const int sx = t >> 3, j = t & 7;
        int q = 0;
        if (!zero_codes) {
            const float r = rintf(w[t] / s);
            if (WF == QMOE_W_INT4_ASYM_G128) q = (int)clamp_d(r + z, 0.0f, 15.0f);
            else if (WF == QMOE_W_INT4_SYM_G128) q = (int)clamp_d(r, -8.0f, 7.0f);
            else q = (int)clamp_d(r, -4.0f, 3.0f);
        }
        const uint32_t u = (uint32_t)(WF == QMOE_W_INT4_ASYM_G128 ? q : q + 8) & 0xFu;
        dw[sx] |= u << ((j & 1) ? 16 + 4 * (j >> 1) : 4 * (j >> 1));
    }
    const size_t blk = (size_t)rb * KB + kb;
    *reinterpret_cast<uint4 *>(codes + blk * 1024 + lane * 16) = make_uint4(dw[0], dw[1], dw[2], dw[3]);
    if (lane < 16) {
        gscale[blk * 16 + i] = half_bits_d(s);
        if (WF == QMOE_W_INT4_ASYM_G128) {
            gzero[blk * 16 + i] = half_bits_d(z);
            // zero-point operand: s z / 128 as a bf16 pair (high, remainder) at
            // group kb of row rb * 16 + i in the 32-group block kb / 32
            const float v = s * z / 128.0f;
            const uint16_t vh = bf16_rne_d(v);
            const uint16_t vl = bf16_rne_d(v - bf16_value_d(vh));
            const int GS = (KB + 31) / 32, g = kb & 31;
            uint16_t *zb = zc + ((size_t)rb * GS + (kb >> 5)) * 1024;
            const int zl = (g >> 3) * 16 + i;
            zb[zl * 8 + (g & 7)] = vh;
            zb[512 + zl * 8 + (g & 7)] = vl;
        }
    }
}

// Per-channel formats, pass 1: the row scale amax / 127 (INT8) or amax / 448
// (FP8), one wave per row; rows whose scale is zero get scale 1 and a flag for
// zero codes.
template <int WF>
__global__ __launch_bounds__(256) void k_quant_rowscale(const uint16_t *__restrict__ a, const uint16_t *__restrict__ b,
                                                        int interleave, int N, int K, float *__restrict__ pscale,
                                                        uint8_t *__restrict__ zero_row) {
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= N) return;
    const uint16_t *row = src_row(a, b, interleave, r, K);
    float amax = 0.0f;
    for (int c = lane * 8; c < K; c += 512) {
        const uint4 v = *reinterpret_cast<const uint4 *>(row + c);
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int h = 0; h < 4; h++) {
            const float x0 = fabsf(bf16_value_d(u[h] & 0xFFFFu)), x1 = fabsf(bf16_value_d(u[h] >> 16));
            amax = amax < x0 ? x0 : amax;
            amax = amax < x1 ? x1 : amax;
        }
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_xor(amax, off);
        amax = amax < o ? o : amax;
    }
    if (lane == 0) {
        const float s = amax / (WF == QMOE_W_INT8_SYM_CH ? 127.0f : 448.0f);
        pscale[r] = s == 0.0f ? 1.0f : s;
        zero_row[r] = s == 0.0f;
    }
}

// Per-channel formats, pass 2: one wave per 16 x 128 block, 32 codes per lane.
template <int WF>
__global__ __launch_bounds__(256) void k_quant_chan(const uint16_t *__restrict__ a, const uint16_t *__restrict__ b,
                                                    int interleave, int NB, int K, const float *__restrict__ pscale,
                                                    const uint8_t *__restrict__ zero_row, uint8_t *__restrict__ codes) {
    const int rb = blockIdx.x * 4 + (threadIdx.x >> 6), kb = blockIdx.y, KB = gridDim.y;
    if (rb >= NB) return;
    const int lane = threadIdx.x & 63, r = rb * 16 + (lane & 15);
    float w[32];
    load_lane(src_row(a, b, interleave, r, K), kb, lane, w);
    const float s = pscale[r];
    const bool zero_codes = zero_row[r] != 0;
    uint32_t out[8];
#pragma unroll
    for (int t = 0; t < 8; t++) out[t] = 0u;
#pragma unroll
    for (int t = 0; t < 32; t++) {
        uint32_t c = 0u;
        if (!zero_codes) {
            const float x = w[t] / s;
            c = WF == QMOE_W_INT8_SYM_CH ? (uint32_t)(uint8_t)(int8_t)clamp_d(rintf(x), -127.0f, 127.0f)
                                         : (uint32_t)e4m3_code_d(x);
        }
        out[t >> 2] |= c << (8 * (t & 3));
    }
    uint4 *dst = reinterpret_cast<uint4 *>(codes + ((size_t)rb * KB + kb) * 2048 + lane * 32);
    dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
    dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
}

}  // namespace

hipError_t launch_quant_matrix(int wformat, const uint16_t *a, const uint16_t *b, int N, int K, uint8_t *codes,
                               uint16_t *gscale, uint16_t *gzero, float *pscale, uint16_t *zc, uint8_t *zero_row,
                               hipStream_t s) {
    const int il = b != nullptr;
    const int NB = N / 16;
    const dim3 blocks((NB + 3) / 4, K / 128);
    switch (wformat) {
    case QMOE_W_INT4_ASYM_G128:
        hipLaunchKernelGGL(k_quant_group<QMOE_W_INT4_ASYM_G128>, blocks, dim3(256), 0, s, a, b, il, NB, K, codes, gscale,
                           gzero, zc);
        break;
    case QMOE_W_INT4_SYM_G128:
        hipLaunchKernelGGL(k_quant_group<QMOE_W_INT4_SYM_G128>, blocks, dim3(256), 0, s, a, b, il, NB, K, codes, gscale,
                           gzero, zc);
        break;
    case QMOE_W_INT3_SYM_G128_IN4:
        hipLaunchKernelGGL(k_quant_group<QMOE_W_INT3_SYM_G128_IN4>, blocks, dim3(256), 0, s, a, b, il, NB, K, codes, gscale,
                           gzero, zc);
        break;
    case QMOE_W_INT8_SYM_CH:
        hipLaunchKernelGGL(k_quant_rowscale<QMOE_W_INT8_SYM_CH>, dim3((N + 3) / 4), dim3(256), 0, s, a, b, il, N, K,
                           pscale, zero_row);
        hipLaunchKernelGGL(k_quant_chan<QMOE_W_INT8_SYM_CH>, blocks, dim3(256), 0, s, a, b, il, NB, K, pscale, zero_row,
                           codes);
        break;
    case QMOE_W_FP8E4M3_CH:
        hipLaunchKernelGGL(k_quant_rowscale<QMOE_W_FP8E4M3_CH>, dim3((N + 3) / 4), dim3(256), 0, s, a, b, il, N, K,
                           pscale, zero_row);
        hipLaunchKernelGGL(k_quant_chan<QMOE_W_FP8E4M3_CH>, blocks, dim3(256), 0, s, a, b, il, NB, K, pscale, zero_row,
                           codes);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace qmoe
