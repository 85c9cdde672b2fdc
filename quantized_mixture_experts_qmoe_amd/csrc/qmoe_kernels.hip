// HIP kernels of the quantized top-k MoE layer for gfx950 (CDNA4).
//
//   router      logits = x . W_r^T (+ bias): bf16 MFMA with fp32 accumulation
//               (fp32 router weights: a plain fp32 dot-product kernel)
//   top-k       one wavefront per token: k rounds of a wave-wide maximum of
//               (logit, ~index) keys on DPP, lowest index wins ties; softmax
//               over the selection. Small batches: top-k and dispatch in one
//               workgroup
//   dispatch    expert-centric task list (OmniMoE page, technical summary 2.2:
//               collect tasks, group by expert id, token order inside a group):
//               per-chunk histogram -> scan + M-tile list -> stable scatter
//   xsum        per-token sums of x over 128-wide groups (offset correction)
//   gemm13      grouped gate/up GEMM over the task list: packed codes become
//               exact bf16 MFMA operands in registers (group scales applied in
//               fp32 per group), gathered token rows are staged in LDS,
//               SiLU(gate) * up is fused in the epilogue
//   gemm2       grouped down GEMM; the epilogue applies the mixing weight
//   combine     y_t = sum_j O[row(t, j)] + sum_s O_shared(t), fp32, bf16 out
#include <hip/hip_runtime.h>
#include <algorithm>
#include <cstdlib>
#include <mutex>
#include <type_traits>

#include "qmoe_internal.h"

namespace qmoe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ __forceinline__ uint16_t to_bf16(float f) {
    __bf16 h = (__bf16)f;   // round to nearest even (v_cvt_pk_bf16_f32)
    return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float half_bits_to_f32(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}
// Loads through the global address space (global_load rather than flat_load, so
// outstanding loads count only against vmcnt and never delay LDS waits).
template <typename T>
__device__ __forceinline__ T gload(const T *p) {
    return *(const __attribute__((address_space(1))) T *)p;
}
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 gload16(const void *p) {
    const u32x4 v = *(const __attribute__((address_space(1))) u32x4 *)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}
// bf16 hi + lo split of an fp32 value (hi = nearest bf16, lo = nearest bf16 of the rest).
__device__ __forceinline__ void split_bf16(float v, __bf16 &hi, __bf16 &lo) {
    hi = (__bf16)v;
    lo = (__bf16)(v - (float)hi);
}

// ---------------------------------------------------------------------------
// Asynchronous global -> LDS copies and raw waits
// ---------------------------------------------------------------------------

// s_waitcnt immediate (gfx9 encoding): wait until at most `vm` vector-memory
// operations are outstanding and all LDS operations have completed.
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(VM >= 0 && VM < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | (0 << 8) | ((VM >> 4) << 14));
}
// Wait until at most n groups of CPW copies each are outstanding (n uniform,
// at most NMAX): s_waitcnt takes only an immediate count.
template <int CPW, int NMAX>
__device__ __forceinline__ void wait_groups(int n) {
    if constexpr (NMAX > 0) {
        if (n >= NMAX) {
            wait_vm_lgkm0<NMAX * CPW>();
            return;
        }
        wait_groups<CPW, NMAX - 1>(n);
    } else {
        wait_vm_lgkm0<0>();
    }
}
// Workgroup barrier without the compiler's fence (which would drain every
// outstanding load); the memory clobber keeps LDS accesses on their side.
__device__ __forceinline__ void raw_barrier() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}
// Global -> LDS copies (16 or 4 bytes per lane; LDS destination in M0)
// addressed as a wave-uniform 64-bit base in SGPRs plus a 32-bit per-lane
// byte offset: advancing through K moves only the scalar base.
__device__ __forceinline__ void dma16s(const void *sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma4s(const void *sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(lds)
                 : "memory", "m0");
}

// ---------------------------------------------------------------------------
// Router
// ---------------------------------------------------------------------------

// Selection helpers used by the router's fused epilogue (defined with the
// gating network below).
__device__ __forceinline__ uint32_t ord_u32(float v);
__device__ __forceinline__ float ord_value(uint32_t u);
template <int EPL16>
__device__ __forceinline__ void topk_row16(const float *__restrict__ lt, int E, int k, int renorm, int lane,
                                           int &my_e, float &my_w);

// Sum over each 16-lane row of a wave, in the row's last lane (DPP row
// shifts: no LDS round trip, unlike a lane shuffle).
__device__ __forceinline__ float row16_sum_last(float v) {
    auto step = [](float x, auto ctrl) {
        return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                         decltype(ctrl)::value, 0xF, 0xF, true));
    };
    v = step(v, std::integral_constant<int, 0x111>{});   // row_shr:1
    v = step(v, std::integral_constant<int, 0x112>{});   // row_shr:2
    v = step(v, std::integral_constant<int, 0x114>{});   // row_shr:4
    v = step(v, std::integral_constant<int, 0x118>{});   // row_shr:8
    return v;
}

// Router for larger batches: a tile of BT tokens x BE experts per workgroup.
// The x rows and router rows of each 128-wide K group are copied into LDS with
// asynchronous global -> LDS copies, whole 256-byte row segments per 16 lanes
// (fragment-shaped global loads of 64 bytes per row run at a third of the L2
// bandwidth), XOR-swizzled (chunk c of row r at c ^ (r & 15)) so the MFMA
// fragment reads are conflict-free, NST groups in flight.
//   WE > 1 (shared): the waves split the tile's experts WE ways and copy each
//     group together, one barrier per group.
//   WE = 1 (streams): every wave computes the whole tile over every fourth
//     group, staged in its own LDS ring with no barrier; the four partial
//     tiles are added through LDS at the end.
// Workgroups of the first expert tile also emit the per-group row sums of x
// (times xscale) read from the staged tile.
// FUSE (one expert tile holds all E experts, k <= 16): the gating network runs
// in the epilogue on the tile's logits staged in LDS (Q-MoE page, section 3:
// the gating network's top-k; weights: softmax over the selection): each
// 16-lane row of a wave selects one token's top k (DPP row maxima, ties to
// the lower expert index) and writes idx, w; the workgroup then writes the
// tile's per-expert task counts (its BT*k tasks are one dispatch chunk).
// Logits go to memory only when `logits` is given.
template <int BT, int BE, int WE, int NST, bool FUSE>
__global__ __launch_bounds__(256) void k_router_lds(const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr,
                                                    const float *__restrict__ rscale,
                                                    const float *__restrict__ bias, float *__restrict__ logits,
                                                    float *__restrict__ xsum, float xscale, int T, int d, int E,
                                                    int net, RouteFuse rf) {
    constexpr bool STREAMS = WE == 1;
    static_assert(WE == 1 || WE == 4, "four waves: streams or a four-way expert split");
    constexpr int MT = BT / 16, NT = BE / (16 * WE);
    static_assert(MT * 16 == BT && NT * 16 * WE == BE, "whole 16-blocks per wave");
    constexpr int ROWS = BT + BE;                       // staged rows per group, x first
    constexpr int CPW = STREAMS ? ROWS / 4 : ROWS / 16;   // 1 KB copies per wave per group
    static_assert(ROWS % (STREAMS ? 4 : 16) == 0, "whole 4-row copies per wave");
    constexpr int ST = ROWS * 256;                      // bytes per stage
    constexpr int RINGS = STREAMS ? 4 : 1;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[RINGS * NST * ST + (STREAMS ? 3 * MT * NT * 1024 : 0)];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // one-dimensional grid of net expert tiles x token tiles (padded to a
    // multiple of 8), numbered XCD-aware: workgroup L runs on XCD L % 8, and
    // the expert tiles of one token tile are consecutive workgroups of one XCD,
    // so its L2 fetches the tile's x rows once
    const int L = blockIdx.x;
    const int xcd = L & 7, j = L >> 3;
    const int et = j % net, tt = (j / net) * 8 + xcd;
    const int t0 = tt * BT;
    const int e0 = et * BE;
    if (t0 >= T) return;
    const uint32_t ring0 = lds_addr(lds) + (STREAMS ? wave * NST * ST : 0);
    const uint8_t *ringp = lds + (STREAMS ? wave * NST * ST : 0);
    const int G = d / 128;
    // groups this wave takes: all (shared) or wave, wave + 4, ... (streams)
    const int gstep = STREAMS ? 4 : 1, gfirst = STREAMS ? wave : 0;
    const int ng = STREAMS ? (G - wave + 3) / 4 : G;

    // copy sources: 4-row slabs, each wholly x or wholly router rows, as the
    // tile's first row in SGPRs plus a per-lane byte offset below 256 * d;
    // rows past T / E read the tile's first row (their results are not stored)
    uint32_t soff[CPW];
    const uint16_t *sbase[CPW];
    const uint16_t *xt = x + (size_t)t0 * d, *wt0 = wr + (size_t)e0 * d;
    const int slab0 = STREAMS ? 0 : CPW * wave;
#pragma unroll
    for (int i = 0; i < CPW; i++) {
        const int row = 4 * (slab0 + i) + (lane >> 4);   // staged row
        const int sw = ((lane & 15) ^ (row & 15)) * 16;   // source chunk of this lane's LDS slot
        const bool is_x = 4 * (slab0 + i) < BT;           // uniform over the slab
        const int r = is_x ? row : row - BT;
        const bool ok = is_x ? t0 + r < T : e0 + r < E;
        sbase[i] = is_x ? xt : wt0;
        soff[i] = (uint32_t)(ok ? r : 0) * (uint32_t)d * 2u + (uint32_t)sw;
    }
    // copies of this wave's q-th group (clamped to its last) into stage st
    auto issue = [&](int q, int st) {
        const int g = gfirst + gstep * min(q, ng - 1);
        const uint32_t sb = ring0 + st * ST;
#pragma unroll
        for (int i = 0; i < CPW; i++)
            dma16s(reinterpret_cast<const uint8_t *>(sbase[i]) + g * 256, soff[i], sb + (slab0 + i) * 1024);
    };

    f32x4 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; i++)
#pragma unroll
        for (int jj = 0; jj < NT; jj++) acc[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
    const bool do_sum = xsum != nullptr && et == 0;
    const int we = STREAMS ? 0 : wave;

    // MFMAs (and the row sums) of this wave's q-th group, staged in stage st
    auto group = [&](int q, int st) __attribute__((always_inline)) {
        const uint16_t *S = reinterpret_cast<const uint16_t *>(ringp + st * ST);
#pragma unroll
        for (int s = 0; s < 4; s++) {
            const int pc = (s * 4 + (lane >> 4)) ^ (lane & 15);
            bf16x8 af[MT], bfr[NT];
#pragma unroll
            for (int i = 0; i < MT; i++)
                af[i] = *reinterpret_cast<const bf16x8 *>(&S[(16 * i + (lane & 15)) * 128 + pc * 8]);
#pragma unroll
            for (int jj = 0; jj < NT; jj++)
                bfr[jj] = *reinterpret_cast<const bf16x8 *>(&S[(BT + 16 * (we * NT + jj) + (lane & 15)) * 128 + pc * 8]);
#pragma unroll
            for (int i = 0; i < MT; i++)
#pragma unroll
                for (int jj = 0; jj < NT; jj++)
                    acc[i][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[jj], acc[i][jj], 0, 0, 0);
        }
        if (do_sum) {
            // 16 lanes per staged x row, one 16-byte chunk each; in shared
            // mode the workgroup's threads split the rows, in streams mode
            // each wave sums its own group
            const int g = gfirst + gstep * q;
            constexpr int NTH = STREAMS ? 64 : 256;
            const int tid = STREAMS ? lane : (int)threadIdx.x;
#pragma unroll
            for (int c0 = 0; c0 < BT * 16; c0 += NTH) {
                const int c = c0 + tid;
                const int row = c >> 4;
                const uint4 q4 = *reinterpret_cast<const uint4 *>(&S[row * 128 + ((c & 15) ^ (row & 15)) * 8]);
                const uint32_t qq[4] = {q4.x, q4.y, q4.z, q4.w};
                float v = 0.0f;
#pragma unroll
                for (int k = 0; k < 4; k++) v += bf16f(qq[k] & 0xFFFFu) + bf16f(qq[k] >> 16);
                // the 16 chunks of a row are one 16-lane DPP row (c & 15 = lane & 15)
                v = row16_sum_last(v);
                const int t = t0 + row;
                if ((c & 15) == 15 && t < T) xsum[(size_t)t * G + g] = v * xscale;
            }
        }
    };
    if (STREAMS && ng <= NST) {
        // a stream whose groups all fit its ring (small batches): every copy
        // in flight at once, then the waits count down group by group
        for (int q = 0; q < ng; q++) issue(q, q);
        for (int q = 0; q < ng; q++) {
            wait_groups<CPW, NST - 1>(ng - 1 - q);
            group(q, q);
        }
        __builtin_amdgcn_s_waitcnt(0);
    } else if (ng > 0) {   // uniform; a stream with no group (G < 4) only adds zeros
#pragma unroll
        for (int p = 0; p < NST - 1; p++) issue(p, p);
        for (int q = 0; q < ng; q++) {
            wait_vm_lgkm0<(NST - 2) * CPW>();
            if constexpr (!STREAMS) raw_barrier();
            // refill the stage read one group ago (in shared mode every wave
            // passed this group's barrier, so all are done with it)
            issue(q + NST - 1, (q + NST - 1) % NST);
            group(q, q % NST);
        }
        // no copy may still be writing LDS when the ring is reused or freed
        __builtin_amdgcn_s_waitcnt(0);
    }

    if constexpr (STREAMS) {
        f32x4 *red = reinterpret_cast<f32x4 *>(lds + RINGS * NST * ST);
        if (wave > 0) {
#pragma unroll
            for (int i = 0; i < MT; i++)
#pragma unroll
                for (int jj = 0; jj < NT; jj++) red[((wave - 1) * MT * NT + i * NT + jj) * 64 + lane] = acc[i][jj];
        }
        __syncthreads();
        if (wave > 0) return;
#pragma unroll
        for (int w = 0; w < 3; w++)
#pragma unroll
            for (int i = 0; i < MT; i++)
#pragma unroll
                for (int jj = 0; jj < NT; jj++) acc[i][jj] += red[(w * MT * NT + i * NT + jj) * 64 + lane];
    } else if constexpr (FUSE) {
        __syncthreads();   // every wave's copies have landed: the ring is free
    }
    // staged logits of the tile (FUSE): [BT][LP] fp32 over the free ring, then
    // the per-expert task counts
    constexpr int LP = BE + 1;
    float *Ls = reinterpret_cast<float *>(lds);
    int *cnt = reinterpret_cast<int *>(lds + BT * LP * 4);
    static_assert(!FUSE || BT * LP * 4 + BE * 4 <= RINGS * NST * ST, "the logit tile fits in the ring");
    if constexpr (FUSE) {
        for (int e = STREAMS ? lane : (int)threadIdx.x; e < BE; e += STREAMS ? 64 : 256) cnt[e] = 0;
    }
#pragma unroll
    for (int jj = 0; jj < NT; jj++) {
        const int el = 16 * (we * NT + jj) + (lane & 15);
        const int e = e0 + el;
        if (e >= E) continue;
        const float b = bias ? bias[e] : 0.0f;
        const float sc = rscale ? rscale[e] : 1.0f;
#pragma unroll
        for (int i = 0; i < MT; i++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int tr = 16 * i + (lane >> 4) * 4 + r;
                const float lv = acc[i][jj][r] * sc + b;
                if (FUSE) Ls[tr * LP + el] = lv;
                if (logits && t0 + tr < T) logits[(size_t)(t0 + tr) * E + e] = lv;
            }
    }
    if constexpr (FUSE) {
        // (streams mode: one wave left, whose LDS accesses stay in order)
        if constexpr (!STREAMS) __syncthreads();
        // 16-lane rows over the tile's tokens: row g of wave w is row 4w + g
        constexpr int NROWS = STREAMS ? 4 : 16;
        const int row0 = (STREAMS ? 0 : 4 * wave) + (lane >> 4);
        for (int tr = row0; tr < BT; tr += NROWS) {
            const int t = t0 + tr;
            int my_e;
            float my_w;
            topk_row16<BE / 16>(Ls + tr * LP, E, rf.k, rf.renorm, lane, my_e, my_w);
            if (t < T && (lane & 15) < rf.k) {
                rf.idx[(size_t)t * rf.k + (lane & 15)] = my_e;
                rf.w[(size_t)t * rf.k + (lane & 15)] = my_w;
                atomicAdd(&cnt[my_e], 1);
            }
        }
        if constexpr (!STREAMS) __syncthreads();
        const int tt = t0 / BT;
        for (int e = STREAMS ? lane : (int)threadIdx.x; e < E; e += STREAMS ? 64 : 256)
            rf.chunk_counts[(size_t)tt * E + e] = cnt[e];
    }
}

__device__ __forceinline__ float wave_sum_f32(float v);   // DPP wave reduction, with the top-k helpers below

__global__ __launch_bounds__(256) void k_router_f32(const uint16_t *__restrict__ x, const float *__restrict__ wr,
                                                    const float *__restrict__ bias, float *__restrict__ logits, int T,
                                                    int d, int E) {
    // one wave per token: lane l takes columns [4l + 256j, 4l + 256j + 4) of x
    // and of each router row (d % 256 == 0), four experts at a time; the
    // partial dots are summed across the wave on DPP
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const uint16_t *xr = x + (size_t)t * d + 4 * lane;
    for (int e0 = 0; e0 < E; e0 += 4) {
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int c = 0; c < d; c += 256) {
            const uint2 xv = *reinterpret_cast<const uint2 *>(xr + c);
            const float x0 = bf16f(xv.x & 0xFFFFu), x1 = bf16f(xv.x >> 16);
            const float x2 = bf16f(xv.y & 0xFFFFu), x3 = bf16f(xv.y >> 16);
#pragma unroll
            for (int u = 0; u < 4; u++) {
                if (e0 + u < E) {
                    const float4 w = *reinterpret_cast<const float4 *>(wr + (size_t)(e0 + u) * d + c + 4 * lane);
                    acc[u] = fmaf(x0, w.x, acc[u]);
                    acc[u] = fmaf(x1, w.y, acc[u]);
                    acc[u] = fmaf(x2, w.z, acc[u]);
                    acc[u] = fmaf(x3, w.w, acc[u]);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < 4; u++) {
            if (e0 + u >= E) break;
            const float sum = wave_sum_f32(acc[u]);
            if (lane == 0) logits[(size_t)t * E + e0 + u] = sum + (bias ? bias[e0 + u] : 0.0f);
        }
    }
}


// ---------------------------------------------------------------------------
// Top-k + softmax weights (gating network)
// ---------------------------------------------------------------------------

// Wave-wide reductions on DPP (row shifts within 16-lane rows, then the
// row-15 and row-31 broadcasts): each step is a VALU op, not an LDS round trip.
// After the six steps lane 63 holds the result.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_zero(float v) {         // lanes without a source read 0
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, true));
}
constexpr int kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114, kDppShr8 = 0x118;
constexpr int kDppBcast15 = 0x142, kDppBcast31 = 0x143;

__device__ __forceinline__ float wave_sum_f32(float v) {
    v += dpp_zero<kDppShr1, 0xF>(v);
    v += dpp_zero<kDppShr2, 0xF>(v);
    v += dpp_zero<kDppShr4, 0xF>(v);
    v += dpp_zero<kDppShr8, 0xF>(v);
    v += dpp_zero<kDppBcast15, 0xA>(v);
    v += dpp_zero<kDppBcast31, 0xC>(v);
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
// Sum over each 16-lane row; the total lands in the row's lane 15.
__device__ __forceinline__ float row16_sum_f32(float v) {
    v += dpp_zero<kDppShr1, 0xF>(v);
    v += dpp_zero<kDppShr2, 0xF>(v);
    v += dpp_zero<kDppShr4, 0xF>(v);
    v += dpp_zero<kDppShr8, 0xF>(v);
    return v;
}
// SwiGLU gate: silu(g) * u = g / (1 + e^-g) * u with the hardware reciprocal
// (about 1 ulp of fp32; the product is rounded to bf16 right after)
__device__ __forceinline__ float silu_mul(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}
// Inclusive prefix sum over the wave (lane i: sum of lanes 0..i).
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, kDppShr1, 0xF, 0xF, true);
    v += __builtin_amdgcn_update_dpp(0, v, kDppShr2, 0xF, 0xF, true);
    v += __builtin_amdgcn_update_dpp(0, v, kDppShr4, 0xF, 0xF, true);
    v += __builtin_amdgcn_update_dpp(0, v, kDppShr8, 0xF, 0xF, true);
    v += __builtin_amdgcn_update_dpp(0, v, kDppBcast15, 0xA, 0xF, true);
    v += __builtin_amdgcn_update_dpp(0, v, kDppBcast31, 0xC, 0xF, true);
    return v;
}

// Selection order: larger logit first, ties to the lower index. Values are
// compared as an order-preserving 32-bit image of the finite fp32 value (+0.0
// and -0.0 equal); every image is above 0, which marks an empty or taken entry.
__device__ __forceinline__ uint32_t ord_u32(float v) {
    const uint32_t u = __float_as_uint(v + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ord_value(uint32_t u) {
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}
// lanes without a source read 0, which is below every image (the step then
// keeps the lane's own value); this form lets the shift fold into the max
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t max_step32(uint32_t v) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, true);
    return o > v ? o : v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max_step32<kDppShr1, 0xF>(v);
    v = max_step32<kDppShr2, 0xF>(v);
    v = max_step32<kDppShr4, 0xF>(v);
    v = max_step32<kDppShr8, 0xF>(v);
    v = max_step32<kDppBcast15, 0xA>(v);
    v = max_step32<kDppBcast31, 0xC>(v);
    return __builtin_amdgcn_readlane(v, 63);
}
// One selection round over entries hv[i] of index lane + 64 i: the largest
// value, ties to the lowest index (the first entry slot i with a match, then
// its lowest lane, from ballots). Takes the winner out (sets it to 0) and
// returns its index (wave-uniform); vmax receives its value image.
template <int EPL>
__device__ __forceinline__ int wave_take_max(uint32_t (&hv)[EPL], int lane, uint32_t &vmax) {
    uint32_t m = hv[0];
#pragma unroll
    for (int i = 1; i < EPL; i++) m = hv[i] > m ? hv[i] : m;
    vmax = wave_max_u32(m);
    int win = -1;
#pragma unroll
    for (int i = 0; i < EPL; i++) {
        const unsigned long long hit = __ballot(hv[i] == vmax);
        if (win < 0 && hit) win = 64 * i + __ffsll(hit) - 1;
    }
#pragma unroll
    for (int i = 0; i < EPL; i++)
        if (lane + 64 * i == win) hv[i] = 0u;
    return win;
}

// Top-k of one token by one wavefront: k selection rounds (largest logit,
// ties to the lower expert index); lane j ends holding slot j. Weights: softmax over the k selected logits
// (renorm) or the full-softmax probabilities of the selected. Writes
// idx_out[0..k) and w_out[0..k); returns this lane's expert (slot = lane) or -1
// for lanes >= k, and this lane's weight in my_w.
template <int EPL>
__device__ __forceinline__ int topk_token(const float *__restrict__ lt, int E, int k, int renorm, int lane,
                                          int32_t *__restrict__ idx_out, float *__restrict__ w_out, float &my_w) {
    float v[EPL];
    uint32_t hv[EPL];
#pragma unroll
    for (int i = 0; i < EPL; i++) {
        const int e = lane + 64 * i;
        v[i] = e < E ? lt[e] : 0.0f;
        hv[i] = e < E ? ord_u32(v[i]) : 0u;
    }
    int my_e = -1;
    uint32_t my_h = 0u, first_h = 0u;
    for (int j = 0; j < k; j++) {
        uint32_t vm;
        const int e = wave_take_max<EPL>(hv, lane, vm);
        if (lane == j) {
            my_e = e;
            my_h = vm;
        }
        if (j == 0) first_h = vm;
    }
    const float vmax = ord_value(first_h);
    const float ex = lane < k ? expf(ord_value(my_h) - vmax) : 0.0f;
    float part;
    if (renorm) {
        part = ex;
    } else {
        part = 0.0f;
#pragma unroll
        for (int i = 0; i < EPL; i++)
            if (lane + 64 * i < E) part += expf(v[i] - vmax);
    }
    const float denom = wave_sum_f32(part);
    my_w = ex / denom;
    if (lane < k) {
        idx_out[lane] = my_e;
        w_out[lane] = my_w;
        return my_e;
    }
    return -1;
}

// Row maximum over a 16-lane row, in every lane of the row: four rotate-and-max
// steps (DPP row_ror 1, 2, 4, 8).
constexpr int kDppRor1 = 0x121, kDppRor2 = 0x122, kDppRor4 = 0x124, kDppRor8 = 0x128;
template <int CTRL>
__device__ __forceinline__ uint32_t ror_max(uint32_t v) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
    return o > v ? o : v;
}
template <int CTRL>
__device__ __forceinline__ float ror_add(float v) {
    return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Top-k of one token by one 16-lane row (the router's fused epilogue): entry e
// of lt[0..E) is held by lane e % 16 of the row (EPL16 entries per lane); k <=
// 16 selection rounds (largest logit, ties to the lower expert index); lane
// j < k of the row ends holding slot j's expert and weight (softmax over the k
// selected, or the full-softmax probability when renorm = 0).
template <int EPL16>
__device__ __forceinline__ void topk_row16(const float *__restrict__ lt, int E, int k, int renorm, int lane,
                                           int &my_e, float &my_w) {
    const int l16 = lane & 15, rshift = lane & 48;
    float v[EPL16];
    uint32_t hv[EPL16];
#pragma unroll
    for (int i = 0; i < EPL16; i++) {
        const int e = l16 + 16 * i;
        v[i] = e < E ? lt[e] : 0.0f;
        hv[i] = e < E ? ord_u32(v[i]) : 0u;
    }
    my_e = -1;
    uint32_t my_h = 0u, first_h = 0u;
    for (int j = 0; j < k; j++) {
        uint32_t m = hv[0];
#pragma unroll
        for (int i = 1; i < EPL16; i++) m = hv[i] > m ? hv[i] : m;
        m = ror_max<kDppRor1>(m);
        m = ror_max<kDppRor2>(m);
        m = ror_max<kDppRor4>(m);
        m = ror_max<kDppRor8>(m);
        // the first entry slot holding the maximum, then its lowest lane
        int win = -1;
#pragma unroll
        for (int i = 0; i < EPL16; i++) {
            const uint32_t bits = (uint32_t)(__ballot(hv[i] == m) >> rshift) & 0xFFFFu;
            if (win < 0 && bits) win = 16 * i + __builtin_ctz(bits);
        }
#pragma unroll
        for (int i = 0; i < EPL16; i++)
            if (l16 + 16 * i == win) hv[i] = 0u;
        if (l16 == j) {
            my_e = win;
            my_h = m;
        }
        if (j == 0) first_h = m;
    }
    const float vmax = ord_value(first_h);
    const float ex = l16 < k ? expf(ord_value(my_h) - vmax) : 0.0f;
    float part;
    if (renorm) {
        part = ex;
    } else {
        part = 0.0f;
#pragma unroll
        for (int i = 0; i < EPL16; i++)
            if (l16 + 16 * i < E) part += expf(v[i] - vmax);
    }
    part = ror_add<kDppRor1>(part);
    part = ror_add<kDppRor2>(part);
    part = ror_add<kDppRor4>(part);
    part = ror_add<kDppRor8>(part);
    my_w = ex / part;
}

template <int EPL>
__global__ __launch_bounds__(256) void k_topk(const float *__restrict__ logits, int T, int E, int k, int renorm,
                                              int32_t *__restrict__ idx, float *__restrict__ w) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;   // uniform per wave
    float my_w;
    topk_token<EPL>(logits + (size_t)t * E, E, k, renorm, lane, idx + (size_t)t * k, w + (size_t)t * k, my_w);
}

// ---------------------------------------------------------------------------
// Dispatch: expert-centric task list
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_dispatch_count(const int32_t *__restrict__ idx, int P, int E,
                                                        int32_t *__restrict__ chunk_counts) {
    extern __shared__ int cnt[];
    for (int e = threadIdx.x; e < E; e += 256) cnt[e] = 0;
    __syncthreads();
    const int p0 = blockIdx.x * kDispatchChunk;
    for (int i = threadIdx.x; i < kDispatchChunk; i += 256) {
        const int p = p0 + i;
        if (p < P) atomicAdd(&cnt[idx[p]], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) chunk_counts[(size_t)blockIdx.x * E + e] = cnt[e];
}

// Exclusive scan over a 1024-thread workgroup (16 waves): DPP scans inside the
// waves, then one wave scans the 16 wave totals.
__device__ int block_exclusive_scan_1024(int v, int *wsum) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int incl = wave_incl_scan(v);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        const int s = lane < 16 ? wsum[lane] : 0;
        const int si = wave_incl_scan(s);
        if (lane < 16) wsum[16 + lane] = si - s;   // exclusive wave bases
    }
    __syncthreads();
    const int r = wsum[16 + wave] + incl - v;
    __syncthreads();
    return r;
}

// One workgroup of 1024 threads; G = 1024 / next_pow2(E) threads per expert
// (thread g * next_pow2(E) + e, so that neighbouring threads read neighbouring
// experts of one chunk: the chunk counts are [chunk][E]), each owning a
// contiguous range of chunks. One exclusive scan of the range sums in
// (expert, range) order, through LDS, gives every range's first row directly
// -- the expert's offset plus the rows of its earlier ranges -- and the
// experts' offsets and counts with it; a second scan places the tiles.
__global__ __launch_bounds__(1024) void k_dispatch_scan(const int32_t *__restrict__ cc, int nchunks, int E, int P,
                                                        int T, int n_shared, int bm, int32_t *__restrict__ chunk_base,
                                                        int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                                        Tile *__restrict__ tiles, int32_t *__restrict__ num_tiles) {
    __shared__ int wsum[32];
    __shared__ int ebase[1025];
    __shared__ int xs[1024];
    int E2 = 1;
    while (E2 < E) E2 <<= 1;
    const int G = 1024 / E2;
    const int tid = threadIdx.x, e = tid % E2, g = tid / E2;
    const bool live = e < E;
    const int b0 = (int)((long)nchunks * g / G), b1 = (int)((long)nchunks * (g + 1) / G);
    // ranges of up to kScanRegs chunks are loaded all at once into registers
    // (every load in flight together; reused for the chunk bases below)
    constexpr int kScanRegs = 32;
    const bool in_regs = b1 - b0 <= kScanRegs;
    int cv[kScanRegs];
    int s = 0;
    if (in_regs) {
#pragma unroll
        for (int i = 0; i < kScanRegs; i++) cv[i] = (live && b0 + i < b1) ? cc[(size_t)(b0 + i) * E + e] : 0;
#pragma unroll
        for (int i = 0; i < kScanRegs; i++) s += cv[i];
    } else if (live) {
        int b = b0;
        for (; b + 4 <= b1; b += 4) {
            const int v0 = cc[(size_t)b * E + e], v1 = cc[(size_t)(b + 1) * E + e];
            const int v2 = cc[(size_t)(b + 2) * E + e], v3 = cc[(size_t)(b + 3) * E + e];
            s += (v0 + v1) + (v2 + v3);
        }
        for (; b < b1; b++) s += cc[(size_t)b * E + e];
    }
    // the range sums in (expert, range) order
    xs[e * G + g] = s;
    __syncthreads();
    const int v = xs[tid];
    const int vx = block_exclusive_scan_1024(v, wsum);   // ends with a barrier: every xs read is done
    xs[tid] = vx;
    __syncthreads();
    const int first_row = xs[e * G + g];
    if (live && g == 0) ebase[e] = first_row;
    if (tid == 0) ebase[E] = P;
    __syncthreads();
    const int cnt = (live && g == 0) ? ebase[e + 1] - first_row : 0;
    const int ntile = (cnt + bm - 1) / bm;
    const int tile_base = block_exclusive_scan_1024(ntile, wsum);
    if (live && g == 0) {
        counts[e] = cnt;
        offsets[e] = first_row;
        for (int m = 0; m < cnt; m += bm) tiles[tile_base + m / bm] = Tile{e, first_row + m, first_row + cnt, 0};
    }
    if (live && in_regs) {
        int run = first_row;
#pragma unroll
        for (int i = 0; i < kScanRegs; i++)
            if (b0 + i < b1) {
                chunk_base[(size_t)(b0 + i) * E + e] = run;
                run += cv[i];
            }
    } else if (live) {
        int run = first_row;
        for (int b = b0; b < b1; b++) {
            chunk_base[(size_t)b * E + e] = run;
            run += cc[(size_t)b * E + e];
        }
    }
    // the last expert's first thread knows the routed tile total
    if (live && g == 0 && e == E - 1) {
        offsets[E] = P;
        int tcount = tile_base + ntile;
        for (int sh = 0; sh < n_shared; sh++)
            for (int m = 0; m < T; m += bm) tiles[tcount++] = Tile{E + sh, P + sh * T + m, P + (sh + 1) * T, 0};
        *num_tiles = tcount;
    }
}

// Stable scatter: ranks inside a chunk (`chunk` consecutive pairs) follow pair
// order. Each round takes 256 consecutive pairs; ranks inside a wave come from
// per-expert 64-bit lane masks.
__global__ __launch_bounds__(256) void k_dispatch_scatter(const int32_t *__restrict__ idx, const float *__restrict__ w,
                                                          int P, int E, int chunk,
                                                          const int32_t *__restrict__ chunk_base,
                                                          int32_t *__restrict__ perm, int32_t *__restrict__ inv,
                                                          float *__restrict__ wrow) {
    extern __shared__ unsigned long long smem64[];
    unsigned long long *masks = smem64;                       // [4][E]
    int *running = reinterpret_cast<int *>(smem64 + 4 * E);  // [E]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int e = threadIdx.x; e < E; e += 256) {
        running[e] = chunk_base[(size_t)blockIdx.x * E + e];
        masks[e] = masks[E + e] = masks[2 * E + e] = masks[3 * E + e] = 0ull;
    }
    __syncthreads();
    const int c0 = blockIdx.x * chunk;
    for (int r0 = 0; r0 < chunk; r0 += 256) {
        const int p = c0 + r0 + threadIdx.x;
        const bool valid = r0 + (int)threadIdx.x < chunk && p < P;
        const int e = valid ? idx[p] : 0;
        const float wp = valid ? w[p] : 0.0f;
        if (valid) atomicOr(&masks[wave * E + e], 1ull << lane);
        __syncthreads();
        if (valid) {
            int rank = __popcll(masks[wave * E + e] & ((1ull << lane) - 1ull));
            for (int w2 = 0; w2 < wave; w2++) rank += __popcll(masks[w2 * E + e]);
            const int row = running[e] + rank;
            perm[row] = p;
            inv[p] = row;
            wrow[row] = wp;
        }
        __syncthreads();
        for (int e2 = threadIdx.x; e2 < E; e2 += 256) {
            running[e2] += __popcll(masks[e2]) + __popcll(masks[E + e2]) + __popcll(masks[2 * E + e2]) +
                           __popcll(masks[3 * E + e2]);
            masks[e2] = masks[E + e2] = masks[2 * E + e2] = masks[3 * E + e2] = 0ull;
        }
        __syncthreads();
    }
}

// Small batches (T <= 64, E <= 256): top-k and the whole dispatch (histogram,
// scan, tile list, stable scatter) in one workgroup of 16 waves, with the same
// outputs as k_topk followed by the three dispatch kernels.
struct RouteSmallSmem {
    int sidx[kSmallRouteMaxT * 64];
    float sw[kSmallRouteMaxT * 64];
    unsigned long long masks[16][kSmallRouteMaxE];
    int base[kSmallRouteMaxE];
    int wsum[32];
};

template <int EPL>
__device__ void route_small_body(RouteSmallSmem &sm, const float *__restrict__ logits, int T, int E, int k,
                                 int renorm, int n_shared, int bm, int32_t *__restrict__ idx, float *__restrict__ w,
                                 int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                 Tile *__restrict__ tiles, int32_t *__restrict__ num_tiles,
                                 int32_t *__restrict__ perm, int32_t *__restrict__ inv, float *__restrict__ wrow) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int P = T * k;
    for (int e = tid; e < E; e += 1024) sm.base[e] = 0;
    for (int i = tid; i < 16 * kSmallRouteMaxE; i += 1024) (&sm.masks[0][0])[i] = 0ull;
    __syncthreads();
    for (int t = wave; t < T; t += 16) {
        float my_w;
        const int e = topk_token<EPL>(logits + (size_t)t * E, E, k, renorm, lane, idx + (size_t)t * k,
                                      w + (size_t)t * k, my_w);
        if (e >= 0) {
            sm.sidx[t * k + lane] = e;
            sm.sw[t * k + lane] = my_w;
            atomicAdd(&sm.base[e], 1);
        }
    }
    __syncthreads();
    // thread e owns expert e
    const int cnt = tid < E ? sm.base[tid] : 0;
    const int ntile = (cnt + bm - 1) / bm;
    const int row0 = block_exclusive_scan_1024(cnt, sm.wsum);
    const int tile0 = block_exclusive_scan_1024(ntile, sm.wsum);
    if (tid < E) {
        counts[tid] = cnt;
        offsets[tid] = row0;
        for (int m = 0; m < cnt; m += bm) tiles[tile0 + m / bm] = Tile{tid, row0 + m, row0 + cnt, 0};
        sm.base[tid] = row0;
    }
    if (tid == E - 1) {
        offsets[E] = P;
        int tcount = tile0 + ntile;
        for (int s = 0; s < n_shared; s++)
            for (int m = 0; m < T; m += bm) tiles[tcount++] = Tile{E + s, P + s * T + m, P + (s + 1) * T, 0};
        *num_tiles = tcount;
    }
    __syncthreads();
    // stable scatter, 1024 pairs per round: rank = earlier pairs of the same expert
    for (int r0 = 0; r0 < P; r0 += 1024) {
        const int p = r0 + tid;
        const bool valid = p < P;
        const int e = valid ? sm.sidx[p] : 0;
        if (valid) atomicOr(&sm.masks[wave][e], 1ull << lane);
        __syncthreads();
        if (valid) {
            int rank = __popcll(sm.masks[wave][e] & ((1ull << lane) - 1ull));
            for (int w2 = 0; w2 < wave; w2++) rank += __popcll(sm.masks[w2][e]);
            const int row = sm.base[e] + rank;
            perm[row] = p;
            inv[p] = row;
            wrow[row] = sm.sw[p];
        }
        __syncthreads();
        if (tid < E) {
            int add = 0;
            for (int w2 = 0; w2 < 16; w2++) {
                add += __popcll(sm.masks[w2][tid]);
                sm.masks[w2][tid] = 0ull;
            }
            sm.base[tid] += add;
        }
        __syncthreads();
    }
}

template <int EPL>
__global__ __launch_bounds__(1024) void k_route_small(const float *__restrict__ logits, int T, int E, int k,
                                                      int renorm, int n_shared, int bm, int32_t *__restrict__ idx,
                                                      float *__restrict__ w, int32_t *__restrict__ counts,
                                                      int32_t *__restrict__ offsets, Tile *__restrict__ tiles,
                                                      int32_t *__restrict__ num_tiles, int32_t *__restrict__ perm,
                                                      int32_t *__restrict__ inv, float *__restrict__ wrow) {
    __shared__ RouteSmallSmem sm;
    route_small_body<EPL>(sm, logits, T, E, k, renorm, n_shared, bm, idx, w, counts, offsets, tiles, num_tiles, perm,
                          inv, wrow);
}

// ---------------------------------------------------------------------------
// Row sums over 128-wide groups (the offset correction of the integer-code GEMM)
// ---------------------------------------------------------------------------

// xsum[t][g] = scale * sum_{c in group g} x[t][c] in fp32 (scale = -ZC, see the
// grouped GEMM). One wave per token row;
// lane l reads 16-byte chunks l, l+64, ...; the 16 chunks of a group sit in 16
// consecutive lanes and are reduced with xor shuffles.
__global__ __launch_bounds__(256) void k_xsum(const uint16_t *__restrict__ x, int T, int d, float scale,
                                              float *__restrict__ xsum) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;
    const int nchunk = d / 8, G = d / 128;
    // 16 lanes per 128-wide group; lanes past the row (d % 512 != 0) add
    // nothing and write nothing
    for (int c0 = 0; c0 < nchunk; c0 += 64) {
        const int c = c0 + lane;
        const bool in = c < nchunk;
        const uint4 v = *reinterpret_cast<const uint4 *>(x + (size_t)t * d + (in ? c : 0) * 8);
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; i++) s += bf16f(u[i] & 0xFFFFu) + bf16f(u[i] >> 16);
        s = in ? s : 0.0f;
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) s += __shfl_xor(s, off);
        if (in && (lane & 15) == 0) xsum[(size_t)t * G + c / 16] = s * scale;
    }
}

// ---------------------------------------------------------------------------
// B operands
// ---------------------------------------------------------------------------

// 4-bit codes -> bf16 integers 128 + u (exact): OR-ing a nibble into the low
// mantissa bits of bf16 128.0 (0x4300) gives 128 + u. One dword holds eight
// codes; (dword >> 4i) & 0x000F000F yields codes 2i, 2i+1 in its two halves.
__device__ __forceinline__ bf16x8 nibbles_to_bf16_128(uint32_t d) {
    uint4 r;
    r.x = (d & 0x000F000Fu) | 0x43004300u;
    r.y = ((d >> 4) & 0x000F000Fu) | 0x43004300u;
    r.z = ((d >> 8) & 0x000F000Fu) | 0x43004300u;
    r.w = ((d >> 12) & 0x000F000Fu) | 0x43004300u;
    return __builtin_bit_cast(bf16x8, r);
}

// Same conversion with the mask and the magic held in registers: gfx9 VOP3
// instructions cannot encode literals, so with register operands each pair of
// codes costs one v_and_or_b32 (plus one shift for the upper three pairs).
struct NibbleConst {
    uint32_t mask;    // 0x000F000F (scalar register)
    uint32_t magic;   // 0x43004300 (vector register)
};
__device__ __forceinline__ NibbleConst nibble_const() {
    NibbleConst c;
    asm volatile("s_mov_b32 %0, 0xf000f" : "=s"(c.mask));
    asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(c.magic));
    return c;
}
__device__ __forceinline__ bf16x8 nibbles_to_bf16_128(uint32_t d, NibbleConst c) {
    uint4 r;
    r.x = (d & c.mask) | c.magic;
    r.y = ((d >> 4) & c.mask) | c.magic;
    r.z = ((d >> 8) & c.mask) | c.magic;
    r.w = ((d >> 12) & c.mask) | c.magic;
    return __builtin_bit_cast(bf16x8, r);
}

template <int DF>
__device__ __forceinline__ bf16x8 codes8_to_bf16(uint32_t d0, uint32_t d1);

// int8: exact in bf16; the per-row scale is applied in the epilogue.
template <>
__device__ __forceinline__ bf16x8 codes8_to_bf16<DF_INT8>(uint32_t d0, uint32_t d1) {
    bf16x8 r;
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const uint32_t dw = j < 4 ? d0 : d1;
        const int v = (int)(int8_t)((dw >> (8 * (j & 3))) & 0xFFu);
        r[j] = (__bf16)(float)v;
    }
    return r;
}

// e4m3 (OCP e4m3fn): exact in bf16. The hardware converts two codes to fp32
// (v_cvt_pk_f32_fp8) and packs two fp32 into bf16 (v_cvt_pk_bf16_f32), one
// instruction per code; the per-row scale is applied in the epilogue.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
template <bool HI_WORD>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t dw) {
    const f32x2 f = __builtin_amdgcn_cvt_pk_f32_fp8(dw, HI_WORD);
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

template <>
__device__ __forceinline__ bf16x8 codes8_to_bf16<DF_FP8>(uint32_t d0, uint32_t d1) {
    uint4 r;
    r.x = e4m3x2_to_bf16x2<false>(d0);
    r.y = e4m3x2_to_bf16x2<true>(d0);
    r.z = e4m3x2_to_bf16x2<false>(d1);
    r.w = e4m3x2_to_bf16x2<true>(d1);
    return __builtin_bit_cast(bf16x8, r);
}

// ---------------------------------------------------------------------------
// Grouped GEMMs over the task list
// ---------------------------------------------------------------------------
//
// MODE 0 (gate/up): A = gathered x rows, B = W13 of the tile's expert; output
//   H[row][F] = silu(gate) * up in bf16 (+ per-group row sums of H for MODE 1).
// MODE 1 (down): A = H rows of the tile, B = W2; output O[row][d] =
//   (mixing weight of the row's task) * (H . W2^T), fp32 on decode tiles and
//   16-bit block codes on prefill tiles.
// Workgroup = 4 waves; tile = BM rows x 256 columns of B's N dimension (for
// MODE 0 these are 128 gate/up column pairs = one 128-wide group of H). Wave w
// owns 64 columns = four 16-row packed blocks, so each packed weight is
// converted by exactly one wave of the workgroup.

// Pointers of expert e from the kernel arguments (a dependent load of its slot
// only for layers with per-expert formats) and the device format of its group.
__device__ __forceinline__ ExpertW expert_at(const GemmArgs &a, int e, int &fmt) {
    int g, i;
    if (a.eslot) {
        const int v = a.eslot[e];
        g = v >> 20;
        i = v & 0xFFFFF;
    } else {
        g = e >= a.E;
        i = g ? e - a.E : e;
    }
    fmt = a.gfmt[g];
    const ExpertW &b = a.ex0[g];
    const int64_t off = a.ex_stride[g] * (int64_t)i;
    auto adv = [off](auto *p) { return p ? (decltype(p))((const uint8_t *)p + off) : p; };
    ExpertW w;
    w.c13 = adv(b.c13);
    w.s13 = adv(b.s13);
    w.z13 = adv(b.z13);
    w.p13 = adv(b.p13);
    w.zc13 = adv(b.zc13);
    w.c2 = adv(b.c2);
    w.s2 = adv(b.s2);
    w.z2 = adv(b.z2);
    w.p2 = adv(b.p2);
    w.zc2 = adv(b.zc2);
    w.F = b.F;
    return w;
}

struct TileCtx {
    Tile tl;
    ExpertW ew;
    int N, K, n0, rows;
};

// Group formats: the MFMA consumes exact integer codes (128 + u as bf16).
// Per 128-wide group g and output (m, n):
//   sum_k a_mk (u_nk - z_ng) = sum_k a_mk (128 + u_nk) - (128 + z_ng) * rowsum_mg
// The chain of four MFMAs of a group starts from C = -ZC * rowsum (ZC = 136 for
// the symmetric formats, whose stored u = q + 8; 128 for asymmetric), and the
// group's result is scaled by s_ng in fp32 into the running accumulator
// (asymmetric: minus s_ng z_ng rowsum_mg as well). Row sums are stored already
// multiplied by -ZC ("nrs"), so the asymmetric term is (s z / 128) * nrs.
template <int DF>
struct GroupConst {
    static constexpr float ZC = DF == DF_I4SYM ? 136.0f : 128.0f;
};

// ---- decode-shaped batches: tiles of at most 16 rows ----------------------
constexpr int kDecodeBlocksPerWave = 4;
constexpr int kDecKC = 2;                     // K blocks per staged chunk
constexpr int kDecPitch = kDecKC * 128 + 8;   // bf16 per LDS row: rows 16 bytes apart in the bank space
//
// Here the packed weights are the whole cost, so the kernel is built to keep
// HBM busy. Workgroup = 4 waves over one tile and 256 columns of B's N
// dimension; each wave owns four 16-row packed blocks (for the gate/up GEMM two
// gate/up pairs) and streams their K blocks through a register ring DEPTH K
// blocks deep, so every load of the ring is in flight at once. The tile's
// activation rows (at most 16) are staged in LDS in chunks of four K blocks,
// double-buffered; the next chunk's loads are issued before the weight loads
// of the current chunk, so waiting for them never drains the weight ring.
// Group formats take their per-128-group row sums from the staged rows.
template <int DF>
struct DecodeCfg {
    static constexpr bool kGroup = DF == DF_I4SYM || DF == DF_I4ASYM;
    static constexpr int kWords = kGroup ? 1 : 2;   // 16-byte words per lane per block and K block
    static constexpr int kDepth = 1;                // K blocks in flight per wave, beyond the one computed
    static constexpr int kNB = kDecodeBlocksPerWave;
    static constexpr int kKC = kDecKC;
};

// One decode tile: B columns [c.n0, c.n0 + 256) of the tile's expert against
// its (at most 16) rows, staged through the calling kernel's LDS.
// Expert outputs O between the down GEMM and the combine: 16-bit codes with
// one power-of-two scale per row and 16 consecutive columns. For a block whose
// largest |v| lies in [2^(e-1), 2^e), every v is stored as the signed
// normalised code q = round(32767 * v / 2^e) (the hardware's fp32 -> snorm16
// conversion) and e as a signed byte; the combine reads v' = q * (2^e /
// 32767). |v' - v| <= 2^(e-16): at most 2^-15 of the block's largest |v|.
// |O| must stay below 2^127.
constexpr float kOInv = 1.0f / 32767.0f;
__device__ __forceinline__ int o_exponent(float amax) {
    return min(max(__builtin_amdgcn_frexp_expf(amax), -126), 127);
}
__device__ __forceinline__ float o_scale(int e) { return __builtin_amdgcn_ldexpf(1.0f, -e); }
// two codes in one dword (a in the low half)
__device__ __forceinline__ uint32_t o_pack(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pknorm_i16(a, b));
}
// Largest |v| over each 16-lane row of the wave (in every lane of the row),
// for the MFMA output layout: lane i holds column i % 16 of a block.
__device__ __forceinline__ float row16_absmax(float v) {
    uint32_t m = __float_as_uint(fabsf(v));   // non-negative floats order as integers
    m = ror_max<kDppRor1>(m);
    m = ror_max<kDppRor2>(m);
    m = ror_max<kDppRor4>(m);
    m = ror_max<kDppRor8>(m);
    return __uint_as_float(m);
}
// Writes value v of O[gr][n] (MFMA output layout: the 16 lanes of a row hold
// 16 consecutive columns n) and, from the row's first lane, the block's
// exponent; every lane of the row takes part (the block maximum), `live`
// selects the rows that store.
__device__ __forceinline__ void o_store_lane(int16_t *__restrict__ O, int8_t *__restrict__ Oe, int d, size_t gr, int n,
                                             float v, bool live, int lane) {
    const int e = o_exponent(row16_absmax(v));
    if (live) {
        O[gr * d + n] = (int16_t)(o_pack(v * o_scale(e), 0.0f) & 0xFFFFu);
        if ((lane & 15) == 0) Oe[gr * (size_t)(d / 16) + n / 16] = (int8_t)e;
    }
}

template <int DF, int MODE>
__device__ __forceinline__ void dec_tile(const GemmArgs &a, const TileCtx &c, uint16_t (*As)[16 * kDecPitch],
                                         float (*Rs)[kDecKC][16]) {
    using CF = DecodeCfg<DF>;
    constexpr int NB = CF::kNB;            // 16-row blocks per wave
    constexpr int KC = CF::kKC;            // K blocks per staged chunk
    constexpr int PITCH = kDecPitch;
    constexpr float ZC = GroupConst<DF>::ZC;
    static_assert(KC % CF::kDepth == 0, "the ring slot must be static inside a chunk");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int KB = c.K / 128;
    const int NC = (KB + KC - 1) / KC;

    // Every path through the K loop issues the same loads (addresses clamped to
    // valid memory, unused data zeroed by selects), so the compiler's wait
    // counts stay exact and the ring keeps its depth.
    // Staging role: row tid/16, SPT consecutive k at SPT * (tid % 16) of the
    // chunk; rows past the tile read its first row and stage zeros.
    constexpr int SPT = KC * 128 / 16;     // k per staging thread
    constexpr int NV = SPT / 8;            // 16-byte words per staging thread
    constexpr int TPG = 128 / SPT;         // staging threads per 128-wide group
    static_assert(SPT % 8 == 0 && TPG >= 1, "chunk size");
    const int sr = tid >> 4, sk = (tid & 15) * SPT;
    const bool srow = sr < c.rows;
    const uint16_t *asrc;
    {
        const int gr = c.tl.row0 + (srow ? sr : 0);
        if (MODE == 0) {
            const int tok = gr < a.P ? a.perm[gr] / a.k : (gr - a.P) % a.T;
            asrc = a.x + (size_t)tok * a.d;
        } else {
            asrc = a.H + (size_t)gr * a.ldh;
        }
    }
    uint4 av[NV];
    bool aok = false;
    auto stage_load = [&](int ch) {
        const int k0 = ch * (KC * 128) + sk;
        aok = srow && k0 < c.K;
        const int kc = min(k0, c.K - SPT);
#pragma unroll
        for (int i = 0; i < NV; i++) av[i] = gload16(asrc + kc + 8 * i);
    };
    auto stage_store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < NV; i++) {
            av[i].x = aok ? av[i].x : 0u;
            av[i].y = aok ? av[i].y : 0u;
            av[i].z = aok ? av[i].z : 0u;
            av[i].w = aok ? av[i].w : 0u;
            *reinterpret_cast<uint4 *>(&As[buf][sr * PITCH + sk + 8 * i]) = av[i];
        }
        if (CF::kGroup) {
            float sum = 0.0f;
#pragma unroll
            for (int i = 0; i < NV; i++) {
                const uint32_t u[4] = {av[i].x, av[i].y, av[i].z, av[i].w};
#pragma unroll
                for (int j = 0; j < 4; j++) sum += bf16f(u[j] & 0xFFFFu) + bf16f(u[j] >> 16);
            }
            // the TPG threads of a 128-wide group are consecutive lanes of one
            // 16-lane row: shifted sums (DPP row_shr 1, 2, 4, ...) leave the
            // group's sum in its last lane
            static_assert(TPG <= 16 && (TPG & (TPG - 1)) == 0, "groups inside a 16-lane row");
            if constexpr (TPG > 1) sum += dpp_zero<kDppShr1, 0xF>(sum);
            if constexpr (TPG > 2) sum += dpp_zero<kDppShr2, 0xF>(sum);
            if constexpr (TPG > 4) sum += dpp_zero<kDppShr4, 0xF>(sum);
            if constexpr (TPG > 8) sum += dpp_zero<kDppShr8, 0xF>(sum);
            if ((tid & (TPG - 1)) == TPG - 1) Rs[buf][(tid & 15) / TPG][sr] = -ZC * sum;
        }
    };

    const uint8_t *codes = MODE == 0 ? c.ew.c13 : c.ew.c2;
    const uint16_t *gsc = MODE == 0 ? c.ew.s13 : c.ew.s2;
    const uint16_t *gzp = MODE == 0 ? c.ew.z13 : c.ew.z2;
    const int ib0 = c.n0 / 16 + NB * wave;
    // Scales and zeros travel as the aligned dword holding this lane's fp16
    // value and its neighbour's; `hsel` picks the half.
    uint4 ring[CF::kDepth][NB][CF::kWords];
    uint32_t rsc[CF::kDepth][NB], rzp[CF::kDepth][NB];
    const int spair = (lane & 15) & ~1;
    const uint32_t hsel = (lane & 1) * 16;
    auto issue = [&](int kb, int slot) {
#pragma unroll
        for (int nb = 0; nb < NB; nb++) {
            const size_t blk = (size_t)(ib0 + nb) * KB + kb;
            if constexpr (CF::kGroup) {
                ring[slot][nb][0] = gload16(codes + blk * 1024 + lane * 16);
                rsc[slot][nb] = gload(reinterpret_cast<const uint32_t *>(gsc + blk * 16 + spair));
                if constexpr (DF == DF_I4ASYM)
                    rzp[slot][nb] = gload(reinterpret_cast<const uint32_t *>(gzp + blk * 16 + spair));
            } else {
                ring[slot][nb][0] = gload16(codes + blk * 2048 + lane * 32);
                ring[slot][nb][1] = gload16(codes + blk * 2048 + lane * 32 + 16);
            }
        }
    };

    f32x4 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; nb++) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int j, int buf, int slot) {
        bf16x8 af[4];
#pragma unroll
        for (int s = 0; s < 4; s++)
            af[s] = *reinterpret_cast<const bf16x8 *>(&As[buf][(lane & 15) * PITCH + j * 128 + s * 32 + (lane >> 4) * 8]);
        if constexpr (CF::kGroup) {
            const f32x4 rs = *reinterpret_cast<const f32x4 *>(&Rs[buf][j][(lane >> 4) * 4]);   // -ZC * rowsum
#pragma unroll
            for (int nb = 0; nb < NB; nb++) {
                const uint4 q = ring[slot][nb][0];
                f32x4 p = rs;
                p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[0], nibbles_to_bf16_128(q.x), p, 0, 0, 0);
                p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[1], nibbles_to_bf16_128(q.y), p, 0, 0, 0);
                p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[2], nibbles_to_bf16_128(q.z), p, 0, 0, 0);
                p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[3], nibbles_to_bf16_128(q.w), p, 0, 0, 0);
                const float sc = half_bits_to_f32((uint16_t)(rsc[slot][nb] >> hsel));
                acc[nb] += sc * p;
                if (DF == DF_I4ASYM)
                    acc[nb] += (sc * half_bits_to_f32((uint16_t)(rzp[slot][nb] >> hsel)) * (1.0f / 128.0f)) * rs;
            }
        } else {
#pragma unroll
            for (int s = 0; s < 4; s++)
#pragma unroll
                for (int nb = 0; nb < NB; nb++) {
                    const uint4 q = ring[slot][nb][s >> 1];
                    acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        af[s], codes8_to_bf16<DF>((s & 1) ? q.z : q.x, (s & 1) ? q.w : q.y), acc[nb], 0, 0, 0);
                }
        }
        // Materialise the accumulators here: otherwise IR-level sinking moves the
        // scale updates (and the last use of the ring's scale registers) to the
        // end of the chunk, past the refills of the same slots.
#pragma unroll
        for (int nb = 0; nb < NB; nb++) asm volatile("" : "+v"(acc[nb]));
    };

    // K blocks past the end (the last chunk's padding) compute on zero rows with
    // a copy of the last block: they add exactly zero.
    // The scheduling barriers keep each refill right after the compute that
    // frees its ring slot: left alone, the scheduler sinks all refills to the
    // end of the chunk (loads stop overlapping compute) or lifts a refill above
    // the last use of its slot (the registers cannot be reused and the loop
    // back-edge gains copies that wait for every load).
    stage_load(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < CF::kDepth; i++) {
        issue(min(i, KB - 1), i);
        __builtin_amdgcn_sched_barrier(0);
    }
    stage_store(0);
    __syncthreads();
    for (int ch = 0; ch < NC; ch++) {
        const int buf = ch & 1;
        stage_load(ch + 1);   // past the last chunk: zeros, never read
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < KC; j++) {
            const int kb = ch * KC + j;
            compute(j, buf, j % CF::kDepth);
            __builtin_amdgcn_sched_barrier(0);
            issue(min(kb + CF::kDepth, KB - 1), j % CF::kDepth);
            __builtin_amdgcn_sched_barrier(0);
        }
        stage_store(buf ^ 1);
        __syncthreads();
    }

    const int lrow = (lane >> 4) * 4;
    if (MODE == 0) {
#pragma unroll
        for (int pr = 0; pr < NB / 2; pr++) {
            const int ibg = ib0 + 2 * pr;
            const int col = (ibg >> 1) * 16 + (lane & 15);
            const float sg = CF::kGroup ? 1.0f : c.ew.p13[ibg * 16 + (lane & 15)];
            const float su = CF::kGroup ? 1.0f : c.ew.p13[(ibg + 1) * 16 + (lane & 15)];
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int row = lrow + r;
                if (row < c.rows) {
                    const float g = acc[2 * pr][r] * sg;
                    const float u = acc[2 * pr + 1][r] * su;
                    a.H[(size_t)(c.tl.row0 + row) * a.ldh + col] = to_bf16(silu_mul(g, u));
                }
            }
        }
    } else {
        float sn[NB];
#pragma unroll
        for (int nb = 0; nb < NB; nb++)
            sn[nb] = CF::kGroup ? 1.0f : c.ew.p2[c.n0 + NB * 16 * wave + 16 * nb + (lane & 15)];
        // (decode tiles: fp32 outputs, read by k_combine_f32; at these
        // sizes the coding would cost more than the bytes it saves)
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int row = lrow + r;
            if (row >= c.rows) continue;
            const int gr = c.tl.row0 + row;
            const float wt = gr < a.P ? a.wrow[gr] : 1.0f;
#pragma unroll
            for (int nb = 0; nb < NB; nb++) {
                const int n = c.n0 + NB * 16 * wave + 16 * nb + (lane & 15);
                a.Of[(size_t)gr * a.d + n] = acc[nb][r] * sn[nb] * wt;
            }
        }
    }
}

// Sets up a decode tile (row range, expert, B column range); false: nothing to do.
__device__ __forceinline__ bool dec_setup(const GemmArgs &a, TileCtx &c, int &fmt) {
    constexpr int WG_COLS = 4 * kDecodeBlocksPerWave * 16;   // columns of B's N dimension per workgroup
    static_assert(kDecodeBlocksPerWave % 2 == 0 && 256 % WG_COLS == 0,
                  "a wave owns whole gate/up pairs; N % 256 == 0 covers the grid");
    const int ntiles = *a.num_tiles;   // issued together with the tile load
    c.tl = a.tiles[blockIdx.y];
    if ((int)blockIdx.y >= ntiles) return false;
    c.ew = expert_at(a, c.tl.e, fmt);
    return true;
}
template <int MODE>
__device__ __forceinline__ bool dec_cols(const GemmArgs &a, TileCtx &c) {
    c.N = MODE == 0 ? 2 * c.ew.F : a.d;
    c.K = MODE == 0 ? a.d : c.ew.F;
    c.n0 = blockIdx.x * (4 * kDecodeBlocksPerWave * 16);
    c.rows = c.tl.row_end - c.tl.row0;
    return c.n0 < c.N;
}

template <int DF, int MODE>
__global__ __launch_bounds__(256) void k_gemm_dec(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t As[2][16 * kDecPitch];
    __shared__ __attribute__((aligned(16))) float Rs[2][kDecKC][16];
    TileCtx c;
    int fmt;
    if (!dec_setup(a, c, fmt) || fmt != DF) return;   // another launch computes another format
    if (!dec_cols<MODE>(a, c)) return;
    dec_tile<DF, MODE>(a, c, As, Rs);
}

// Decode tiles of a layer with per-expert formats: one launch for all of them
// (one HBM stream instead of one per format), each workgroup running its
// expert's format.
template <int MODE>
__global__ __launch_bounds__(256) void k_gemm_dec_mixed(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t As[2][16 * kDecPitch];
    __shared__ __attribute__((aligned(16))) float Rs[2][kDecKC][16];
    TileCtx c;
    int fmt;
    if (!dec_setup(a, c, fmt) || !dec_cols<MODE>(a, c)) return;
    switch (fmt) {
    case DF_INT8: dec_tile<DF_INT8, MODE>(a, c, As, Rs); break;
    case DF_I4ASYM: dec_tile<DF_I4ASYM, MODE>(a, c, As, Rs); break;
    case DF_I4SYM: dec_tile<DF_I4SYM, MODE>(a, c, As, Rs); break;
    case DF_FP8: dec_tile<DF_FP8, MODE>(a, c, As, Rs); break;
    default: break;
    }
}


// ---- prefill tiles: XCD-aware work order -----------------------------------
//
// Work items (M-tile of the task list, N-tile) are numbered in bands
// of 4 N-tiles with the M-tile slower inside a band, so concurrently running
// workgroups share both activation rows and packed weights; the numbering is
// split into 8 contiguous chunks, one per XCD (workgroup L runs on XCD L % 8),
// so each XCD's L2 sees a contiguous window of the work.
__device__ __forceinline__ bool map_work(int L, int ntiles, int NT, int &tile, int &nt) {
    const int total = ntiles * NT;
    const int C = (total + 7) >> 3;
    if ((L >> 3) >= C) return false;
    const int w = (L & 7) * C + (L >> 3);
    if (w >= total) return false;
    constexpr int GN = 4;
    const int band = w / (ntiles * GN);
    const int rem = w - band * ntiles * GN;
    const int gw = min(GN, NT - band * GN);
    tile = rem / gw;
    nt = band * GN + rem % gw;
    return true;
}

// ---- prefill tiles: activation ring in LDS ------------------------------------
//
// Every prefill format (group formats: 4-bit codes with an fp16 scale per
// 128-group; per-channel formats: INT8 / e4m3 codes with one scale per column).
// Tiles of 16*MI rows x 256 columns: each of the NW waves owns all the rows
// and 16*NB columns. With MULTI, a workgroup computes nsub such tiles side by
// side (the same rows, consecutive 256-column ranges), running one load
// pipeline through all of them, so the fixed start and drain of a tile is paid
// once per workgroup rather than once per tile: the next tile's first operands
// are in flight while the previous one's results are stored. Per wave and
// group (128 K positions): the gathered activation rows (and, for the group
// formats, their row sums) travel as asynchronous global -> LDS copies issued
// from inline assembly (so the compiler neither waits on them before LDS
// reads nor counts them), one group ahead in a two-stage ring; the wave's own
// packed codes and scales are ordinary loads into a two-slot register ring,
// two groups ahead. Every group ends with the next group's copies landed and
// one barrier that publishes them to the workgroup.
// LDS of a workgroup: the two activation stages, then the per-row H sums of
// each wave (gate/up) or the rows' mixing weights (down)
template <int DF, int MODE, int MI, int NW>
constexpr int gpf_lds_bytes() {
    return 2 * (16 * MI * 256 + ((DF == DF_I4SYM || DF == DF_I4ASYM) ? 16 * MI * 4 : 0)) +
           (MODE == 0 ? NW * 16 * MI : 16 * MI) * 4;
}

// The tile(s) of one workgroup with MI 16-row blocks (tl: the task-list tile,
// ew: its expert's weights, ngrp: the workgroup's group of N-tiles).
template <int DF, int MODE, int MI, int NB, int NW, bool MULTI>
__device__ __forceinline__ void gpf_tiles(const GemmArgs &a, uint8_t *lds, int ngrp, const Tile &tl,
                                          const ExpertW &ew) {
    constexpr int BM = 16 * MI, RPW = BM / NW;   // activation rows copied per wave
    static_assert(RPW % 4 == 0 && RPW <= 64, "each wave copies whole 4-row slabs");
    constexpr int ADMA = RPW / 4;                 // 1 KB activation copies per wave
    // Packed codes and scales go straight to registers (each wave owns its B
    // blocks, so nothing would be shared through LDS); the two stages hold only
    // the activation tile and its row sums. Per-channel 8-bit codes need no
    // row sums: the column scale multiplies the finished accumulator.
    constexpr bool GRP = DF == DF_I4SYM || DF == DF_I4ASYM;
    constexpr int BW = GRP ? 1 : 2;               // 16-byte code words per lane, block and group
    constexpr int ST_A = 0, ST_R = BM * 256, ST_BYTES = ST_R + (GRP ? BM * 4 : 0);
    constexpr int WCOLS = 16 * NB;                // B columns per wave
    constexpr int NTILE = WCOLS * NW;             // B columns per tile
    // N (2F or d) is a multiple of 256 = NTILE: every wave of a tile with
    // n0 < N owns columns below N
    static_assert(NTILE == 256, "tiles of 256 columns");
    constexpr int RS = 2;                         // B register slots
    constexpr int NST = 2;                        // activation stages
    // apart from the ring (which holds the next tile's first activations
    // while a tile ends): gate/up, the per-row H sums of each wave, [NW][BM]
    // floats; down, the rows' mixing weights, [BM] floats
    constexpr int RED = NST * ST_BYTES;
    static_assert(RED + (MODE == 0 ? NW * BM : BM) * 4 == gpf_lds_bytes<DF, MODE, MI, NW>(), "LDS layout");
    constexpr float ZC = GroupConst<DF>::ZC;

    const int N = MODE == 0 ? 2 * ew.F : a.d;
    const int K = MODE == 0 ? a.d : ew.F;
    const int nt0 = ngrp * a.nsub;                // first 256-column tile
    if (nt0 * NTILE >= N) return;
    // (one tile per workgroup: nothing is carried past the last group)
    const int nsub = MULTI ? min(a.nsub, N / NTILE - nt0) : 1;
    const int KB = K / 128;
    const int V = nsub * KB;                      // groups through all the tiles
    const int rows = tl.row_end - tl.row0;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform, kept in an SGPR
    const int lrow = (lane >> 4) * 4;
    const uint32_t lds0 = lds_addr(lds);

    // sources of this lane's ADMA 16-byte activation chunks per group: rows
    // RPW*w + 4i + lane/16, chunk (lane & 15) ^ (row & 15) (the swizzle), as
    // 32-bit byte offsets from a base in SGPRs: gathered x rows from x itself
    // (the host keeps max_tokens * d below 2^31), the tile's contiguous H rows
    // from its first row
    const int lda = MODE == 0 ? a.d : a.ldh;
    const int ldr = MODE == 0 ? a.d / 128 : a.ldh / 128;
    const uint16_t *abase = MODE == 0 ? a.x : a.H + (size_t)tl.row0 * lda;
    const float *rbase = MODE == 0 ? a.xsum : a.hsum + (size_t)tl.row0 * ldr;
    // source row of tile row r (rows past the tile read its first row), the
    // tile's nr rows starting at row0
    auto src_row = [&](int r, int row0, int nr) {
        const int rr = r < nr ? r : 0;
        if (MODE == 1) return rr;
        const int gr = row0 + rr;
        return gr < a.P ? a.perm[gr] / a.k : (gr - a.P) % a.T;
    };
    uint32_t aoffb[ADMA];
#pragma unroll
    for (int i = 0; i < ADMA; i++) {
        const int row = RPW * wave + 4 * i + (lane >> 4);
        aoffb[i] = 2u * ((uint32_t)src_row(row, tl.row0, rows) * (uint32_t)lda + (uint32_t)(((lane & 15) ^ (row & 15)) * 8));
    }
    const uint32_t roffb = 4u * (uint32_t)src_row(RPW * wave + (lane < RPW ? lane : 0), tl.row0, rows) * (uint32_t)ldr;
    const uint8_t *codes = MODE == 0 ? ew.c13 : ew.c2;
    const uint16_t *gsc = MODE == 0 ? ew.s13 : ew.s2;
    // this wave's first 16-column block in the first tile
    const int ib0 = nt0 * (NTILE / 16) + NB * wave;
    const int last = V - 1;

    // Pipeline position v = j * KB + kb is group kb of tile j. The copies'
    // per-lane byte offsets are constant through K; only the scalar bases
    // advance with the group index.
    auto issue = [&](int kb, int st) __attribute__((always_inline)) {
        // wave-uniform by construction; readfirstlane keeps them in SGPRs
        kb = __builtin_amdgcn_readfirstlane(kb);
        st = __builtin_amdgcn_readfirstlane(st);
        const uint32_t sb = lds0 + st * ST_BYTES;
        const uint16_t *as = abase + kb * 128;
#pragma unroll
        for (int i = 0; i < ADMA; i++) dma16s(as, aoffb[i], sb + ST_A + (RPW * wave + 4 * i) * 256);
        if (GRP && lane < RPW) dma4s(rbase + kb, roffb, sb + ST_R + wave * RPW * 4);
    };
    // B register ring: codes, and the dword holding this lane's fp16 scale and
    // its neighbour's
    uint4 bring[RS][NB][BW];
    uint32_t sring[RS][NB];
    const int spair2 = (lane & 15) & ~1;
    const uint32_t hsel = (lane & 1) * 16;
    auto load_b = [&](int j, int kb, int slot) __attribute__((always_inline)) {
        j = __builtin_amdgcn_readfirstlane(j);
        kb = __builtin_amdgcn_readfirstlane(kb);
#pragma unroll
        for (int nb = 0; nb < NB; nb++) {
            const size_t blk = (size_t)(ib0 + (NTILE / 16) * j + nb) * KB + kb;
            if constexpr (GRP) {
                bring[slot][nb][0] = gload16(codes + blk * 1024 + lane * 16);
                sring[slot][nb] = gload(reinterpret_cast<const uint32_t *>(gsc + blk * 16 + spair2));
            } else {
                bring[slot][nb][0] = gload16(codes + blk * 2048 + lane * 32);
                bring[slot][nb][1] = gload16(codes + blk * 2048 + lane * 32 + 16);
            }
        }
    };

    f32x4 acc[MI][NB];
    // scale of the previous group per column block (accumulators in scale units)
    float s_prev[NB];
    auto reset = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int mi = 0; mi < MI; mi++)
#pragma unroll
            for (int nb = 0; nb < NB; nb++) acc[mi][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int nb = 0; nb < NB; nb++) s_prev[nb] = 1.0f;
    };
    reset();
    const NibbleConst nc = nibble_const();

    // One group: this wave's codes and scales, then the group's MFMAs.
    // Accumulators in units of the current group's scale: per column,
    // X = X * (s_prev / s_cur) + nrs, then the group's MFMAs add the
    // integer-code products straight into X (nrs = -ZC * row sum folds in the
    // code offset, as a chain's start value would); the tile ends with
    // X * s_last. With no chain partials live, the codes are converted half a
    // group (two k-steps) at a time, each half right before its MFMAs, and the
    // A fragments stream one k-step ahead through a two-slot ring (each LDS
    // read in flight behind four MFMAs). Once the first half's codes are
    // converted the next group's activation copies are issued; once the second
    // half's are, the slot is refilled for two groups ahead.
    auto group = [&](int st, int slot, int next_j, int next_kb, int copy_kb, int copy_st) __attribute__((always_inline)) {
        const uint8_t *S = lds + st * ST_BYTES;
        const uint16_t *Ab = reinterpret_cast<const uint16_t *>(S + ST_A);
        const float *Rb = reinterpret_cast<const float *>(S + ST_R);
        // A fragment of row block mi, k-step s (XOR-swizzled chunks)
        auto afrag = [&](int mi, int s) __attribute__((always_inline)) {
            const int pc = (s * 4 + (lane >> 4)) ^ (lane & 15);
            return *reinterpret_cast<const bf16x8 *>(&Ab[(mi * 16 + (lane & 15)) * 128 + pc * 8]);
        };
        float r[NB];
#pragma unroll
        for (int nb = 0; nb < NB; nb++) {
            if constexpr (GRP) {
                const float sc_cur = half_bits_to_f32((uint16_t)(sring[slot][nb] >> hsel));
                r[nb] = s_prev[nb] * __builtin_amdgcn_rcpf(sc_cur);
                s_prev[nb] = sc_cur;
            } else {
                r[nb] = 1.0f;
            }
        }
        bf16x8 afr[2];
        afr[0] = afrag(0, 0);
#pragma unroll
        for (int h = 0; h < 2; h++) {
            bf16x8 bh[NB][2];
#pragma unroll
            for (int nb = 0; nb < NB; nb++) {
                if constexpr (GRP) {
                    bh[nb][0] = nibbles_to_bf16_128(h == 0 ? bring[slot][nb][0].x : bring[slot][nb][0].z, nc);
                    bh[nb][1] = nibbles_to_bf16_128(h == 0 ? bring[slot][nb][0].y : bring[slot][nb][0].w, nc);
                } else {
                    // k-steps 2h and 2h+1: the low and high half of word h
                    const uint4 q = bring[slot][nb][h];
                    bh[nb][0] = codes8_to_bf16<DF>(q.x, q.y);
                    bh[nb][1] = codes8_to_bf16<DF>(q.z, q.w);
                }
            }
            // The converted operands (and the scale ratios) as inputs of an
            // empty volatile asm: the copies and loads below cannot move above
            // the conversion, which is where the compiler waits for this
            // slot's loads, so that wait does not catch them.
#pragma unroll
            for (int nb = 0; nb < NB; nb++)
                asm volatile("" ::"v"(bh[nb][0]), "v"(bh[nb][1]), "v"(r[nb]));
            if (h == 0) issue(copy_kb, copy_st);
            else load_b(next_j, next_kb, slot);
            // The rescale of row block mi + 1 runs beside row block mi's
            // MFMAs, two FMAs after each MFMA (the rescale is the group's
            // largest VALU block, and an MFMA leaves the VALU free for about
            // two). The asymmetric down kernel rescales each row block right
            // before its MFMAs instead: its 96-row body would spill with the
            // next block's row sums held ahead.
            constexpr bool SPREAD = GRP && !(DF == DF_I4ASYM && MODE == 1);
            f32x4 nrs_next;
            if (SPREAD && h == 0) {
                const f32x4 nrs = *reinterpret_cast<const f32x4 *>(&Rb[lrow]);
#pragma unroll
                for (int nb = 0; nb < NB; nb++) acc[0][nb] = acc[0][nb] * r[nb] + nrs;
                if (MI > 1) nrs_next = *reinterpret_cast<const f32x4 *>(&Rb[16 + lrow]);
            }
#pragma unroll
            for (int mi = 0; mi < MI; mi++) {
                if (GRP && !SPREAD && h == 0) {
                    const f32x4 nrs = *reinterpret_cast<const f32x4 *>(&Rb[mi * 16 + lrow]);
#pragma unroll
                    for (int nb = 0; nb < NB; nb++) acc[mi][nb] = acc[mi][nb] * r[nb] + nrs;
                }
#pragma unroll
                for (int ss = 0; ss < 2; ss++) {
                    const int q = (h * MI + mi) * 2 + ss;   // fragment sequence number
                    // next fragment: (mi, s+1), then (mi+1, 2h), then (0, 2) after half 0
                    if (ss == 0) afr[(q + 1) & 1] = afrag(mi, 2 * h + 1);
                    else if (mi + 1 < MI) afr[(q + 1) & 1] = afrag(mi + 1, 2 * h);
                    else if (h == 0) afr[(q + 1) & 1] = afrag(0, 2);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int nb = 0; nb < NB; nb++)
                        acc[mi][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[q & 1], bh[nb][ss], acc[mi][nb], 0, 0, 0);
                    if (SPREAD && h == 0 && mi + 1 < MI) {
                        // half of row block mi + 1's columns beside each block of four MFMAs
#pragma unroll
                        for (int nb = ss * (NB / 2); nb < (ss + 1) * (NB / 2); nb++)
                            acc[mi + 1][nb] = acc[mi + 1][nb] * r[nb] + nrs_next;
                        if (ss == 1 && mi + 2 < MI) nrs_next = *reinterpret_cast<const f32x4 *>(&Rb[(mi + 2) * 16 + lrow]);
#pragma unroll
                        for (int i = 0; i < 4; i++) {
                            __builtin_amdgcn_sched_group_barrier(0x8, 1, 0);   // one MFMA
                            __builtin_amdgcn_sched_group_barrier(0x2, 2, 0);   // two VALU ops
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    };
    // tile and group of pipeline position t, from tile j starting at vs
    auto locate = [&](int t, int j, int vs, int &jt, int &kb) __attribute__((always_inline)) {
        jt = j;
        kb = t - vs;
        if (MULTI)
            while (kb >= KB) {
                kb -= KB;
                ++jt;
            }
    };
    // group v of tile j (which starts at vs); afterwards group v+1's copies
    // have landed (group v+2's B loads may still be in flight) and the
    // barrier has published them
    auto step = [&](int v, int st, int slot, int j, int vs) __attribute__((always_inline)) {
        int nj, nkb, cj, ckb;
        locate(min(v + 2, last), j, vs, nj, nkb);
        locate(min(v + 1, last), j, vs, cj, ckb);
        group(st, slot, nj, nkb, ckb, st ^ 1);
        wait_vm_lgkm0<2 * NB>();
        raw_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    // Results of tile j (its columns start at 256 * (nt0 + j)); st_free: the
    // stage the tile's last group read (idle until the next group's copies).
    auto finish = [&](int j, int st_free) __attribute__((always_inline)) {
        const int n0 = (nt0 + j) * NTILE;
        const int ibj = ib0 + (NTILE / 16) * j;
        // the tile's rows and the output pitches as opaque values here: the
        // row addresses and bounds below are computed per tile, not hoisted
        // out of the loop into registers live through every group
        int row0 = tl.row0, nrows = rows, ld_out = MODE == 0 ? a.ldh : a.d, lrow = (lane >> 4) * 4;
        asm volatile("" : "+s"(row0), "+s"(nrows), "+s"(ld_out), "+v"(lrow));
        if constexpr (GRP) {
            // back from scale units
#pragma unroll
            for (int mi = 0; mi < MI; mi++)
#pragma unroll
                for (int nb = 0; nb < NB; nb++) acc[mi][nb] *= s_prev[nb];
        } else {
            // per-channel scales of the tile's columns (W13: interleaved gate /
            // up blocks, as the codes)
            const float *ps = MODE == 0 ? ew.p13 : ew.p2;
#pragma unroll
            for (int nb = 0; nb < NB; nb++) {
                const float cs = ps[(ibj + nb) * 16 + (lane & 15)];
#pragma unroll
                for (int mi = 0; mi < MI; mi++) acc[mi][nb] *= cs;
            }
        }

        if (DF == DF_I4ASYM) {
            // zero points: acc[m][n] += sum_g (s_ng z_ng / 128) * nrs_mg, one MFMA
            // contraction over the group index with bf16 hi/lo splits of both sides
            // (hi*hi + hi*lo + lo*hi; relative error ~2^-16 of the correction)
            const uint16_t *zcp = MODE == 0 ? ew.zc13 : ew.zc2;
            const int GS = (KB + 31) / 32;
            uint32_t zrow[MI];
#pragma unroll
            for (int mi = 0; mi < MI; mi++) zrow[mi] = (uint32_t)src_row(mi * 16 + (lane & 15), row0, nrows) * (uint32_t)ldr;
            // the eight row sums a lane needs per row block and K range are
            // consecutive floats: two 16-byte loads when rows and ranges keep them
            // aligned (uniform), else eight single loads
            const bool vec = ldr % 8 == 0 && KB % 8 == 0;
            for (int gs = 0; gs < GS; gs++) {
                bf16x8 bh[NB], bl[NB];
#pragma unroll
                for (int nb = 0; nb < NB; nb++) {
                    const uint16_t *q = zcp + ((size_t)(ibj + nb) * GS + gs) * 1024 + lane * 8;
                    bh[nb] = __builtin_bit_cast(bf16x8, gload16(q));
                    bl[nb] = __builtin_bit_cast(bf16x8, gload16(q + 512));
                }
                const int g0 = gs * 32 + (lane >> 4) * 8;
                float rv[MI][8];
                if (vec) {
                    // past the last group (KB % 32 != 0): the last 8 groups are
                    // read and zeroed
                    const bool gin = g0 < KB;
                    const int gc = gin ? g0 : KB - 8;
#pragma unroll
                    for (int mi = 0; mi < MI; mi++) {
                        const uint4 u0 = gload16(rbase + zrow[mi] + gc);
                        const uint4 u1 = gload16(rbase + zrow[mi] + gc + 4);
                        const uint32_t uu[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
                        for (int jj = 0; jj < 8; jj++) rv[mi][jj] = gin ? __uint_as_float(uu[jj]) : 0.0f;
                    }
                } else {
#pragma unroll
                    for (int mi = 0; mi < MI; mi++)
#pragma unroll
                        for (int jj = 0; jj < 8; jj++) rv[mi][jj] = g0 + jj < KB ? gload(rbase + zrow[mi] + g0 + jj) : 0.0f;
                }
#pragma unroll
                for (int mi = 0; mi < MI; mi++) {
                    bf16x8 ah, al;
#pragma unroll
                    for (int jj = 0; jj < 8; jj++) {
                        __bf16 hh, ll;
                        split_bf16(rv[mi][jj], hh, ll);
                        ah[jj] = hh;
                        al[jj] = ll;
                    }
#pragma unroll
                    for (int nb = 0; nb < NB; nb++) {
                        acc[mi][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh[nb], acc[mi][nb], 0, 0, 0);
                        acc[mi][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl[nb], acc[mi][nb], 0, 0, 0);
                        acc[mi][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh[nb], acc[mi][nb], 0, 0, 0);
                    }
                }
            }
        }

        if (MODE == 0) {
            // H = silu(gate) * up; the tile's columns are two groups of 128 H
            // columns, whose per-row sums (of the bf16 values) feed the down
            // GEMM's zero-offset term
            constexpr int WPG = 16 / NB;   // waves per 128-wide H group
            static_assert(NB % 2 == 0 && NW % WPG == 0, "a tile covers whole 128-wide H groups");
            float hs[MI][4];
#pragma unroll
            for (int mi = 0; mi < MI; mi++)
#pragma unroll
                for (int r = 0; r < 4; r++) hs[mi][r] = 0.0f;
            // the tile's H rows: a uniform base and 32-bit per-lane offsets
            uint8_t *Hb = reinterpret_cast<uint8_t *>(a.H + (size_t)row0 * ld_out);
#pragma unroll
            for (int pr = 0; pr < NB / 2; pr++) {
                const int col = ((ibj + 2 * pr) >> 1) * 16 + (lane & 15);
#pragma unroll
                for (int mi = 0; mi < MI; mi++)
#pragma unroll
                    for (int r = 0; r < 4; r++) {
                        const int row = mi * 16 + lrow + r;
                        const float g = acc[mi][2 * pr][r];
                        const float u = acc[mi][2 * pr + 1][r];
                        const uint16_t hb = to_bf16(silu_mul(g, u));
                        hs[mi][r] += bf16f(hb);
                        if (row < nrows) *reinterpret_cast<uint16_t *>(Hb + 2u * (uint32_t)(row * ld_out + col)) = hb;
                    }
            }
            // (per-channel formats: their down GEMM takes no row sums)
            if constexpr (GRP) {
                float *red = reinterpret_cast<float *>(lds + RED);
                // 16-lane row sums, the 4*MI independent chains interleaved step by
                // step (a DPP read right after the write of its source needs wait states)
                auto row_step = [&](auto ctrl) {
#pragma unroll
                    for (int mi = 0; mi < MI; mi++)
#pragma unroll
                        for (int r = 0; r < 4; r++) hs[mi][r] += dpp_zero<decltype(ctrl)::value, 0xF>(hs[mi][r]);
                };
                row_step(std::integral_constant<int, kDppShr1>{});
                row_step(std::integral_constant<int, kDppShr2>{});
                row_step(std::integral_constant<int, kDppShr4>{});
                row_step(std::integral_constant<int, kDppShr8>{});
#pragma unroll
                for (int mi = 0; mi < MI; mi++)
#pragma unroll
                    for (int r = 0; r < 4; r++)
                        if ((lane & 15) == 15) red[wave * BM + mi * 16 + lrow + r] = hs[mi][r];
                // LDS writes done, then the barrier (no wait for the B loads in
                // flight); the group barriers that follow order these reads
                // before the next tile's writes
                wait_vm_lgkm0<63>();
                raw_barrier();
                for (int t = threadIdx.x; t < BM * (NW / WPG); t += 64 * NW) {
                    const int h = t / BM, row = t % BM;
                    const int grp = n0 / 256 + h;   // 128-wide H group
                    if (row < nrows && grp < ew.F / 128) {
                        const float *rr = red + WPG * h * BM + row;
                        float v = 0.0f;
#pragma unroll
                        for (int w = 0; w < WPG; w++) v += rr[w * BM];
                        a.hsum[(size_t)(row0 + row) * (a.ldh / 128) + grp] = -ZC * v;
                    }
                }
            }
        } else if constexpr (MI >= 4) {
            // O (16-bit codes, one scale per row and 16 columns) through this
            // wave's own activation rows of the idle stage (4 KB of at least
            // 4 KB; the wave's next copies into them come after its reads, in
            // its own program order), so that each lane holds four
            // consecutive columns of one row: the 16-column block is a lane
            // quad, and the stores are 8 bytes per lane.
            const float *wts = reinterpret_cast<const float *>(lds + RED);
            float *Sw = reinterpret_cast<float *>(lds + st_free * ST_BYTES + ST_A + wave * RPW * 256);
            static_assert(RPW * 256 >= 16 * WCOLS * 4, "a 16-row block fits the wave's rows");
            // rows padded by four floats where they fit (addresses linear in
            // the row: immediate offsets), else a 16-byte-chunk XOR swizzle
            constexpr bool PAD = RPW * 256 >= 16 * (WCOLS + 4) * 4;
            constexpr int OP = PAD ? WCOLS + 4 : WCOLS;
            auto sidx = [&](int row, int col) __attribute__((always_inline)) {
                return PAD ? row * OP + col : row * OP + (((col >> 2) ^ row) << 2) + (col & 3);
            };
            const int c4 = lane & 15;
            // the tile's O rows and exponents: uniform bases, 32-bit offsets
            uint8_t *Ob = reinterpret_cast<uint8_t *>(a.O + (size_t)row0 * ld_out);
            int8_t *Eb = a.Oe + (size_t)row0 * (ld_out / 16);
            const int col0 = n0 + WCOLS * wave + 4 * c4;
#pragma unroll
            for (int mi = 0; mi < MI; mi++) {
                const f32x4 wt = *reinterpret_cast<const f32x4 *>(&wts[mi * 16 + lrow]);
#pragma unroll
                for (int nb = 0; nb < NB; nb++)
#pragma unroll
                    for (int r = 0; r < 4; r++) Sw[sidx(lrow + r, 16 * nb + (lane & 15))] = acc[mi][nb][r] * wt[r];
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int row = 4 * i + (lane >> 4);
                    const f32x4 v = *reinterpret_cast<const f32x4 *>(&Sw[sidx(row, 4 * c4)]);
                    uint32_t m = __float_as_uint(fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
                    // quad maximum (DPP quad_perm [1,0,3,2], then [2,3,0,1])
                    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, false));
                    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, false));
                    const int e = o_exponent(__uint_as_float(m));
                    const float sc = o_scale(e);
                    const int grow = mi * 16 + row;
                    if (grow < nrows) {
                        *reinterpret_cast<uint2 *>(Ob + 2u * (uint32_t)(grow * ld_out + col0)) =
                            make_uint2(o_pack(v[0] * sc, v[1] * sc), o_pack(v[2] * sc, v[3] * sc));
                        if ((c4 & 3) == 0) Eb[(uint32_t)(grow * (ld_out / 16) + col0 / 16)] = (int8_t)e;
                    }
                }
            }
        } else {
            // (32-row tiles) O straight from the MFMA layout: the 16 lanes of
            // a row hold a 16-column block
            const float *wts = reinterpret_cast<const float *>(lds + RED);
#pragma unroll
            for (int mi = 0; mi < MI; mi++) {
                const f32x4 wt = *reinterpret_cast<const f32x4 *>(&wts[mi * 16 + lrow]);
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const int row = mi * 16 + lrow + r;
#pragma unroll
                    for (int nb = 0; nb < NB; nb++) {
                        const int n = n0 + WCOLS * wave + 16 * nb + (lane & 15);
                        o_store_lane(a.O, a.Oe, ld_out, (size_t)(row0 + row), n, acc[mi][nb][r] * wt[r], row < nrows,
                                     lane);
                    }
                }
            }
        }
    };

    // The compiler counts only the B loads (the copies are inline assembly),
    // so before it reads a slot it waits for everything issued before the
    // other slot's loads, the next group's copies included: both operands are
    // in hand at the start of the group they feed, as the barrier requires
    // anyway.
    if (MODE == 1 && threadIdx.x < BM) {
        // mixing weight per row (1 for shared-expert rows and rows past the tile)
        const int gr = tl.row0 + threadIdx.x;
        reinterpret_cast<float *>(lds + RED)[threadIdx.x] = threadIdx.x < rows && gr < a.P ? a.wrow[gr] : 1.0f;
    }
    issue(0, 0);
    load_b(0, 0, 0);
    {
        int j1, kb1;
        locate(min(1, last), 0, 0, j1, kb1);
        load_b(j1, kb1, 1);
    }
    wait_vm_lgkm0<2 * NB>();
    raw_barrier();
    // Group v reads stage and slot v & 1; a tile's groups run in pairs (one
    // lone group first when it starts at an odd v, one last when it ends
    // before a pair is complete).
    int v = 0, j = 0, vend = KB;
    for (;;) {
        const int vs = vend - KB;
        if (v & 1) step(v++, 1, 1, j, vs);
        for (; v + 1 < vend; v += 2) {
            step(v, 0, 0, j, vs);
            step(v + 1, 1, 1, j, vs);
        }
        if (v < vend) step(v++, 0, 0, j, vs);
        finish(j, (v - 1) & 1);
        if (++j == nsub) break;
        vend += KB;
        reset();
    }
    // no copy into LDS may be in flight when the workgroup ends
    __builtin_amdgcn_s_waitcnt(0);
}

// Prefill GEMM: tiles of up to 16*MI rows. The last tile of an expert usually
// holds fewer rows: such a tile runs only the 32-row steps it needs (MI = 2 or
// 4), converting the same codes for fewer MFMAs.
template <int DF, int MODE, int MI, int NB, int NW, bool MULTI>
__global__ __launch_bounds__(64 * NW, 2) void k_gemm_gpf(GemmArgs a) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[gpf_lds_bytes<DF, MODE, MI, NW>()];
    int tile_id, ngrp;
    if (!map_work(blockIdx.x, *a.num_tiles, a.n_groups, tile_id, ngrp)) return;
    const Tile tl = a.tiles[tile_id];
    int efmt;
    const ExpertW ew = expert_at(a, tl.e, efmt);
    if (efmt != DF) return;   // another launch computes this expert
    const int rows = tl.row_end - tl.row0;
    static_assert(MI == 4 || MI == 6, "64- or 96-row tiles");
    if (rows <= 32) gpf_tiles<DF, MODE, 2, NB, NW, MULTI>(a, lds, ngrp, tl, ew);
    else if (MI == 4 || rows <= 64) gpf_tiles<DF, MODE, 4, NB, NW, MULTI>(a, lds, ngrp, tl, ew);
    else gpf_tiles<DF, MODE, MI, NB, NW, MULTI>(a, lds, ngrp, tl, ew);
}

// ---------------------------------------------------------------------------
// Combine
// ---------------------------------------------------------------------------

// y[t] = sum_j O[inv[t*k+j]] + sum_s O[P + s*T + t], summed in fp32 in slot
// order, rounded once to bf16. Each thread takes four consecutive columns of
// one token; the rows are loaded eight at a time so that the loads overlap.
// O is read exactly once: non-temporal loads keep it from displacing cached
// data. This kernel reads the 16-bit codes of the layer's down GEMM (four
// codes and their block's exponent per row).
__global__ __launch_bounds__(256) void k_combine(const int16_t *__restrict__ O, const int8_t *__restrict__ Oe,
                                                 const int32_t *__restrict__ inv, int T, int d, int k, int P,
                                                 int n_shared, uint16_t *__restrict__ y) {
    const int t = blockIdx.x;
    const int c4 = blockIdx.y * 256 + threadIdx.x;
    if (c4 >= d / 4) return;
    const int nrows = k + n_shared;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j0 = 0; j0 < nrows; j0 += 8) {
        uint2 q[8];
        int e[8];
#pragma unroll
        for (int u = 0; u < 8; u++) {
            const int j = j0 + u;
            if (j < nrows) {
                const size_t row = j < k ? (size_t)inv[(size_t)t * k + j] : (size_t)P + (size_t)(j - k) * T + t;
                q[u] = __builtin_bit_cast(uint2, __builtin_nontemporal_load(
                                                     reinterpret_cast<const unsigned long long *>(O + row * d) + c4));
                e[u] = Oe[row * (size_t)(d / 16) + c4 / 4];
            }
        }
#pragma unroll
        for (int u = 0; u < 8; u++)
            if (j0 + u < nrows) {
                const float f = __builtin_amdgcn_ldexpf(kOInv, e[u]);
                acc.x += (float)(int16_t)(q[u].x & 0xFFFFu) * f;
                acc.y += (float)(int16_t)(q[u].x >> 16) * f;
                acc.z += (float)(int16_t)(q[u].y & 0xFFFFu) * f;
                acc.w += (float)(int16_t)(q[u].y >> 16) * f;
            }
    }
    uint2 out;
    out.x = (uint32_t)to_bf16(acc.x) | ((uint32_t)to_bf16(acc.y) << 16);
    out.y = (uint32_t)to_bf16(acc.z) | ((uint32_t)to_bf16(acc.w) << 16);
    *reinterpret_cast<uint2 *>(y + (size_t)t * d + c4 * 4) = out;
}

// The same sum over fp32 rows (the decode GEMM's outputs, the atomic-expert
// layer's task rows).
constexpr int kCombineCPT = 1;
__device__ __forceinline__ float4 load_o(const float *p) {
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
    return make_float4(v[0], v[1], v[2], v[3]);
}
__global__ __launch_bounds__(256) void k_combine_f32(const float *__restrict__ O, const int32_t *__restrict__ inv,
                                                     int T, int d, int k, int P, int n_shared,
                                                     uint16_t *__restrict__ y) {
    constexpr int CPT = kCombineCPT;
    const int t = blockIdx.x;
    const int d4 = d / 4;
    const int c0 = blockIdx.y * 256 * CPT + threadIdx.x;
    const int nrows = k + n_shared;
    float4 acc[CPT];
#pragma unroll
    for (int c = 0; c < CPT; c++) acc[c] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j0 = 0; j0 < nrows; j0 += 8) {
        float4 v[8][CPT];
#pragma unroll
        for (int u = 0; u < 8; u++) {
            const int j = j0 + u;
            if (j < nrows) {
                const size_t row = j < k ? (size_t)inv[(size_t)t * k + j] : (size_t)P + (size_t)(j - k) * T + t;
#pragma unroll
                for (int c = 0; c < CPT; c++)
                    if (c0 + 256 * c < d4) v[u][c] = load_o(O + row * d + (c0 + 256 * c) * 4);
            }
        }
#pragma unroll
        for (int u = 0; u < 8; u++)
            if (j0 + u < nrows)
#pragma unroll
                for (int c = 0; c < CPT; c++) {
                    acc[c].x += v[u][c].x;
                    acc[c].y += v[u][c].y;
                    acc[c].z += v[u][c].z;
                    acc[c].w += v[u][c].w;
                }
    }
#pragma unroll
    for (int c = 0; c < CPT; c++) {
        const int c4 = c0 + 256 * c;
        if (c4 >= d4) continue;
        uint2 out;
        out.x = (uint32_t)to_bf16(acc[c].x) | ((uint32_t)to_bf16(acc[c].y) << 16);
        out.y = (uint32_t)to_bf16(acc[c].z) | ((uint32_t)to_bf16(acc[c].w) << 16);
        *reinterpret_cast<uint2 *>(y + (size_t)t * d + c4 * 4) = out;
    }
}

// ---------------------------------------------------------------------------
// Atomic experts (OmniMoE technical summary 2.1, 2.2): N = N_r x N_c vector
// experts E_i(x) = silu(x . w_in_i) w_out_i held in two global bf16 matrices
// W, V [N][d], chosen by a Cartesian product router.
// ---------------------------------------------------------------------------

// Cartesian product routing, one wavefront per token: score(a, b) = l_r[a] +
// l_c[b] in fp32, expert a * N_c + b; the k best scores win, ties to the lower
// flat index; weights: softmax over the k selected scores. Also writes each
// task's dispatch key (its expert's group of B consecutive expert ids).
//
// fp32 addition is monotone in each operand, so every pair outside the best
// min(k, N_r) rows R x best min(k, N_c) columns C scores at most the k-th best
// score s_k among the <= 64 pairs of R x C (k pairs of R x C dominate it in its
// own column or row). The k rounds over R x C are therefore exact unless an
// outside pair rounds to exactly s_k and has a lower flat index than a selected
// pair of score s_k. That needs an outside row a with l_r[a] + max l_c >= s_k
// or an outside column b with max l_r + l_c[b] >= s_k; only then (exact ties,
// rare) are the slots of score s_k refilled with the tied pairs of lowest flat
// index, found row by row in ascending order.
template <int EPL>
__global__ __launch_bounds__(256) void k_cart_topk(const float *__restrict__ logits, int T, int Nr, int Nc, int k,
                                                   int B, int32_t *__restrict__ idx, float *__restrict__ w,
                                                   int32_t *__restrict__ gidx) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    // a token's row logits and then its column logits, one row of Nr + Nc
    const float *lrt = logits + (size_t)t * (Nr + Nc), *lct = lrt + Nr;
    const int kr = min(k, Nr), kc = min(k, Nc);
    // best rows and columns; taken entries' images become 0
    float vr[EPL], vc[EPL];
    uint32_t hr[EPL], hc[EPL];
#pragma unroll
    for (int i = 0; i < EPL; i++) {
        const int a = lane + 64 * i;
        vr[i] = a < Nr ? lrt[a] : 0.0f;
        hr[i] = a < Nr ? ord_u32(vr[i]) : 0u;
        vc[i] = a < Nc ? lct[a] : 0.0f;
        hc[i] = a < Nc ? ord_u32(vc[i]) : 0u;
    }
    int ra = -1, cb = -1;
    for (int j = 0; j < kr; j++) {
        uint32_t vm;
        const int e = wave_take_max<EPL>(hr, lane, vm);
        if (lane == j) ra = e;
    }
    for (int j = 0; j < kc; j++) {
        uint32_t vm;
        const int e = wave_take_max<EPL>(hc, lane, vm);
        if (lane == j) cb = e;
    }
    const int a = __shfl(ra, lane / kc), b = __shfl(cb, lane % kc);
    const bool cand = lane < kr * kc;
    // candidate pairs are not in index order across lanes: each round takes
    // the largest score, then among the lanes holding it the lowest flat index
    // (the largest complement)
    uint32_t h = 0u;
    if (cand) h = ord_u32(lrt[a] + lct[b]);
    const uint32_t nflat = ~(uint32_t)(a * Nc + b);
    uint32_t mine_h = 0u, mine_n = 0u, first_h = 0u, sk = 0u;
    for (int j = 0; j < k; j++) {
        const uint32_t vm = wave_max_u32(h);
        const uint32_t nw = wave_max_u32(h == vm ? nflat : 0u);
        if (h == vm && nflat == nw) h = 0u;   // the winner: pairs have distinct flat indices
        if (lane == j) {
            mine_h = vm;
            mine_n = nw;
        }
        if (j == 0) first_h = vm;
        sk = vm;
    }
    // can a pair outside R x C reach s_k? (only by an exact tie)
    const float lrmax = lrt[__shfl(ra, 0)], lcmax = lct[__shfl(cb, 0)];
    bool reach = false;
#pragma unroll
    for (int i = 0; i < EPL; i++) {
        const int e = lane + 64 * i;
        reach = reach || (e < Nr && hr[i] != 0u && ord_u32(vr[i] + lcmax) >= sk);
        reach = reach || (e < Nc && hc[i] != 0u && ord_u32(lrmax + vc[i]) >= sk);
    }
    if (__ballot(reach) != 0ull) {   // wave-uniform
        // slots [keep, k) hold score s_k: refill them with the tied pairs of
        // lowest flat index over every row that can reach s_k (the taken rows
        // and the outside rows that passed), rows ascending, columns ascending
        const int keep = __popcll(__ballot(lane < k && mine_h > sk));
        const int m = k - keep;
        int got = 0;
#pragma unroll
        for (int i = 0; i < EPL; i++) {
            const int e = lane + 64 * i;
            const bool rel = e < Nr && (hr[i] == 0u || ord_u32(vr[i] + lcmax) >= sk);
            unsigned long long rm = __ballot(rel);
            while (rm != 0ull && got < m) {
                const int row = 64 * i + __ffsll(rm) - 1;
                rm &= rm - 1ull;
                const float lrow = lrt[row];
                for (int c0 = 0; c0 < Nc && got < m; c0 += 64) {
                    const int col = c0 + lane;
                    unsigned long long tm = __ballot(col < Nc && ord_u32(lrow + lct[col < Nc ? col : 0]) == sk);
                    while (tm != 0ull && got < m) {
                        const int cc = c0 + __ffsll(tm) - 1;
                        tm &= tm - 1ull;
                        if (lane == keep + got) {
                            mine_h = sk;
                            mine_n = ~(uint32_t)(row * Nc + cc);
                        }
                        got++;
                    }
                }
            }
        }
    }
    const float ex = lane < k ? expf(ord_value(mine_h) - ord_value(first_h)) : 0.0f;
    const float denom = wave_sum_f32(ex);
    if (lane < k) {
        const int e = (int)~mine_n;
        idx[(size_t)t * k + lane] = e;
        w[(size_t)t * k + lane] = ex / denom;
        gidx[(size_t)t * k + lane] = e / B;
    }
}

// dot of eight bf16 pairs (one 16-byte chunk of each operand) into acc
__device__ __forceinline__ float dot8_bf16(uint4 a, uint4 b, float acc) {
    const uint32_t au[4] = {a.x, a.y, a.z, a.w}, bu[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int h = 0; h < 4; h++) {
        acc = fmaf(bf16f(au[h] & 0xFFFFu), bf16f(bu[h] & 0xFFFFu), acc);
        acc = fmaf(bf16f(au[h] >> 16), bf16f(bu[h] >> 16), acc);
    }
    return acc;
}
// p[0..8) = g * (eight bf16 of v), fp32
__device__ __forceinline__ void store_scaled8(float *p, float g, uint4 v) {
    float4 lo, hi;
    lo.x = g * bf16f(v.x & 0xFFFFu); lo.y = g * bf16f(v.x >> 16);
    lo.z = g * bf16f(v.y & 0xFFFFu); lo.w = g * bf16f(v.y >> 16);
    hi.x = g * bf16f(v.z & 0xFFFFu); hi.y = g * bf16f(v.z >> 16);
    hi.z = g * bf16f(v.w & 0xFFFFu); hi.w = g * bf16f(v.w >> 16);
    *reinterpret_cast<float4 *>(p) = lo;
    *reinterpret_cast<float4 *>(p + 4) = hi;
}

// Expert-centric: the task rows in expert-group order (groups of B
// consecutive expert ids, tokens ascending inside a group), one wavefront per
// row: h = silu(x_t . w_in_e) * (mixing weight), O[row] = h * w_out_e in fp32
// (the combine adds a token's k rows). Neighbouring wavefronts hold the rows of
// one group, so W and V rows that several tasks share come through the cache.
// d = 512 * NCH; each lane owns 16-byte chunk `lane` of every 512-wide column
// chunk. The row's x, w_in and w_out loads are issued together (up to eight
// chunks at a time), one memory round trip per row for d <= 4096.
template <int NCH>
__global__ __launch_bounds__(256) void k_atomic_rows(const uint16_t *__restrict__ x, const uint16_t *__restrict__ W,
                                                     const uint16_t *__restrict__ V, const int32_t *__restrict__ perm,
                                                     const int32_t *__restrict__ idx, const float *__restrict__ wrow,
                                                     int P, int k, float *__restrict__ O) {
    constexpr int d = NCH * 512, CB = NCH < 8 ? NCH : 8;
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= P) return;   // uniform per wave
    const int pair = perm[row];
    const int t = pair / k, e = idx[pair];
    const float wt = wrow[row];
    const uint16_t *xr = x + (size_t)t * d + lane * 8, *wi = W + (size_t)e * d + lane * 8;
    const uint16_t *wo = V + (size_t)e * d + lane * 8;
    float *orow = O + (size_t)row * d + lane * 8;
    if constexpr (NCH == CB) {
        uint4 xv[NCH], wv[NCH], vv[NCH];
#pragma unroll
        for (int c = 0; c < NCH; c++) {
            xv[c] = gload16(xr + c * 512);
            wv[c] = gload16(wi + c * 512);
        }
#pragma unroll
        for (int c = 0; c < NCH; c++) vv[c] = gload16(wo + c * 512);
        float dot = 0.0f;
#pragma unroll
        for (int c = 0; c < NCH; c++) dot = dot8_bf16(xv[c], wv[c], dot);
        const float g = silu_mul(wave_sum_f32(dot), wt);
#pragma unroll
        for (int c = 0; c < NCH; c++) store_scaled8(orow + c * 512, g, vv[c]);
    } else {
        float dot = 0.0f;
#pragma unroll
        for (int c0 = 0; c0 < NCH; c0 += CB) {
            uint4 xv[CB], wv[CB];
#pragma unroll
            for (int c = 0; c < CB; c++)
                if (c0 + c < NCH) {
                    xv[c] = gload16(xr + (c0 + c) * 512);
                    wv[c] = gload16(wi + (c0 + c) * 512);
                }
#pragma unroll
            for (int c = 0; c < CB; c++)
                if (c0 + c < NCH) dot = dot8_bf16(xv[c], wv[c], dot);
        }
        const float g = silu_mul(wave_sum_f32(dot), wt);
#pragma unroll
        for (int c0 = 0; c0 < NCH; c0 += CB) {
            uint4 vv[CB];
#pragma unroll
            for (int c = 0; c < CB; c++)
                if (c0 + c < NCH) vv[c] = gload16(wo + (c0 + c) * 512);
#pragma unroll
            for (int c = 0; c < CB; c++)
                if (c0 + c < NCH) store_scaled8(orow + (c0 + c) * 512, g, vv[c]);
        }
    }
}

// Token-centric (the scheduling the OmniMoE page replaces, kept as the
// ablation): one wavefront per token takes its k experts in slot order and
// accumulates y_t in registers. Each expert's w_in and w_out rows are loaded
// together; for d <= 2048 the next expert's rows are loaded while the current
// one is computed (two register slots).
template <int NCH>
__global__ __launch_bounds__(256) void k_atomic_token(const uint16_t *__restrict__ x, const uint16_t *__restrict__ W,
                                                      const uint16_t *__restrict__ V, const int32_t *__restrict__ idx,
                                                      const float *__restrict__ w, int T, int k,
                                                      uint16_t *__restrict__ y) {
    constexpr int d = NCH * 512;
    constexpr bool kAhead = NCH <= 4;
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;   // uniform per wave
    // lane j < k holds slot j's expert and weight (k <= 8)
    const int my_e = lane < k ? idx[(size_t)t * k + lane] : 0;
    const float my_w = lane < k ? w[(size_t)t * k + lane] : 0.0f;
    const uint16_t *xr = x + (size_t)t * d + lane * 8;
    uint4 xv[NCH];
#pragma unroll
    for (int c = 0; c < NCH; c++) xv[c] = gload16(xr + c * 512);
    float acc[NCH][8];
#pragma unroll
    for (int c = 0; c < NCH; c++)
#pragma unroll
        for (int q = 0; q < 8; q++) acc[c][q] = 0.0f;
    auto load = [&](int j, uint4 (&wv)[NCH], uint4 (&vv)[NCH]) {
        const int e = __builtin_amdgcn_readlane(my_e, j);
        const uint16_t *wi = W + (size_t)e * d + lane * 8, *wo = V + (size_t)e * d + lane * 8;
#pragma unroll
        for (int c = 0; c < NCH; c++) {
            wv[c] = gload16(wi + c * 512);
            vv[c] = gload16(wo + c * 512);
        }
    };
    auto expert = [&](int j, const uint4 (&wv)[NCH], const uint4 (&vv)[NCH]) {
        float dot = 0.0f;
#pragma unroll
        for (int c = 0; c < NCH; c++) dot = dot8_bf16(xv[c], wv[c], dot);
        const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_w), j));
        const float g = silu_mul(wave_sum_f32(dot), wj);
#pragma unroll
        for (int c = 0; c < NCH; c++) {
            const uint32_t vu[4] = {vv[c].x, vv[c].y, vv[c].z, vv[c].w};
#pragma unroll
            for (int h = 0; h < 4; h++) {
                acc[c][2 * h] += g * bf16f(vu[h] & 0xFFFFu);
                acc[c][2 * h + 1] += g * bf16f(vu[h] >> 16);
            }
        }
    };
    if constexpr (kAhead) {
        uint4 wv[2][NCH], vv[2][NCH];
        load(0, wv[0], vv[0]);
#pragma unroll
        for (int j = 0; j < 8; j++) {   // k <= 8; unrolled so the slots are static
            if (j >= k) break;
            if (j + 1 < k) load(j + 1, wv[(j + 1) & 1], vv[(j + 1) & 1]);
            expert(j, wv[j & 1], vv[j & 1]);
        }
    } else {
        for (int j = 0; j < k; j++) {
            uint4 wv[NCH], vv[NCH];
            load(j, wv, vv);
            expert(j, wv, vv);
        }
    }
    uint16_t *yr = y + (size_t)t * d + lane * 8;
#pragma unroll
    for (int c = 0; c < NCH; c++) {
        uint4 out;
        out.x = (uint32_t)to_bf16(acc[c][0]) | ((uint32_t)to_bf16(acc[c][1]) << 16);
        out.y = (uint32_t)to_bf16(acc[c][2]) | ((uint32_t)to_bf16(acc[c][3]) << 16);
        out.z = (uint32_t)to_bf16(acc[c][4]) | ((uint32_t)to_bf16(acc[c][5]) << 16);
        out.w = (uint32_t)to_bf16(acc[c][6]) | ((uint32_t)to_bf16(acc[c][7]) << 16);
        *reinterpret_cast<uint4 *>(yr + c * 512) = out;
    }
}

// ---------------------------------------------------------------------------
// Shader clock probe (measurement)
// ---------------------------------------------------------------------------

// One wave that samples the shader-cycle counter (s_memtime) and the
// constant-rate real-time counter (s_memrealtime) every ~`period` real-time
// ticks until `duration` ticks have passed (a bounded wait on the wall clock:
// it always ends), writing (cycles, ticks) pairs to out[2 i], out[2 i + 1] for
// i < max_samples. Run beside other work on another stream, the cycle/tick
// ratio over a window gives the shader clock during that window.
__global__ __launch_bounds__(64) void k_clock_probe(unsigned long long *out, unsigned long long duration,
                                                    unsigned long long period, int max_samples) {
    if (threadIdx.x != 0) return;
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    unsigned long long next = r0;
    int i = 0;
    for (;;) {
        const unsigned long long c = __builtin_amdgcn_s_memtime();
        const unsigned long long r = __builtin_amdgcn_s_memrealtime();
        if (r >= next && i < max_samples) {
            out[2 * i] = c;
            out[2 * i + 1] = r;
            i++;
            next = r + period;
        }
        if (r - r0 >= duration || i >= max_samples) break;
        __builtin_amdgcn_s_sleep(8);
    }
}

hipError_t launch_clock_probe(unsigned long long *out, unsigned long long duration, unsigned long long period,
                              int max_samples, hipStream_t s) {
    hipLaunchKernelGGL(k_clock_probe, dim3(1), dim3(64), 0, s, out, duration, period, max_samples);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Static scratch for the allocation-free forward
// ---------------------------------------------------------------------------

// Workspace of qmoe_forward_static. Each device holds its own copy for the
// life of the process. In host code `scratch` names a host-side stand-in, not
// device memory: its device address comes from hipGetSymbolAddress, looked up
// once per device with that device current.
static __device__ __attribute__((aligned(256))) uint8_t scratch[kStaticScratchBytes];

hipError_t static_scratch(void **ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

// Expert tiles of 64 for many experts, 32, or 16 when E <= 16 (no idle half tile).
// rf != NULL: the gating epilogue runs in the router when one expert tile
// holds every expert (and k <= 16); *chunk receives the tasks per dispatch
// chunk it used (BT * k), or 0 when it did not run.
template <int BT, int BE, int WE, int NST>
static void launch_router_lds(const uint16_t *x, const uint16_t *wr, const float *rscale, const float *bias,
                              float *logits, float *xsum, float xscale, int T, int d, int E, const RouteFuse *rf,
                              int *chunk, hipStream_t s) {
    const long gx = 8L * ((T + BT * 8 - 1) / (BT * 8));   // token tiles, padded to a multiple of 8
    const int net = (E + BE - 1) / BE;
    if (rf && net == 1 && rf->k <= 16) {
        *chunk = BT * rf->k;
        hipLaunchKernelGGL((k_router_lds<BT, BE, WE, NST, true>), dim3((unsigned)gx), dim3(256), 0, s, x, wr, rscale,
                           bias, logits, xsum, xscale, T, d, E, net, *rf);
        return;
    }
    if (chunk) *chunk = 0;
    hipLaunchKernelGGL((k_router_lds<BT, BE, WE, NST, false>), dim3((unsigned)(gx * net)), dim3(256), 0, s, x, wr,
                       rscale, bias, logits, xsum, xscale, T, d, E, net, RouteFuse{});
}

// The expert tile width launch_router_bf16 picks, and whether the gating
// epilogue fuses for that shape (one expert tile covers every expert, k <= 16).
static int router_tile_experts(int T, int E) { return (T < 256 || E <= 16) ? 16 : E <= 32 ? 32 : E <= 64 ? 64 : 128; }
bool router_fuses(int T, int E, int k) { return E <= router_tile_experts(T, E) && k <= 16; }

hipError_t launch_router_bf16(const uint16_t *x, const uint16_t *wr, const float *rscale, const float *bias,
                              float *logits, float *xsum, float xscale, int T, int d, int E, const RouteFuse *rf,
                              int *chunk, hipStream_t s) {
    // 16 x 16 tiles as four independent streams for small batches and few
    // experts (LDS: 4 rings of 3 x 8 KB, 4 x 8 KB up to 64 tokens, where a
    // stream of d <= 2048 has all its groups in flight at once); wider expert tiles for large batches
    // (4 rings of 3 x 12 KB; shared rings of 3 x 20 KB, and 3 x 40 KB while
    // the 32-token tiles fit one round of one workgroup per CU, else 2 x 40 KB
    // for two per CU)
    if (T <= 64) launch_router_lds<16, 16, 1, 4>(x, wr, rscale, bias, logits, xsum, xscale, T, d, E, rf, chunk, s);
    else if (T < 256 || E <= 16) launch_router_lds<16, 16, 1, 3>(x, wr, rscale, bias, logits, xsum, xscale, T, d, E, rf, chunk, s);
    else if (E <= 32) launch_router_lds<16, 32, 1, 3>(x, wr, rscale, bias, logits, xsum, xscale, T, d, E, rf, chunk, s);
    else if (E <= 64) launch_router_lds<16, 64, 4, 3>(x, wr, rscale, bias, logits, xsum, xscale, T, d, E, rf, chunk, s);
    else if ((T + 31) / 32 <= 256) launch_router_lds<32, 128, 4, 3>(x, wr, rscale, bias, logits, xsum, xscale, T, d, E, rf, chunk, s);
    else launch_router_lds<32, 128, 4, 2>(x, wr, rscale, bias, logits, xsum, xscale, T, d, E, rf, chunk, s);
    return hipGetLastError();
}

hipError_t launch_router_f32(const uint16_t *x, const float *wr, const float *bias, float *logits, int T, int d, int E,
                             hipStream_t s) {
    hipLaunchKernelGGL(k_router_f32, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, x, wr, bias, logits, T, d, E);
    return hipGetLastError();
}

hipError_t launch_topk(const float *logits, int T, int E, int k, int renorm, int32_t *idx, float *w, hipStream_t s) {
    dim3 grid((T + 3) / 4);
    if (E <= 64)
        hipLaunchKernelGGL(k_topk<1>, grid, dim3(256), 0, s, logits, T, E, k, renorm, idx, w);
    else if (E <= 128)
        hipLaunchKernelGGL(k_topk<2>, grid, dim3(256), 0, s, logits, T, E, k, renorm, idx, w);
    else if (E <= 256)
        hipLaunchKernelGGL(k_topk<4>, grid, dim3(256), 0, s, logits, T, E, k, renorm, idx, w);
    else if (E <= 512)
        hipLaunchKernelGGL(k_topk<8>, grid, dim3(256), 0, s, logits, T, E, k, renorm, idx, w);
    else
        hipLaunchKernelGGL(k_topk<16>, grid, dim3(256), 0, s, logits, T, E, k, renorm, idx, w);
    return hipGetLastError();
}

hipError_t launch_route_small(const float *logits, int T, int E, int k, int renorm, int n_shared, int bm,
                              int32_t *idx, float *w, int32_t *counts, int32_t *offsets, Tile *tiles,
                              int32_t *num_tiles, int32_t *perm, int32_t *inv, float *wrow, hipStream_t s) {
    if (T > kSmallRouteMaxT || E > kSmallRouteMaxE) return hipErrorInvalidValue;
    if (E <= 64)
        hipLaunchKernelGGL(k_route_small<1>, dim3(1), dim3(1024), 0, s, logits, T, E, k, renorm, n_shared, bm, idx, w,
                           counts, offsets, tiles, num_tiles, perm, inv, wrow);
    else if (E <= 128)
        hipLaunchKernelGGL(k_route_small<2>, dim3(1), dim3(1024), 0, s, logits, T, E, k, renorm, n_shared, bm, idx, w,
                           counts, offsets, tiles, num_tiles, perm, inv, wrow);
    else
        hipLaunchKernelGGL(k_route_small<4>, dim3(1), dim3(1024), 0, s, logits, T, E, k, renorm, n_shared, bm, idx, w,
                           counts, offsets, tiles, num_tiles, perm, inv, wrow);
    return hipGetLastError();
}

hipError_t launch_dispatch_count(const int32_t *idx, int P, int E, int32_t *chunk_counts, hipStream_t s) {
    const int nchunks = (P + kDispatchChunk - 1) / kDispatchChunk;
    hipLaunchKernelGGL(k_dispatch_count, dim3(nchunks), dim3(256), E * sizeof(int), s, idx, P, E, chunk_counts);
    return hipGetLastError();
}

hipError_t launch_dispatch_scan(const int32_t *chunk_counts, int nchunks, int E, int P, int T, int n_shared, int bm,
                                int32_t *chunk_base, int32_t *counts, int32_t *offsets, Tile *tiles,
                                int32_t *num_tiles, hipStream_t s) {
    hipLaunchKernelGGL(k_dispatch_scan, dim3(1), dim3(1024), 0, s, chunk_counts, nchunks, E, P, T, n_shared, bm,
                       chunk_base, counts, offsets, tiles, num_tiles);
    return hipGetLastError();
}

hipError_t launch_dispatch_scatter(const int32_t *idx, const float *w, int P, int E, int chunk,
                                   const int32_t *chunk_base, int32_t *perm, int32_t *inv, float *wrow, hipStream_t s) {
    const int nchunks = (P + chunk - 1) / chunk;
    const size_t lds = (size_t)E * (4 * sizeof(unsigned long long) + sizeof(int));
    hipLaunchKernelGGL(k_dispatch_scatter, dim3(nchunks), dim3(256), lds, s, idx, w, P, E, chunk, chunk_base, perm,
                       inv, wrow);
    return hipGetLastError();
}

template <int MODE>
static hipError_t launch_gemm_dec(int df, dim3 grid, const GemmArgs &a, hipStream_t s) {
    switch (df) {
    case kDfAllFormats: hipLaunchKernelGGL(k_gemm_dec_mixed<MODE>, grid, dim3(256), 0, s, a); break;
    case DF_INT8: hipLaunchKernelGGL((k_gemm_dec<DF_INT8, MODE>), grid, dim3(256), 0, s, a); break;
    case DF_I4ASYM: hipLaunchKernelGGL((k_gemm_dec<DF_I4ASYM, MODE>), grid, dim3(256), 0, s, a); break;
    case DF_I4SYM: hipLaunchKernelGGL((k_gemm_dec<DF_I4SYM, MODE>), grid, dim3(256), 0, s, a); break;
    case DF_FP8: hipLaunchKernelGGL((k_gemm_dec<DF_FP8, MODE>), grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Consecutive 256-column tiles per prefill workgroup: with short K (the down
// projection of narrow experts) a tile spends a large part of its time on
// filling and draining its load pipeline, which one pipeline through several
// tiles pays once. Fewer, longer workgroups also quantize worse onto the
// machine's 512 workgroup slots (two per CU): a workgroup takes up to
// kGemmGroupTarget / KB tiles, as long as the launch keeps at least
// kGemmMinWorkgroups workgroups (six rounds of the slots). The environment
// variable QMOE_PREFILL_TILES_PER_WG = n >= 1 sets the count instead (capped
// at the tiles there are; for tuning and tests).
#ifndef QMOE_GEMM_GROUP_TARGET
#define QMOE_GEMM_GROUP_TARGET 12
#endif
constexpr int kGemmGroupTarget = QMOE_GEMM_GROUP_TARGET;
constexpr long kGemmMinWorkgroups = 6 * 512;

static int gemm_nsub(int df, int bm, int KB, int n_tiles, int max_tiles) {
    // the 96-row INT4-asym and 8-bit variants have no registers to spare for
    // the operands in flight while a tile ends (zero-point correction,
    // 8-bit code words)
    if (bm == 96 && df != DF_I4SYM) return 1;
    if (const char *env = std::getenv("QMOE_PREFILL_TILES_PER_WG")) {
        const int n = std::atoi(env);
        if (n >= 1) return std::min(n, n_tiles);
    }
    int nsub = std::min(n_tiles, std::max(1, (kGemmGroupTarget + KB - 1) / KB));
    while (nsub > 1 && (long)max_tiles * ((n_tiles + nsub - 1) / nsub) < kGemmMinWorkgroups) nsub--;
    return nsub;
}

template <int DF, int MODE, int MI>
static void launch_gpf(bool multi, dim3 grid, const GemmArgs &a, hipStream_t s) {
    if constexpr (DF != DF_I4SYM && MI == 6) {
        hipLaunchKernelGGL((k_gemm_gpf<DF, MODE, MI, 4, 4, false>), grid, dim3(256), 0, s, a);
    } else {
        if (multi) hipLaunchKernelGGL((k_gemm_gpf<DF, MODE, MI, 4, 4, true>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((k_gemm_gpf<DF, MODE, MI, 4, 4, false>), grid, dim3(256), 0, s, a);
    }
}

template <int MODE>
static hipError_t launch_gemm(int df, int bm, int max_tiles, int maxN, const GemmArgs &a0, hipStream_t s) {
    GemmArgs a = a0;
    a.n_tiles = (maxN + 255) / 256;
    if ((bm == 64 || bm == 96) && (df == DF_I4SYM || df == DF_I4ASYM)) {
        // prefill tiles: bm rows x 256 columns, 4 waves of bm x 64, two stages,
        // two workgroups per CU (<= 256 VGPRs; 34 KB / 52 KB LDS each); K of
        // the down projection taken as the widest expert's
        a.nsub = gemm_nsub(df, bm, (MODE == 0 ? a.d : a.ldh) / 128, a.n_tiles, max_tiles);
        a.n_groups = (a.n_tiles + a.nsub - 1) / a.nsub;
        const long total = (long)max_tiles * a.n_groups;
        dim3 grid((unsigned)(8 * ((total + 7) / 8)));
        const bool multi = a.nsub > 1;
        if (bm == 64) {
            if (df == DF_I4SYM) launch_gpf<DF_I4SYM, MODE, 4>(multi, grid, a, s);
            else launch_gpf<DF_I4ASYM, MODE, 4>(multi, grid, a, s);
        } else {
            if (df == DF_I4SYM) launch_gpf<DF_I4SYM, MODE, 6>(multi, grid, a, s);
            else launch_gpf<DF_I4ASYM, MODE, 6>(multi, grid, a, s);
        }
        return hipGetLastError();
    }
    if (bm == 16) {
        const int cols = 4 * kDecodeBlocksPerWave * 16;
        return launch_gemm_dec<MODE>(df, dim3((maxN + cols - 1) / cols, max_tiles), a, s);
    }
    // per-channel formats (8-bit codes): the same kernel; e4m3 in 64-row
    // tiles only (its 96-row variant would spill)
    if (!((bm == 64 && (df == DF_INT8 || df == DF_FP8)) || (bm == 96 && df == DF_INT8))) return hipErrorInvalidValue;
    a.nsub = gemm_nsub(df, bm, (MODE == 0 ? a.d : a.ldh) / 128, a.n_tiles, max_tiles);
    a.n_groups = (a.n_tiles + a.nsub - 1) / a.nsub;
    const long total = (long)max_tiles * a.n_groups;
    dim3 grid((unsigned)(8 * ((total + 7) / 8)));
    if (bm == 64) {
        if (df == DF_INT8) launch_gpf<DF_INT8, MODE, 4>(a.nsub > 1, grid, a, s);
        else launch_gpf<DF_FP8, MODE, 4>(a.nsub > 1, grid, a, s);
    } else {
        launch_gpf<DF_INT8, MODE, 6>(false, grid, a, s);
    }
    return hipGetLastError();
}

hipError_t launch_gemm13(int df, int bm, const GemmArgs &a, int max_tiles, int maxN13, hipStream_t s) {
    return launch_gemm<0>(df, bm, max_tiles, maxN13, a, s);
}

hipError_t launch_gemm2(int df, int bm, const GemmArgs &a, int max_tiles, hipStream_t s) {
    return launch_gemm<1>(df, bm, max_tiles, a.d, a, s);
}

hipError_t launch_xsum(const uint16_t *x, int T, int d, float scale, float *xsum, hipStream_t s) {
    hipLaunchKernelGGL(k_xsum, dim3((T + 3) / 4), dim3(256), 0, s, x, T, d, scale, xsum);
    return hipGetLastError();
}

hipError_t launch_combine(const int16_t *O, const int8_t *Oe, const int32_t *inv, int T, int d, int k, int P,
                          int n_shared, uint16_t *y, hipStream_t s) {
    hipLaunchKernelGGL(k_combine, dim3(T, (d / 4 + 255) / 256), dim3(256), 0, s, O, Oe, inv, T, d, k, P, n_shared, y);
    return hipGetLastError();
}

hipError_t launch_combine_f32(const float *O, const int32_t *inv, int T, int d, int k, int P, int n_shared,
                              uint16_t *y, hipStream_t s) {
    hipLaunchKernelGGL(k_combine_f32, dim3(T, (d / 4 + 256 * kCombineCPT - 1) / (256 * kCombineCPT)), dim3(256), 0, s, O, inv,
                       T, d, k, P, n_shared, y);
    return hipGetLastError();
}

hipError_t launch_cart_topk(const float *logits, int T, int Nr, int Nc, int k, int B, int32_t *idx, float *w,
                            int32_t *gidx, hipStream_t s) {
    const dim3 grid((T + 3) / 4);
    const int n = Nr > Nc ? Nr : Nc;
    if (n <= 64) hipLaunchKernelGGL(k_cart_topk<1>, grid, dim3(256), 0, s, logits, T, Nr, Nc, k, B, idx, w, gidx);
    else if (n <= 256) hipLaunchKernelGGL(k_cart_topk<4>, grid, dim3(256), 0, s, logits, T, Nr, Nc, k, B, idx, w, gidx);
    else hipLaunchKernelGGL(k_cart_topk<16>, grid, dim3(256), 0, s, logits, T, Nr, Nc, k, B, idx, w, gidx);
    return hipGetLastError();
}

// d = 512 * NCH with 1 <= NCH <= 16 (checked by the caller)
#define QMOE_NCH_CASES(F) \
    F(1) F(2) F(3) F(4) F(5) F(6) F(7) F(8) F(9) F(10) F(11) F(12) F(13) F(14) F(15) F(16)

hipError_t launch_atomic_rows(const uint16_t *x, const uint16_t *W, const uint16_t *V, const int32_t *perm,
                              const int32_t *idx, const float *wrow, int P, int d, int k, float *O, hipStream_t s) {
    const dim3 grid((P + 3) / 4);
    switch (d / 512) {
#define QMOE_ROWS_CASE(n) \
    case n: hipLaunchKernelGGL(k_atomic_rows<n>, grid, dim3(256), 0, s, x, W, V, perm, idx, wrow, P, k, O); break;
        QMOE_NCH_CASES(QMOE_ROWS_CASE)
#undef QMOE_ROWS_CASE
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_atomic_token(const uint16_t *x, const uint16_t *W, const uint16_t *V, const int32_t *idx,
                               const float *w, int T, int d, int k, uint16_t *y, hipStream_t s) {
    const dim3 grid((T + 3) / 4);
    switch (d / 512) {
#define QMOE_TOKEN_CASE(n) \
    case n: hipLaunchKernelGGL(k_atomic_token<n>, grid, dim3(256), 0, s, x, W, V, idx, w, T, k, y); break;
        QMOE_NCH_CASES(QMOE_TOKEN_CASE)
#undef QMOE_TOKEN_CASE
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}
#undef QMOE_NCH_CASES

}  // namespace qmoe
