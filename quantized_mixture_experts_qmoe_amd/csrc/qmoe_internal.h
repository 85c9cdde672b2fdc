// Internal declarations shared by the HIP library's translation units
// (packer, kernels, C-ABI layer). Not installed; not part of the ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "../../include/qmoe.h"

namespace qmoe {

// ---------------------------------------------------------------------------
// Device weight layout.
//
// A packed block covers 16 output rows x 128 input positions (k) of one matrix.
// 4-bit formats: 1024 bytes. Lane l (0..63) of a wave owns bytes [16l, 16l+16);
//   its dword s (0..3) holds the eight codes of row (l % 16) at
//   k = 32s + 8(l/16) + j, j = 0..7. Code j occupies bits [4(j/2), 4(j/2)+4) when
//   j is even and bits [16 + 4(j/2), 16 + 4(j/2)+4) when j is odd, so that
//   (dword >> 4i) & 0x000F000F yields codes 2i and 2i+1 in the two 16-bit halves.
//   Stored values are unsigned: q + 8 for the symmetric formats, q for INT4_ASYM.
// 8-bit formats: 2048 bytes. Lane l owns bytes [32l, 32l+32); dwords 2s and 2s+1
//   hold the eight codes of row (l % 16) at k = 32s + 8(l/16) + j in byte j.
// In both cases a lane's dword pair for step s is exactly the B operand of one
// v_mfma_f32_16x16x32_bf16 (lane l supplies column l%16, k = 8(l/16)..+8).
// Blocks are stored row-block major: block (rb, kb) at index rb*(K/128) + kb.
// Group scales / zeros (fp16 bits): [N/16][K/128][16], the block's 16 rows
// contiguous. Per-channel scales (fp32): [N].
// Zero-point correction operand (INT4_ASYM only): v_ng = s_ng * z_ng / 128 split
// exactly into bf16 hi + lo and laid out as MFMA B operands over the group
// index: block (rb, gs) of 1024 bf16 = hi[64 lanes][8] then lo[64 lanes][8];
// lane l holds row rb*16 + l%16, groups g = 32gs + 8(l/16) + j (0 past the last
// group).
//
// The gate and up matrices of one expert are packed as a single matrix "W13"
// of 2F rows whose 16-row blocks alternate: block 2b = gate rows 16b..16b+15,
// block 2b+1 = up rows 16b..16b+15. The down matrix "W2" is [d][F].
// ---------------------------------------------------------------------------
constexpr int kBlockRows = 16;
constexpr int kBlockK = 128;

enum DevFormat : int {
    DF_INT8 = 0,   // signed int8 codes, fp32 per-row scale
    DF_I4ASYM = 1, // 4-bit codes, fp16 scale + zero per (row, group)
    DF_I4SYM = 2,  // 4-bit codes (q+8), fp16 scale per (row, group); INT3 uses it too
    DF_FP8 = 4     // e4m3 codes, fp32 per-row scale
};

inline int dev_format(int wformat) {
    switch (wformat) {
    case QMOE_W_INT8_SYM_CH: return DF_INT8;
    case QMOE_W_INT4_ASYM_G128: return DF_I4ASYM;
    case QMOE_W_INT4_SYM_G128: return DF_I4SYM;
    case QMOE_W_INT3_SYM_G128_IN4: return DF_I4SYM;
    case QMOE_W_FP8E4M3_CH: return DF_FP8;
    default: return -1;
    }
}
inline bool is_group_wformat(int wformat) {
    return wformat == QMOE_W_INT4_ASYM_G128 || wformat == QMOE_W_INT4_SYM_G128 ||
           wformat == QMOE_W_INT3_SYM_G128_IN4;
}
inline int block_bytes(int df) { return (df == DF_INT8 || df == DF_FP8) ? 2048 : 1024; }

// Device pointers of one expert's packed matrices.
struct ExpertW {
    const uint8_t *c13;   // W13 codes
    const uint16_t *s13;  // W13 group scales (fp16 bits) or nullptr
    const uint16_t *z13;  // W13 group zeros (fp16 bits) or nullptr
    const float *p13;     // W13 per-channel scales [2F] or nullptr
    const uint16_t *zc13; // W13 zero-point correction operand (INT4_ASYM) or nullptr
    const uint8_t *c2;    // W2 codes
    const uint16_t *s2;
    const uint16_t *z2;
    const float *p2;      // W2 per-channel scales [d]
    const uint16_t *zc2;
    int32_t F;            // d_ff of this expert
    int32_t pad[3];
};

// One M-tile of the grouped GEMMs: rows [row0, row_end) of expert e.
struct Tile {
    int32_t e, row0, row_end, pad;
};

// ---------------------------------------------------------------------------
// Host packer (qmoe_pack.cpp)
// ---------------------------------------------------------------------------
struct CanonMatrix {      // canonical quantized matrix, row-major [N][K]
    int N = 0, K = 0;
    std::vector<int8_t> q;     // codes as exported
    std::vector<float> scale;  // [N][G] or [N]
    std::vector<float> zero;   // same shape as scale
};

// Quantize w[N][K] by the format rules. Returns QMOE_OK or a QMOE_E* code.
int quantize_matrix(int wformat, int N, int K, const float *w, CanonMatrix &out);

// Router weight w[E][d] quantized per expert row (router_quant: QMOE_RQ_INT8_CH
// or QMOE_RQ_FP8E4M3_CH, the rules of the per-channel expert formats): the
// codes' values as bf16 bits (exact) and the fp32 row scales.
int quantize_router(int router_quant, int E, int d, const float *w, std::vector<uint16_t> &codes_bf16,
                    std::vector<float> &scale);

// Device layout of a canonical matrix (codes blocks, group scales/zeros as fp16
// bits, per-channel scales). For W13 the caller passes the interleaved matrix.
struct PackedMatrix {
    std::vector<uint8_t> codes;
    std::vector<uint16_t> gscale, gzero;
    std::vector<float> pscale;
    std::vector<uint16_t> zc;   // zero-point correction operand (INT4_ASYM)
};
void layout_matrix(int wformat, const CanonMatrix &m, PackedMatrix &out);
// Build the interleaved W13 canonical matrix from gate and up.
void interleave_gate_up(const CanonMatrix &gate, const CanonMatrix &up, CanonMatrix &w13, bool group_format);
// Inverse of layout_matrix (for export): fills codes/scales/zeros of m (N, K preset).
void unlayout_matrix(int wformat, const PackedMatrix &p, CanonMatrix &m);

// Element counts of a packed matrix (what layout_matrix produces), without packing.
struct PackSizes {
    size_t codes = 0, gscale = 0, gzero = 0, pscale = 0, zc = 0;
};
PackSizes pack_sizes(int wformat, int N, int K);

// On-device quantizer (qmoe_quant.hip): matrix [N][K] of bf16 values at `a`
// (for W13: gate at `a`, up at `b`, interleaved by 16-row blocks; otherwise b
// is NULL) into the packed arrays at their arena addresses. zero_row: N bytes
// of scratch (per-channel formats). The zc array must be zeroed beforehand.
hipError_t launch_quant_matrix(int wformat, const uint16_t *a, const uint16_t *b, int N, int K, uint8_t *codes,
                               uint16_t *gscale, uint16_t *gzero, float *pscale, uint16_t *zc, uint8_t *zero_row,
                               hipStream_t s);

// ---------------------------------------------------------------------------
// Kernel launchers (qmoe_kernels.hip). All asynchronous on `s`.
// ---------------------------------------------------------------------------
// xsum (may be NULL): receives xscale * per-128-group row sums of x.
// rscale (may be NULL): per-expert scale of a quantized router (logit =
// rscale[e] * x.wr[e] + bias[e]).
// rf (may be NULL): the gating network's outputs when it runs fused in the
// router's epilogue (possible where one router workgroup holds every expert of
// its tokens, k <= 16): top-k indices and weights and the per-expert task
// counts of each token tile (one dispatch chunk of BT * k tasks). *chunk (may
// be NULL when rf is) receives BT * k when the fused epilogue ran, else 0.
// logits may be NULL when it runs.
struct RouteFuse {
    int32_t *idx;           // [T][k] selected experts
    float *w;               // [T][k] mixing weights
    int32_t *chunk_counts;  // [token tiles][E] tasks per expert of each tile
    int32_t k, renorm;
};
hipError_t launch_router_bf16(const uint16_t *x, const uint16_t *wr, const float *rscale, const float *bias,
                              float *logits, float *xsum, float xscale, int T, int d, int E, const RouteFuse *rf,
                              int *chunk, hipStream_t s);
// Whether launch_router_bf16 runs the fused gating epilogue for this shape.
bool router_fuses(int T, int E, int k);
hipError_t launch_router_f32(const uint16_t *x, const float *wr, const float *bias, float *logits, int T, int d, int E,
                             hipStream_t s);
hipError_t launch_topk(const float *logits, int T, int E, int k, int renorm, int32_t *idx, float *w, hipStream_t s);
// Dispatch: per-chunk histogram, scan + tile list, stable scatter. The
// histogram kernel's chunk is kDispatchChunk tasks; the fused router's is one
// token tile (BT * k tasks, BT >= 16).
constexpr int kDispatchChunk = 1024;
constexpr int kMinRouterTile = 16;
// One-workgroup top-k + dispatch for small batches.
constexpr int kSmallRouteMaxT = 64;
constexpr int kSmallRouteMaxE = 256;
hipError_t launch_dispatch_count(const int32_t *idx, int P, int E, int32_t *chunk_counts, hipStream_t s);
hipError_t launch_dispatch_scan(const int32_t *chunk_counts, int nchunks, int E, int P, int T, int n_shared, int bm,
                                int32_t *chunk_base, int32_t *counts, int32_t *offsets, Tile *tiles,
                                int32_t *num_tiles, hipStream_t s);
// Also writes wrow[row] = w[pair of row] (the mixing weight in row order).
// chunk: tasks per chunk of the counts the scan consumed.
hipError_t launch_dispatch_scatter(const int32_t *idx, const float *w, int P, int E, int chunk,
                                   const int32_t *chunk_base, int32_t *perm, int32_t *inv, float *wrow, hipStream_t s);
// Top-k and the whole dispatch in one workgroup (T <= kSmallRouteMaxT, E <= kSmallRouteMaxE).
hipError_t launch_route_small(const float *logits, int T, int E, int k, int renorm, int n_shared, int bm,
                              int32_t *idx, float *w, int32_t *counts, int32_t *offsets, Tile *tiles,
                              int32_t *num_tiles, int32_t *perm, int32_t *inv, float *wrow, hipStream_t s);

// Experts are laid out in groups of one kind (routed / shared) and one device
// format, each group uniformly strided in the arena: at most 2 x 4 groups.
constexpr int kMaxExpertGroups = 8;

struct GemmArgs {
    // Expert pointers: expert e is group g's first expert advanced by i *
    // ex_stride[g] bytes. Without a slot table (every expert in one format) g
    // is 0 for routed and 1 for shared experts and i the index among them, with
    // no dependent load; with one (per-expert formats), eslot[e] = g << 20 | i.
    // A launch computes only the experts whose group format gfmt[g] is its own.
    ExpertW ex0[kMaxExpertGroups];
    int64_t ex_stride[kMaxExpertGroups];
    int32_t gfmt[kMaxExpertGroups];
    const int32_t *eslot;
    const Tile *tiles;
    const int32_t *num_tiles;
    const int32_t *perm;     // task list (pair id per routed row)
    const float *wrow;       // mixing weight per routed row [P] (row order)
    const uint16_t *x;       // [T][d] bf16 (gate/up input)
    const float *xsum;       // [T][d/128] group sums of x
    uint16_t *H;             // [rows][ldh] bf16 intermediate
    float *hsum;             // [rows][ldh/128] group sums of H (bf16-rounded values)
    int16_t *O;              // [rows][d] weighted expert outputs of prefill tiles, 16-bit codes (see k_combine)
    int8_t *Oe;              // [rows][d/16] their exponents, one per 16 columns
    float *Of;               // [rows][d] fp32 weighted expert outputs of decode tiles (same memory as O)
    int32_t ldh;
    int32_t d;
    int32_t k;               // top-k
    int32_t P;               // routed rows (T*k)
    int32_t T;
    int32_t E;               // routed experts
    int32_t n_tiles;         // 256-column N-tiles of the widest expert (set by the launcher)
    int32_t nsub;            // prefill: consecutive N-tiles per workgroup (set by the launcher)
    int32_t n_groups;        // prefill: ceil(n_tiles / nsub)
};
// bm: rows per M-tile (16: weight-streaming decode kernel; 64: prefill
// kernels); max_tiles: grid bound; maxN13: max 2F. df = kDfAllFormats (decode
// tiles only): one launch for every expert of a layer with per-expert formats.
constexpr int kDfAllFormats = -1;
hipError_t launch_gemm13(int df, int bm, const GemmArgs &a, int max_tiles, int maxN13, hipStream_t s);
hipError_t launch_gemm2(int df, int bm, const GemmArgs &a, int max_tiles, hipStream_t s);
// O: the prefill down GEMM's 16-bit codes and per-16-column exponents; the
// _f32 variant sums fp32 rows (decode tiles, atomic experts).
hipError_t launch_combine(const int16_t *O, const int8_t *Oe, const int32_t *inv, int T, int d, int k, int P,
                          int n_shared, uint16_t *y, hipStream_t s);
hipError_t launch_combine_f32(const float *O, const int32_t *inv, int T, int d, int k, int P, int n_shared,
                              uint16_t *y, hipStream_t s);
hipError_t launch_xsum(const uint16_t *x, int T, int d, float scale, float *xsum, hipStream_t s);

// Shader clock probe: one wave sampling (shader cycles, real-time ticks) pairs.
hipError_t launch_clock_probe(unsigned long long *out, unsigned long long duration, unsigned long long period,
                              int max_samples, hipStream_t s);

// Static per-device scratch (qmoe_forward_static): a file-scope device array of
// kStaticScratchBytes in qmoe_kernels.hip. static_scratch() returns its
// address on the current device (looked up once per device, then cached).
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
hipError_t static_scratch(void **ptr);

// Atomic experts: Cartesian top-k over logits [T][Nr + Nc] (each token's row
// logits, then its column logits; k <= 8; Nr, Nc <= 1024), writing idx / w
// [T][k] and the dispatch key idx / B; the expert-centric kernel (the task rows
// of the dispatch, one wavefront each) into O [rows][d] fp32; the token-centric
// ablation straight into y [T][d] bf16 (d = 512 * n, n <= 16).
hipError_t launch_cart_topk(const float *logits, int T, int Nr, int Nc, int k, int B, int32_t *idx, float *w,
                            int32_t *gidx, hipStream_t s);
hipError_t launch_atomic_rows(const uint16_t *x, const uint16_t *W, const uint16_t *V, const int32_t *perm,
                              const int32_t *idx, const float *wrow, int P, int d, int k, float *O, hipStream_t s);
hipError_t launch_atomic_token(const uint16_t *x, const uint16_t *W, const uint16_t *V, const int32_t *idx,
                               const float *w, int T, int d, int k, uint16_t *y, hipStream_t s);

}  // namespace qmoe
