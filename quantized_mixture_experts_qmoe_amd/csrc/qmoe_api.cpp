// C-ABI entry points of the quantized top-k MoE layer (see include/qmoe.h).
//
// qmoe_pack_experts  : expert quantizer (host) + device weight arena + workspace
// qmoe_route_topk    : top-k selection and expert-centric task list from logits
// qmoe_forward       : router -> top-k -> dispatch -> grouped gate/up -> grouped
//                      down -> combine, all HIP kernels on the caller's stream
// qmoe_destroy       : frees the context
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <thread>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "qmoe_internal.h"

using namespace qmoe;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

const char *kKernelNames[QMOE_NUM_KERNELS] = {"router",     "topk",         "dispatch_count", "dispatch_scan",
                                              "dispatch_scatter", "xsum", "gemm_gate_up", "gemm_down",
                                              "combine",    "topk_dispatch"};
enum Slot { K_ROUTER = 0, K_TOPK, K_DCOUNT, K_DSCAN, K_DSCATTER, K_XSUM, K_GEMM13, K_GEMM2, K_COMBINE, K_TOPKD };

struct MatInfo {
    int N = 0, K = 0;
    size_t codes_off = 0, codes_bytes = 0;
    size_t gs_off = 0, gz_off = 0, ps_off = 0, zc_off = 0;   // byte offsets in the arena (0 = absent)
    size_t gs_count = 0, ps_count = 0;
};

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

// Device buffers one forward works in, carved out of a single region: the
// context's own allocation (sized for max_tokens at pack time) or, for
// qmoe_forward_static, the library's static per-device scratch array.
struct QmoeWorkspace {
    float *logits = nullptr, *wpair = nullptr, *wrow = nullptr;
    int32_t *idx = nullptr, *chunk_counts = nullptr, *chunk_base = nullptr, *counts = nullptr, *offsets = nullptr;
    int32_t *perm = nullptr, *inv = nullptr, *num_tiles = nullptr;
    Tile *tiles = nullptr;
    uint16_t *H = nullptr;
    float *xsum = nullptr, *xsum_asym = nullptr, *hsum = nullptr;
    // expert outputs: fp32 (decode tiles) or 16-bit codes in the same memory
    // (prefill tiles) with their exponents, one per 16 columns
    float *O = nullptr;
    int8_t *Oe = nullptr;
};

struct qmoe_ctx {
    qmoe_config cfg{};
    int df = 0;                     // device format of every expert (uniform layers)
    std::vector<int> wfmt;          // per expert: qmoe_wformat
    bool mixed = false;             // experts in more than one device format
    bool any_group = false, any_8bit = false, any_fp8 = false;
    int fmt_mask = 0;               // bit f: some expert uses device format f
    int32_t *eslot = nullptr;       // per expert: group << 20 | index (mixed layers)
    int E = 0, S = 0, F = 0, Fs = 0, d = 0, k = 0;
    int maxT = 0;
    // weights
    uint8_t *arena = nullptr;
    size_t arena_bytes = 0;
    std::vector<MatInfo> m13, m2;   // per expert (E + S)
    ExpertW ex0[kMaxExpertGroups] = {};        // first expert of each group (see GemmArgs)
    int64_t ex_stride[kMaxExpertGroups] = {};  // byte stride between consecutive experts of a group
    int32_t gfmt[kMaxExpertGroups] = {};       // device format of each group
    void *router_w = nullptr;       // bf16 [E][d] or fp32 [E][d] (quantized router: the codes' values as bf16)
    float *router_b = nullptr;
    float *router_s = nullptr;      // quantized router: per-expert scale [E]
    bool router_bf16 = true;        // the bf16 MFMA router runs (bf16 weights or quantized codes)
    // workspace for max_tokens
    QmoeWorkspace ws;
    int ldh = 0;
    std::vector<void *> allocs;
    // profiling
    uint32_t prof = 0;   // bit i: time kernel slot i
    struct Rec {
        int slot;
        hipEvent_t a, b;
    };
    std::vector<Rec> recs;
    std::vector<hipEvent_t> pool;
    double tot_ms[QMOE_NUM_KERNELS] = {};
    int64_t launches[QMOE_NUM_KERNELS] = {};
    bool debug_sync = false;
    int gemm_bm = 64;   // rows per M-tile of the prefill GEMMs
};

namespace {

int dalloc(qmoe_ctx *c, void **p, size_t bytes) {
    if (bytes == 0) bytes = 256;
    if (getenv("QMOE_TEST_FAIL_ALLOC")) return fail(QMOE_ENOMEM, "allocation failure injected (QMOE_TEST_FAIL_ALLOC)");
    hipError_t e = hipMalloc(p, bytes);
    if (e != hipSuccess) {
        *p = nullptr;
        return fail(QMOE_ENOMEM, "hipMalloc(%zu) failed: %s", bytes, hipGetErrorString(e));
    }
    c->allocs.push_back(*p);
    return QMOE_OK;
}

// Device formats as a dense index 0..3 (format masks, expert groups).
int fmt_index(int df) { return df == DF_FP8 ? 3 : df; }
int fmt_of_index(int fi) { return fi == 3 ? DF_FP8 : fi; }

int validate(const qmoe_config *cfg) {
    if (!cfg) return fail(QMOE_EINVAL, "cfg is NULL");
    if (cfg->d_model <= 0 || cfg->d_ff <= 0 || cfg->n_experts <= 0 || cfg->max_tokens <= 0)
        return fail(QMOE_EINVAL, "d_model, d_ff, n_experts and max_tokens must be positive");
    if (cfg->top_k < 1 || cfg->top_k > cfg->n_experts)
        return fail(QMOE_EINVAL, "top_k=%d must be in [1, n_experts=%d]", cfg->top_k, cfg->n_experts);
    if (cfg->n_shared < 0) return fail(QMOE_EINVAL, "n_shared must be >= 0");
    if (cfg->n_shared > 0 && cfg->d_ff_shared <= 0) return fail(QMOE_EINVAL, "d_ff_shared must be positive");
    if (dev_format(cfg->wformat) < 0) return fail(QMOE_EINVAL, "unknown wformat %d", cfg->wformat);
    if (cfg->expert_wformat && cfg->n_experts > 0 && cfg->n_shared >= 0) {
        for (int i = 0; i < cfg->n_experts + cfg->n_shared; i++)
            if (dev_format(cfg->expert_wformat[i]) < 0)
                return fail(QMOE_EINVAL, "unknown wformat %d for expert %d", cfg->expert_wformat[i], i);
    }
    if (cfg->d_model % 256 != 0) return fail(QMOE_EUNSUPPORTED, "d_model=%d is not a multiple of 256", cfg->d_model);
    if (cfg->d_ff % 128 != 0) return fail(QMOE_EUNSUPPORTED, "d_ff=%d is not a multiple of 128", cfg->d_ff);
    if (cfg->n_shared > 0 && cfg->d_ff_shared % 128 != 0)
        return fail(QMOE_EUNSUPPORTED, "d_ff_shared=%d is not a multiple of 128", cfg->d_ff_shared);
    bool group = is_group_wformat(cfg->wformat);
    if (cfg->expert_wformat && cfg->n_experts > 0 && cfg->n_shared >= 0)
        for (int i = 0; i < cfg->n_experts + cfg->n_shared; i++) group = group || is_group_wformat(cfg->expert_wformat[i]);
    if (group && cfg->group_size != 128)
        return fail(QMOE_EUNSUPPORTED, "group_size=%d: only 128 is supported", cfg->group_size);
    if (cfg->n_experts > 1024) return fail(QMOE_EUNSUPPORTED, "n_experts=%d exceeds 1024", cfg->n_experts);
    if (cfg->top_k > 64) return fail(QMOE_EUNSUPPORTED, "top_k=%d exceeds 64", cfg->top_k);
    // launch grids index token tiles and M-tiles in their y dimension (< 65536)
    const long long rows = (long long)cfg->max_tokens * (cfg->top_k + cfg->n_shared);
    if (cfg->max_tokens > (1 << 20) || rows > (1ll << 21))
        return fail(QMOE_EUNSUPPORTED, "max_tokens=%d too large (max_tokens <= 2^20 and max_tokens * (top_k + "
                                       "n_shared) <= 2^21)", cfg->max_tokens);
    // the prefill GEMM addresses gathered x rows as 32-bit byte offsets from x
    if ((long long)cfg->max_tokens * cfg->d_model >= (1ll << 31))
        return fail(QMOE_EUNSUPPORTED, "max_tokens * d_model = %lld: must stay below 2^31",
                    (long long)cfg->max_tokens * cfg->d_model);
    if (cfg->renormalize != 0 && cfg->renormalize != 1) return fail(QMOE_EINVAL, "renormalize must be 0 or 1");
    if (cfg->router_fp32 != 0 && cfg->router_fp32 != 1) return fail(QMOE_EINVAL, "router_fp32 must be 0 or 1");
    if (cfg->router_quant < QMOE_RQ_NONE || cfg->router_quant > QMOE_RQ_FP8E4M3_CH)
        return fail(QMOE_EINVAL, "unknown router_quant %d", cfg->router_quant);
    return QMOE_OK;
}

// Quantize + lay out one expert (all three matrices).
struct ExpertPack {
    PackedMatrix w13, w2;
    int rc = QMOE_OK;
};

void pack_one(int wformat, int F, int d, const float *wg, const float *wu, const float *wd, ExpertPack &out) {
    CanonMatrix g, u, dn, w13;
    int rc = quantize_matrix(wformat, F, d, wg, g);
    if (rc == QMOE_OK) rc = quantize_matrix(wformat, F, d, wu, u);
    if (rc == QMOE_OK) rc = quantize_matrix(wformat, d, F, wd, dn);
    if (rc != QMOE_OK) {
        out.rc = rc;
        return;
    }
    interleave_gate_up(g, u, w13, is_group_wformat(wformat));
    layout_matrix(wformat, w13, out.w13);
    layout_matrix(wformat, dn, out.w2);
}

PackSizes sizes_of(const PackedMatrix &p) {
    PackSizes z;
    z.codes = p.codes.size();
    z.gscale = p.gscale.size();
    z.gzero = p.gzero.size();
    z.pscale = p.pscale.size();
    z.zc = p.zc.size();
    return z;
}

MatInfo plan_matrix(const PackSizes &p, int N, int K, size_t &cursor) {
    MatInfo m;
    m.N = N;
    m.K = K;
    m.codes_off = cursor;
    m.codes_bytes = p.codes;
    cursor = align256(cursor + m.codes_bytes);
    if (p.gscale) {
        m.gs_off = cursor;
        m.gs_count = p.gscale;
        cursor = align256(cursor + p.gscale * 2);
    }
    if (p.gzero) {
        m.gz_off = cursor;
        cursor = align256(cursor + p.gzero * 2);
    }
    if (p.pscale) {
        m.ps_off = cursor;
        m.ps_count = p.pscale;
        cursor = align256(cursor + p.pscale * 4);
    }
    if (p.zc) {
        m.zc_off = cursor;
        cursor = align256(cursor + p.zc * 2);
    }
    return m;
}

int upload_matrix(qmoe_ctx *c, const MatInfo &m, const PackedMatrix &p) {
    hipError_t e = hipMemcpy(c->arena + m.codes_off, p.codes.data(), p.codes.size(), hipMemcpyHostToDevice);
    if (e == hipSuccess && m.gs_off)
        e = hipMemcpy(c->arena + m.gs_off, p.gscale.data(), p.gscale.size() * 2, hipMemcpyHostToDevice);
    if (e == hipSuccess && m.gz_off)
        e = hipMemcpy(c->arena + m.gz_off, p.gzero.data(), p.gzero.size() * 2, hipMemcpyHostToDevice);
    if (e == hipSuccess && m.ps_off)
        e = hipMemcpy(c->arena + m.ps_off, p.pscale.data(), p.pscale.size() * 4, hipMemcpyHostToDevice);
    if (e == hipSuccess && m.zc_off)
        e = hipMemcpy(c->arena + m.zc_off, p.zc.data(), p.zc.size() * 2, hipMemcpyHostToDevice);
    if (e != hipSuccess) return fail(QMOE_EHIP, "hipMemcpy of packed weights failed: %s", hipGetErrorString(e));
    return QMOE_OK;
}

void free_ctx(qmoe_ctx *c) {
    if (!c) return;
    for (void *p : c->allocs) (void)hipFree(p);
    for (auto &r : c->recs) {
        (void)hipEventDestroy(r.a);
        (void)hipEventDestroy(r.b);
    }
    for (auto ev : c->pool) (void)hipEventDestroy(ev);
    delete c;
}

hipEvent_t take_event(qmoe_ctx *c) {
    if (!c->pool.empty()) {
        hipEvent_t e = c->pool.back();
        c->pool.pop_back();
        return e;
    }
    // timing-only events: no system-scope fence (no cache writeback or
    // invalidation between the timed kernels)
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    return e;
}

// Runs `launch` (returning hipError_t) with optional event timing around it.
// prof: the kernel slots to time on this call (c->prof, or 0 where the call
// may create no events).
template <typename Fn>
int timed(qmoe_ctx *c, uint32_t prof, int slot, hipStream_t s, Fn launch) {
    hipEvent_t a = nullptr, b = nullptr;
    const bool on = (prof >> slot) & 1u;
    if (on) {
        a = take_event(c);
        b = take_event(c);
        if (a && b) {
            (void)hipEventRecord(a, s);
        } else {   // creation failed: this launch goes untimed
            if (a) c->pool.push_back(a);
            if (b) c->pool.push_back(b);
            a = b = nullptr;
        }
    }
    hipError_t e = launch();
    if (e != hipSuccess) {
        if (a) c->pool.push_back(a);
        if (b) c->pool.push_back(b);
        return fail(QMOE_EHIP, "launch of %s failed: %s", kKernelNames[slot], hipGetErrorString(e));
    }
    if (a && b) {
        (void)hipEventRecord(b, s);
        c->recs.push_back({slot, a, b});
    }
    if (c->debug_sync) {
        e = hipStreamSynchronize(s);
        if (e == hipSuccess) e = hipGetLastError();
        if (e != hipSuccess) return fail(QMOE_EHIP, "%s failed: %s", kKernelNames[slot], hipGetErrorString(e));
    }
    return QMOE_OK;
}

int rows_per_tile(const qmoe_ctx *c, int T) {
    const long P = (long)T * c->k;
    const long active = std::min<long>(c->E, P);
    const double avg = (double)P / (double)std::max<long>(1, active);
    if (avg <= 16.0) return 16;
    if (c->any_fp8) return 64;   // the e4m3 prefill GEMM takes 64-row tiles (96 would spill)
    // 96-row tiles convert each packed code for 1.5x more MFMA work, which pays
    // once an expert's rows fill a few tiles (160 rows: two 96-row tiles
    // against three of 64); below that their ragged tails cost more than the
    // conversions save
    if (avg >= 160.0) return 96;
    return c->gemm_bm;
}

int max_tiles_for(const qmoe_ctx *c, int T, int bm) {
    const long P = (long)T * c->k;
    return (int)((P + bm - 1) / bm + std::min<long>(c->E, P) + (long)c->S * ((T + bm - 1) / bm));
}

// Carves the workspace of a forward over up to T tokens out of `base` (NULL:
// only measures) and returns its size in bytes. Every buffer starts on a
// 256-byte boundary. Nothing in it needs clearing: each forward writes every
// entry it later reads.
size_t carve_workspace(const qmoe_ctx *c, size_t T, uint8_t *base, QmoeWorkspace &w) {
    const size_t P = T * c->k;
    // dispatch chunks: kDispatchChunk tasks, or one router token tile
    const size_t nchunks = std::max((P + kDispatchChunk - 1) / kDispatchChunk,
                                    (T + kMinRouterTile - 1) / kMinRouterTile);
    const size_t rows_total = P + (size_t)c->S * T;
    // 16-row tiles give the most tiles of any tile height
    const size_t tiles_cap = (size_t)max_tiles_for(c, (int)T, 16) + 16;
    const bool both_sums = ((c->fmt_mask >> fmt_index(DF_I4SYM)) & 1) && ((c->fmt_mask >> fmt_index(DF_I4ASYM)) & 1);
    size_t cur = 0;
    auto take = [&](auto *&ptr, size_t bytes) {
        ptr = base ? reinterpret_cast<std::remove_reference_t<decltype(ptr)>>(base + cur) : nullptr;
        cur = align256(cur + std::max<size_t>(bytes, 4));
    };
    take(w.logits, T * c->E * 4);
    take(w.wpair, P * 4);
    take(w.wrow, P * 4);
    take(w.idx, P * 4);
    take(w.chunk_counts, nchunks * c->E * 4);
    take(w.chunk_base, nchunks * c->E * 4);
    take(w.counts, (size_t)c->E * 4);
    take(w.offsets, (size_t)(c->E + 1) * 4);
    take(w.perm, P * 4);
    take(w.inv, P * 4);
    take(w.num_tiles, 4);
    take(w.tiles, tiles_cap * sizeof(Tile));
    take(w.H, rows_total * c->ldh * 2);
    take(w.O, rows_total * c->d * 4);
    take(w.Oe, rows_total * (c->d / 16));
    take(w.xsum, T * (c->d / 128) * 4);
    // layers mixing INT4_SYM / INT3 (row sums scaled by -136) with INT4_ASYM (-128)
    if (both_sums) take(w.xsum_asym, T * (c->d / 128) * 4);
    else w.xsum_asym = nullptr;
    take(w.hsum, rows_total * (c->ldh / 128) * 4);
    return cur;
}

// Top-k + dispatch shared by route_topk and forward. fused_chunk > 0: the
// router's epilogue already selected the top k and wrote the per-expert counts
// of chunks of fused_chunk tasks; only the scan and the scatter remain.
int run_route(qmoe_ctx *c, const QmoeWorkspace &w, uint32_t prof, const float *logits, int T, int bm, int n_shared,
              int fused_chunk, hipStream_t s) {
    const int P = T * c->k;
    if (!fused_chunk && T <= kSmallRouteMaxT && c->E <= kSmallRouteMaxE)
        return timed(c, prof, K_TOPKD, s, [&] {
            return launch_route_small(logits, T, c->E, c->k, c->cfg.renormalize, n_shared, bm, w.idx, w.wpair,
                                      w.counts, w.offsets, w.tiles, w.num_tiles, w.perm, w.inv, w.wrow, s);
        });
    int rc = QMOE_OK;
    const int chunk = fused_chunk ? fused_chunk : kDispatchChunk;
    const int nchunks = (P + chunk - 1) / chunk;
    if (!fused_chunk) {
        rc = timed(c, prof, K_TOPK, s,
                   [&] { return launch_topk(logits, T, c->E, c->k, c->cfg.renormalize, w.idx, w.wpair, s); });
        if (rc) return rc;
        rc = timed(c, prof, K_DCOUNT, s, [&] { return launch_dispatch_count(w.idx, P, c->E, w.chunk_counts, s); });
        if (rc) return rc;
    }
    rc = timed(c, prof, K_DSCAN, s, [&] {
        return launch_dispatch_scan(w.chunk_counts, nchunks, c->E, P, T, n_shared, bm, w.chunk_base, w.counts,
                                    w.offsets, w.tiles, w.num_tiles, s);
    });
    if (rc) return rc;
    return timed(c, prof, K_DSCATTER, s, [&] {
        return launch_dispatch_scatter(w.idx, w.wpair, P, c->E, chunk, w.chunk_base, w.perm, w.inv, w.wrow, s);
    });
}

int copy_out(void *dst, const void *src, size_t bytes, hipStream_t s) {
    if (!dst || bytes == 0) return QMOE_OK;
    hipError_t e = hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return fail(QMOE_EHIP, "hipMemcpyAsync failed: %s", hipGetErrorString(e));
    return QMOE_OK;
}

int copy_route(const qmoe_ctx *c, const QmoeWorkspace &w, const qmoe_route_out *o, int T, hipStream_t s) {
    if (!o) return QMOE_OK;
    const size_t P = (size_t)T * c->k;
    int rc = copy_out(o->topk_idx, w.idx, P * 4, s);
    if (!rc) rc = copy_out(o->topk_w, w.wpair, P * 4, s);
    if (!rc) rc = copy_out(o->counts, w.counts, (size_t)c->E * 4, s);
    if (!rc) rc = copy_out(o->offsets, w.offsets, (size_t)(c->E + 1) * 4, s);
    if (!rc) rc = copy_out(o->perm, w.perm, P * 4, s);
    return rc;
}

}  // namespace

namespace {

// Where the expert weights come from: host fp32 arrays (host quantizer) or
// device bf16 arrays (device quantizer).
struct WeightSource {
    const float *const *hg = nullptr, *const *hu = nullptr, *const *hd = nullptr;
    const uint16_t *const *dg = nullptr, *const *du = nullptr, *const *dd = nullptr;
    hipStream_t stream = nullptr;
    bool device() const { return dg != nullptr; }
};

int pack_layer(const qmoe_config *cfg, const WeightSource &src, const void *w_router, const float *router_bias,
               qmoe_ctx **out) {
    g_last_error.clear();
    if (!out) return fail(QMOE_EINVAL, "out is NULL");
    *out = nullptr;
    int rc = validate(cfg);
    if (rc) return rc;
    const bool dev = src.device();
    if ((dev ? (!src.dg || !src.du || !src.dd) : (!src.hg || !src.hu || !src.hd)) || !w_router)
        return fail(QMOE_EINVAL, "weight array pointer is NULL");
    const int nexp = cfg->n_experts + cfg->n_shared;
    for (int i = 0; i < nexp; i++) {
        const void *g = dev ? (const void *)src.dg[i] : (const void *)src.hg[i];
        const void *u = dev ? (const void *)src.du[i] : (const void *)src.hu[i];
        const void *d = dev ? (const void *)src.dd[i] : (const void *)src.hd[i];
        if (!g || !u || !d) return fail(QMOE_EINVAL, "weights of expert %d are NULL", i);
        if (dev && (((uintptr_t)g | (uintptr_t)u | (uintptr_t)d) & 15))
            return fail(QMOE_EINVAL, "device weights of expert %d are not 16-byte aligned", i);
    }

    int ndev = 0;
    hipError_t he = hipGetDeviceCount(&ndev);
    if (he != hipSuccess || ndev == 0) return fail(QMOE_EHIP, "no HIP device available");
    if (cfg->device < 0 || cfg->device >= ndev) return fail(QMOE_EINVAL, "device %d out of range", cfg->device);
    he = hipSetDevice(cfg->device);
    if (he != hipSuccess) return fail(QMOE_EHIP, "hipSetDevice: %s", hipGetErrorString(he));

    qmoe_ctx *c = new qmoe_ctx();
    c->cfg = *cfg;
    c->df = dev_format(cfg->wformat);
    c->E = cfg->n_experts;
    c->S = cfg->n_shared;
    c->F = cfg->d_ff;
    c->Fs = cfg->n_shared > 0 ? cfg->d_ff_shared : 0;
    c->d = cfg->d_model;
    c->k = cfg->top_k;
    c->maxT = cfg->max_tokens;
    c->debug_sync = getenv("QMOE_DEBUG") != nullptr;

    // Per-expert formats: device format groups, one kernel launch per format.
    c->wfmt.resize(nexp);
    for (int i = 0; i < nexp; i++) {
        c->wfmt[i] = cfg->expert_wformat ? cfg->expert_wformat[i] : cfg->wformat;
        c->fmt_mask |= 1 << fmt_index(dev_format(c->wfmt[i]));
        c->any_group = c->any_group || is_group_wformat(c->wfmt[i]);
        c->any_8bit = c->any_8bit || !is_group_wformat(c->wfmt[i]);
        c->any_fp8 = c->any_fp8 || c->wfmt[i] == QMOE_W_FP8E4M3_CH;
    }
    c->mixed = (c->fmt_mask & (c->fmt_mask - 1)) != 0;
    c->df = dev_format(c->wfmt[0]);   // the format of every expert when not mixed

    // Arena order: groups of one kind (routed, shared) and one device format,
    // experts ascending inside a group, so every group is uniformly strided.
    auto group_of = [&](int i) {
        return c->mixed ? (i >= c->E ? 4 : 0) + fmt_index(dev_format(c->wfmt[i])) : (i >= c->E ? 1 : 0);
    };
    std::vector<int> order(nexp);
    for (int i = 0; i < nexp; i++) order[i] = i;
    std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return group_of(x) < group_of(y); });
    c->m13.resize(nexp);
    c->m2.resize(nexp);
    size_t cursor = 0;
    if (!dev) {
        // Quantize and lay out every expert on the host, several experts at a time.
        std::vector<ExpertPack> packs(nexp);
        {
            const int nthreads = std::max(1, std::min<int>(nexp, (int)std::thread::hardware_concurrency()));
            std::vector<std::thread> pool;
            for (int tid = 0; tid < nthreads; tid++)
                pool.emplace_back([&, tid] {
                    for (int i = tid; i < nexp; i += nthreads) {
                        const int f = i < c->E ? c->F : c->Fs;
                        pack_one(c->wfmt[i], f, c->d, src.hg[i], src.hu[i], src.hd[i], packs[i]);
                    }
                });
            for (auto &t : pool) t.join();
        }
        for (int i = 0; i < nexp; i++)
            if (packs[i].rc) {
                free_ctx(c);
                return fail(packs[i].rc, "quantization of expert %d failed", i);
            }
        for (int i : order) {
            const int f = i < c->E ? c->F : c->Fs;
            c->m13[i] = plan_matrix(sizes_of(packs[i].w13), 2 * f, c->d, cursor);
            c->m2[i] = plan_matrix(sizes_of(packs[i].w2), c->d, f, cursor);
        }
        c->arena_bytes = cursor;
        rc = dalloc(c, (void **)&c->arena, c->arena_bytes);
        for (int i = 0; !rc && i < nexp; i++) {
            rc = upload_matrix(c, c->m13[i], packs[i].w13);
            if (!rc) rc = upload_matrix(c, c->m2[i], packs[i].w2);
            packs[i] = ExpertPack();   // release host copies as we go
        }
    } else {
        // Quantize and lay out every expert on the device, straight into the
        // arena (zeroed first: the zero-point operand has padding entries).
        for (int i : order) {
            const int f = i < c->E ? c->F : c->Fs;
            c->m13[i] = plan_matrix(pack_sizes(c->wfmt[i], 2 * f, c->d), 2 * f, c->d, cursor);
            c->m2[i] = plan_matrix(pack_sizes(c->wfmt[i], c->d, f), c->d, f, cursor);
        }
        c->arena_bytes = cursor;
        rc = dalloc(c, (void **)&c->arena, c->arena_bytes);
        uint8_t *zero_row = nullptr;
        const size_t zr_bytes = (size_t)std::max(2 * std::max(c->F, c->Fs), c->d);
        if (!rc) rc = dalloc(c, (void **)&zero_row, zr_bytes);
        if (!rc && hipMemsetAsync(c->arena, 0, c->arena_bytes, src.stream) != hipSuccess)
            rc = fail(QMOE_EHIP, "clearing the weight arena failed");
        auto quant = [&](int wf, const MatInfo &m, const uint16_t *a, const uint16_t *b) {
            hipError_t e = launch_quant_matrix(
                wf, a, b, m.N, m.K, c->arena + m.codes_off, m.gs_off ? (uint16_t *)(c->arena + m.gs_off) : nullptr,
                m.gz_off ? (uint16_t *)(c->arena + m.gz_off) : nullptr,
                m.ps_off ? (float *)(c->arena + m.ps_off) : nullptr,
                m.zc_off ? (uint16_t *)(c->arena + m.zc_off) : nullptr, zero_row, src.stream);
            return e == hipSuccess ? QMOE_OK : fail(QMOE_EHIP, "quantization kernel launch failed: %s", hipGetErrorString(e));
        };
        for (int i = 0; !rc && i < nexp; i++) {
            rc = quant(c->wfmt[i], c->m13[i], src.dg[i], src.du[i]);
            if (!rc) rc = quant(c->wfmt[i], c->m2[i], src.dd[i], nullptr);
            // the row-flag scratch is reused by the next matrix: keep the stream ordered
        }
        if (!rc) {
            const hipError_t e = hipStreamSynchronize(src.stream);
            if (e != hipSuccess) rc = fail(QMOE_EHIP, "device quantization failed: %s", hipGetErrorString(e));
        }
    }
    if (rc) {
        free_ctx(c);
        return rc;
    }
    std::vector<ExpertW> hexp(nexp);
    for (int i = 0; i < nexp; i++) {
        ExpertW &w = hexp[i];
        const MatInfo &a = c->m13[i], &b = c->m2[i];
        w.c13 = c->arena + a.codes_off;
        w.s13 = a.gs_off ? (const uint16_t *)(c->arena + a.gs_off) : nullptr;
        w.z13 = a.gz_off ? (const uint16_t *)(c->arena + a.gz_off) : nullptr;
        w.p13 = a.ps_off ? (const float *)(c->arena + a.ps_off) : nullptr;
        w.zc13 = a.zc_off ? (const uint16_t *)(c->arena + a.zc_off) : nullptr;
        w.c2 = c->arena + b.codes_off;
        w.s2 = b.gs_off ? (const uint16_t *)(c->arena + b.gs_off) : nullptr;
        w.z2 = b.gz_off ? (const uint16_t *)(c->arena + b.gz_off) : nullptr;
        w.p2 = b.ps_off ? (const float *)(c->arena + b.ps_off) : nullptr;
        w.zc2 = b.zc_off ? (const uint16_t *)(c->arena + b.zc_off) : nullptr;
        w.F = i < c->E ? c->F : c->Fs;
    }
    // each group's first expert and uniform stride; the slot table of mixed layers
    std::vector<int32_t> slot(nexp, 0);
    for (int grp = 0; grp < kMaxExpertGroups && !rc; grp++) {
        std::vector<int> mem;
        for (int i : order)
            if (group_of(i) == grp) mem.push_back(i);
        if (mem.empty()) continue;
        const int first = mem[0], count = (int)mem.size();
        c->ex0[grp] = hexp[first];
        c->gfmt[grp] = dev_format(c->wfmt[first]);
        c->ex_stride[grp] = count > 1 ? (int64_t)(c->m13[mem[1]].codes_off - c->m13[first].codes_off) : 0;
        for (int j = 0; j < count; j++) slot[mem[j]] = (grp << 20) | j;
        for (int j = 1; j < count && !rc; j++) {
            const int64_t off = c->ex_stride[grp] * j;
            const MatInfo &a0 = c->m13[first], &b0 = c->m2[first], &a = c->m13[mem[j]], &b = c->m2[mem[j]];
            const size_t z0[10] = {a0.codes_off, a0.gs_off, a0.gz_off, a0.ps_off, a0.zc_off,
                                   b0.codes_off, b0.gs_off, b0.gz_off, b0.ps_off, b0.zc_off};
            const size_t zi[10] = {a.codes_off, a.gs_off, a.gz_off, a.ps_off, a.zc_off,
                                   b.codes_off, b.gs_off, b.gz_off, b.ps_off, b.zc_off};
            // fields 0 and 5 (codes) are always present (offset 0 is valid there);
            // for the others offset 0 means "absent"
            for (int f = 0; f < 10; f++)
                if ((f % 5 && (z0[f] == 0) != (zi[f] == 0)) || ((f % 5 == 0 || z0[f]) && (int64_t)(zi[f] - z0[f]) != off))
                    rc = fail(QMOE_EHIP, "internal: expert %d is not uniformly strided in the arena", mem[j]);
        }
    }
    if (!rc && c->mixed) {
        rc = dalloc(c, (void **)&c->eslot, sizeof(int32_t) * nexp);
        if (!rc && hipMemcpy(c->eslot, slot.data(), sizeof(int32_t) * nexp, hipMemcpyHostToDevice) != hipSuccess)
            rc = fail(QMOE_EHIP, "upload of the expert slot table failed");
    }

    // Router weight (as given, or quantized per expert row) and bias.
    c->router_bf16 = !cfg->router_fp32 || cfg->router_quant != QMOE_RQ_NONE;
    if (!rc && cfg->router_quant != QMOE_RQ_NONE) {
        const size_t n = (size_t)c->E * c->d;
        std::vector<float> wf(n);
        for (size_t i = 0; i < n; i++) {
            if (cfg->router_fp32) {
                wf[i] = ((const float *)w_router)[i];
            } else {
                const uint32_t u = (uint32_t)((const uint16_t *)w_router)[i] << 16;
                memcpy(&wf[i], &u, 4);
            }
        }
        std::vector<uint16_t> codes;
        std::vector<float> rs;
        rc = quantize_router(cfg->router_quant, c->E, c->d, wf.data(), codes, rs);
        if (rc) rc = fail(rc, "router quantization failed");
        if (!rc) rc = dalloc(c, &c->router_w, n * 2);
        if (!rc && hipMemcpy(c->router_w, codes.data(), n * 2, hipMemcpyHostToDevice) != hipSuccess)
            rc = fail(QMOE_EHIP, "upload of router weight failed");
        if (!rc) rc = dalloc(c, (void **)&c->router_s, sizeof(float) * c->E);
        if (!rc && hipMemcpy(c->router_s, rs.data(), sizeof(float) * c->E, hipMemcpyHostToDevice) != hipSuccess)
            rc = fail(QMOE_EHIP, "upload of router scales failed");
    } else if (!rc) {
        const size_t wr_bytes = (size_t)c->E * c->d * (cfg->router_fp32 ? 4 : 2);
        rc = dalloc(c, &c->router_w, wr_bytes);
        if (!rc && hipMemcpy(c->router_w, w_router, wr_bytes, hipMemcpyHostToDevice) != hipSuccess)
            rc = fail(QMOE_EHIP, "upload of router weight failed");
    }
    if (!rc && router_bias) {
        rc = dalloc(c, (void **)&c->router_b, sizeof(float) * c->E);
        if (!rc && hipMemcpy(c->router_b, router_bias, sizeof(float) * c->E, hipMemcpyHostToDevice) != hipSuccess)
            rc = fail(QMOE_EHIP, "upload of router bias failed");
    }

    // Workspace sized for max_tokens: one allocation, carved.
    c->ldh = std::max(c->F, c->Fs);
    if (!rc) {
        uint8_t *wsb = nullptr;
        rc = dalloc(c, (void **)&wsb, carve_workspace(c, (size_t)c->maxT, nullptr, c->ws));
        if (!rc) carve_workspace(c, (size_t)c->maxT, wsb, c->ws);
    }
    if (rc) {
        free_ctx(c);
        return rc;
    }
    *out = c;
    return QMOE_OK;
}

}  // namespace

extern "C" {

const char *qmoe_last_error(void) { return g_last_error.c_str(); }

const char *qmoe_kernel_name(int32_t slot) {
    return (slot >= 0 && slot < QMOE_NUM_KERNELS) ? kKernelNames[slot] : "";
}

int qmoe_pack_experts(const qmoe_config *cfg, const float *const *w_gate, const float *const *w_up,
                      const float *const *w_down, const void *w_router, const float *router_bias, qmoe_ctx **out) {
    WeightSource src;
    src.hg = w_gate;
    src.hu = w_up;
    src.hd = w_down;
    if (!w_gate || !w_up || !w_down) return fail(QMOE_EINVAL, "weight array pointer is NULL");
    return pack_layer(cfg, src, w_router, router_bias, out);
}

int qmoe_pack_experts_device(const qmoe_config *cfg, const uint16_t *const *w_gate, const uint16_t *const *w_up,
                             const uint16_t *const *w_down, const void *w_router, const float *router_bias,
                             void *stream, qmoe_ctx **out) {
    if (!w_gate || !w_up || !w_down) return fail(QMOE_EINVAL, "weight array pointer is NULL");
    WeightSource src;
    src.dg = w_gate;
    src.du = w_up;
    src.dd = w_down;
    src.stream = (hipStream_t)stream;
    return pack_layer(cfg, src, w_router, router_bias, out);
}

void qmoe_destroy(qmoe_ctx *ctx) {
    if (!ctx) return;
    (void)hipSetDevice(ctx->cfg.device);
    free_ctx(ctx);
}

int qmoe_route_topk(qmoe_ctx *c, const float *logits, int32_t T, qmoe_route_out *out, void *stream) {
    g_last_error.clear();
    if (!c) return fail(QMOE_EINVAL, "ctx is NULL");
    if (T < 0 || T > c->maxT) return fail(QMOE_EINVAL, "T=%d outside [0, max_tokens=%d]", T, c->maxT);
    if (T == 0) return QMOE_OK;
    if (!logits) return fail(QMOE_EINVAL, "logits is NULL");
    hipStream_t s = (hipStream_t)stream;
    if (hipSetDevice(c->cfg.device) != hipSuccess) return fail(QMOE_EHIP, "hipSetDevice failed");
    int rc = run_route(c, c->ws, c->prof, logits, T, 128, 0, 0, s);
    if (rc) return rc;
    return copy_route(c, c->ws, out, T, s);
}

}  // extern "C"

namespace {

int check_forward_args(const qmoe_ctx *c, const uint16_t *x, int32_t T, const uint16_t *y) {
    if (!c) return fail(QMOE_EINVAL, "ctx is NULL");
    if (T < 0 || T > c->maxT) return fail(QMOE_EINVAL, "T=%d outside [0, max_tokens=%d]", T, c->maxT);
    if (T == 0) return QMOE_OK;
    if (!x || !y) return fail(QMOE_EINVAL, "x or y is NULL");
    if ((const void *)x == (const void *)y) return fail(QMOE_EINVAL, "y may not alias x");
    return QMOE_OK;
}

// The forward's launches (router -> top-k/dispatch -> row sums -> grouped
// gate/up -> grouped down -> combine) on the workspace w.
int run_forward(qmoe_ctx *c, const QmoeWorkspace &w, uint32_t prof, const uint16_t *x, int32_t T, uint16_t *y,
                qmoe_route_out *dbg, hipStream_t s) {
    const int P = T * c->k;
    const int bm = rows_per_tile(c, T);
    const int max_tiles = max_tiles_for(c, T, bm);
    const bool grouped = c->any_group;
    // row-sum scale of the integer-code GEMM: -136 for INT4_SYM / INT3 (stored
    // code q + 8), -128 for INT4_ASYM; a layer with both computes the second
    // set of sums separately
    const bool sym_present = (c->fmt_mask >> fmt_index(DF_I4SYM)) & 1;
    const bool asym_present = (c->fmt_mask >> fmt_index(DF_I4ASYM)) & 1;
    const float zc = sym_present ? -136.0f : -128.0f;
    // Row sums of x: the prefill GEMMs of the group formats read them; the
    // decode kernel (bm == 16) computes its own while staging rows.
    const bool need_sums = grouped && bm > 16;
    // the bf16 router emits the row sums from its staged x tiles
    const bool fused_sums = need_sums && c->router_bf16;
    int rc;
    // the gating network runs in the router's epilogue where one router
    // workgroup holds every expert of its tokens (larger batches; the small
    // ones take the one-workgroup top-k + dispatch)
    int fused_chunk = 0;
    const bool try_fuse = c->router_bf16 && T > kSmallRouteMaxT && router_fuses(T, c->E, c->k);
    RouteFuse rf{w.idx, w.wpair, w.chunk_counts, c->k, c->cfg.renormalize};
    // logits are written only when the caller asks for them (or the top-k runs separately)
    float *lg = (dbg && dbg->logits) || !try_fuse ? w.logits : nullptr;
    if (!c->router_bf16)
        rc = timed(c, prof, K_ROUTER, s, [&] {
            return launch_router_f32(x, (const float *)c->router_w, c->router_b, w.logits, T, c->d, c->E, s);
        });
    else
        rc = timed(c, prof, K_ROUTER, s, [&] {
            return launch_router_bf16(x, (const uint16_t *)c->router_w, c->router_s, c->router_b, lg,
                                      fused_sums ? w.xsum : nullptr, zc, T, c->d, c->E, try_fuse ? &rf : nullptr,
                                      &fused_chunk, s);
        });
    if (rc) return rc;
    if (try_fuse && !fused_chunk) return fail(QMOE_EHIP, "internal: the router's gating epilogue did not run");
    rc = run_route(c, w, prof, w.logits, T, bm, c->S, fused_chunk, s);
    if (rc) return rc;
    if (need_sums && !fused_sums) {
        rc = timed(c, prof, K_XSUM, s, [&] { return launch_xsum(x, T, c->d, zc, w.xsum, s); });
        if (rc) return rc;
    }
    if (need_sums && sym_present && asym_present) {
        rc = timed(c, prof, K_XSUM, s, [&] { return launch_xsum(x, T, c->d, -128.0f, w.xsum_asym, s); });
        if (rc) return rc;
    }

    GemmArgs a{};
    for (int g = 0; g < kMaxExpertGroups; g++) {
        a.ex0[g] = c->ex0[g];
        a.ex_stride[g] = c->ex_stride[g];
        a.gfmt[g] = c->gfmt[g];
    }
    a.eslot = c->eslot;
    a.tiles = w.tiles;
    a.num_tiles = w.num_tiles;
    a.perm = w.perm;
    a.wrow = w.wrow;
    a.x = x;
    a.xsum = w.xsum;
    a.H = w.H;
    a.hsum = w.hsum;
    a.O = reinterpret_cast<int16_t *>(w.O);
    a.Oe = w.Oe;
    a.Of = w.O;
    a.ldh = c->ldh;
    a.d = c->d;
    a.k = c->k;
    a.P = P;
    a.T = T;
    a.E = c->E;
    const int maxN13 = 2 * std::max(c->F, c->Fs);
    // one gate/up launch per device format present, then one down launch per
    // format (each computes only its own experts' tiles)
    // (decode tiles of a mixed layer: one launch, each workgroup in its expert's format)
    const bool one_launch = !c->mixed || bm == 16;
    for (int fi = 0; fi < 4; fi++) {
        if (!((c->fmt_mask >> fi) & 1)) continue;
        const int df = c->mixed && bm == 16 ? kDfAllFormats : fmt_of_index(fi);
        a.xsum = df == DF_I4ASYM && sym_present ? w.xsum_asym : w.xsum;
        rc = timed(c, prof, K_GEMM13, s, [&] { return launch_gemm13(df, bm, a, max_tiles, maxN13, s); });
        if (rc) return rc;
        if (one_launch) break;
    }
    for (int fi = 0; fi < 4; fi++) {
        if (!((c->fmt_mask >> fi) & 1)) continue;
        const int df = c->mixed && bm == 16 ? kDfAllFormats : fmt_of_index(fi);
        rc = timed(c, prof, K_GEMM2, s, [&] { return launch_gemm2(df, bm, a, max_tiles, s); });
        if (rc) return rc;
        if (one_launch) break;
    }
    rc = timed(c, prof, K_COMBINE, s, [&] {
        return bm == 16 ? launch_combine_f32(w.O, w.inv, T, c->d, c->k, P, c->S, y, s)
                        : launch_combine(a.O, w.Oe, w.inv, T, c->d, c->k, P, c->S, y, s);
    });
    if (rc) return rc;
    if (dbg) {
        rc = copy_out(dbg->logits, w.logits, (size_t)T * c->E * 4, s);
        if (!rc) rc = copy_route(c, w, dbg, T, s);
    }
    return rc;
}

}  // namespace

extern "C" {

int qmoe_forward(qmoe_ctx *c, const uint16_t *x, int32_t T, uint16_t *y, qmoe_route_out *dbg, void *stream) {
    g_last_error.clear();
    int rc = check_forward_args(c, x, T, y);
    if (rc || T == 0) return rc;
    if (hipSetDevice(c->cfg.device) != hipSuccess) return fail(QMOE_EHIP, "hipSetDevice failed");
    return run_forward(c, c->ws, c->prof, x, T, y, dbg, (hipStream_t)stream);
}

int qmoe_forward_static(qmoe_ctx *c, const uint16_t *x, int32_t T, uint16_t *y, qmoe_route_out *dbg, void *stream) {
    g_last_error.clear();
    int rc = check_forward_args(c, x, T, y);
    if (rc || T == 0) return rc;
    if (hipSetDevice(c->cfg.device) != hipSuccess) return fail(QMOE_EHIP, "hipSetDevice failed");
    QmoeWorkspace w;
    const size_t need = carve_workspace(c, (size_t)T, nullptr, w);
    if (need > kStaticScratchBytes)
        return fail(QMOE_EUNSUPPORTED, "T=%d needs %zu bytes of workspace; the static scratch holds %zu", T, need,
                    kStaticScratchBytes);
    void *base = nullptr;
    const hipError_t e = static_scratch(&base);
    if (e != hipSuccess) return fail(QMOE_EHIP, "static scratch address: %s", hipGetErrorString(e));
    carve_workspace(c, (size_t)T, static_cast<uint8_t *>(base), w);
    // no profiling events here: the call creates nothing
    return run_forward(c, w, 0u, x, T, y, dbg, (hipStream_t)stream);
}

int qmoe_export_packed(qmoe_ctx *c, int32_t expert, int32_t matrix, int8_t *codes, float *scales, float *zeros) {
    g_last_error.clear();
    if (!c || !codes || !scales) return fail(QMOE_EINVAL, "NULL argument");
    if (expert < 0 || expert >= c->E + c->S || matrix < 0 || matrix > 2)
        return fail(QMOE_EINVAL, "expert %d / matrix %d out of range", expert, matrix);
    if (hipSetDevice(c->cfg.device) != hipSuccess) return fail(QMOE_EHIP, "hipSetDevice failed");
    const MatInfo &m = matrix == 2 ? c->m2[expert] : c->m13[expert];
    PackedMatrix p;
    p.codes.resize(m.codes_bytes);
    hipError_t e = hipMemcpy(p.codes.data(), c->arena + m.codes_off, m.codes_bytes, hipMemcpyDeviceToHost);
    if (e == hipSuccess && m.gs_off) {
        p.gscale.resize(m.gs_count);
        e = hipMemcpy(p.gscale.data(), c->arena + m.gs_off, m.gs_count * 2, hipMemcpyDeviceToHost);
    }
    if (e == hipSuccess && m.gz_off) {
        p.gzero.resize(m.gs_count);
        e = hipMemcpy(p.gzero.data(), c->arena + m.gz_off, m.gs_count * 2, hipMemcpyDeviceToHost);
    }
    if (e == hipSuccess && m.ps_off) {
        p.pscale.resize(m.ps_count);
        e = hipMemcpy(p.pscale.data(), c->arena + m.ps_off, m.ps_count * 4, hipMemcpyDeviceToHost);
    }
    if (e != hipSuccess) return fail(QMOE_EHIP, "hipMemcpy D2H failed: %s", hipGetErrorString(e));
    CanonMatrix full;
    full.N = m.N;
    full.K = m.K;
    unlayout_matrix(c->wfmt[expert], p, full);
    const int G = is_group_wformat(c->wfmt[expert]) ? m.K / kBlockK : 1;
    // W13 rows alternate gate / up in 16-row blocks; select the requested half.
    const int outN = matrix == 2 ? m.N : m.N / 2;
    for (int r = 0; r < outN; r++) {
        const int src = matrix == 2 ? r : ((r / kBlockRows) * 2 + matrix) * kBlockRows + r % kBlockRows;
        memcpy(codes + (size_t)r * m.K, &full.q[(size_t)src * m.K], (size_t)m.K);
        for (int g = 0; g < G; g++) {
            scales[(size_t)r * G + g] = full.scale[(size_t)src * G + g];
            if (zeros) zeros[(size_t)r * G + g] = full.zero[(size_t)src * G + g];
        }
    }
    return QMOE_OK;
}

int qmoe_profile_enable(qmoe_ctx *c, int32_t slot_mask) {
    if (!c) return fail(QMOE_EINVAL, "ctx is NULL");
    c->prof = (uint32_t)slot_mask & ((1u << QMOE_NUM_KERNELS) - 1u);
    if (c->prof) {
        for (auto &r : c->recs) {
            c->pool.push_back(r.a);
            c->pool.push_back(r.b);
        }
        c->recs.clear();
        for (int i = 0; i < QMOE_NUM_KERNELS; i++) {
            c->tot_ms[i] = 0.0;
            c->launches[i] = 0;
        }
    }
    return QMOE_OK;
}

int qmoe_profile_read(qmoe_ctx *c, double *total_ms, int64_t *launches) {
    if (!c || !total_ms || !launches) return fail(QMOE_EINVAL, "NULL argument");
    size_t done = 0;   // records read so far; their events are back in the pool
    int rc = QMOE_OK;
    for (; done < c->recs.size(); done++) {
        const auto &r = c->recs[done];
        float ms = 0.0f;
        if (hipEventSynchronize(r.b) != hipSuccess) {
            rc = fail(QMOE_EHIP, "hipEventSynchronize failed");
            break;
        }
        if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
            rc = fail(QMOE_EHIP, "hipEventElapsedTime failed");
            break;
        }
        c->tot_ms[r.slot] += ms;
        c->launches[r.slot] += 1;
        c->pool.push_back(r.a);
        c->pool.push_back(r.b);
    }
    c->recs.erase(c->recs.begin(), c->recs.begin() + (std::ptrdiff_t)done);
    if (rc) return rc;
    for (int i = 0; i < QMOE_NUM_KERNELS; i++) {
        total_ms[i] = c->tot_ms[i];
        launches[i] = c->launches[i];
    }
    return QMOE_OK;
}

int qmoe_clock_probe(void *stream, int64_t duration_ticks, int64_t period_ticks, int32_t max_samples,
                     uint64_t *samples, int64_t *wall_khz) {
    if (!samples || !wall_khz || duration_ticks <= 0 || period_ticks <= 0 || max_samples < 1)
        return fail(QMOE_EINVAL, "clock probe: bad arguments");
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
        return fail(QMOE_EHIP, "clock probe: wall clock rate unavailable");
    *wall_khz = khz;
    const hipError_t e = launch_clock_probe(reinterpret_cast<unsigned long long *>(samples),
                                            (unsigned long long)duration_ticks, (unsigned long long)period_ticks,
                                            max_samples, (hipStream_t)stream);
    return e == hipSuccess ? QMOE_OK : fail(QMOE_EHIP, "clock probe launch failed: %s", hipGetErrorString(e));
}

// ---- Atomic experts ---------------------------------------------------------

struct qmoe_atomic_ctx {
    qmoe_atomic_config cfg{};
    int N = 0, B = 1, NG = 1, P = 0, max_tiles = 0;
    uint16_t *W = nullptr, *V = nullptr, *R = nullptr;   // R: router rows, then router columns [Nr + Nc][d]
    float *logits = nullptr, *w = nullptr, *wrow = nullptr, *O = nullptr;   // logits [T][Nr + Nc]
    int32_t *idx = nullptr, *gidx = nullptr, *chunk_counts = nullptr, *chunk_base = nullptr, *counts = nullptr;
    int32_t *offsets = nullptr, *perm = nullptr, *inv = nullptr, *num_tiles = nullptr;
    Tile *tiles = nullptr;
    std::vector<void *> allocs;
};

namespace {

// The dispatch scan also emits a tile list (rows per tile below); the
// expert-centric kernel walks the sorted rows directly and does not read it.
constexpr int kAtomicRows = 64;

void atomic_free(qmoe_atomic_ctx *c) {
    if (!c) return;
    for (void *p : c->allocs) (void)hipFree(p);
    delete c;
}

int atomic_alloc(qmoe_atomic_ctx *c, void **p, size_t bytes) {
    *p = nullptr;
    if (getenv("QMOE_TEST_FAIL_ALLOC")) return fail(QMOE_ENOMEM, "allocation failure injected (QMOE_TEST_FAIL_ALLOC)");
    const hipError_t e = hipMalloc(p, std::max<size_t>(bytes, 4));
    if (e != hipSuccess) {
        *p = nullptr;
        return fail(QMOE_ENOMEM, "hipMalloc(%zu) failed: %s", bytes, hipGetErrorString(e));
    }
    c->allocs.push_back(*p);
    return QMOE_OK;
}

int atomic_validate(const qmoe_atomic_config *cfg) {
    if (!cfg) return fail(QMOE_EINVAL, "cfg is NULL");
    if (cfg->d_model <= 0 || cfg->n_rows <= 0 || cfg->n_cols <= 0 || cfg->max_tokens <= 0)
        return fail(QMOE_EINVAL, "d_model, n_rows, n_cols and max_tokens must be positive");
    const long long N = (long long)cfg->n_rows * cfg->n_cols;
    if (cfg->top_k < 1 || cfg->top_k > N) return fail(QMOE_EINVAL, "top_k=%d must be in [1, N=%lld]", cfg->top_k, N);
    if (cfg->d_model % 512 != 0 || cfg->d_model > 8192)
        return fail(QMOE_EUNSUPPORTED, "d_model=%d: must be a multiple of 512 and at most 8192", cfg->d_model);
    if (cfg->n_rows > 1024 || cfg->n_cols > 1024)
        return fail(QMOE_EUNSUPPORTED, "n_rows=%d, n_cols=%d: at most 1024 each", cfg->n_rows, cfg->n_cols);
    if (cfg->top_k > 8) return fail(QMOE_EUNSUPPORTED, "top_k=%d exceeds 8", cfg->top_k);
    if (cfg->max_tokens > (1 << 20) || (long long)cfg->max_tokens * cfg->top_k > (1ll << 21))
        return fail(QMOE_EUNSUPPORTED, "max_tokens=%d too large (<= 2^20 and max_tokens * top_k <= 2^21)",
                    cfg->max_tokens);
    return QMOE_OK;
}

}  // namespace

int qmoe_atomic_create(const qmoe_atomic_config *cfg, const uint16_t *w_in, const uint16_t *w_out,
                       const uint16_t *router_rows, const uint16_t *router_cols, qmoe_atomic_ctx **out) {
    g_last_error.clear();
    if (!out) return fail(QMOE_EINVAL, "out is NULL");
    *out = nullptr;
    int rc = atomic_validate(cfg);
    if (rc) return rc;
    if (!w_in || !w_out || !router_rows || !router_cols) return fail(QMOE_EINVAL, "weight pointer is NULL");
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev == 0) return fail(QMOE_EHIP, "no HIP device available");
    if (cfg->device < 0 || cfg->device >= ndev) return fail(QMOE_EINVAL, "device %d out of range", cfg->device);
    if (hipSetDevice(cfg->device) != hipSuccess) return fail(QMOE_EHIP, "hipSetDevice failed");
    qmoe_atomic_ctx *c = new qmoe_atomic_ctx();
    c->cfg = *cfg;
    const size_t d = (size_t)cfg->d_model;
    c->N = cfg->n_rows * cfg->n_cols;
    // experts per dispatch group: at most 256 groups, which keeps the one-
    // workgroup scan of the dispatch short (four threads per group)
    c->B = (c->N + 255) / 256;
    c->NG = (c->N + c->B - 1) / c->B;
    c->P = cfg->max_tokens * cfg->top_k;
    c->max_tiles = (c->P + kAtomicRows - 1) / kAtomicRows + std::min(c->NG, c->P);
    auto up = [&](uint16_t *dst, const uint16_t *src, size_t n) {
        return hipMemcpy(dst, src, n * 2, hipMemcpyHostToDevice) == hipSuccess
                   ? QMOE_OK
                   : fail(QMOE_EHIP, "upload of atomic-expert weights failed");
    };
    const size_t nr = (size_t)cfg->n_rows, nc = (size_t)cfg->n_cols;
    rc = atomic_alloc(c, (void **)&c->W, (size_t)c->N * d * 2);
    if (!rc) rc = up(c->W, w_in, (size_t)c->N * d);
    if (!rc) rc = atomic_alloc(c, (void **)&c->V, (size_t)c->N * d * 2);
    if (!rc) rc = up(c->V, w_out, (size_t)c->N * d);
    // one router matrix, so that one pass over x yields both logit sets
    if (!rc) rc = atomic_alloc(c, (void **)&c->R, (nr + nc) * d * 2);
    if (!rc) rc = up(c->R, router_rows, nr * d);
    if (!rc) rc = up(c->R + nr * d, router_cols, nc * d);
    const size_t T = (size_t)cfg->max_tokens, P = (size_t)c->P;
    const size_t nchunks = (P + kDispatchChunk - 1) / kDispatchChunk;
    if (!rc) rc = atomic_alloc(c, (void **)&c->logits, T * (nr + nc) * 4);
    if (!rc) rc = atomic_alloc(c, (void **)&c->idx, P * 4);
    if (!rc) rc = atomic_alloc(c, (void **)&c->gidx, P * 4);
    if (!rc) rc = atomic_alloc(c, (void **)&c->w, P * 4);
    if (!rc) rc = atomic_alloc(c, (void **)&c->wrow, P * 4);
    if (!rc) rc = atomic_alloc(c, (void **)&c->perm, P * 4);
    if (!rc) rc = atomic_alloc(c, (void **)&c->inv, P * 4);
    if (!rc) rc = atomic_alloc(c, (void **)&c->chunk_counts, nchunks * c->NG * 4);
    if (!rc) rc = atomic_alloc(c, (void **)&c->chunk_base, nchunks * c->NG * 4);
    if (!rc) rc = atomic_alloc(c, (void **)&c->counts, (size_t)c->NG * 4);
    if (!rc) rc = atomic_alloc(c, (void **)&c->offsets, ((size_t)c->NG + 1) * 4);
    if (!rc) rc = atomic_alloc(c, (void **)&c->num_tiles, 256);
    if (!rc) rc = atomic_alloc(c, (void **)&c->tiles, ((size_t)c->max_tiles + 16) * sizeof(Tile));
    if (!rc) rc = atomic_alloc(c, (void **)&c->O, P * d * 4);
    if (rc) {
        atomic_free(c);
        return rc;
    }
    *out = c;
    return QMOE_OK;
}

int qmoe_atomic_forward(qmoe_atomic_ctx *c, const uint16_t *x, int32_t T, uint16_t *y, int32_t schedule,
                        qmoe_atomic_route_out *dbg, void *stream) {
    g_last_error.clear();
    if (!c) return fail(QMOE_EINVAL, "ctx is NULL");
    if (T < 0 || T > c->cfg.max_tokens) return fail(QMOE_EINVAL, "T=%d outside [0, max_tokens=%d]", T, c->cfg.max_tokens);
    if (schedule != QMOE_SCHEDULE_EXPERT_CENTRIC && schedule != QMOE_SCHEDULE_TOKEN_CENTRIC)
        return fail(QMOE_EINVAL, "unknown schedule %d", schedule);
    if (T == 0) return QMOE_OK;
    if (!x || !y) return fail(QMOE_EINVAL, "x or y is NULL");
    if ((const void *)x == (const void *)y) return fail(QMOE_EINVAL, "y may not alias x");
    if (hipSetDevice(c->cfg.device) != hipSuccess) return fail(QMOE_EHIP, "hipSetDevice failed");
    hipStream_t s = (hipStream_t)stream;
    const int d = c->cfg.d_model, k = c->cfg.top_k, Nr = c->cfg.n_rows, Nc = c->cfg.n_cols, P = T * k;
    auto ok = [](hipError_t e, const char *what) {
        return e == hipSuccess ? QMOE_OK : fail(QMOE_EHIP, "%s failed: %s", what, hipGetErrorString(e));
    };
    int rc = ok(launch_router_bf16(x, c->R, nullptr, nullptr, c->logits, nullptr, 0.0f, T, d, Nr + Nc, nullptr,
                                   nullptr, s), "router");
    if (!rc) rc = ok(launch_cart_topk(c->logits, T, Nr, Nc, k, c->B, c->idx, c->w, c->gidx, s), "cartesian top-k");
    if (!rc && schedule == QMOE_SCHEDULE_TOKEN_CENTRIC) {
        rc = ok(launch_atomic_token(x, c->W, c->V, c->idx, c->w, T, d, k, y, s), "token-centric experts");
    } else if (!rc) {
        const int nchunks = (P + kDispatchChunk - 1) / kDispatchChunk;
        rc = ok(launch_dispatch_count(c->gidx, P, c->NG, c->chunk_counts, s), "dispatch count");
        if (!rc)
            rc = ok(launch_dispatch_scan(c->chunk_counts, nchunks, c->NG, P, T, 0, kAtomicRows, c->chunk_base,
                                         c->counts, c->offsets, c->tiles, c->num_tiles, s),
                    "dispatch scan");
        if (!rc)
            rc = ok(launch_dispatch_scatter(c->gidx, c->w, P, c->NG, kDispatchChunk, c->chunk_base, c->perm, c->inv,
                                            c->wrow, s),
                    "dispatch scatter");
        if (!rc)
            rc = ok(launch_atomic_rows(x, c->W, c->V, c->perm, c->idx, c->wrow, P, d, k, c->O, s),
                    "expert-centric experts");
        if (!rc) rc = ok(launch_combine_f32(c->O, c->inv, T, d, k, P, 0, y, s), "combine");
    }
    if (!rc && dbg) {
        const size_t ld = (size_t)(Nr + Nc) * 4;
        auto copy_cols = [&](float *dst, const float *src, int n) {
            const hipError_t e = hipMemcpy2DAsync(dst, (size_t)n * 4, src, ld, (size_t)n * 4, (size_t)T,
                                                  hipMemcpyDeviceToDevice, s);
            return e == hipSuccess ? QMOE_OK : fail(QMOE_EHIP, "logit copy failed: %s", hipGetErrorString(e));
        };
        if (dbg->logits_rows) rc = copy_cols(dbg->logits_rows, c->logits, Nr);
        if (!rc && dbg->logits_cols) rc = copy_cols(dbg->logits_cols, c->logits + Nr, Nc);
        if (!rc && dbg->topk_idx) rc = copy_out(dbg->topk_idx, c->idx, (size_t)P * 4, s);
        if (!rc && dbg->topk_w) rc = copy_out(dbg->topk_w, c->w, (size_t)P * 4, s);
        if (!rc && dbg->perm && schedule == QMOE_SCHEDULE_EXPERT_CENTRIC)
            rc = copy_out(dbg->perm, c->perm, (size_t)P * 4, s);
    }
    return rc;
}

void qmoe_atomic_destroy(qmoe_atomic_ctx *c) {
    if (!c) return;
    (void)hipSetDevice(c->cfg.device);
    atomic_free(c);
}

}  // extern "C"
