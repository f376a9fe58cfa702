// C-ABI surface of libxattn: argument validation, workspace sizing, tile-size
// choice and kernel dispatch.  The operation and the conventions are stated in
// include/xattn.h.
#include "xattn.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <new>
#include <string>

#include "internal.h"
#include "plan_layout.h"

struct xattn_ctx {
    xattn_config cfg;
    xattn::Tuning tune;   // overrides from the environment, read at creation
    int n_cu = 0;         // compute units of cfg.device, read on first use
};

namespace {

thread_local std::string g_last_error;

xattn_status fail(xattn_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

xattn_status hip_fail(hipError_t e, const char* what) {
    return fail(XATTN_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool bf16_dh_supported(int dh) { return dh == 32 || dh == 64 || dh == 128; }

// The XATTN_* tuning overrides (internal.h), read once per context.
xattn::Tuning read_tuning() {
    xattn::Tuning t;
    if (const char* env = getenv("XATTN_VARIANT")) {
        int rb = 0, ks = 0;
        if (sscanf(env, "%d,%d", &rb, &ks) == 2) t.variant_rb = rb, t.variant_ks = ks;
    }
    if (const char* env = getenv("XATTN_SHORT")) t.short_path = env[0] == '1' ? 1 : 0;
    if (const char* env = getenv("XATTN_CODEC_DECODE")) t.codec_decode = env[0] == '0' ? 0 : 1;
    if (const char* env = getenv("XATTN_CODEC_QW")) {
        const int v = atoi(env);
        if (v == 2 || v == 4 || v == 8) t.codec_qw = v;
    }
    if (const char* env = getenv("XATTN_FUSED_OUTPUT")) t.fused_output = env[0] == '1' ? 1 : 0;
    if (const char* env = getenv("XATTN_GEMM")) {
        int te = 0, tc = 0, kc = 0;
        if (sscanf(env, "%d,%d,%d", &te, &tc, &kc) == 3) t.gemm_te = te, t.gemm_tc = tc, t.gemm_kc = kc;
    }
    if (const char* env = getenv("XATTN_DQ_KS")) {
        const int v = atoi(env);
        if (v == 1 || v == 2) t.dq_ks = v;
    }
    return t;
}

// Work-group shape of the bf16 kernel: rb query blocks of 32 candidates and
// ksplit memory splits (rb * ksplit waves).  Long memories favour splitting
// the memory so that every SIMD holds several waves; batches with many query
// tiles favour wide query blocks that share each staged memory tile.
// The context's XATTN_VARIANT="rb,ksplit" overrides the choice (tuning and
// tests).
struct Variant {
    int rb, ksplit;
};

// Batches of at most kInPlanMaxRequests requests on a model of at most
// kAttnProjMaxD features run as one launch: the attention kernel plans the
// batch and projects its own queries.  Larger ones run the projection GEMM
// (with the planner) and then the attention kernel over its output.
bool fused_shape(const xattn_config& c, int R) {
    return c.d_model <= xattn::kAttnProjMaxD && R <= xattn::kInPlanMaxRequests;
}

// Batches of short memories (mean L_r no longer than what LDS holds at once)
// on a 256-feature bf16 model run the planner and then the short-memory
// kernel, which projects and attends in one launch (short_bf16.hip); small
// batches keep the single launch.  The context's XATTN_SHORT=0 / 1 turns the
// path off / on for every batch it supports (tuning and tests).
bool short_shape(const xattn_ctx* ctx, int R, int total_kv, int heads) {
    const xattn_config& c = ctx->cfg;
    if (c.dtype != XATTN_BF16 || c.d_model != xattn::kShortD || heads < 1 || c.d_model % heads)
        return false;
    const int dh = c.d_model / heads;
    if (dh != 32 && dh != 64 && dh != 128) return false;
    if (ctx->tune.short_path >= 0) return ctx->tune.short_path == 1;
    if (fused_shape(c, R)) return false;
    return (int64_t)total_kv <=
           (int64_t)R * xattn::short_max_rows(c.kv_mode == XATTN_KV_SEPARATE);
}

// Compute units of the context's device (read once).
int cu_count(xattn_ctx* ctx) {
    if (ctx->n_cu <= 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, ctx->cfg.device) !=
                hipSuccess ||
            n <= 0)
            n = 256;
        ctx->n_cu = n;
    }
    return ctx->n_cu;
}

// Work-groups of the short-memory kernel: one per compute unit (its LDS
// footprint admits one), never more than there are work items.
int short_grid(xattn_ctx* ctx, int64_t max_tiles) {
    const int n = cu_count(ctx);
    return (int)(max_tiles < n ? max_tiles : n);
}

// LDS bytes of a variant as this batch shape launches it.  The choice depends
// only on the batch shape, never on the entry point: a plan built by one call
// is read by the next, and its tile size is the variant's.
int variant_smem(const xattn_config& c, int R, int dh, int rb, int ks) {
    const bool sep = c.kv_mode == XATTN_KV_SEPARATE;
    const int proj = fused_shape(c, R) ? xattn::attn_bf16_variant_smem(dh, rb, ks, sep, true) : 0;
    return proj > 0 ? proj : xattn::attn_bf16_variant_smem(dh, rb, ks, sep, false);
}

Variant choose_variant(const xattn_ctx* ctx, int R, int total_cand, int total_kv, int heads) {
    const xattn_config& c = ctx->cfg;
    const int dh = c.d_model / heads;
    {
        const int rb = ctx->tune.variant_rb, ks = ctx->tune.variant_ks;
        if (rb > 0 && variant_smem(c, R, dh, rb, ks) > 0) return {rb, ks};
    }
    const double rows = (double)total_cand * c.n_slots * heads;   // query rows x heads
    const double mean_L = R > 0 ? (double)total_kv / R : 0.0;
    const double mean_N = R > 0 ? (double)total_cand / R : 0.0;
    // Measured on MI355X over the benchmark batches and synthetic shapes
    // (query tiles of 64 x heads from 24 to 16384, mean memory 600 to 16384):
    Variant v{2, 2};
    if (rows / 64.0 < 256.0 && mean_L >= 1024.0)
        v = {1, 4};   // few query tiles, long memories: split the memory
    else if (rows / 64.0 >= 1024.0 && mean_N >= 128.0)
        v = {4, 1};   // many full tiles already fill the chip
    else if (mean_N <= 64.0 && mean_L >= 1024.0 && !fused_shape(c, R))
        v = {2, 1};   // one 64-candidate tile per request and slot, long memories
    // Take the preferred variant if it leaves room for two work-groups per
    // compute unit, else the first such fallback, else the smallest built one.
    const Variant order[] = {v, {2, 2}, {4, 1}, {1, 4}, {2, 1}};
    for (const Variant& o : order) {
        const int sm = variant_smem(c, R, dh, o.rb, o.ksplit);
        if (sm > 0 && sm <= 81920) return o;
    }
    Variant best{2, 1};
    int best_sm = 1 << 30;
    for (const Variant& o : order) {
        const int sm = variant_smem(c, R, dh, o.rb, o.ksplit);
        if (sm > 0 && sm < best_sm) best = o, best_sm = sm;
    }
    return best;
}

int tile_m_for(const xattn_ctx* ctx, int R, int total_cand, int total_kv, int heads) {
    if (ctx->cfg.dtype != XATTN_BF16) return 64;
    return 32 * choose_variant(ctx, R, total_cand, total_kv, heads).rb;
}

int64_t max_tiles_for(const xattn_config& c, int R, int total_cand, int tile_m) {
    // sum_r ceil(N_r / tile_m) <= (total_cand + R * (tile_m - 1)) / tile_m
    return (int64_t)c.n_slots * (((int64_t)total_cand + (int64_t)R * (tile_m - 1)) / tile_m);
}

// The workspace is sized for the smallest tile (32 candidates), which bounds
// the tile count of every variant.
int64_t max_tiles_any(const xattn_config& c, int R, int total_cand) {
    return max_tiles_for(c, R, total_cand, 32);
}

// Workspace layout: plan header and tiles, then (256-byte aligned) the
// projected queries [total_cand][q][d] in the context's element type.
size_t q_offset(const xattn_config& c, int R, int total_cand) {
    const size_t plan = (size_t)xattn::kPlanHeaderBytes + 16 * (size_t)max_tiles_any(c, R, total_cand);
    return (plan + 255) & ~(size_t)255;
}

size_t elem_bytes(const xattn_config& c) { return c.dtype == XATTN_BF16 ? 2 : 4; }

size_t workspace_bytes(const xattn_config& c, int R, int total_cand) {
    return q_offset(c, R, total_cand) + (size_t)total_cand * c.n_slots * c.d_model * elem_bytes(c);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Coded-memory workspace: the forward's, then (256-byte aligned) the decoded
// planes, [total_kv][d] bf16 each: one in shared mode, key and value in
// separate mode.
size_t codec_plane_offset(const xattn_config& c, int R, int total_cand) {
    return align256(workspace_bytes(c, R, total_cand));
}
size_t codec_plane_bytes(const xattn_config& c, int total_kv) {
    return align256((size_t)total_kv * c.d_model * 2);
}
size_t codec_workspace_bytes(const xattn_config& c, int R, int total_cand, int total_kv) {
    const int planes = c.kv_mode == XATTN_KV_SEPARATE ? 2 : 1;
    return codec_plane_offset(c, R, total_cand) + planes * codec_plane_bytes(c, total_kv);
}

struct DeviceGuard {
    int prev = -1;
    hipError_t err = hipSuccess;
    explicit DeviceGuard(int dev) {
        err = hipGetDevice(&prev);
        if (err == hipSuccess && prev != dev) err = hipSetDevice(dev);
        else if (err == hipSuccess) prev = -1;
    }
    ~DeviceGuard() {
        if (prev >= 0) (void)hipSetDevice(prev);
    }
};

xattn_status check_shape(const xattn_ctx* ctx, int R, int total_cand, int total_kv, int heads) {
    if (!ctx) return fail(XATTN_EINVAL, "ctx is NULL");
    if (R < 0 || total_cand < 0 || total_kv < 0)
        return fail(XATTN_EINVAL, "negative count (num_requests=%d total_cand=%d total_kv=%d)", R,
                    total_cand, total_kv);
    if (heads < 1 || ctx->cfg.d_model % heads != 0)
        return fail(XATTN_EINVAL, "heads=%d must be >= 1 and divide d_model=%d", heads,
                    ctx->cfg.d_model);
    const int dh = ctx->cfg.d_model / heads;
    if (ctx->cfg.dtype == XATTN_BF16 && !bf16_dh_supported(dh))
        return fail(XATTN_EUNSUPPORTED, "bf16 path supports d_h in {32, 64, 128}, got %d", dh);
    if (ctx->cfg.dtype == XATTN_FP32 && dh > 128)
        return fail(XATTN_EUNSUPPORTED, "fp32 path supports d_h <= 128, got %d", dh);
    if (R > xattn::kPlanMaxRequests)
        return fail(XATTN_EUNSUPPORTED, "num_requests=%d exceeds the planner limit %d", R,
                    xattn::kPlanMaxRequests);
    if ((int64_t)total_cand * ctx->cfg.n_slots > INT32_MAX)
        return fail(XATTN_EUNSUPPORTED, "total_cand * q exceeds int32");
    return XATTN_OK;
}

}  // namespace

extern "C" {

const char* xattn_last_error(void) { return g_last_error.c_str(); }

xattn_status xattn_create(const xattn_config* cfg, xattn_ctx** out) {
    g_last_error.clear();
    if (!out) return fail(XATTN_EINVAL, "out is NULL");
    *out = nullptr;
    if (!cfg) return fail(XATTN_EINVAL, "cfg is NULL");
    if (cfg->d_model < 1) return fail(XATTN_EINVAL, "d_model=%d must be >= 1", cfg->d_model);
    if (cfg->n_slots < 1 || cfg->n_slots > 64)
        return fail(XATTN_EINVAL, "n_slots=%d must be in [1, 64]", cfg->n_slots);
    if (cfg->dtype != XATTN_BF16 && cfg->dtype != XATTN_FP32)
        return fail(XATTN_EINVAL, "unknown dtype %d", (int)cfg->dtype);
    if (cfg->kv_mode != XATTN_KV_SHARED && cfg->kv_mode != XATTN_KV_SEPARATE)
        return fail(XATTN_EINVAL, "unknown kv_mode %d", (int)cfg->kv_mode);
    if (cfg->device < 0) return fail(XATTN_EINVAL, "device=%d must be >= 0", cfg->device);
    if (cfg->dtype == XATTN_BF16 && cfg->d_model % 32 != 0)
        return fail(XATTN_EUNSUPPORTED, "bf16 path needs d_model %% 32 == 0, got %d",
                    cfg->d_model);
    xattn_ctx* ctx = new (std::nothrow) xattn_ctx;
    if (!ctx) return fail(XATTN_EINVAL, "out of host memory");
    ctx->cfg = *cfg;
    ctx->tune = read_tuning();
    *out = ctx;
    return XATTN_OK;
}

void xattn_destroy(xattn_ctx* ctx) { delete ctx; }

int64_t xattn_max_tiles(const xattn_ctx* ctx, int32_t R, int32_t total_cand, int32_t heads) {
    if (!ctx || R < 0 || total_cand < 0 || heads < 1) return 0;
    return max_tiles_any(ctx->cfg, R, total_cand);
}

int32_t xattn_forward_path(const xattn_ctx* ctx, int32_t R, int32_t total_cand,
                           int32_t total_kv, int32_t heads) {
    if (!ctx || R <= 0 || total_cand <= 0 || total_kv < 0 || heads < 1 ||
        ctx->cfg.d_model % heads != 0)
        return 0;
    const xattn_config& c = ctx->cfg;
    if (c.dtype != XATTN_BF16) return XATTN_PATH_FP32;
    if (short_shape(ctx, R, total_kv, heads)) return XATTN_PATH_SHORT;
    const Variant var = choose_variant(ctx, R, total_cand, total_kv, heads);
    return fused_shape(c, R) && xattn::attn_bf16_variant_smem(c.d_model / heads, var.rb, var.ksplit,
                                                              c.kv_mode == XATTN_KV_SEPARATE, true) > 0
               ? XATTN_PATH_SINGLE : XATTN_PATH_GEMM;
}

int32_t xattn_forward_launches(const xattn_ctx* ctx, int32_t R, int32_t total_cand,
                               int32_t total_kv, int32_t heads) {
    switch (xattn_forward_path(ctx, R, total_cand, total_kv, heads)) {
        case XATTN_PATH_SINGLE: return 1;
        case XATTN_PATH_GEMM: return 2;
        case XATTN_PATH_FP32: return 3;
        case XATTN_PATH_SHORT: return 1;
        default: return 0;
    }
}

size_t xattn_workspace_size(const xattn_ctx* ctx, int32_t R, int32_t total_cand, int32_t heads) {
    if (!ctx || R < 0 || total_cand < 0 || heads < 1) return 0;
    return workspace_bytes(ctx->cfg, R, total_cand);
}

size_t xattn_codec_workspace_size(const xattn_ctx* ctx, int32_t R, int32_t total_cand,
                                  int32_t total_kv, int32_t heads) {
    if (!ctx || R < 0 || total_cand < 0 || total_kv < 0 || heads < 1) return 0;
    return codec_workspace_bytes(ctx->cfg, R, total_cand, total_kv);
}

xattn_status xattn_plan(xattn_ctx* ctx, const int32_t* cu_kv, const int32_t* cu_cand, int32_t R,
                        int32_t total_cand, int32_t total_kv, int32_t heads, int32_t* cu_q,
                        int32_t* row_req, int32_t* tiles, int32_t* n_tiles, int32_t* tile_m,
                        void* workspace, size_t workspace_bytes, void* stream) {
    g_last_error.clear();
    xattn_status st = check_shape(ctx, R, total_cand, total_kv, heads);
    if (st != XATTN_OK) return st;
    if (!cu_kv || !cu_cand || !cu_q || !tiles || !n_tiles)
        return fail(XATTN_EINVAL, "NULL offset or output pointer");
    if (!workspace || workspace_bytes < xattn_workspace_size(ctx, R, total_cand, heads))
        return fail(XATTN_EWORKSPACE, "workspace needs %zu bytes, got %zu",
                    xattn_workspace_size(ctx, R, total_cand, heads), workspace_bytes);
    const int tm = tile_m_for(ctx, R, total_cand, total_kv, heads);
    if (tile_m) *tile_m = tm;
    DeviceGuard dg(ctx->cfg.device);
    if (dg.err != hipSuccess) return hip_fail(dg.err, "hipSetDevice");
    hipError_t e = xattn::launch_plan(cu_kv, cu_cand, R, ctx->cfg.n_slots, tm, total_cand,
                                      total_kv, workspace, max_tiles_for(ctx->cfg, R, total_cand, tm),
                                      cu_q, row_req, tiles, n_tiles,
                                      static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "plan kernel launch");
    return XATTN_OK;
}

namespace {

enum class Mode { kForward, kAttend, kAttendQ };

// Workspace bytes a forward pass (plan + projection + attention, no prefix
// cutoff) really touches on the path this batch takes: the plan alone on the
// single-launch and short-memory paths (their queries never leave the chip),
// the plan and the projected queries on the others.
size_t forward_path_ws_bytes(const xattn_ctx* ctx, int R, int total_cand, int total_kv,
                             int heads) {
    const int path = xattn_forward_path(ctx, R, total_cand, total_kv, heads);
    if (path == XATTN_PATH_SHORT || path == XATTN_PATH_SINGLE) return q_offset(ctx->cfg, R, total_cand);
    return workspace_bytes(ctx->cfg, R, total_cand);
}

// Shared body of xattn_forward (plan + projection + attention), xattn_attend
// (projection + attention over the plan in the workspace), xattn_attend_q
// (attention over caller-projected queries and the plan in the workspace) and
// xattn_forward_prefix (xattn_forward with a per-candidate memory prefix,
// cand_len not NULL) and xattn_forward_train (lse not NULL: the attention
// kernel also stores each row's log2 softmax normaliser per head).
xattn_status run_forward(Mode mode, xattn_ctx* ctx, const void* Z, const void* W_Q, const void* Qin,
                         const void* K, const void* V, const int32_t* cu_kv,
                         const int32_t* cu_cand, int32_t R, int32_t total_cand, int32_t total_kv,
                         int32_t heads, void* O, void* workspace, size_t workspace_bytes_,
                         void* stream, const int32_t* cand_len = nullptr, float* lse = nullptr,
                         bool use_scratch = false) {
    g_last_error.clear();
    xattn_status st = check_shape(ctx, R, total_cand, total_kv, heads);
    if (st != XATTN_OK) return st;
    const xattn_config& c = ctx->cfg;
    if (c.kv_mode == XATTN_KV_SHARED && V)
        return fail(XATTN_EINVAL, "V must be NULL in XATTN_KV_SHARED mode (V = K = H)");
    if (!cu_kv || !cu_cand) return fail(XATTN_EINVAL, "NULL offset array");
    if (total_cand > 0 && !O) return fail(XATTN_EINVAL, "NULL O");
    if (lse && c.dtype != XATTN_BF16)
        return fail(XATTN_EUNSUPPORTED, "stored statistics need a bf16 context");
    if (total_cand > 0 && mode != Mode::kAttendQ && (!Z || !W_Q))
        return fail(XATTN_EINVAL, "NULL Z or W_Q");
    if (total_cand > 0 && mode == Mode::kAttendQ && !Qin) return fail(XATTN_EINVAL, "NULL Q");
    if (total_kv > 0 && !K) return fail(XATTN_EINVAL, "NULL K");
    if (total_kv > 0 && c.kv_mode == XATTN_KV_SEPARATE && !V)
        return fail(XATTN_EINVAL, "V is NULL in XATTN_KV_SEPARATE mode");
    if (R == 0 && (total_cand != 0 || total_kv != 0))
        return fail(XATTN_EINVAL, "num_requests=0 with total_cand=%d total_kv=%d", total_cand,
                    total_kv);
    if (use_scratch) {
        // the library's own array stands in for the workspace: the batch must
        // fit what its path touches
        const size_t need = forward_path_ws_bytes(ctx, R, total_cand, total_kv, heads);
        if (need > xattn::scratch_capacity())
            return fail(XATTN_EUNSUPPORTED,
                        "batch needs %zu bytes of scratch, more than the %zu the no-alloc "
                        "forward holds (use xattn_forward with a workspace)",
                        need, xattn::scratch_capacity());
    } else {
        const size_t need = workspace_bytes(c, R, total_cand);
        if (!workspace || workspace_bytes_ < need)
            return fail(XATTN_EWORKSPACE, "workspace needs %zu bytes, got %zu", need,
                        workspace_bytes_);
    }
    if (R == 0 || total_cand == 0) return XATTN_OK;  // no query rows: nothing to compute

    const Variant var = c.dtype == XATTN_BF16 ? choose_variant(ctx, R, total_cand, total_kv, heads)
                                              : Variant{2, 1};
    const int tm = tile_m_for(ctx, R, total_cand, total_kv, heads);
    const int64_t max_tiles = max_tiles_for(c, R, total_cand, tm);
    if (max_tiles * heads > INT32_MAX)
        return fail(XATTN_EUNSUPPORTED, "grid of %lld work-groups is too large",
                    (long long)(max_tiles * heads));
    hipStream_t s = static_cast<hipStream_t>(stream);
    DeviceGuard dg(c.device);
    if (dg.err != hipSuccess) return hip_fail(dg.err, "hipSetDevice");
    hipError_t e = hipSuccess;
    if (use_scratch) {
        // the array's device address on this (now current) device; the
        // host-side name of the array is never passed to a kernel
        e = xattn::scratch_on_device(c.device, &workspace);
        if (e != hipSuccess) return hip_fail(e, "no-alloc scratch address (hipGetSymbolAddress)");
        workspace_bytes_ = xattn::scratch_capacity();
    }
    void* qws = static_cast<char*>(workspace) + q_offset(c, R, total_cand);
    const void* Qp = mode == Mode::kAttendQ ? Qin : qws;
    if (c.dtype == XATTN_BF16) {
        xattn::AttnArgs a{};
        a.K = K;
        a.V = c.kv_mode == XATTN_KV_SEPARATE ? V : nullptr;
        a.ws = workspace;
        a.cu_kv = cu_kv;
        a.cu_cand = cu_cand;
        a.max_tiles = max_tiles;
        a.R = R;
        a.total_cand = total_cand;
        a.total_kv = total_kv;
        a.q = c.n_slots;
        a.d = c.d_model;
        a.heads = heads;
        a.O = O;
        a.cand_len = cand_len;
        a.lse = lse;
        a.ncu = cu_count(ctx);
        if (mode != Mode::kAttendQ && !cand_len && short_shape(ctx, R, total_kv, heads)) {
            // projection and attention in one launch; a forward pass also
            // plans the batch in that launch (request order) and stores the
            // plan in the workspace
            a.Z = Z;
            a.Wq = W_Q;
            a.tile_m = tm;
            a.inplan = mode == Mode::kForward;
            e = xattn::launch_short_bf16(a, short_grid(ctx, max_tiles), s);
            if (e != hipSuccess) return hip_fail(e, "short-memory kernel launch");
            return XATTN_OK;
        }
        // small batches, with or without prefix cutoffs: one launch
        const bool fused_proj =
            fused_shape(c, R) &&
            xattn::attn_bf16_variant_smem(c.d_model / heads, var.rb, var.ksplit,
                                          c.kv_mode == XATTN_KV_SEPARATE, true) > 0;
        if (mode == Mode::kAttendQ) {
            a.Qp = Qin;   // caller-projected queries, stored plan
        } else if (fused_proj) {
            // one launch: the attention kernel projects its own queries, and
            // plans a small batch itself (forward) or reads the stored plan
            a.Z = Z;
            a.Wq = W_Q;
            a.inplan = mode == Mode::kForward;
        } else {
            // projection GEMM into the workspace (its launch also runs the
            // planner for a forward pass), then attention over those queries
            e = xattn::launch_project_plan_bf16(Z, W_Q, total_cand, c.n_slots, c.d_model, qws, cu_kv,
                                                cu_cand, R, tm, total_kv,
                                                mode == Mode::kForward ? workspace : nullptr,
                                                max_tiles, s, nullptr, 1.0f, nullptr, &ctx->tune);
            if (e != hipSuccess) return hip_fail(e, "projection kernel launch");
            a.Qp = qws;
        }
        e = xattn::launch_attn_bf16(a, var.rb, var.ksplit, s);
    } else {
        if (mode == Mode::kForward) {
            e = xattn::launch_plan(cu_kv, cu_cand, R, c.n_slots, tm, total_cand, total_kv, workspace,
                                   max_tiles, nullptr, nullptr, nullptr, nullptr, s);
            if (e != hipSuccess) return hip_fail(e, "plan kernel launch");
        }
        if (mode != Mode::kAttendQ) {
            e = xattn::launch_project_f32(static_cast<const float*>(Z),
                                          static_cast<const float*>(W_Q), total_cand, c.n_slots,
                                          c.d_model, static_cast<float*>(qws), s);
            if (e != hipSuccess) return hip_fail(e, "projection kernel launch");
        }
        e = xattn::launch_attn_f32(static_cast<const float*>(Qp), static_cast<const float*>(K),
                                   c.kv_mode == XATTN_KV_SEPARATE ? static_cast<const float*>(V)
                                                                  : nullptr,
                                   workspace, cand_len, max_tiles, c.n_slots, c.d_model, heads,
                                   static_cast<float*>(O), s);
    }
    if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
    return XATTN_OK;
}

}  // namespace

xattn_status xattn_forward(xattn_ctx* ctx, const void* Z, const void* W_Q, const void* K,
                           const void* V, const int32_t* cu_kv, const int32_t* cu_cand,
                           int32_t R, int32_t total_cand, int32_t total_kv, int32_t heads,
                           void* O, void* workspace, size_t workspace_bytes_, void* stream) {
    return run_forward(Mode::kForward, ctx, Z, W_Q, nullptr, K, V, cu_kv, cu_cand, R, total_cand,
                       total_kv, heads, O, workspace, workspace_bytes_, stream);
}

xattn_status xattn_forward_noalloc(xattn_ctx* ctx, const void* Z, const void* W_Q, const void* K,
                                   const void* V, const int32_t* cu_kv, const int32_t* cu_cand,
                                   int32_t R, int32_t total_cand, int32_t total_kv, int32_t heads,
                                   void* O, void* stream) {
    return run_forward(Mode::kForward, ctx, Z, W_Q, nullptr, K, V, cu_kv, cu_cand, R, total_cand,
                       total_kv, heads, O, nullptr, 0, stream, nullptr, nullptr,
                       /*use_scratch=*/true);
}

xattn_status xattn_forward_prefix(xattn_ctx* ctx, const void* Z, const void* W_Q, const void* K,
                                  const void* V, const int32_t* cu_kv, const int32_t* cu_cand,
                                  const int32_t* cand_kv_len, int32_t R, int32_t total_cand,
                                  int32_t total_kv, int32_t heads, void* O, void* workspace,
                                  size_t workspace_bytes_, void* stream) {
    if (ctx && total_cand > 0 && !cand_kv_len) {
        g_last_error.clear();
        return fail(XATTN_EINVAL, "NULL cand_kv_len");
    }
    return run_forward(Mode::kForward, ctx, Z, W_Q, nullptr, K, V, cu_kv, cu_cand, R, total_cand,
                       total_kv, heads, O, workspace, workspace_bytes_, stream, cand_kv_len);
}

xattn_status xattn_forward_train(xattn_ctx* ctx, const void* Z, const void* W_Q, const void* K,
                                 const void* V, const int32_t* cu_kv, const int32_t* cu_cand,
                                 const int32_t* cand_kv_len, int32_t R, int32_t total_cand,
                                 int32_t total_kv, int32_t heads, void* O, float* lse,
                                 void* workspace, size_t workspace_bytes_, void* stream) {
    g_last_error.clear();
    if (ctx && total_cand > 0 && !lse) return fail(XATTN_EINVAL, "NULL lse");
    return run_forward(Mode::kForward, ctx, Z, W_Q, nullptr, K, V, cu_kv, cu_cand, R, total_cand,
                       total_kv, heads, O, workspace, workspace_bytes_, stream, cand_kv_len,
                       total_cand > 0 ? lse : nullptr);
}

xattn_status xattn_attend(xattn_ctx* ctx, const void* Z, const void* W_Q, const void* K,
                          const void* V, const int32_t* cu_kv, const int32_t* cu_cand,
                          int32_t R, int32_t total_cand, int32_t total_kv, int32_t heads,
                          void* O, void* workspace, size_t workspace_bytes_, void* stream) {
    return run_forward(Mode::kAttend, ctx, Z, W_Q, nullptr, K, V, cu_kv, cu_cand, R, total_cand,
                       total_kv, heads, O, workspace, workspace_bytes_, stream);
}

xattn_status xattn_attend_q(xattn_ctx* ctx, const void* Q, const void* K, const void* V,
                            const int32_t* cu_kv, const int32_t* cu_cand, int32_t R,
                            int32_t total_cand, int32_t total_kv, int32_t heads, void* O,
                            void* workspace, size_t workspace_bytes_, void* stream) {
    return run_forward(Mode::kAttendQ, ctx, nullptr, nullptr, Q, K, V, cu_kv, cu_cand, R,
                       total_cand, total_kv, heads, O, workspace, workspace_bytes_, stream);
}

xattn_status xattn_attend_q_prefix(xattn_ctx* ctx, const void* Q, const void* K, const void* V,
                                   const int32_t* cu_kv, const int32_t* cu_cand,
                                   const int32_t* cand_kv_len, int32_t R, int32_t total_cand,
                                   int32_t total_kv, int32_t heads, void* O, void* workspace,
                                   size_t workspace_bytes_, void* stream) {
    if (ctx && total_cand > 0 && !cand_kv_len) {
        g_last_error.clear();
        return fail(XATTN_EINVAL, "NULL cand_kv_len");
    }
    return run_forward(Mode::kAttendQ, ctx, nullptr, nullptr, Q, K, V, cu_kv, cu_cand, R,
                       total_cand, total_kv, heads, O, workspace, workspace_bytes_, stream,
                       cand_kv_len);
}

namespace {

// Backward workspace: the query-tile plan (tiles of 64 candidates), the
// memory-tile plan (64 rows), the projected (bf16: pre-scaled) queries, the
// forward statistics lse and D, dQ, the transposed W_Q and, in bf16, the
// split-K partials of dW_Q.  Every region starts 256-byte aligned.
struct BwdLayout {
    size_t plan, kplan, qs, lse, dsum, dq, wt, part, vis, total;
    int nch;
    int64_t max_q, max_k;
};

BwdLayout bwd_layout(const xattn_config& c, int R, int total_cand, int total_kv, int heads) {
    BwdLayout L{};
    const size_t eb = elem_bytes(c);
    const size_t rows = (size_t)total_cand * c.n_slots, d = (size_t)c.d_model;
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    L.max_q = max_tiles_for(c, R, total_cand, 64);
    L.max_k = ((int64_t)total_kv + (int64_t)R * 63) / 64;
    L.nch = c.dtype == XATTN_BF16 ? xattn::bwd_dw_chunks(total_cand, c.n_slots, c.d_model) : 0;
    size_t off = 0;
    L.plan = off;
    off = al(off + xattn::kPlanHeaderBytes + 16 * (size_t)(L.max_q > 0 ? L.max_q : 1));
    L.kplan = off;
    off = al(off + xattn::kPlanHeaderBytes + 16 * (size_t)(L.max_k > 0 ? L.max_k : 1));
    L.qs = off;
    off = al(off + rows * d * eb);
    L.lse = off;
    off = al(off + rows * heads * 4);
    L.dsum = off;
    off = al(off + rows * heads * 4);
    L.dq = off;
    off = al(off + rows * d * eb);
    L.wt = off;
    off = al(off + (size_t)c.n_slots * d * d * eb);
    L.part = off;
    off = al(off + (size_t)L.nch * c.n_slots * d * d * 4);
    L.vis = off;
    off = al(off + (size_t)total_cand * 4);
    L.total = off;
    return L;
}

}  // namespace

size_t xattn_backward_workspace_size(const xattn_ctx* ctx, int32_t R, int32_t total_cand,
                                     int32_t total_kv, int32_t heads) {
    if (!ctx || R < 0 || total_cand < 0 || total_kv < 0 || heads < 1 ||
        ctx->cfg.d_model % heads != 0)
        return 0;
    return bwd_layout(ctx->cfg, R, total_cand, total_kv, heads).total;
}

namespace {

// Body of xattn_backward (O_saved and lse_saved NULL: the forward statistics
// are recomputed) and xattn_backward_saved (the forward's output and
// normalisers are given; only D = <dO, O> is computed).
xattn_status run_backward(xattn_ctx* ctx, const void* Z, const void* W_Q, const void* K,
                          const void* V, const void* dO, const void* O_saved,
                          const float* lse_saved, const int32_t* cu_kv, const int32_t* cu_cand,
                          const int32_t* cand_kv_len, int32_t R, int32_t total_cand,
                          int32_t total_kv, int32_t heads, void* dZ, float* dW_Q, void* dK,
                          void* dV, void* workspace, size_t workspace_bytes_, void* stream) {
    g_last_error.clear();
    xattn_status st = check_shape(ctx, R, total_cand, total_kv, heads);
    if (st != XATTN_OK) return st;
    const xattn_config& c = ctx->cfg;
    const bool sep = c.kv_mode == XATTN_KV_SEPARATE;
    const bool saved = O_saved || lse_saved;
    if (saved && c.dtype != XATTN_BF16)
        return fail(XATTN_EUNSUPPORTED, "stored statistics need a bf16 context");
    if (saved && total_cand > 0 && (!O_saved || !lse_saved))
        return fail(XATTN_EINVAL, "NULL O or lse");
    // dO (and the stored O) are read in 16-byte pieces by both paths
    if (total_cand > 0 &&
        ((reinterpret_cast<uintptr_t>(saved ? O_saved : nullptr) |
          reinterpret_cast<uintptr_t>(dO)) & 15) != 0)
        return fail(XATTN_EINVAL, saved ? "O and dO must be 16-byte aligned"
                                        : "dO must be 16-byte aligned");
    if (!sep && (V || dV))
        return fail(XATTN_EINVAL, "V and dV must be NULL in XATTN_KV_SHARED mode (dK is dH)");
    if (!cu_kv || !cu_cand) return fail(XATTN_EINVAL, "NULL offset array");
    if (!dW_Q) return fail(XATTN_EINVAL, "NULL dW_Q");
    if (total_cand > 0 && (!Z || !dO || !dZ)) return fail(XATTN_EINVAL, "NULL Z, dO or dZ");
    if (!W_Q) return fail(XATTN_EINVAL, "NULL W_Q");
    if (total_kv > 0 && (!K || !dK)) return fail(XATTN_EINVAL, "NULL K or dK");
    if (total_kv > 0 && sep && (!V || !dV))
        return fail(XATTN_EINVAL, "V or dV is NULL in XATTN_KV_SEPARATE mode");
    if (R == 0 && (total_cand != 0 || total_kv != 0))
        return fail(XATTN_EINVAL, "num_requests=0 with total_cand=%d total_kv=%d", total_cand,
                    total_kv);
    const BwdLayout Lw = bwd_layout(c, R, total_cand, total_kv, heads);
    if (!workspace || workspace_bytes_ < Lw.total)
        return fail(XATTN_EWORKSPACE, "workspace needs %zu bytes, got %zu", Lw.total,
                    workspace_bytes_);
    if ((Lw.max_q + Lw.max_k) * heads > INT32_MAX)
        return fail(XATTN_EUNSUPPORTED, "grid too large");
    DeviceGuard dg(c.device);
    if (dg.err != hipSuccess) return hip_fail(dg.err, "hipSetDevice");
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    const int q = c.n_slots, d = c.d_model, dh = d / heads;
    const bool bf = c.dtype == XATTN_BF16;
    hipError_t e = hipSuccess;
#define XATTN_TRY(call, what)                     \
    do {                                          \
        e = (call);                               \
        if (e != hipSuccess) return hip_fail(e, what); \
    } while (0)
    if (R == 0) {   // no parameters were used: a zero weight gradient
        XATTN_TRY(bf ? xattn::launch_bwd_dw_bf16(nullptr, nullptr, 0, q, d, nullptr, 0, dW_Q, s)
                     : xattn::launch_bwd_dw_f32(nullptr, nullptr, 0, q, d, dW_Q, s),
                  "weight-gradient launch");
        return XATTN_OK;
    }
    // 1. plans: query tiles of 64 candidates, memory tiles of 64 rows (the
    //    planner with memory and candidates exchanged)
    // 2. queries (bf16: scaled by log2(e)/sqrt(d_h) exactly as the forward
    //    kernel scales them)
    if (bf) {
        // one launch: pre-scaled projection, query-tile planner, memory-tile
        // planner, W_Q transposed
        const xattn::PrepExtra ex{reinterpret_cast<int*>(ws + Lw.kplan), Lw.max_k, W_Q,
                                  ws + Lw.wt};
        XATTN_TRY(xattn::launch_project_plan_bf16(Z, W_Q, total_cand, q, d, ws + Lw.qs, cu_kv,
                                                  cu_cand, R, 64, total_kv, ws + Lw.plan, Lw.max_q,
                                                  s, nullptr,
                                                  1.4426950408889634f / sqrtf((float)dh), &ex,
                                                  &ctx->tune),
                  "projection kernel launch");
    } else {
        XATTN_TRY(xattn::launch_plan(cu_kv, cu_cand, R, q, 64, total_cand, total_kv, ws + Lw.plan,
                                     Lw.max_q, nullptr, nullptr, nullptr, nullptr, s),
                  "plan kernel launch");
        XATTN_TRY(xattn::launch_project_f32(static_cast<const float*>(Z),
                                            static_cast<const float*>(W_Q), total_cand, q, d,
                                            reinterpret_cast<float*>(ws + Lw.qs), s),
                  "projection kernel launch");
    }
    if (!bf)
        XATTN_TRY(xattn::launch_plan(cu_cand, cu_kv, R, 1, 64, total_kv, total_cand,
                                     ws + Lw.kplan, Lw.max_k, nullptr, nullptr, nullptr, nullptr, s),
                  "memory plan kernel launch");
    // per-candidate prefix: absolute end of each candidate's visible memory
    int* vis = cand_kv_len ? reinterpret_cast<int*>(ws + Lw.vis) : nullptr;
    if (vis)
        XATTN_TRY(xattn::launch_prefix_vis(cu_kv, cu_cand, cand_kv_len, R, total_cand, vis, s),
                  "prefix kernel launch");
    // 3. forward statistics lse and D = <dO, O> per row and head
    float* lse = reinterpret_cast<float*>(ws + Lw.lse);
    float* dsum = reinterpret_cast<float*>(ws + Lw.dsum);
    if (saved) {
        XATTN_TRY(xattn::launch_bwd_dsum_bf16(dO, O_saved, (int64_t)total_cand * q, d, heads, dsum,
                                              s),
                  "statistics kernel launch");
    } else if (bf) {
        xattn::AttnArgs a{};
        a.Qp = ws + Lw.qs;
        a.K = K;
        a.V = sep ? V : nullptr;
        a.ws = ws + Lw.plan;
        a.cu_kv = cu_kv;
        a.cu_cand = cu_cand;
        a.max_tiles = Lw.max_q;
        a.R = R;
        a.total_cand = total_cand;
        a.total_kv = total_kv;
        a.q = q;
        a.d = d;
        a.heads = heads;
        a.prescaled = 1;
        a.cand_len = cand_kv_len;
        a.lse = lse;
        a.Dsum = dsum;
        a.dO = dO;
        // 64-candidate tiles (the plan above); 32-wide heads over one K = V
        // memory take the (2, 1) shape, which runs as head pairs
        const bool pairs = dh == 32 && !sep && heads % 2 == 0;
        const int ks = !pairs && xattn::attn_bf16_variant_smem(dh, 2, 2, sep, false) > 0 ? 2 : 1;
        XATTN_TRY(xattn::launch_attn_bf16(a, 2, ks, s), "statistics kernel launch");
    } else {
        XATTN_TRY(xattn::launch_attn_f32_stats(reinterpret_cast<const float*>(ws + Lw.qs),
                                               static_cast<const float*>(K),
                                               sep ? static_cast<const float*>(V) : nullptr,
                                               ws + Lw.plan, cand_kv_len, Lw.max_q, q, d, heads,
                                               static_cast<const float*>(dO), lse, dsum, s),
                  "statistics kernel launch");
    }
    // 4. dQ (per query tile) and dK, dV (per memory tile, summed over the
    //    request's query rows)
    xattn::BwdArgs b{};
    b.Qs = ws + Lw.qs;
    b.K = K;
    b.V = sep ? V : nullptr;
    b.dO = dO;
    b.lse = saved ? lse_saved : lse;
    b.Dsum = dsum;
    b.plan = reinterpret_cast<const int*>(ws + Lw.plan);
    b.kplan = reinterpret_cast<const int*>(ws + Lw.kplan);
    b.vis = vis;
    b.dQ = ws + Lw.dq;
    b.dK = dK;
    b.dV = sep ? dV : nullptr;
    b.q = q;
    b.d = d;
    b.heads = heads;
    b.scale = 1.0f / sqrtf((float)dh);
    XATTN_TRY(bf ? xattn::launch_bwd_attn_bf16(b, sep, Lw.max_q, Lw.max_k, s, ctx->tune.dq_ks)
                 : xattn::launch_bwd_attn_f32(b, sep, Lw.max_q, Lw.max_k, s),
              "attention backward launch");
    // 5. dZ = dQ W_Q[slot] through the transposed weights; 6. dW_Q
    if (!bf)
        XATTN_TRY(xattn::launch_transpose_weights(W_Q, q, d, true, ws + Lw.wt, s),
                  "transpose kernel launch");
    if (bf) {
        XATTN_TRY(xattn::launch_project_plan_bf16(ws + Lw.dq, ws + Lw.wt, total_cand, q, d, dZ,
                                                  nullptr, nullptr, 0, 0, 0, nullptr, 0, s,
                                                  nullptr, 1.0f, nullptr, &ctx->tune),
                  "input-gradient launch");
        XATTN_TRY(xattn::launch_bwd_dw_bf16(ws + Lw.dq, Z, total_cand, q, d,
                                            reinterpret_cast<float*>(ws + Lw.part), Lw.nch, dW_Q,
                                            s),
                  "weight-gradient launch");
    } else {
        XATTN_TRY(xattn::launch_project_f32(reinterpret_cast<const float*>(ws + Lw.dq),
                                            reinterpret_cast<const float*>(ws + Lw.wt),
                                            total_cand, q, d, static_cast<float*>(dZ), s),
                  "input-gradient launch");
        XATTN_TRY(xattn::launch_bwd_dw_f32(reinterpret_cast<const float*>(ws + Lw.dq),
                                           static_cast<const float*>(Z), total_cand, q, d, dW_Q,
                                           s),
                  "weight-gradient launch");
    }
#undef XATTN_TRY
    return XATTN_OK;
}

}  // namespace

xattn_status xattn_backward(xattn_ctx* ctx, const void* Z, const void* W_Q, const void* K,
                            const void* V, const void* dO, const int32_t* cu_kv,
                            const int32_t* cu_cand, const int32_t* cand_kv_len, int32_t R,
                            int32_t total_cand, int32_t total_kv, int32_t heads, void* dZ,
                            float* dW_Q, void* dK, void* dV, void* workspace,
                            size_t workspace_bytes_, void* stream) {
    return run_backward(ctx, Z, W_Q, K, V, dO, nullptr, nullptr, cu_kv, cu_cand, cand_kv_len, R,
                        total_cand, total_kv, heads, dZ, dW_Q, dK, dV, workspace, workspace_bytes_,
                        stream);
}

xattn_status xattn_backward_saved(xattn_ctx* ctx, const void* Z, const void* W_Q, const void* K,
                                  const void* V, const void* dO, const void* O, const float* lse,
                                  const int32_t* cu_kv, const int32_t* cu_cand,
                                  const int32_t* cand_kv_len, int32_t R, int32_t total_cand,
                                  int32_t total_kv, int32_t heads, void* dZ, float* dW_Q,
                                  void* dK, void* dV, void* workspace, size_t workspace_bytes_,
                                  void* stream) {
    if (ctx && total_cand > 0 && (!O || !lse)) {
        g_last_error.clear();
        return fail(XATTN_EINVAL, "NULL O or lse");
    }
    // with no query rows there is nothing to reuse: the plain pass zeroes dW_Q and the memory
    // gradients
    return run_backward(ctx, Z, W_Q, K, V, dO, total_cand > 0 ? O : nullptr,
                        total_cand > 0 ? lse : nullptr, cu_kv, cu_cand, cand_kv_len, R,
                        total_cand, total_kv, heads, dZ, dW_Q, dK, dV, workspace,
                        workspace_bytes_, stream);
}

namespace {

xattn_status codec_book(const xattn_config& c, const xattn_codebook* cb, int heads,
                        xattn::CodecBook* out) {
    if (!cb) return fail(XATTN_EINVAL, "NULL codebook");
    if (!cb->bits || !cb->center || !cb->half_range || !cb->rotation)
        return fail(XATTN_EINVAL, "NULL codebook array");
    const int dh = c.d_model / heads;
    if (cb->budget_bits <= 0 || cb->budget_bits % 32 != 0 || cb->budget_bits > 8 * dh)
        return fail(XATTN_EUNSUPPORTED, "budget_bits %d: need a positive multiple of 32 <= %d",
                    cb->budget_bits, 8 * dh);
    *out = xattn::CodecBook{cb->budget_bits, cb->bits, cb->center, cb->half_range, cb->rotation};
    return XATTN_OK;
}

xattn_status codec_shape(const xattn_ctx* ctx, int heads) {
    if (!ctx) return fail(XATTN_EINVAL, "ctx is NULL");
    const xattn_config& c = ctx->cfg;
    if (heads < 1 || c.d_model % heads != 0)
        return fail(XATTN_EINVAL, "heads=%d does not divide d_model=%d", heads, c.d_model);
    if (c.dtype != XATTN_BF16) return fail(XATTN_EUNSUPPORTED, "coded memory needs a bf16 context");
    if (!bf16_dh_supported(c.d_model / heads))
        return fail(XATTN_EUNSUPPORTED, "head width %d not built", c.d_model / heads);
    return XATTN_OK;
}

}  // namespace

xattn_status xattn_codec_encode(xattn_ctx* ctx, const xattn_codebook* cb, int32_t heads,
                                const void* X, int32_t n_rows, uint32_t* codes, float* norms,
                                void* stream) {
    g_last_error.clear();
    xattn_status st = codec_shape(ctx, heads);
    if (st != XATTN_OK) return st;
    xattn::CodecBook b{};
    if ((st = codec_book(ctx->cfg, cb, heads, &b)) != XATTN_OK) return st;
    if (n_rows < 0) return fail(XATTN_EINVAL, "negative n_rows");
    if (n_rows == 0) return XATTN_OK;
    if (!X || !codes || !norms) return fail(XATTN_EINVAL, "NULL X, codes or norms");
    DeviceGuard dg(ctx->cfg.device);
    if (dg.err != hipSuccess) return hip_fail(dg.err, "hipSetDevice");
    hipError_t e = xattn::launch_codec_encode(b, X, n_rows, ctx->cfg.d_model, heads, codes, norms,
                                              static_cast<hipStream_t>(stream));
    return e == hipSuccess ? XATTN_OK : hip_fail(e, "encode kernel launch");
}

xattn_status xattn_codec_fold_query_weights(xattn_ctx* ctx, const xattn_codebook* cb_k,
                                            int32_t heads, const void* W_Q, void* W_Q_rot,
                                            void* stream) {
    g_last_error.clear();
    xattn_status st = codec_shape(ctx, heads);
    if (st != XATTN_OK) return st;
    xattn::CodecBook b{};
    if ((st = codec_book(ctx->cfg, cb_k, heads, &b)) != XATTN_OK) return st;
    if (!W_Q || !W_Q_rot) return fail(XATTN_EINVAL, "NULL W_Q or W_Q_rot");
    DeviceGuard dg(ctx->cfg.device);
    if (dg.err != hipSuccess) return hip_fail(dg.err, "hipSetDevice");
    hipError_t e = xattn::launch_codec_fold(b, W_Q, ctx->cfg.n_slots, ctx->cfg.d_model, heads,
                                            W_Q_rot, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? XATTN_OK : hip_fail(e, "fold kernel launch");
}

xattn_status xattn_forward_codec(xattn_ctx* ctx, const xattn_codebook* cb_k,
                                 const xattn_codebook* cb_v, const void* Z, const void* W_Q_rot,
                                 const uint32_t* k_codes, const float* k_norms,
                                 const uint32_t* v_codes, const float* v_norms,
                                 const int32_t* cu_kv, const int32_t* cu_cand, int32_t R,
                                 int32_t total_cand, int32_t total_kv, int32_t heads, void* O,
                                 void* workspace, size_t workspace_bytes_, void* stream) {
    g_last_error.clear();
    xattn_status st = check_shape(ctx, R, total_cand, total_kv, heads);
    if (st != XATTN_OK) return st;
    if ((st = codec_shape(ctx, heads)) != XATTN_OK) return st;
    const xattn_config& c = ctx->cfg;
    const bool sep = c.kv_mode == XATTN_KV_SEPARATE;
    xattn::CodecArgs a{};
    if ((st = codec_book(c, cb_k, heads, &a.kb)) != XATTN_OK) return st;
    if (sep) {
        if ((st = codec_book(c, cb_v, heads, &a.vb)) != XATTN_OK) return st;
        if (a.vb.budget != a.kb.budget)
            return fail(XATTN_EUNSUPPORTED, "key and value budgets differ (%d, %d)", a.kb.budget,
                        a.vb.budget);
        if (total_kv > 0 && (!v_codes || !v_norms))
            return fail(XATTN_EINVAL, "NULL value codes or norms in XATTN_KV_SEPARATE mode");
    } else if (cb_v || v_codes || v_norms) {
        return fail(XATTN_EINVAL, "value codebook given in XATTN_KV_SHARED mode");
    }
    if (!cu_kv || !cu_cand) return fail(XATTN_EINVAL, "NULL offset array");
    if (total_cand > 0 && (!Z || !W_Q_rot || !O)) return fail(XATTN_EINVAL, "NULL Z, W_Q_rot or O");
    if (total_kv > 0 && (!k_codes || !k_norms)) return fail(XATTN_EINVAL, "NULL key codes or norms");
    const size_t need = workspace_bytes(c, R, total_cand);
    if (!workspace || workspace_bytes_ < need)
        return fail(XATTN_EWORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace_bytes_);
    if (R == 0 && (total_cand != 0 || total_kv != 0))
        return fail(XATTN_EINVAL, "num_requests=0 with total_cand=%d total_kv=%d", total_cand,
                    total_kv);
    if (R == 0 || total_cand == 0) return XATTN_OK;
    DeviceGuard dg0(c.device);
    if (dg0.err != hipSuccess) return hip_fail(dg0.err, "hipSetDevice");
    // Short memories on a 256-feature model (the TransX memory): the
    // short-memory kernel decodes each request's memory once per work-group
    // (keys in the rotated basis, values rotated back) after a planner launch
    // (request order).  The same rule as the bf16 short path, with at most
    // 96 rows in both modes (two decoded planes).  The context's XATTN_SHORT
    // overrides.
    {
        const int dh = c.d_model / heads;
        const int forced = ctx->tune.short_path;
        const bool short_codec =
            c.d_model == xattn::kShortD && (dh == 32 || dh == 64 || dh == 128) &&
            (forced >= 0 ? forced == 1
                         : !fused_shape(c, R) &&
                               (int64_t)total_kv <= (int64_t)R * xattn::short_max_rows(true));
        if (short_codec) {
            const int64_t mt = max_tiles_for(c, R, total_cand, 64);
            hipStream_t s0 = static_cast<hipStream_t>(stream);
            hipError_t e0 = xattn::launch_plan(cu_kv, cu_cand, R, c.n_slots, 64, total_cand,
                                               total_kv, workspace, mt, nullptr, nullptr, nullptr,
                                               nullptr, s0, /*rank=*/false);
            if (e0 != hipSuccess) return hip_fail(e0, "plan kernel launch");
            xattn::AttnArgs aa{};
            aa.Z = Z;
            aa.Wq = W_Q_rot;
            aa.O = O;
            aa.ws = workspace;
            aa.cu_kv = cu_kv;
            aa.cu_cand = cu_cand;
            aa.max_tiles = mt;
            aa.R = R;
            aa.total_cand = total_cand;
            aa.total_kv = total_kv;
            aa.q = c.n_slots;
            aa.d = c.d_model;
            aa.heads = heads;
            aa.tile_m = 64;
            xattn::ShortCodec cd{};
            cd.kb = a.kb;
            cd.vb = a.vb;
            cd.kcodes = k_codes;
            cd.knorms = k_norms;
            cd.vcodes = sep ? v_codes : nullptr;
            cd.vnorms = sep ? v_norms : nullptr;
            cd.total_kv = total_kv;
            e0 = xattn::launch_short_codec_bf16(aa, cd, sep, short_grid(ctx, mt), s0);
            return e0 == hipSuccess ? XATTN_OK : hip_fail(e0, "short-memory codec kernel launch");
        }
    }
    // Memories that many query tiles read: when the caller's workspace holds
    // the decoded planes (xattn_codec_workspace_size), the memory is decoded
    // once per call and the plain forward runs over it, its queries projected
    // over W_Q_rot.  Separate mode: keys in the rotated basis, values rotated
    // back.  Shared mode: one plane in the rotated basis serves as key and
    // value, and the output rows are rotated back afterwards.
    // The context's XATTN_CODEC_DECODE=0 keeps the per-tile reconstruction
    // below.
    {
        const bool decode = ctx->tune.codec_decode != 0 &&
                            workspace_bytes_ >= codec_workspace_bytes(c, R, total_cand, total_kv);
        if (decode) {
            char* planes = static_cast<char*>(workspace) + codec_plane_offset(c, R, total_cand);
            xattn::CodecDecodeArgs da{};
            da.kb = a.kb;
            da.vb = a.vb;
            da.kcodes = k_codes;
            da.knorms = k_norms;
            da.vcodes = sep ? v_codes : nullptr;
            da.vnorms = sep ? v_norms : nullptr;
            da.Kout = planes;
            da.Vout = sep ? planes + codec_plane_bytes(c, total_kv) : nullptr;
            da.d = c.d_model;
            da.total_kv = total_kv;
            hipStream_t s0 = static_cast<hipStream_t>(stream);
            hipError_t e0 = xattn::launch_codec_decode(da, sep, heads, 128, s0);
            if (e0 != hipSuccess) return hip_fail(e0, "codec decode kernel launch");
            st = run_forward(Mode::kForward, ctx, Z, W_Q_rot, nullptr, da.Kout, da.Vout, cu_kv,
                             cu_cand, R, total_cand, total_kv, heads, O, workspace,
                             workspace_bytes_, stream);
            if (st != XATTN_OK || sep) return st;
            e0 = xattn::launch_codec_rotate_out(a.kb, O, total_cand * c.n_slots, c.d_model, heads,
                                                512, s0);
            return e0 == hipSuccess ? XATTN_OK : hip_fail(e0, "codec output rotation launch");
        }
    }
    // Query waves sharing each reconstructed memory tile (the reconstruction
    // is paid once per tile and work-group): as many as the requests' query
    // rows fill, up to 8 x 32 rows, except that grids of more than 4096
    // eight-wave work-groups run faster with four (measured: 4 waves on a
    // batch of 256 requests x 1024 candidates, 8 on 4-8 requests of
    // 768-1536 rows, 2 on 1..64 candidates per user).  XATTN_CODEC_QW
    // overrides.
    const double rows_per_req = (double)total_cand * c.n_slots / R;
    int qw = rows_per_req >= 512 ? 8 : (rows_per_req >= 128 ? 4 : 2);
    if (qw == 8 && max_tiles_for(c, R, total_cand, 256) * heads > 4096) qw = 4;
    if (ctx->tune.codec_qw) qw = ctx->tune.codec_qw;
    const int64_t max_tiles = max_tiles_for(c, R, total_cand, 32 * qw);
    if (max_tiles * heads > INT32_MAX) return fail(XATTN_EUNSUPPORTED, "grid too large");
    DeviceGuard dg(c.device);
    if (dg.err != hipSuccess) return hip_fail(dg.err, "hipSetDevice");
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* qws = static_cast<char*>(workspace) + q_offset(c, R, total_cand);
    hipError_t e = xattn::launch_project_plan_bf16(Z, W_Q_rot, total_cand, c.n_slots, c.d_model,
                                                   qws, cu_kv, cu_cand, R, 32 * qw, total_kv,
                                                   workspace, max_tiles, s, nullptr, 1.0f,
                                                   nullptr, &ctx->tune);
    if (e != hipSuccess) return hip_fail(e, "projection kernel launch");
    a.Qr = qws;
    a.kcodes = k_codes;
    a.knorms = k_norms;
    a.vcodes = sep ? v_codes : nullptr;
    a.vnorms = sep ? v_norms : nullptr;
    a.plan = static_cast<const int*>(workspace);
    a.O = O;
    a.q = c.n_slots;
    a.d = c.d_model;
    a.heads = heads;
    a.total_kv = total_kv;
    a.scale_log2 = 1.4426950408889634f / sqrtf((float)(c.d_model / heads));
    e = xattn::launch_codec_attn(a, sep, qw, max_tiles, s);
    return e == hipSuccess ? XATTN_OK : hip_fail(e, "codec attention kernel launch");
}

xattn_status xattn_project(xattn_ctx* ctx, const void* Z, const void* W_Q, int32_t total_cand,
                           void* Q, void* stream) {
    g_last_error.clear();
    if (!ctx) return fail(XATTN_EINVAL, "ctx is NULL");
    if (total_cand < 0) return fail(XATTN_EINVAL, "negative total_cand");
    if (total_cand == 0) return XATTN_OK;
    if (!Z || !W_Q || !Q) return fail(XATTN_EINVAL, "NULL Z, W_Q or Q");
    const xattn_config& c = ctx->cfg;
    DeviceGuard dg(c.device);
    if (dg.err != hipSuccess) return hip_fail(dg.err, "hipSetDevice");
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = c.dtype == XATTN_BF16
                       ? xattn::launch_project_plan_bf16(Z, W_Q, total_cand, c.n_slots, c.d_model,
                                                         Q, nullptr, nullptr, 0, 0, 0, nullptr, 0,
                                                         s, nullptr, 1.0f, nullptr, &ctx->tune)
                       : xattn::launch_project_f32(static_cast<const float*>(Z),
                                                   static_cast<const float*>(W_Q), total_cand,
                                                   c.n_slots, c.d_model, static_cast<float*>(Q), s);
    if (e != hipSuccess) return hip_fail(e, "projection kernel launch");
    return XATTN_OK;
}

xattn_status xattn_output(xattn_ctx* ctx, const void* Z, const void* W_go, const void* O,
                          const void* W_o, int32_t total_cand, void* Y, void* workspace,
                          size_t workspace_bytes_, void* stream) {
    g_last_error.clear();
    if (!ctx) return fail(XATTN_EINVAL, "ctx is NULL");
    if (total_cand < 0) return fail(XATTN_EINVAL, "negative total_cand");
    if (total_cand == 0) return XATTN_OK;
    if (!Z || !W_go || !O || !W_o || !Y) return fail(XATTN_EINVAL, "NULL Z, W_go, O, W_o or Y");
    const xattn_config& c = ctx->cfg;
    if ((int64_t)total_cand * c.n_slots > INT32_MAX)
        return fail(XATTN_EUNSUPPORTED, "total_cand * q exceeds int32");
    const size_t xbytes = (size_t)total_cand * c.n_slots * c.d_model * elem_bytes(c);
    if (!workspace || workspace_bytes_ < xbytes)
        return fail(XATTN_EWORKSPACE, "workspace needs %zu bytes, got %zu", xbytes,
                    workspace_bytes_);
    // the gated values go to the end of the workspace, 256-byte aligned
    const size_t xoff = (workspace_bytes_ - xbytes) & ~(size_t)255;
    void* X = static_cast<char*>(workspace) + xoff;
    DeviceGuard dg(c.device);
    if (dg.err != hipSuccess) return hip_fail(dg.err, "hipSetDevice");
    hipStream_t s = static_cast<hipStream_t>(stream);
    // bf16 on a 256-feature model with at least one unit of 64 candidates
    // per compute unit (measured crossover; smaller batches run faster as two
    // GEMM launches that spread over the chip): one kernel keeps the gated
    // values on chip.  The context's XATTN_FUSED_OUTPUT=0 / 1 forces either.
    const int64_t units = (int64_t)c.n_slots * ((total_cand + 63) / 64);
    const int forced = ctx->tune.fused_output;
    const bool fused = c.dtype == XATTN_BF16 && c.d_model == xattn::kShortD &&
                       (forced >= 0 ? forced == 1 : units >= short_grid(ctx, INT64_MAX));
    if (fused) {
        hipError_t e = xattn::launch_gate_output_fused_bf16(Z, W_go, O, W_o, Y, total_cand,
                                                            c.n_slots, c.d_model,
                                                            short_grid(ctx, units), s);
        if (e != hipSuccess) return hip_fail(e, "output kernel launch");
        return XATTN_OK;
    }
    hipError_t e = c.dtype == XATTN_BF16
                       ? xattn::launch_gate_output_bf16(Z, W_go, O, W_o, total_cand, c.n_slots,
                                                        c.d_model, X, Y, s, &ctx->tune)
                       : xattn::launch_gate_output_f32(
                             static_cast<const float*>(Z), static_cast<const float*>(W_go),
                             static_cast<const float*>(O), static_cast<const float*>(W_o),
                             total_cand, c.n_slots, c.d_model, static_cast<float*>(X),
                             static_cast<float*>(Y), s);
    if (e != hipSuccess) return hip_fail(e, "output kernel launch");
    return XATTN_OK;
}

xattn_status xattn_device_error(xattn_ctx* ctx, const void* workspace, int32_t* flag,
                                void* stream) {
    g_last_error.clear();
    if (!ctx || !workspace || !flag) return fail(XATTN_EINVAL, "NULL argument");
    DeviceGuard dg(ctx->cfg.device);
    if (dg.err != hipSuccess) return hip_fail(dg.err, "hipSetDevice");
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    int32_t v = 0;
    e = hipMemcpy(&v, static_cast<const char*>(workspace) + sizeof(int32_t) * xattn::kPlanError,
                  sizeof v, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy");
    *flag = v;
    if (v != 0)
        return fail(XATTN_EDEVICE_VALIDATION,
                    "the device found the offset arrays inconsistent (flag %d: %s%s)", v,
                    (v & xattn::kErrCuKv) ? "cu_seqlens_kv " : "",
                    (v & xattn::kErrCuCand) ? "cu_cand" : "");
    return XATTN_OK;
}

}  // extern "C"
