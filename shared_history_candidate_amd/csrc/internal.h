// Host-side launchers shared between the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xattn {

// Tuning overrides, read from the environment once when a context is
// created (tests and tuning runs force kernel choices this way); 0 / -1 keep
// the library's own choice.
//   XATTN_VARIANT="rb,ks"   attention work-group shape
//   XATTN_SHORT=0|1         short-memory path off / on where it applies
//   XATTN_CODEC_DECODE=0    coded memory: per-tile reconstruction, never decode once
//   XATTN_CODEC_QW=2|4|8    coded memory: query waves per work-group
//   XATTN_FUSED_OUTPUT=0|1  output stage as two GEMM launches / one launch
//   XATTN_GEMM="te,tc,kc"   projection GEMM tile shape
//   XATTN_DQ_KS=1|2         backward dQ kernel: memory splits per work-group
struct Tuning {
    int variant_rb = 0, variant_ks = 0;
    int short_path = -1;
    int codec_decode = -1;
    int codec_qw = 0;
    int fused_output = -1;
    int gemm_te = 0, gemm_tc = 0, gemm_kc = 0;
    int dq_ks = 0;
};

// Library-owned scratch of xattn_forward_noalloc (scratch.hip): its size,
// and its device address on `device`, which must be the current device
// (resolved with hipGetSymbolAddress on the first call per device, then
// cached).
size_t scratch_capacity();
hipError_t scratch_on_device(int device, void** out);

hipError_t launch_plan(const int* cu_kv, const int* cu_cand, int R, int q, int tile_m,
                       int total_cand, int total_kv, void* ws, int64_t max_tiles, int* cu_q,
                       int* row_req, int* tiles, int* n_tiles, hipStream_t stream,
                       bool rank = true);

// bf16 attention (attn_bf16.hip).  A work-group has rb x ksplit waves: rb
// query blocks of 32 candidates (tile_m = 32 * rb) and ksplit memory splits
// merged on chip.  With Z and Wq set the kernel projects its own queries
// (d <= 256; otherwise it reads Qp); with inplan set every wave plans the
// batch itself (R <= kInPlanMaxRequests) instead of reading the plan from
// ws, and the first one writes the plan there.  V is NULL in
// projection-free mode.
struct AttnArgs {
    const void* Qp;
    const void* Z;
    const void* Wq;
    const void* K;
    const void* V;
    void* ws;
    const int* cu_kv;
    const int* cu_cand;
    const int* cand_len;   // per-candidate prefix cutoff, or NULL (Qp path only)
    int64_t max_tiles;
    int R, total_cand, total_kv, inplan, q, d, heads;
    int tile_m;         // candidates per plan tile (short-memory kernel's plan check)
    // Qp already holds bf16(Q * log2(e)/sqrt(d_h)) (backward pass)
    int prescaled;
    float scale_log2;   // set by the launcher
    void* O;            // may be NULL when lse is set
    // Statistics for the backward pass, [rows][heads] fp32 (row = c*q + s):
    // lse = log2 of the row's softmax normaliser in the scaled exp2 units of
    // the scores; Dsum = <dO_row, O_row> of the head (fp32 O), if dO is set.
    float* lse;
    float* Dsum;
    const void* dO;
    // compute units of the device (0: unknown); the attention kernel's
    // pacing reads a work-group's dispatch round from it
    int ncu;
};
// Widest model (d) whose queries the attention kernel projects itself.
constexpr int kAttnProjMaxD = 256;
// LDS bytes of variant (rb, ksplit) for head width dh, K/V mode and query
// source, 0 if not built.
int attn_bf16_variant_smem(int dh, int rb, int ksplit, bool sep, bool proj);
hipError_t launch_attn_bf16(const AttnArgs& a, int rb, int ksplit, hipStream_t stream);

// Short-memory kernel (short_bf16.hip): projection and attention in one
// launch over the plan in a.ws, for a model of kShortD features.  Memories of
// up to short_max_rows() rows stay in LDS whole; longer ones are streamed in
// chunks of that size.  `grid` work-groups walk the plan's items.
constexpr int kShortD = 256;
constexpr int short_max_rows(bool sep) { return sep ? 96 : 192; }
hipError_t launch_short_bf16(const AttnArgs& a, int grid, hipStream_t stream);
// Output gate and W_o in one launch (output_bf16.hip), d = kShortD only;
// `grid` work-groups (at most one per unit of 64 candidates and slot).
hipError_t launch_gate_output_fused_bf16(const void* Z, const void* Wgo, const void* O,
                                         const void* Wo, void* Y, int total_cand, int q, int d,
                                         int grid, hipStream_t stream);

// bf16 TSP projection Q = Z W_Q[slot] into Qp; when ws is not NULL the same
// launch also runs the planner into ws (one extra work-group).
// Backward-pass side jobs run by extra work-groups of the projection launch:
// the memory-tile plan into kws (max_ktiles items) and wdst = wsrc
// transposed per slot ([q][d][d] bf16).
struct PrepExtra {
    int* kws;
    int64_t max_ktiles;
    const void* wsrc;
    void* wdst;
};
// With oscale != 1 the stored value is bf16(float(bf16(acc)) * oscale): the
// queries pre-scaled exactly as the attention kernel scales them.
// tune (may be NULL): the context's tile-shape override.
hipError_t launch_project_plan_bf16(const void* Z, const void* Wq, int total_cand, int q, int d,
                                    void* Qp, const int* cu_kv, const int* cu_cand, int R,
                                    int tile_m, int total_kv, void* ws, int64_t max_tiles,
                                    hipStream_t stream, const void* Og = nullptr,
                                    float oscale = 1.0f, const PrepExtra* ex = nullptr,
                                    const Tuning* tune = nullptr);

// Output gate and projection of Eq. (7): X = O * sigmoid(Z W_go[slot]) (bf16,
// [total_cand][q][d]), then Y = X W_o; two launches of the projection kernel.
hipError_t launch_gate_output_bf16(const void* Z, const void* Wgo, const void* O, const void* Wo,
                                   int total_cand, int q, int d, void* X, void* Y,
                                   hipStream_t stream, const Tuning* tune = nullptr);

// Backward pass (bwd_bf16.hip, bwd in attn_f32.hip).  plan: query tiles of
// 64 candidates (the forward's plan layout); kplan: memory tiles of 64 rows,
// the same planner with memory and candidates exchanged.  Qs holds the
// queries scaled by log2(e)/sqrt(d_h) in bf16 mode (unscaled in fp32 mode),
// lse and Dsum the forward statistics ([rows][heads]).  dK is dH (both
// roles) when V is NULL.
struct BwdArgs {
    const void* Qs;
    const void* K;
    const void* V;
    const void* dO;
    const float* lse;
    const float* Dsum;
    const int* plan;
    const int* kplan;
    // per-candidate end of the visible memory (absolute row), or NULL
    const int* vis;
    void* dQ;
    void* dK;
    void* dV;
    int q, d, heads;
    float scale;   // 1/sqrt(d_h)
};
// dq_ks: memory splits of the dQ kernel (0: the library's choice, 1 or 2).
hipError_t launch_bwd_attn_bf16(const BwdArgs& a, bool sep, int64_t q_items, int64_t k_items,
                                hipStream_t stream, int dq_ks = 0);
// dsum[row][h] = <dO_row, O_row> over head h's features (bf16 [rows][d], rows
// 16-byte aligned, d/heads in {32, 64, 128}; fp32 sums in a fixed order)
hipError_t launch_bwd_dsum_bf16(const void* dO, const void* O, int64_t rows, int d, int heads,
                                float* dsum, hipStream_t stream);
// vis[c] = cu_kv[r] + clamp(len[c], 0, L_r) for each candidate c of request r
hipError_t launch_prefix_vis(const int* cu_kv, const int* cu_cand, const int* len, int R,
                             int total_cand, int* vis, hipStream_t stream);
// dW_Q = sum over rows of slot s of dQ^T Z (fp32 [q][d][d], output-major),
// nch split-K chunks through part ([nch][q][d][d] fp32) reduced in order.
int bwd_dw_chunks(int total_cand, int q, int d);
hipError_t launch_bwd_dw_bf16(const void* dQ, const void* Z, int total_cand, int q, int d,
                              float* part, int nch, float* dW, hipStream_t stream);
hipError_t launch_transpose_weights(const void* wt, int q, int d, bool fp32, void* wT,
                                    hipStream_t stream);
hipError_t launch_bwd_attn_f32(const BwdArgs& a, bool sep, int64_t q_items, int64_t k_items,
                               hipStream_t stream);
hipError_t launch_bwd_dw_f32(const float* dQ, const float* Z, int total_cand, int q, int d,
                             float* dW, hipStream_t stream);
// fp32 forward statistics (lse, Dsum for the backward pass), O may be NULL.
hipError_t launch_attn_f32_stats(const float* Qp, const float* K, const float* V, const void* ws,
                                 const int* cand_len, int64_t max_tiles, int q, int d, int heads,
                                 const float* dO, float* lse, float* Dsum, hipStream_t stream);

// Memory codec (codec_bf16.hip).  A codebook per memory role: budget bits
// per (row, head) vector (a multiple of 32, at most 8 per coordinate), bits
// [heads][d_h] (0..8), center/half [heads][d_h] of the rotated coordinates'
// quantiser, rot [heads][d_h][d_h] (rot[h][o][i]: column i = eigenvector i).
struct CodecBook {
    int budget;
    const uint8_t* bits;
    const float* center;
    const float* half;
    const float* rot;
};
struct CodecArgs {
    const void* Qr;              // rotated projected queries [rows][d] (bf16)
    CodecBook kb, vb;            // vb unused when the memory is both K and V
    const uint32_t* kcodes;      // [heads][total_kv][budget/32]
    const float* knorms;         // [heads][total_kv]
    const uint32_t* vcodes;
    const float* vnorms;
    const int* plan;             // query-tile plan, tile_m = 64
    void* O;
    int q, d, heads, total_kv;
    float scale_log2;
};
hipError_t launch_codec_encode(const CodecBook& cb, const void* X, int n, int d, int heads,
                               uint32_t* codes, float* norms, hipStream_t stream);
hipError_t launch_codec_fold(const CodecBook& cb, const void* Wq, int q, int d, int heads,
                             void* Wr, hipStream_t stream);
// Decoded planes of a coded memory: Kout [total_kv][d] bf16 in the keys'
// rotated basis; separate mode also Vout [total_kv][d] bf16, rotated back.
struct CodecDecodeArgs {
    CodecBook kb, vb;
    const uint32_t* kcodes;
    const float* knorms;
    const uint32_t* vcodes;
    const float* vnorms;
    void* Kout;
    void* Vout;
    int d, total_kv;
};
hipError_t launch_codec_decode(const CodecDecodeArgs& a, bool sep, int heads, int grid_x,
                               hipStream_t stream);
// O_h <- E_h O_h in place for rows [rows][d] (shared-mode decoded memory).
hipError_t launch_codec_rotate_out(const CodecBook& cb, void* O, int rows, int d, int heads,
                                   int grid_x, hipStream_t stream);
// qw query waves (2, 4 or 8) share each reconstructed tile: tile_m = 32 qw.
hipError_t launch_codec_attn(const CodecArgs& a, bool sep, int qw, int64_t items,
                             hipStream_t stream);
// Short-memory kernel over a coded memory (short_bf16.hip): memories of up
// to short_max_rows(true) rows are decoded once per work-group into LDS
// (keys in the rotated basis, values rotated back); a.Wq is W_Q folded into
// the keys' basis, the plan comes from the workspace (a.inplan = 0).
struct ShortCodec {
    CodecBook kb, vb;            // vb unused when the memory is both K and V
    const uint32_t* kcodes;      // [heads][total_kv][budget/32]
    const float* knorms;         // [heads][total_kv]
    const uint32_t* vcodes;
    const float* vnorms;
    int total_kv;
};
hipError_t launch_short_codec_bf16(const AttnArgs& a, const ShortCodec& cd, bool sep, int grid,
                                   hipStream_t stream);

// fp32 path (tile_m = 64): attention over projected queries (cand_len: the
// per-candidate prefix cutoff, or NULL), projection.
hipError_t launch_attn_f32(const float* Qp, const float* K, const float* V, const void* ws,
                           const int* cand_len, int64_t max_tiles, int q, int d, int heads,
                           float* O, hipStream_t stream);

hipError_t launch_project_f32(const float* Z, const float* Wq, int total_cand, int q, int d,
                              float* Q, hipStream_t stream);

// fp32 output gate and projection (same definition, one thread per output).
hipError_t launch_gate_output_f32(const float* Z, const float* Wgo, const float* O,
                                  const float* Wo, int total_cand, int q, int d, float* X,
                                  float* Y, hipStream_t stream);

}  // namespace xattn
