// TSP query projection on the gfx950 matrix cores, bf16 in, fp32 accumulate,
// bf16 out (ReST reading note, s.3.3.2 Eq. (8) applied to W_Q of s.3.3.1
// Eq. (7): query slot s of every candidate has its own W_Q[s]):
//
//     Q[c][s][o] = sum_i Z[c][s][i] * W_Q[s][o][i]
//
// Each slot is an independent GEMM over all candidates.  A work-group of four
// waves computes a TE (output features) x TC (candidates) tile of Q^T =
// W_Q[s] . Z_s^T, the waves arranged 2 x 2, each holding (TE/64) x (TC/64)
// 32x32 accumulators.  Input features stream through LDS in stages (256 wide
// for small tiles, so that d <= 256 is one memory round trip; 64 wide and
// double-buffered for wide tiles), the next stage's loads in flight during
// the current stage's products.  Operands arrive through bounds-checked
// buffer loads, so rows past the last candidate (or output feature) read as
// zeros and are never stored.
//
// The same launch can carry the varlen planner in one extra work-group
// (blockIdx.x == 0): the plan and the projection are independent, and the
// attention kernel that follows on the stream needs both.
//
// With a gate operand Og the kernel is the output gate of Eq. (7) instead
// (ReST reading note, s.3.3.1; per-slot W_go as in s.3.3.2 Eq. (8)): it
// stores O[c][s][o] * sigmoid(Z[c][s] . W_go[s][o]) rounded to bf16, the
// operand of the output projection, which is this kernel again with one
// slot (W_o shared by all slots).
#include <cstdio>
#include <cstdlib>

#include "internal.h"
#include "plan_device.h"

namespace xattn {

namespace {

// Tile shapes: TE output features x TC candidates, KC input features per LDS
// stage.  Small tiles stage up to 256 input features at once, so a d = 256
// projection costs a single memory round trip per work-group; wide tiles
// (large batches, where many work-groups hide the latency) stage 64.
template <int TE, int TC, int KC>
struct GCfg {
    static constexpr int LDP = KC + 8;   // LDS row pitch (elements, 16-byte aligned rows)
    static constexpr int NBUF = KC >= 256 ? 1 : 2;   // LDS stages (register prefetch either way)
    static constexpr int BE = TE / 64;   // 32-row accumulator blocks per wave along o
    static constexpr int BC = TC / 64;   // ... along candidates
    static constexpr int A_ELEMS = TE * LDP;
    static constexpr int B_ELEMS = TC * LDP;
    static constexpr int STAGE = A_ELEMS + B_ELEMS;
    static constexpr int BYTES = NBUF * STAGE * 2;
    static constexpr int A_CPT = TE * (KC / 8) / 256;   // 16-byte chunks per thread per stage
    static constexpr int B_CPT = TC * (KC / 8) / 256;
    static constexpr int SMEM = BYTES > (int)sizeof(PlanSmem) ? BYTES : (int)sizeof(PlanSmem);
};

struct PlanArgs {
    const int* cu_kv;
    const int* cu_cand;
    int* ws;
    int64_t max_tiles;
    int R, tile_m, total_kv;
    int enabled;
    PrepExtra ex;   // backward-pass side jobs (memory planner, W transpose)
    int tr_blocks;  // work-groups of the transpose job
};

// Side jobs of the backward pass's projection launch: the memory-tile plan
// (the planner with memory and candidates exchanged, tiles of 64 rows) and
// W_Q transposed for dZ.
__device__ void prep_side_jobs(const PlanArgs& pa, int job, int total_cand, int q, int d,
                               char* smem) {
    const PrepExtra& ex = pa.ex;
    if (job == 0) {
        run_plan<256>(pa.cu_cand, pa.cu_kv, pa.R, 1, 64, pa.total_kv, total_cand, ex.kws,
                      ex.max_ktiles, nullptr, nullptr, nullptr, nullptr,
                      *reinterpret_cast<PlanSmem*>(smem));
        return;
    }
    // transpose tile (job - 1): wT[s][i][o] = wt[s][o][i], 32 x 32 per work-group
    const int t = job - 1, tpd = (d + 31) / 32;
    const int s = t / (tpd * tpd), rem = t - s * tpd * tpd;
    const int o0 = (rem / tpd) * 32, i0 = (rem % tpd) * 32;
    bf16 (*tileb)[33] = reinterpret_cast<bf16 (*)[33]>(smem);
    const bf16* src = static_cast<const bf16*>(ex.wsrc) + (size_t)s * d * d;
    bf16* dst = static_cast<bf16*>(ex.wdst) + (size_t)s * d * d;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8
    for (int y = ty; y < 32; y += 8) {
        const int o = o0 + y, i = i0 + tx;
        if (o < d && i < d) tileb[y][tx] = src[(size_t)o * d + i];
    }
    __syncthreads();
    for (int y = ty; y < 32; y += 8) {
        const int i = i0 + y, o = o0 + tx;
        if (o < d && i < d) dst[(size_t)i * d + o] = tileb[tx][y];
    }
}

__device__ __forceinline__ uint32_t clamp_bytes(size_t b) {
    return b > 0xFFFFFFF0u ? 0xFFFFFFF0u : (uint32_t)b;
}

template <int TE, int TC, int KC>
__global__ __launch_bounds__(256) void prep_kernel(const bf16* __restrict__ Z,
                                                   const bf16* __restrict__ Wq, int total_cand,
                                                   int q, int d, bf16* __restrict__ Q,
                                                   int tiles_e, int tiles_c, PlanArgs pa,
                                                   const bf16* __restrict__ Og, float oscale) {
    using C = GCfg<TE, TC, KC>;
    constexpr int LDP = C::LDP;
    __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
    int bid = blockIdx.x;
    if (pa.enabled) {
        if (bid == 0) {
            run_plan<256>(pa.cu_kv, pa.cu_cand, pa.R, q, pa.tile_m, total_cand, pa.total_kv, pa.ws,
                          pa.max_tiles, nullptr, nullptr, nullptr, nullptr,
                          *reinterpret_cast<PlanSmem*>(smem));
            return;
        }
        --bid;
    }
    if (pa.ex.kws) {   // side jobs of the backward pass
        if (bid < 1 + pa.tr_blocks) {
            prep_side_jobs(pa, bid, total_cand, q, d, smem);
            return;
        }
        bid -= 1 + pa.tr_blocks;
    }
    // Work-groups are dealt to the 8 XCDs (each with its own L2) in turn, so
    // tile number n runs on XCD n % 8.  Remap so that tiles adjacent in
    // (slot, candidate tile, output-feature tile) order - which read the same
    // query tokens - run on the same XCD: logical tile = x * per + y for
    // physical n = y * 8 + x (the last partial round keeps its order).
    const int per_slot = tiles_e * tiles_c;
    {
        const int nb = q * per_slot;
        const int per = nb / 8;
        if (bid < 8 * per) bid = (bid % 8) * per + bid / 8;
    }
    const int s = bid / per_slot;
    const int rem = bid - s * per_slot;
    const int tc = rem / tiles_e, te = rem - tc * tiles_e;
    const int e0 = te * TE, c0 = tc * TC;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = w >> 1, wc = w & 1;
    const int g = lane >> 5, l32 = lane & 31;

    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(Wq + ((size_t)s * d + e0) * d), (short)0,
        clamp_bytes((size_t)(d - e0) * d * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(Z + ((size_t)c0 * q + s) * d), (short)0,
        clamp_bytes(((size_t)(total_cand - c0) * q - s) * d * 2), 0x00020000);

    bf16* lds = reinterpret_cast<bf16*>(smem);
    uint4 areg[C::A_CPT], breg[C::B_CPT];
    auto gload = [&](int k0) {
#pragma unroll
        for (int u = 0; u < C::A_CPT; ++u) {
            const int i = tid + u * 256, row = i / (KC / 8), col = i % (KC / 8);
            areg[u] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, (row * d + k0 + col * 8) * 2, 0, 0));
        }
#pragma unroll
        for (int u = 0; u < C::B_CPT; ++u) {
            const int i = tid + u * 256, row = i / (KC / 8), col = i % (KC / 8);
            breg[u] = __builtin_bit_cast(
                uint4,
                __builtin_amdgcn_raw_buffer_load_b128(rz, (row * q * d + k0 + col * 8) * 2, 0, 0));
        }
    };
    auto lstore = [&](int buf) {
        bf16* a = lds + buf * C::STAGE;
        bf16* b = a + C::A_ELEMS;
#pragma unroll
        for (int u = 0; u < C::A_CPT; ++u) {
            const int i = tid + u * 256, row = i / (KC / 8), col = i % (KC / 8);
            *reinterpret_cast<uint4*>(a + row * LDP + col * 8) = areg[u];
        }
#pragma unroll
        for (int u = 0; u < C::B_CPT; ++u) {
            const int i = tid + u * 256, row = i / (KC / 8), col = i % (KC / 8);
            *reinterpret_cast<uint4*>(b + row * LDP + col * 8) = breg[u];
        }
    };

    f32x16 acc[C::BE][C::BC];
#pragma unroll
    for (int i = 0; i < C::BE; ++i)
#pragma unroll
        for (int j = 0; j < C::BC; ++j) acc[i][j] = f32x16{};

    // d is a multiple of 32: the last stage may be partly empty (its columns
    // past d are loaded but never multiplied)
    const int nk = (d + KC - 1) / KC;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kc = 0; kc < nk; ++kc) {
        const int buf = C::NBUF == 2 ? (kc & 1) : 0;
        if (kc + 1 < nk) gload((kc + 1) * KC);
        const bf16* a = lds + buf * C::STAGE;
        const bf16* b = a + C::A_ELEMS;
        const int ksteps = min(KC, d - kc * KC) / 16;
        for (int kk = 0; kk < ksteps; ++kk) {
            bf16x8 af[C::BE], bfr[C::BC];
#pragma unroll
            for (int i = 0; i < C::BE; ++i)
                af[i] = *reinterpret_cast<const bf16x8*>(
                    a + (wr * (TE / 2) + i * 32 + l32) * LDP + kk * 16 + 8 * g);
#pragma unroll
            for (int j = 0; j < C::BC; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8*>(
                    b + (wc * (TC / 2) + j * 32 + l32) * LDP + kk * 16 + 8 * g);
#pragma unroll
            for (int i = 0; i < C::BE; ++i)
#pragma unroll
                for (int j = 0; j < C::BC; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
        }
        if (kc + 1 < nk) {
            if constexpr (C::NBUF == 1) __syncthreads();   // stage fully consumed
            lstore(C::NBUF == 2 ? buf ^ 1 : 0);
        }
        __syncthreads();
    }

    // accumulator (i, j) reg 4*b4 + t holds o = e0 + wr*TE/2 + 32i + 8*b4 + 4g + t
    // for candidate c0 + wc*TC/2 + 32j + l32.  Runs b4 = 2bp and 2bp + 1 are
    // exchanged between the lane halves (join_runs / split_runs, common.h),
    // so that each lane stores (and, gated, loads) 16 bytes: features
    // 16bp + 8g .. +7 of the 32-wide block.  Both halves of a pair hold the
    // same candidate, so they skip (c past the batch) together.
#pragma unroll
    for (int j = 0; j < C::BC; ++j) {
        const int c = c0 + wc * (TC / 2) + j * 32 + l32;
        if (c >= total_cand) continue;
        bf16* qrow = Q + ((size_t)c * q + s) * d;
#pragma unroll
        for (int i = 0; i < C::BE; ++i)
#pragma unroll
            for (int bp = 0; bp < 2; ++bp) {
                const int o0 = e0 + wr * (TE / 2) + i * 32 + 16 * bp;   // the pair's first feature
                const int o = o0 + 8 * g;                                 // this lane's run
                bf16x4 v[2];
                if (Og) {
                    u32x2 og[2] = {u32x2{0u, 0u}, u32x2{0u, 0u}};
                    if (o0 < d) {
                        const u32x4 ol = o < d ? *reinterpret_cast<const u32x4*>(Og + ((size_t)c * q + s) * d + o)
                                               : u32x4{0u, 0u, 0u, 0u};
                        split_runs(ol, og[0], og[1]);
                    }
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const bf16x4 ov = __builtin_bit_cast(bf16x4, og[h2]);
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            const float e = __builtin_amdgcn_exp2f(-acc[i][j][8 * bp + 4 * h2 + t] *
                                                                   1.4426950408889634f);
                            v[h2][t] = (bf16)((float)ov[t] * __builtin_amdgcn_rcpf(1.0f + e));
                        }
                    }
                } else if (oscale == 1.0f) {
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                        for (int t = 0; t < 4; ++t) v[h2][t] = (bf16)acc[i][j][8 * bp + 4 * h2 + t];
                } else {
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            v[h2][t] = (bf16)((float)(bf16)acc[i][j][8 * bp + 4 * h2 + t] * oscale);
                }
                const u32x4 out = join_runs(v[0], v[1]);
                if (o < d) *reinterpret_cast<u32x4*>(qrow + o) = out;
            }
    }
}

template <int TE, int TC, int KC>
hipError_t launch_prep(const void* Z, const void* Wq, int total_cand, int q, int d, void* Q,
                       const PlanArgs& pa, hipStream_t stream, const void* Og, float oscale) {
    const int tiles_e = (d + TE - 1) / TE;
    const int tiles_c = (total_cand + TC - 1) / TC;
    const int64_t blocks = (int64_t)q * tiles_e * tiles_c + (pa.enabled ? 1 : 0) +
                           (pa.ex.kws ? 1 + pa.tr_blocks : 0);
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL((prep_kernel<TE, TC, KC>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const bf16*>(Z), static_cast<const bf16*>(Wq), total_cand, q, d,
                       static_cast<bf16*>(Q), tiles_e, tiles_c, pa,
                       static_cast<const bf16*>(Og), oscale);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_project_plan_bf16(const void* Z, const void* Wq, int total_cand, int q, int d,
                                    void* Q, const int* cu_kv, const int* cu_cand, int R,
                                    int tile_m, int total_kv, void* ws, int64_t max_tiles,
                                    hipStream_t stream, const void* Og, float oscale,
                                    const PrepExtra* ex, const Tuning* tune) {
    PlanArgs pa{cu_kv, cu_cand, static_cast<int*>(ws), max_tiles, R, tile_m, total_kv,
                ws != nullptr ? 1 : 0, ex ? *ex : PrepExtra{}, 0};
    if (ex) {
        const int tpd = (d + 31) / 32;
        pa.tr_blocks = q * tpd * tpd;
    }
    if (total_cand <= 0 && !pa.enabled) return hipSuccess;
    // the context's tile-shape override (tuning), if it names a built shape
    if (tune && tune->gemm_te > 0) {
        const int te = tune->gemm_te, tc = tune->gemm_tc, kc = tune->gemm_kc;
        {
#define XATTN_GEMM_CASE(A_, B_, C_) \
    if (te == A_ && tc == B_ && kc == C_) return launch_prep<A_, B_, C_>(Z, Wq, total_cand, q, d, Q, pa, stream, Og, oscale);
            XATTN_GEMM_CASE(128, 128, 64)
            XATTN_GEMM_CASE(64, 64, 256)
            XATTN_GEMM_CASE(128, 128, 32)
            XATTN_GEMM_CASE(128, 64, 64)
            XATTN_GEMM_CASE(64, 128, 64)
            XATTN_GEMM_CASE(256, 64, 32)
            XATTN_GEMM_CASE(64, 64, 64)
#undef XATTN_GEMM_CASE
        }
    }
    // wide tiles when they still give at least two work-groups per compute
    // unit; else 64 x 64 tiles, with the whole reduction in one LDS stage up
    // to d = 256 and in 64-wide stages beyond (d = 512: 67.6 KB of staging
    // allowed two work-groups per CU for 1.5 rounds of them; 64-wide stages
    // take 18 KB: projection 11.05 -> 9.4 us on the long history)
    const int64_t big = (int64_t)q * ((d + 127) / 128) * ((total_cand + 127) / 128);
    if (big >= 512) return launch_prep<128, 128, 64>(Z, Wq, total_cand, q, d, Q, pa, stream, Og, oscale);
    if (d > 256) return launch_prep<64, 64, 64>(Z, Wq, total_cand, q, d, Q, pa, stream, Og, oscale);
    return launch_prep<64, 64, 256>(Z, Wq, total_cand, q, d, Q, pa, stream, Og, oscale);
}

hipError_t launch_gate_output_bf16(const void* Z, const void* Wgo, const void* O, const void* Wo,
                                   int total_cand, int q, int d, void* X, void* Y,
                                   hipStream_t stream, const Tuning* tune) {
    hipError_t e = launch_project_plan_bf16(Z, Wgo, total_cand, q, d, X, nullptr, nullptr, 0, 0, 0,
                                            nullptr, 0, stream, O, 1.0f, nullptr, tune);
    if (e != hipSuccess) return e;
    return launch_project_plan_bf16(X, Wo, total_cand * q, 1, d, Y, nullptr, nullptr, 0, 0, 0,
                                    nullptr, 0, stream, nullptr, 1.0f, nullptr, tune);
}

}  // namespace xattn
