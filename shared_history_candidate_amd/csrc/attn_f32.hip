// fp32 path (the full-precision mode: nothing is rounded below fp32): the
// TSP projection and the shared-memory cross-attention over its output.
//
// Same definition as the bf16 path (ReST reading note, s.3.3.1 Eq. (7) with
// the per-slot W_Q of s.3.3.2 Eq. (8); separate K/V as in the TransX report
// s.2).  Projection: one thread per output element.  Attention: one
// work-group of 64 threads per plan work item and head, thread i owning query
// column c0 + i; memory rows stream through LDS in tiles of 32 and each
// thread applies the online-softmax update once per tile.
#include <climits>

#include "common.h"
#include "internal.h"

namespace xattn {

namespace {

constexpr int kRows = 64;  // candidates per work item (tile_m of the fp32 path)
constexpr int kBN = 32;    // memory rows per tile

template <int DHMAX>
__global__ __launch_bounds__(kRows) void attn_f32_kernel(
    const float* __restrict__ Qp, const float* __restrict__ K, const float* __restrict__ V,
    const int* __restrict__ ws, const int* __restrict__ cand_len, int q, int d, int heads,
    float scale_log2, float* __restrict__ O, const float* __restrict__ dO,
    float* __restrict__ lse, float* __restrict__ Dsum) {
    __shared__ float ks[kBN][DHMAX];
    __shared__ float vs[kBN][DHMAX];
    const int dh = d / heads;
    const int n_tiles = ws[kPlanNTiles];
    const int tile = blockIdx.x / heads;
    const int h = blockIdx.x - tile * heads;
    if (tile >= n_tiles || ws[kPlanTileM] != kRows) return;
    const int4 item = reinterpret_cast<const int4*>(
        reinterpret_cast<const char*>(ws) + kPlanHeaderBytes)[tile];
    const int kv0 = item.x, L = item.y, c0 = item.z;
    const int nc = item.w & kItemNcMask, s = item.w >> 16;
    const int i = threadIdx.x;
    const bool valid = i < nc;
    const int cand = c0 + i;
    // per-candidate prefix cutoff: this row sees memory rows [0, Lc)
    int Lc = L;
    if (cand_len && valid) {
        const int want = cand_len[cand];
        Lc = want < 0 ? 0 : (want < L ? want : L);
    }

    // this thread's projected query (head slice)
    float qv[DHMAX];
    {
        const float* qrow = Qp + ((size_t)(valid ? cand : c0) * q + s) * d + h * dh;
#pragma unroll
        for (int e = 0; e < DHMAX; ++e) qv[e] = e < dh ? qrow[e] : 0.f;
    }

    float acc[DHMAX];
#pragma unroll
    for (int e = 0; e < DHMAX; ++e) acc[e] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    const float* Vm = V ? V : K;

    for (int j0 = 0; j0 < L; j0 += kBN) {
        const int nj = min(kBN, L - j0);
        __syncthreads();
        for (int idx = i; idx < kBN * DHMAX; idx += kRows) {
            const int j = idx / DHMAX, e = idx % DHMAX;
            const bool ok = j < nj && e < dh;
            const size_t off = (size_t)(kv0 + j0 + j) * d + h * dh + e;
            ks[j][e] = ok ? K[off] : 0.f;
            vs[j][e] = ok ? Vm[off] : 0.f;
        }
        __syncthreads();
        float sc[kBN];
        float mt = -INFINITY;
#pragma unroll
        for (int j = 0; j < kBN; ++j) {
            float a = 0.f;
#pragma unroll
            for (int e = 0; e < DHMAX; ++e) a = fmaf(qv[e], ks[j][e], a);
            sc[j] = (j < nj && j0 + j < Lc) ? a : -INFINITY;
            mt = fmaxf(mt, sc[j]);
        }
        const float m_new = fmaxf(m_run, mt);
        if (m_new == -INFINITY) continue;   // no visible row yet
        const float alpha = exp2f((m_run - m_new) * scale_log2);
        const float mb = m_new * scale_log2;
        l_run *= alpha;
#pragma unroll
        for (int e = 0; e < DHMAX; ++e) acc[e] *= alpha;
#pragma unroll
        for (int j = 0; j < kBN; ++j) {
            const float p = exp2f(fmaf(sc[j], scale_log2, -mb));
            l_run += p;
#pragma unroll
            for (int e = 0; e < DHMAX; ++e) acc[e] = fmaf(p, vs[j][e], acc[e]);
        }
        m_run = m_new;
    }

    if (valid) {
        const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
        const size_t rbase = ((size_t)cand * q + s) * d + h * dh;
        if (O) {
#pragma unroll
            for (int e = 0; e < DHMAX; ++e)
                if (e < dh) O[rbase + e] = acc[e] * inv;
        }
        if (lse) {
            // backward statistics: log2 normaliser in scaled units, <dO, O>
            const size_t idx = ((size_t)cand * q + s) * heads + h;
            lse[idx] = l_run > 0.f ? m_run * scale_log2 + log2f(l_run) : -INFINITY;
            float dsum = 0.f;
#pragma unroll
            for (int e = 0; e < DHMAX; ++e)
                if (e < dh) dsum = fmaf(acc[e] * inv, dO[rbase + e], dsum);
            Dsum[idx] = dsum;
        }
    }
}

__global__ void project_f32_kernel(const float* __restrict__ Z, const float* __restrict__ Wq,
                                   int64_t n, int q, int d, float* __restrict__ Q) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= n) return;
    const int64_t row = idx / d;
    const int o = (int)(idx - row * d);
    const int s = (int)(row % q);
    const float* zrow = Z + (size_t)row * d;
    const float* w = Wq + ((size_t)s * d + o) * d;
    float a = 0.f;
    for (int k = 0; k < d; ++k) a = fmaf(zrow[k], w[k], a);
    Q[idx] = a;
}

// Output gate of Eq. (7) in fp32: X[row][o] = O[row][o] * sigmoid(Z[row] . W_go[row % q][o]).
__global__ void gate_f32_kernel(const float* __restrict__ Z, const float* __restrict__ Wgo,
                                const float* __restrict__ O, int64_t n, int q, int d,
                                float* __restrict__ X) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= n) return;
    const int64_t row = idx / d;
    const int o = (int)(idx - row * d);
    const float* zrow = Z + (size_t)row * d;
    const float* w = Wgo + ((size_t)(row % q) * d + o) * d;
    float a = 0.f;
    for (int k = 0; k < d; ++k) a = fmaf(zrow[k], w[k], a);
    X[idx] = O[idx] / (1.0f + expf(-a));
}

template <int DHMAX>
hipError_t launch_f32(const float* Qp, const float* K, const float* V,
                      const void* ws, const int* cand_len, int64_t max_tiles, int q,
                      int d, int heads, float* O, hipStream_t stream,
                      const float* dO = nullptr, float* lse = nullptr, float* Dsum = nullptr) {
    const int dh = d / heads;
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)dh);
    const int64_t blocks = max_tiles * heads;
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL((attn_f32_kernel<DHMAX>), dim3((unsigned)blocks), dim3(kRows), 0, stream,
                       Qp, K, V, static_cast<const int*>(ws), cand_len, q, d, heads, scale_log2,
                       O, dO, lse, Dsum);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Backward pass in fp32 (same definitions as bwd_bf16.hip, scalar arithmetic).
// dQ: one thread per query row of a plan item (64 rows), memory rows through
// LDS in tiles of 32.  dK/dV: one thread per memory row of a memory-tile item
// (64 rows), the request's query rows through LDS in tiles of 32.
// ---------------------------------------------------------------------------
template <int DHMAX>
__global__ __launch_bounds__(kRows) void bwd_dq_f32_kernel(BwdArgs a) {
    __shared__ float ks[kBN][DHMAX];
    __shared__ float vs[kBN][DHMAX];
    const int q = a.q, d = a.d, heads = a.heads, dh = d / heads;
    const float scale_log2 = 1.4426950408889634f * a.scale;
    const int tile = blockIdx.x / heads;
    const int h = blockIdx.x - tile * heads;
    if (tile >= a.plan[kPlanNTiles] || a.plan[kPlanTileM] != kRows) return;
    const int4 item = reinterpret_cast<const int4*>(
        reinterpret_cast<const char*>(a.plan) + kPlanHeaderBytes)[tile];
    const int kv0 = item.x, L = item.y, c0 = item.z;
    const int nc = item.w & kItemNcMask, s = item.w >> 16;
    const int i = threadIdx.x;
    const bool valid = i < nc;
    const size_t row = (size_t)(valid ? c0 + i : c0) * q + s;
    const float* Qp = static_cast<const float*>(a.Qs);
    const float* dO = static_cast<const float*>(a.dO);
    const float* K = static_cast<const float*>(a.K);
    const float* V = a.V ? static_cast<const float*>(a.V) : K;
    float qv[DHMAX], dov[DHMAX], dq[DHMAX];
#pragma unroll
    for (int e = 0; e < DHMAX; ++e) {
        qv[e] = e < dh ? Qp[row * d + h * dh + e] : 0.f;
        dov[e] = e < dh ? dO[row * d + h * dh + e] : 0.f;
        dq[e] = 0.f;
    }
    const float lse = a.lse[row * heads + h], Dr = a.Dsum[row * heads + h];
    // visible memory rows of this thread's candidate (prefix cutoff)
    const int Lc = a.vis && valid ? a.vis[c0 + i] - kv0 : L;
    for (int j0 = 0; j0 < L; j0 += kBN) {
        const int nj = min(kBN, L - j0);
        __syncthreads();
        for (int idx = i; idx < kBN * DHMAX; idx += kRows) {
            const int j = idx / DHMAX, e = idx % DHMAX;
            const bool ok = j < nj && e < dh;
            const size_t off = (size_t)(kv0 + j0 + j) * d + h * dh + e;
            ks[j][e] = ok ? K[off] : 0.f;
            vs[j][e] = ok ? V[off] : 0.f;
        }
        __syncthreads();
        for (int j = 0; j < nj; ++j) {
            if (j0 + j >= Lc) break;
            float sc = 0.f, dp = 0.f;
#pragma unroll
            for (int e = 0; e < DHMAX; ++e) {
                sc = fmaf(qv[e], ks[j][e], sc);
                dp = fmaf(dov[e], vs[j][e], dp);
            }
            const float ds = exp2f(fmaf(sc, scale_log2, -lse)) * (dp - Dr);
#pragma unroll
            for (int e = 0; e < DHMAX; ++e) dq[e] = fmaf(ds, ks[j][e], dq[e]);
        }
    }
    if (valid) {
        float* out = static_cast<float*>(a.dQ) + row * d + h * dh;
#pragma unroll
        for (int e = 0; e < DHMAX; ++e)
            if (e < dh) out[e] = dq[e] * a.scale;
    }
}

template <int DHMAX>
__global__ __launch_bounds__(kRows) void bwd_dkv_f32_kernel(BwdArgs a) {
    __shared__ float qs[kBN][DHMAX];
    __shared__ float ds_[kBN][DHMAX];
    __shared__ float ls[kBN], Ds[kBN];
    __shared__ int vis_[kBN];
    const int q = a.q, d = a.d, heads = a.heads, dh = d / heads;
    const float scale_log2 = 1.4426950408889634f * a.scale;
    const int tile = blockIdx.x / heads;
    const int h = blockIdx.x - tile * heads;
    if (tile >= a.kplan[kPlanNTiles] || a.kplan[kPlanTileM] != kRows) return;
    // memory-tile item: {first candidate, candidates, first memory row, rows}
    const int4 item = reinterpret_cast<const int4*>(
        reinterpret_cast<const char*>(a.kplan) + kPlanHeaderBytes)[tile];
    const int c_lo = item.x, N = item.y, key0 = item.z, nk = item.w & kItemNcMask;
    const int j = threadIdx.x;
    const bool valid = j < nk;
    const size_t key = (size_t)key0 + (valid ? j : 0);
    const float* Qp = static_cast<const float*>(a.Qs);
    const float* dO = static_cast<const float*>(a.dO);
    const float* K = static_cast<const float*>(a.K);
    const float* V = a.V ? static_cast<const float*>(a.V) : K;
    float kv[DHMAX], vv[DHMAX], dk[DHMAX], dv[DHMAX];
#pragma unroll
    for (int e = 0; e < DHMAX; ++e) {
        kv[e] = e < dh ? K[key * d + h * dh + e] : 0.f;
        vv[e] = e < dh ? V[key * d + h * dh + e] : 0.f;
        dk[e] = 0.f;
        dv[e] = 0.f;
    }
    const int row0 = c_lo * q, M = N * q;
    for (int i0 = 0; i0 < M; i0 += kBN) {
        const int ni = min(kBN, M - i0);
        __syncthreads();
        for (int idx = j; idx < kBN * DHMAX; idx += kRows) {
            const int i = idx / DHMAX, e = idx % DHMAX;
            const bool ok = i < ni && e < dh;
            const size_t off = (size_t)(row0 + i0 + i) * d + h * dh + e;
            qs[i][e] = ok ? Qp[off] : 0.f;
            ds_[i][e] = ok ? dO[off] : 0.f;
        }
        if (j < ni) {
            ls[j] = a.lse[(size_t)(row0 + i0 + j) * heads + h];
            Ds[j] = a.Dsum[(size_t)(row0 + i0 + j) * heads + h];
            vis_[j] = a.vis ? a.vis[(row0 + i0 + j) / q] : INT_MAX;
        }
        __syncthreads();
        for (int i = 0; i < ni; ++i) {
            if ((int)key >= vis_[i]) continue;   // the row does not see this memory row
            float sc = 0.f, dp = 0.f;
#pragma unroll
            for (int e = 0; e < DHMAX; ++e) {
                sc = fmaf(qs[i][e], kv[e], sc);
                dp = fmaf(ds_[i][e], vv[e], dp);
            }
            const float p = exp2f(fmaf(sc, scale_log2, -ls[i]));
            const float g = p * (dp - Ds[i]);
#pragma unroll
            for (int e = 0; e < DHMAX; ++e) {
                dv[e] = fmaf(p, ds_[i][e], dv[e]);
                dk[e] = fmaf(g, qs[i][e], dk[e]);
            }
        }
    }
    if (valid) {
        float* ko = static_cast<float*>(a.dK) + key * d + h * dh;
        float* vo = a.V ? static_cast<float*>(a.dV) + key * d + h * dh : nullptr;
#pragma unroll
        for (int e = 0; e < DHMAX; ++e)
            if (e < dh) {
                if (vo) {
                    ko[e] = dk[e] * a.scale;
                    vo[e] = dv[e];
                } else {
                    ko[e] = dk[e] * a.scale + dv[e];
                }
            }
    }
}

// dW[s][o][i] = sum over candidates c of dQ[c*q+s][o] Z[c*q+s][i], one thread
// per output element, candidates in order.
__global__ void bwd_dw_f32_kernel(const float* __restrict__ dQ, const float* __restrict__ Z,
                                  int total_cand, int q, int d, float* __restrict__ dW) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)q * d * d) return;
    const int i = (int)(idx % d);
    const int o = (int)((idx / d) % d);
    const int s = (int)(idx / ((int64_t)d * d));
    float acc = 0.f;
    for (int c = 0; c < total_cand; ++c) {
        const size_t r = ((size_t)c * q + s) * d;
        acc = fmaf(dQ[r + o], Z[r + i], acc);
    }
    dW[idx] = acc;
}

template <int DHMAX>
hipError_t launch_bwd_f32_dh(const BwdArgs& a, int64_t q_items, int64_t k_items,
                             hipStream_t stream) {
    if (q_items > 0)
        hipLaunchKernelGGL((bwd_dq_f32_kernel<DHMAX>), dim3((unsigned)(q_items * a.heads)),
                           dim3(kRows), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (k_items > 0)
        hipLaunchKernelGGL((bwd_dkv_f32_kernel<DHMAX>), dim3((unsigned)(k_items * a.heads)),
                           dim3(kRows), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(const float* Qp, const float* K, const float* V,
                           const void* ws, const int* cand_len, int64_t max_tiles, int q,
                           int d, int heads, float* O, hipStream_t stream) {
    const int dh = d / heads;
    if (dh <= 8) return launch_f32<8>(Qp, K, V, ws, cand_len, max_tiles, q, d, heads, O, stream);
    if (dh <= 16) return launch_f32<16>(Qp, K, V, ws, cand_len, max_tiles, q, d, heads, O, stream);
    if (dh <= 32) return launch_f32<32>(Qp, K, V, ws, cand_len, max_tiles, q, d, heads, O, stream);
    if (dh <= 64) return launch_f32<64>(Qp, K, V, ws, cand_len, max_tiles, q, d, heads, O, stream);
    if (dh <= 128) return launch_f32<128>(Qp, K, V, ws, cand_len, max_tiles, q, d, heads, O, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_attn_f32_stats(const float* Qp, const float* K, const float* V, const void* ws,
                                 const int* cand_len, int64_t max_tiles, int q, int d, int heads,
                                 const float* dO, float* lse, float* Dsum, hipStream_t stream) {
    const int dh = d / heads;
#define XATTN_F32S(N_) \
    if (dh <= N_) return launch_f32<N_>(Qp, K, V, ws, cand_len, max_tiles, q, d, heads, nullptr, stream, dO, lse, Dsum);
    XATTN_F32S(8)
    XATTN_F32S(16)
    XATTN_F32S(32)
    XATTN_F32S(64)
    XATTN_F32S(128)
#undef XATTN_F32S
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_attn_f32(const BwdArgs& a, bool sep, int64_t q_items, int64_t k_items,
                               hipStream_t stream) {
    (void)sep;   // V == NULL selects the projection-free reading
    const int dh = a.d / a.heads;
    if (dh <= 8) return launch_bwd_f32_dh<8>(a, q_items, k_items, stream);
    if (dh <= 16) return launch_bwd_f32_dh<16>(a, q_items, k_items, stream);
    if (dh <= 32) return launch_bwd_f32_dh<32>(a, q_items, k_items, stream);
    if (dh <= 64) return launch_bwd_f32_dh<64>(a, q_items, k_items, stream);
    if (dh <= 128) return launch_bwd_f32_dh<128>(a, q_items, k_items, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_dw_f32(const float* dQ, const float* Z, int total_cand, int q, int d,
                             float* dW, hipStream_t stream) {
    const int64_t n = (int64_t)q * d * d;
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(bwd_dw_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       dQ, Z, total_cand, q, d, dW);
    return hipGetLastError();
}

hipError_t launch_project_f32(const float* Z, const float* Wq, int total_cand, int q, int d,
                              float* Q, hipStream_t stream) {
    const int64_t n = (int64_t)total_cand * q * d;
    if (n <= 0) return hipSuccess;
    const int threads = 256;
    hipLaunchKernelGGL(project_f32_kernel, dim3((unsigned)((n + threads - 1) / threads)),
                       dim3(threads), 0, stream, Z, Wq, n, q, d, Q);
    return hipGetLastError();
}

hipError_t launch_gate_output_f32(const float* Z, const float* Wgo, const float* O,
                                  const float* Wo, int total_cand, int q, int d, float* X,
                                  float* Y, hipStream_t stream) {
    const int64_t n = (int64_t)total_cand * q * d;
    if (n <= 0) return hipSuccess;
    const int threads = 256;
    hipLaunchKernelGGL(gate_f32_kernel, dim3((unsigned)((n + threads - 1) / threads)),
                       dim3(threads), 0, stream, Z, Wgo, O, n, q, d, X);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_project_f32(X, Wo, total_cand * q, 1, d, Y, stream);
}

}  // namespace xattn
