// fp32 path (the full-precision mode: nothing is rounded below fp32): the
// TSP projection and the shared-memory cross-attention over its output.
//
// Same definition as the bf16 path (ReST reading note, s.3.3.1 Eq. (7) with
// the per-slot W_Q of s.3.3.2 Eq. (8); separate K/V as in the TransX report
// s.2).  Projection: one thread per output element.  Attention: one
// work-group of 64 threads per plan work item and head, thread i owning query
// column c0 + i; memory rows stream through LDS in tiles of 32 and each
// thread applies the online-softmax update once per tile.
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
    float scale_log2, float* __restrict__ O) {
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
        float* orow = O + ((size_t)cand * q + s) * d + h * dh;
#pragma unroll
        for (int e = 0; e < DHMAX; ++e)
            if (e < dh) orow[e] = acc[e] * inv;
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
                      int d, int heads, float* O, hipStream_t stream) {
    const int dh = d / heads;
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)dh);
    const int64_t blocks = max_tiles * heads;
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL((attn_f32_kernel<DHMAX>), dim3((unsigned)blocks), dim3(kRows), 0, stream,
                       Qp, K, V, static_cast<const int*>(ws), cand_len, q, d, heads, scale_log2,
                       O);
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
