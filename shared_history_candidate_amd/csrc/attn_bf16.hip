// Fused TSP query projection + shared-memory cross-attention, bf16 in, fp32
// accumulate, bf16 out, for gfx950 matrix cores.
//
// Computes, for every work item {r, s, c0, nc} of the plan and every head h,
//   Q_h   = Z[c, s, :] . W_Q[s][h*d_h:(h+1)*d_h, :]^T   (ReST reading note,
//           s.3.3.2 Eq. (8): slot s has its own W_Q[s])
//   O_h   = softmax(Q_h K_h^T / sqrt(d_h)) V_h          (s.3.3.1 Eq. (7);
//           K = V = H in projection-free mode, separate K, V for the TransX
//           behaviour memory, TransX report s.2)
// for the nc candidates c in [c0, c0+nc) of request r.  All candidates of a
// request stream the same memory rows (shared-prefix serving, ReST reading
// note s.3.5).
//
// Work decomposition.  One work-group handles one work item and one head with
// `WAVES` waves; wave w owns query columns c0 + 32w .. c0 + 32w + 31.  The
// product is computed transposed, S^T = K Q^T, so that each lane holds one
// query row's scores and the softmax reductions along the key axis stay
// inside a lane (plus one exchange between the two 32-lane halves):
//   projection  Q_h^T (d_h x 32)  = W_h (d_h x d)   . Z^T (d x 32)
//   scores      S^T   (32 x 32)   = K_tile (32 x d_h) . Q_h^T
//   output      O^T   (d_h x 32) += V_tile^T (d_h x 32) . P^T (32 x 32)
// The memory is streamed in tiles of 32 rows through double-buffered LDS
// (one buffer serves as both K and V in projection-free mode).  V^T operands
// are read from the row-major tile with LDS transpose reads.  The scores'
// k-index (feature e) and the PV k-index (memory row j) follow the
// accumulator layout of the previous product, so Q and P go from
// accumulators to operands without any data movement.
#include "common.h"
#include "internal.h"

namespace xattn {

namespace {

constexpr int BN = 32;  // memory rows per tile

// One 32(e) x 32(query) block of Q^T for the lane's query row:
//   acc[reg r] = sum_i W[s][erow0 + (r/4)*8 + 4*g + r%4][i] * Z[cand][s][i].
// wrow points at W[s][erow0 + lane%32][0]; zrow at Z[cand][s][0] (or nullptr
// for an out-of-range query column, which then contributes zeros).
__device__ __forceinline__ void project_acc(const bf16* __restrict__ wrow,
                                            const bf16* __restrict__ zrow, int d, int g,
                                            f32x16& acc) {
    const bf16x8 zero = {};
    for (int k0 = 0; k0 < d; k0 += 16) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(wrow + k0 + 8 * g);
        const bf16x8 b = zrow ? *reinterpret_cast<const bf16x8*>(zrow + k0 + 8 * g) : zero;
        acc = mfma32(a, b, acc);
    }
}

template <int DH, int WAVES, bool SEPARATE>
__global__ __launch_bounds__(64 * WAVES) void attn_bf16_kernel(
    const bf16* __restrict__ Z, const bf16* __restrict__ Wq, const bf16* __restrict__ K,
    const bf16* __restrict__ V, const int* __restrict__ cu_kv, const int* __restrict__ ws,
    int q, int d, int heads, float scale_log2, bf16* __restrict__ O) {
    constexpr int NT = 64 * WAVES;
    constexpr int LDK = DH + 8;             // LDS row pitch (elements)
    constexpr int EB = DH / 32;             // 32-wide feature blocks
    constexpr int KS = DH / 16;             // k-steps of the score product
    constexpr int CHUNKS = BN * DH / 8;     // 16-byte chunks per memory tile
    constexpr int CPT = (CHUNKS + NT - 1) / NT;
    constexpr int NBUF = SEPARATE ? 2 : 1;  // K (and V) planes per stage
    __shared__ __attribute__((aligned(16))) bf16 lds[2][NBUF][BN * LDK];

    const int n_tiles = ws[kPlanNTiles];
    const int tile = blockIdx.x / heads;
    const int h = blockIdx.x - tile * heads;
    // A plan built for another tile size (another batch shape) is not ours.
    if (tile >= n_tiles || ws[kPlanTileM] != 32 * WAVES) return;
    const int4 item = reinterpret_cast<const int4*>(
        reinterpret_cast<const char*>(ws) + kPlanHeaderBytes)[tile];
    const int r = item.x, s = item.y, c0 = item.z, nc = item.w;
    const int kv0 = cu_kv[r];
    const int L = cu_kv[r + 1] - kv0;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 5;         // 32-lane half
    const int l32 = lane & 31;
    const int qcol = wave * 32 + l32;  // query column inside the tile
    const bool qvalid = qcol < nc;
    const int cand = c0 + qcol;

    // ---- 1. projection: Q_h^T for this wave's 32 query columns ----
    bf16x8 qb[KS];
    {
        const bf16* zrow = qvalid ? Z + ((size_t)cand * q + s) * d : nullptr;
#pragma unroll
        for (int eb = 0; eb < EB; ++eb) {
            f32x16 acc = {};
            const bf16* wrow = Wq + ((size_t)s * d + h * DH + eb * 32 + l32) * d;
            project_acc(wrow, zrow, d, g, acc);
            // accumulator reg 8u+t holds feature e = eb*32 + 16u + (t/4)*8 + 4g + t%4,
            // which is exactly k-slot t of score k-step 2*eb+u.
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int t = 0; t < 8; ++t) qb[2 * eb + u][t] = (bf16)acc[8 * u + t];
        }
    }

    // ---- 2. stream the memory rows ----
    f32x16 oacc[EB];
#pragma unroll
    for (int eb = 0; eb < EB; ++eb) oacc[eb] = f32x16{};
    float m_run = -INFINITY;  // running max of raw scores (same in both halves)
    float l_run = 0.f;        // running sum of weights over this half's keys

    const int ntiles_kv = (L + BN - 1) / BN;
    uint4 kreg[CPT];
    uint4 vreg[SEPARATE ? CPT : 1];
    const bf16* Kh = K + (size_t)kv0 * d + h * DH;
    const bf16* Vh = SEPARATE ? V + (size_t)kv0 * d + h * DH : nullptr;

    auto gload = [&](int kt) {
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            const int c = threadIdx.x + u * NT;
            const int j = c / (DH / 8), c8 = c % (DH / 8);
            const int jj = kt * BN + j;
            const bool ok = (c < CHUNKS) && (jj < L);
            const size_t off = (size_t)jj * d + c8 * 8;
            kreg[u] = ok ? *reinterpret_cast<const uint4*>(Kh + off) : make_uint4(0, 0, 0, 0);
            if constexpr (SEPARATE)
                vreg[u] = ok ? *reinterpret_cast<const uint4*>(Vh + off) : make_uint4(0, 0, 0, 0);
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            const int c = threadIdx.x + u * NT;
            if (c < CHUNKS) {
                const int j = c / (DH / 8), c8 = c % (DH / 8);
                *reinterpret_cast<uint4*>(&lds[buf][0][j * LDK + c8 * 8]) = kreg[u];
                if constexpr (SEPARATE)
                    *reinterpret_cast<uint4*>(&lds[buf][NBUF - 1][j * LDK + c8 * 8]) = vreg[u];
            }
        }
    };

    if (ntiles_kv > 0) {
        gload(0);
        lstore(0);
    }
    __syncthreads();

    // Per-lane constants of the transposed V read (see lds_read_tr16): in each
    // 16-lane group G, source lane k addresses row 4*(G/2) + k/4 and column
    // 16*(G%2) + 4*(k%4) of the 16-row slab, so lane l receives
    // V[16u + 4g + t][eb*32 + l%32] for t = 0..3.
    const int G = lane >> 4, k16 = lane & 15;
    const int tr_row = 4 * (G >> 1) + (k16 >> 2);
    const int tr_col = 16 * (G & 1) + 4 * (k16 & 3);

    for (int kt = 0; kt < ntiles_kv; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < ntiles_kv) gload(kt + 1);
        const bf16* kb = lds[buf][0];
        const bf16* vb = lds[buf][NBUF - 1];

        // scores S^T: lane holds query l32, keys j = (r/4)*8 + 4g + r%4
        f32x16 sacc = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int e0 = 32 * (ks >> 1) + 16 * (ks & 1);
            const bf16x4 lo = *reinterpret_cast<const bf16x4*>(kb + l32 * LDK + e0 + 4 * g);
            const bf16x4 hi = *reinterpret_cast<const bf16x4*>(kb + l32 * LDK + e0 + 8 + 4 * g);
            sacc = mfma32(cat(lo, hi), qb[ks], sacc);
        }
        const int jleft = L - kt * BN;  // valid keys in this tile
        if (jleft < BN) {
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int j = (rr >> 2) * 8 + 4 * g + (rr & 3);
                if (j >= jleft) sacc[rr] = -INFINITY;
            }
        }
        float mt = sacc[0];
#pragma unroll
        for (int rr = 1; rr < 16; ++rr) mt = fmaxf(mt, sacc[rr]);
        mt = fmaxf(mt, xor32(mt));
        const float m_new = fmaxf(m_run, mt);
        const float alpha = exp2f((m_run - m_new) * scale_log2);
        const float mb = m_new * scale_log2;
        bf16x8 pb[2];
        float psum = 0.f;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const float p = exp2f(fmaf(sacc[rr], scale_log2, -mb));
            psum += p;
            pb[rr >> 3][rr & 7] = (bf16)p;
        }
        l_run = fmaf(l_run, alpha, psum);
        m_run = m_new;
#pragma unroll
        for (int eb = 0; eb < EB; ++eb) oacc[eb] *= alpha;

        // O^T += V^T P^T over the two 16-key halves of the tile
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
            for (int eb = 0; eb < EB; ++eb) {
                const bf16* base = vb + (16 * u + tr_row) * LDK + eb * 32 + tr_col;
                const bf16x4 lo = lds_read_tr16(base);
                const bf16x4 hi = lds_read_tr16(base + 8 * LDK);
                oacc[eb] = mfma32(cat(lo, hi), pb[u], oacc[eb]);
            }
        }
        if (kt + 1 < ntiles_kv) lstore(buf ^ 1);
        __syncthreads();
    }

    // ---- 3. normalise and store ----
    const float l_tot = l_run + xor32(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (qvalid) {
        bf16* orow = O + ((size_t)cand * q + s) * d + h * DH;
#pragma unroll
        for (int eb = 0; eb < EB; ++eb) {
#pragma unroll
            for (int b4 = 0; b4 < 4; ++b4) {
                bf16x4 v;
#pragma unroll
                for (int t = 0; t < 4; ++t) v[t] = (bf16)(oacc[eb][4 * b4 + t] * inv);
                *reinterpret_cast<bf16x4*>(orow + eb * 32 + b4 * 8 + 4 * g) = v;
            }
        }
    }
}

// Standalone projection: Q[c][s][e] for a 32(e) x 32(cand) block per wave.
template <int WAVES>
__global__ __launch_bounds__(64 * WAVES) void project_bf16_kernel(
    const bf16* __restrict__ Z, const bf16* __restrict__ Wq, int total_cand, int q, int d,
    bf16* __restrict__ Q) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 5, l32 = lane & 31;
    const int cand = (blockIdx.x * WAVES + wave) * 32 + l32;
    const int e0 = blockIdx.y * 32;
    const int s = blockIdx.z;
    const bool valid = cand < total_cand;
    const bf16* zrow = valid ? Z + ((size_t)cand * q + s) * d : nullptr;
    f32x16 acc = {};
    project_acc(Wq + ((size_t)s * d + e0 + l32) * d, zrow, d, g, acc);
    if (valid) {
        bf16* qrow = Q + ((size_t)cand * q + s) * d + e0;
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) {
            bf16x4 v;
#pragma unroll
            for (int t = 0; t < 4; ++t) v[t] = (bf16)acc[4 * b4 + t];
            *reinterpret_cast<bf16x4*>(qrow + b4 * 8 + 4 * g) = v;
        }
    }
}

template <int DH, int WAVES, bool SEP>
hipError_t launch_one(const void* Z, const void* Wq, const void* K, const void* V,
                      const int* cu_kv, const void* ws, int64_t max_tiles, int q, int d,
                      int heads, void* O, hipStream_t stream) {
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)DH);
    const int64_t blocks = max_tiles * heads;
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL((attn_bf16_kernel<DH, WAVES, SEP>), dim3((unsigned)blocks),
                       dim3(64 * WAVES), 0, stream, static_cast<const bf16*>(Z),
                       static_cast<const bf16*>(Wq), static_cast<const bf16*>(K),
                       static_cast<const bf16*>(V), cu_kv, static_cast<const int*>(ws), q, d,
                       heads, scale_log2, static_cast<bf16*>(O));
    return hipGetLastError();
}

template <int DH, int WAVES>
hipError_t launch_dh_w(const void* Z, const void* Wq, const void* K, const void* V,
                       const int* cu_kv, const void* ws, int64_t max_tiles, int q, int d,
                       int heads, void* O, hipStream_t stream) {
    if (V) return launch_one<DH, WAVES, true>(Z, Wq, K, V, cu_kv, ws, max_tiles, q, d, heads, O, stream);
    return launch_one<DH, WAVES, false>(Z, Wq, K, V, cu_kv, ws, max_tiles, q, d, heads, O, stream);
}

template <int DH>
hipError_t launch_dh(const void* Z, const void* Wq, const void* K, const void* V,
                     const int* cu_kv, const void* ws, int64_t max_tiles, int q, int d,
                     int heads, int waves, void* O, hipStream_t stream) {
    if (waves == 4) return launch_dh_w<DH, 4>(Z, Wq, K, V, cu_kv, ws, max_tiles, q, d, heads, O, stream);
    return launch_dh_w<DH, 2>(Z, Wq, K, V, cu_kv, ws, max_tiles, q, d, heads, O, stream);
}

}  // namespace

hipError_t launch_attn_bf16(const void* Z, const void* Wq, const void* K, const void* V,
                            const int* cu_kv, const void* ws, int64_t max_tiles, int q, int d,
                            int heads, int waves, void* O, hipStream_t stream) {
    switch (d / heads) {
        case 32: return launch_dh<32>(Z, Wq, K, V, cu_kv, ws, max_tiles, q, d, heads, waves, O, stream);
        case 64: return launch_dh<64>(Z, Wq, K, V, cu_kv, ws, max_tiles, q, d, heads, waves, O, stream);
        case 128: return launch_dh<128>(Z, Wq, K, V, cu_kv, ws, max_tiles, q, d, heads, waves, O, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_project_bf16(const void* Z, const void* Wq, int total_cand, int q, int d,
                               void* Q, hipStream_t stream) {
    constexpr int W = 2;
    if (total_cand <= 0) return hipSuccess;
    dim3 grid((total_cand + 32 * W - 1) / (32 * W), d / 32, q);
    hipLaunchKernelGGL((project_bf16_kernel<W>), grid, dim3(64 * W), 0, stream,
                       static_cast<const bf16*>(Z), static_cast<const bf16*>(Wq), total_cand, q,
                       d, static_cast<bf16*>(Q));
    return hipGetLastError();
}

}  // namespace xattn
