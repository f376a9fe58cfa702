// Output gate and output projection of Eq. (7) in one launch, bf16 in, fp32
// accumulate, bf16 out, for a model of d = 256 features (gfx950 matrix cores):
//
//   Y[row] = ( O[row] * sigmoid( Z[row] . W_go[s] ) ) . W_o     (row = c*q + s)
//
// (ReST reading note s.3.3.1 Eq. (7); the gate projection token-specific as
// in s.3.3.2 Eq. (8), W_o shared by all slots).  Same arithmetic as the two
// GEMM launches of gemm_bf16.hip (fp32 gate, sigmoid via exp2 and the
// hardware reciprocal, the gated values rounded to bf16 before the W_o
// product), without the gated values' round trip through HBM: they stay in
// LDS.
//
// Work decomposition.  A persistent grid of one 8-wave work-group per compute
// unit walks the units (slot s, 64 candidates), slot-major, in equal
// contiguous shares.  Wave w holds rows 32w..32w+31 of W_go[s] and of W_o in
// registers as A operands (reloaded only when the slot changes).  Per unit:
//   1. the unit's Z rows (staged in LDS, loaded into registers one unit
//      ahead) give G^T rows 32w.. = W_go[s] rows 32w.. . Z^T on the matrix
//      cores; the unit's O values are loaded 16 bytes per lane and moved
//      into the accumulator's layout by an exchange between the lane halves;
//   2. gated = O * sigmoid(G), rounded to bf16, replaces the Z rows in LDS;
//   3. Y^T rows 32w.. = W_o rows 32w.. . gated^T, rounded to bf16 and stored
//      16 bytes per lane (the same exchange) through a descriptor that covers
//      the unit's rows only.
#include "common.h"
#include "internal.h"

namespace xattn {

namespace {

constexpr int D = kShortD;   // model features
constexpr int NW = 8;
constexpr int NT = 64 * NW;
constexpr int UR = 64;       // candidates per unit
constexpr int LDK = D + 8;   // LDS pitch (elements): 16-byte rows
constexpr int Z_CPT = UR * (D / 8) / NT;   // 16-byte Z chunks per thread
static_assert(UR * (D / 8) % NT == 0, "even staging split");


struct OutArgs {
    const bf16* Z;
    const bf16* Wgo;
    const bf16* O;
    const bf16* Wo;
    bf16* Y;
    int total_cand, q;
};

__global__ __launch_bounds__(NT) void gate_output_kernel(OutArgs a) {
    __shared__ __attribute__((aligned(16))) bf16 buf[UR * LDK];   // Z rows, then gated rows
    const int q = a.q, total_cand = a.total_cand;
    const int n_chunks = (total_cand + UR - 1) / UR;
    const int U = q * n_chunks;
    const int G = gridDim.x;
    const int u_end = (int)((int64_t)(blockIdx.x + 1) * U / G);
    int u = (int)((int64_t)blockIdx.x * U / G);
    if (u >= u_end) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, l32 = lane & 31;

    // Every pointer the unit loop uses, in scalar registers before it: a
    // scalar load still in flight in the loop would make each wait for an
    // LDS read there a wait for all of them (no LDS read ahead of the
    // products).
    const bf16* const Zp = a.Z;
    const bf16* const Op = a.O;
    const bf16* const Wgop = a.Wgo;
    bf16* const Yp = a.Y;
    asm volatile("" ::"s"(Zp), "s"(Op), "s"(Wgop), "s"(Yp));

    // unit u: slot s = u / n_chunks, candidates [cb, cb + nr)
    auto unit = [&](int uu, int& s, int& cb, int& nr) {
        s = uu / n_chunks;
        cb = (uu - s * n_chunks) * UR;
        nr = min(UR, total_cand - cb);
    };
    // a descriptor over the unit's rows c*q + s of a [total_cand][q][D]
    // tensor: rows past the unit's candidates lie outside it (loads read
    // zeros, stores are dropped)
    auto rows_rsrc = [&](const bf16* base, int s, int cb, int nr) {
        return __builtin_amdgcn_make_buffer_rsrc(
            (void*)(base + ((size_t)cb * q + s) * D), (short)0,
            (uint32_t)(((size_t)(nr - 1) * q + 1) * D * 2), 0x00020000);
    };

    uint4 zr[Z_CPT];
    auto zload = [&](int s, int cb, int nr) {
        const __amdgpu_buffer_rsrc_t rz = rows_rsrc(Zp, s, cb, nr);
#pragma unroll
        for (int i = 0; i < Z_CPT; ++i) {
            const int idx = tid + i * NT, row = idx >> 5, col = idx & 31;
            zr[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rz, (row * q * D + col * 8) * 2, 0, 0));
        }
    };
    auto zstore = [&]() {
#pragma unroll
        for (int i = 0; i < Z_CPT; ++i) {
            const int idx = tid + i * NT, row = idx >> 5, col = idx & 31;
            *reinterpret_cast<uint4*>(buf + row * LDK + col * 8) = zr[i];
        }
    };

    // this wave's rows of W_go[s] and of W_o: k-step kk holds inputs
    // 16kk + 8g .. +7 of output feature 32w + l32
    bf16x8 wg[D / 16], wo[D / 16];
    auto wload = [&](bf16x8 (&wr)[D / 16], const bf16* rowp) {
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) wr[kk] = *reinterpret_cast<const bf16x8*>(rowp + 16 * kk);
    };

    // acc[rb] = wr . (rows 32rb.. of the LDS tile)^T over the D inputs, with
    // each k-step's B fragments read one k-step ahead of its products
    auto gemm = [&](const bf16x8 (&wr)[D / 16], f32x16 (&acc)[2]) {
        auto frag = [&](int kk, int rb) {
            return *reinterpret_cast<const bf16x8*>(buf + (rb * 32 + l32) * LDK + 16 * kk + 8 * g);
        };
        bf16x8 b[2][2];
        b[0][0] = frag(0, 0);
        b[0][1] = frag(0, 1);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            if (kk + 1 < D / 16) {
                b[(kk + 1) & 1][0] = frag(kk + 1, 0);
                b[(kk + 1) & 1][1] = frag(kk + 1, 1);
            }
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) acc[rb] = mfma32(wr[kk], b[kk & 1][rb], acc[rb]);
        }
    };

    int s, cb, nr;
    unit(u, s, cb, nr);
    int wslot = s;
    wload(wo, a.Wo + (size_t)(32 * w + l32) * D + 8 * g);
    wload(wg, Wgop + ((size_t)s * D + 32 * w + l32) * D + 8 * g);
    zload(s, cb, nr);
    zstore();   // its wait covers the weight rows loaded before the Z rows
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) asm volatile("" : "+v"(wg[kk]), "+v"(wo[kk]));

    for (;;) {
        const bool has_next = u + 1 < u_end;
        int s2 = s, cb2 = cb, nr2 = nr;
        if (has_next) unit(u + 1, s2, cb2, nr2);
        __syncthreads();   // the unit's Z rows are in LDS
        // O rows 32rb + l32, features 32w + 16jp + 8g .. +7 (16 bytes per
        // lane), requested before the next unit's Z rows: the vector-memory
        // counter completes in order, so waiting for them in the gate
        // epilogue does not wait for the Z rows
        const __amdgpu_buffer_rsrc_t ro = rows_rsrc(Op, s, cb, nr);
        u32x4 ol[2][2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int jp = 0; jp < 2; ++jp)
                ol[rb][jp] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                               ro, ((rb * 32 + l32) * q * D + 32 * w + 16 * jp + 8 * g) * 2, 0, 0));
        if (has_next) zload(s2, cb2, nr2);
        if (s != wslot) {
            // a new slot (rare): wait for its rows here
            wslot = s;
            wload(wg, Wgop + ((size_t)s * D + 32 * w + l32) * D + 8 * g);
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) asm volatile("" : "+v"(wg[kk]));
        }

        // 1. gate: G^T rows 32w.. = W_go[s] rows 32w.. . Z^T
        f32x16 acc[2] = {f32x16{}, f32x16{}};
        gemm(wg, acc);
        __syncthreads();   // every wave is done reading Z

        // 2. gated = O * sigmoid(G), bf16, into LDS (acc reg 4*j4 + t:
        //    feature 32w + 8j4 + 4g + t of row 32rb + l32).  A lane holds
        //    features 16jp + 8g .. +7 of O; split_runs leaves runs j4 = 2jp
        //    and 2jp + 1 of the accumulator layout.
        u32x2 ov[2][4];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int jp = 0; jp < 2; ++jp) split_runs(ol[rb][jp], ov[rb][2 * jp], ov[rb][2 * jp + 1]);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) {
                const bf16x4 o = __builtin_bit_cast(bf16x4, ov[rb][j4]);
                bf16x4 v;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const float e = __builtin_amdgcn_exp2f(-acc[rb][4 * j4 + t] * 1.4426950408889634f);
                    v[t] = (bf16)((float)o[t] * __builtin_amdgcn_rcpf(1.0f + e));
                }
                *reinterpret_cast<bf16x4*>(buf + (rb * 32 + l32) * LDK + 32 * w + 8 * j4 + 4 * g) = v;
            }
        __syncthreads();   // the gated rows are in LDS

        // 3. Y^T rows 32w.. = W_o rows 32w.. . gated^T
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) acc[rb] = f32x16{};
        gemm(wo, acc);
        // Y rows, 16 bytes per lane (join_runs)
        const __amdgpu_buffer_rsrc_t ry = rows_rsrc(Yp, s, cb, nr);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int jp = 0; jp < 2; ++jp) {
                bf16x4 ve, vo;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    ve[t] = (bf16)acc[rb][8 * jp + t];
                    vo[t] = (bf16)acc[rb][8 * jp + 4 + t];
                }
                __builtin_amdgcn_raw_buffer_store_b128(
                    join_runs(ve, vo), ry, ((rb * 32 + l32) * q * D + 32 * w + 16 * jp + 8 * g) * 2, 0, 0);
            }
        if (!has_next) break;
        __syncthreads();   // every wave is done reading the gated rows
        zstore();
        ++u;
        s = s2;
        cb = cb2;
        nr = nr2;
    }
}

}  // namespace

hipError_t launch_gate_output_fused_bf16(const void* Z, const void* Wgo, const void* O,
                                         const void* Wo, void* Y, int total_cand, int q, int d,
                                         int grid, hipStream_t stream) {
    if (d != kShortD || total_cand <= 0 || q < 1) return hipErrorInvalidValue;
    const int64_t units = (int64_t)q * ((total_cand + UR - 1) / UR);
    const int g = (int)(units < grid ? units : grid);
    if (g <= 0) return hipErrorInvalidValue;
    const OutArgs a{static_cast<const bf16*>(Z), static_cast<const bf16*>(Wgo),
                    static_cast<const bf16*>(O), static_cast<const bf16*>(Wo), static_cast<bf16*>(Y),
                    total_cand, q};
    hipLaunchKernelGGL(gate_output_kernel, dim3((unsigned)g), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace xattn
