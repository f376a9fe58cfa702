// Backward pass of the shared-memory cross-attention on gfx950 matrix cores,
// bf16 operands, fp32 accumulation.
//
// For the loss gradient dO of O = softmax(Q_h K_h^T / sqrt(d_h)) V_h (ReST
// reading note, s.3.3.1 Eq. (7); per-slot W_Q of Eq. (8); K = V = H in
// projection-free mode), with P the softmax weights, the chain rule gives
//   dV_h = P^T dO_h,  dP = dO_h V_h^T,  dS = P o (dP - D),  D_i = <dO_i, O_i>,
//   dQ_h = dS K_h / sqrt(d_h),  dK_h = dS^T Q_h / sqrt(d_h),
// summed, for the memory, over every query row of the request: all candidates
// of a user send their gradients back into the one memory (TransX report s.2,
// trajectory packing; ReST reading note s.3.5, ULT).  In projection-free mode
// H receives dK + dV.
//
// The queries arrive pre-scaled (Qs = Q log2(e)/sqrt(d_h), the forward's own
// operand) together with the forward's per-row statistics lse (log2 of the
// softmax normaliser in those units) and D, so a weight is exp2(Qs.k - lse)
// and both kernels recompute P without any running maximum.
//
// bwd_dq_kernel: one work-group (2 x KS waves, 64 query rows) per plan item
// and head, streaming the request's memory tiles through LDS like the
// forward kernel; KS memory splits (tiles t with t % KS == split), their
// partial dQ summed on chip in split order.  Per 64-row tile and wave:
//   S^T - lse  (64 x 32) = K_tile . Qs^T     (accumulator seeded with -lse)
//   dP^T - D   (64 x 32) = V_tile . dO^T     (seeded with -D)
//   dQ^T      (d_h x 32) += K_tile^T . dS^T  (K^T from LDS transpose reads)
// Each lane owns one query row, so P and dS never leave the lane.
//
// bwd_dkv_kernel: one work-group per 64 memory rows of a request and head
// (a plan over memory tiles), 2 x 2 waves: two waves of 32 memory rows times
// two splits of the request's query rows, merged on chip in a fixed order.
// Per 32-row query tile and wave (mirror image of the above: each lane owns
// one memory row):
//   S - lse   (32 x 32) = Qs_tile . K^T        (K, V rows held in registers)
//   dP - D    (32 x 32) = dO_tile . V^T
//   dV^T     (d_h x 32) += dO_tile^T . P
//   dK^T     (d_h x 32) += Qs_tile^T . dS      (dK = ln 2 * this: Qs carries log2 e / sqrt(d_h))
// No atomics anywhere: every output element is written once, after a
// reduction in a fixed order, so the result is deterministic bit for bit.
//
// bwd_dw_kernel: dW_Q[s] = dQ_s^T Z_s (output-major, fp32) as split-K
// partial tiles over candidate chunks, summed in chunk order by
// bwd_dw_reduce (many threads: a reduction inside the last work-group of a
// tile measured 25x slower, its loads mostly missing its XCD's L2).  dZ =
// dQ W_Q[s] is the projection GEMM over a transposed copy of W_Q, made by
// side work-groups of the projection launch (bf16) or bwd_transpose_kernel
// (fp32).
#include <cstdlib>

#include "common.h"
#include "internal.h"

namespace xattn {

namespace {

constexpr int kBN = 64;   // memory rows per tile of the dQ kernel
constexpr int kBQ = 32;   // query rows per tile of the dK/dV kernel
constexpr float kLn2 = 0.69314718055994531f;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, long long bytes) {
    const uint32_t b = bytes <= 0 ? 0u : (bytes > 0xFFFFFFF0ll ? 0xFFFFFFF0u : (uint32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, b, 0x00020000);
}

__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// 16-byte load of eight bf16 values (global or LDS)
__device__ __forceinline__ bf16x8 ld8(const bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
template <int DH, bool SEP, int KS>
struct DqCfg {
    static constexpr int NT = 128 * KS;
    static constexpr int GT = 128;               // threads of one memory split
    static constexpr int EB = DH / 32, KST = DH / 16;
    static constexpr int LDK = DH + 8;           // 16-byte rows
    static constexpr int PLANES = SEP ? 2 : 1;
    static constexpr int TILE = kBN * LDK;
    static constexpr int STG = KS * 2 * PLANES * TILE * 2;
    static constexpr int CMB = (KS - 1) * 2 * EB * 16 * 64 * 4;
    static constexpr int SMEM = STG > CMB ? STG : CMB;
    static constexpr int CPT = kBN * DH / 8 / GT;   // 16-byte chunks per thread and plane
};

template <int DH, bool SEP, bool CUT, int KS>
__global__ __launch_bounds__(128 * KS) void bwd_dq_kernel(BwdArgs a) {
    using C = DqCfg<DH, SEP, KS>;
    __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
    const int q = a.q, d = a.d, heads = a.heads;
    const int* __restrict__ ws = a.plan;
    const int tile = blockIdx.x / heads;
    const int h = blockIdx.x - tile * heads;
    if (tile >= ws[kPlanNTiles] || ws[kPlanTileM] != 64) return;
    const int4 item = reinterpret_cast<const int4*>(reinterpret_cast<const char*>(ws) +
                                                    kPlanHeaderBytes)[tile];
    const int kv0 = __builtin_amdgcn_readfirstlane(item.x);
    const int L = __builtin_amdgcn_readfirstlane(item.y);
    const int c0 = __builtin_amdgcn_readfirstlane(item.z);
    const int iw = __builtin_amdgcn_readfirstlane(item.w);
    const int nc = iw & kItemNcMask, s = iw >> 16;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qblk = w & 1, ksg = w >> 1;        // query block, memory split
    const int gt = tid - ksg * C::GT;            // thread index inside the split
    const int g = lane >> 5, l32 = lane & 31;
    const int qcol = qblk * 32 + l32;
    const bool qvalid = qcol < nc;
    const size_t row = (size_t)(qvalid ? c0 + qcol : c0 + nc - 1) * q + s;

    // this lane's pre-scaled query and output gradient (head slices), as the
    // B operands of the two score-shaped products
    const bf16* __restrict__ Qs = static_cast<const bf16*>(a.Qs);
    const bf16* __restrict__ dO = static_cast<const bf16*>(a.dO);
    bf16x8 qb[C::KST], db[C::KST];
#pragma unroll
    for (int k = 0; k < C::KST; ++k) {
        qb[k] = ld8(Qs + row * d + h * DH + 16 * k + 8 * g);
        db[k] = ld8(dO + row * d + h * DH + 16 * k + 8 * g);
    }
    const float lse = a.lse[row * heads + h];
    const float Dr = a.Dsum[row * heads + h];
    f32x16 seed_s, seed_p;
#pragma unroll
    for (int r = 0; r < 16; ++r) seed_s[r] = -lse, seed_p[r] = -Dr;

    // Per-candidate prefix (CUT): this lane's query row sees memory rows
    // [0, cut); the tile loop runs to the largest cut of the work-group's
    // candidates (computed identically by both waves).
    int cut = L, L_loop = L;
    if constexpr (CUT) {
        cut = qvalid ? a.vis[c0 + qcol] - kv0 : L;
        int mx = 0;
        for (int i = lane; i < nc; i += 64) mx = max(mx, a.vis[c0 + i] - kv0);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) mx = max(mx, __shfl_xor(mx, off, 64));
        L_loop = __builtin_amdgcn_readfirstlane(mx);
    }

    const bf16* Kh = static_cast<const bf16*>(a.K) + (size_t)kv0 * d + h * DH;
    const bf16* Vh = SEP ? static_cast<const bf16*>(a.V) + (size_t)kv0 * d + h * DH : Kh;
    int goff[C::CPT], loff[C::CPT];
#pragma unroll
    for (int u = 0; u < C::CPT; ++u) {
        const int c = gt + u * C::GT;
        const int j = c / (DH / 8), c8 = c % (DH / 8);
        goff[u] = (j * d + c8 * 8) * 2;
        loff[u] = j * C::LDK + c8 * 8;
    }
    uint4 kr[C::CPT], vr[SEP ? C::CPT : 1];
    // tile t of the request's memory; rows past L read as zeros
    auto gload = [&](int t) {
        const long long left = (long long)(L_loop - t * kBN) * d * 2;
        const __amdgpu_buffer_rsrc_t rk = rsrc(Kh + (size_t)t * kBN * d, left);
#pragma unroll
        for (int u = 0; u < C::CPT; ++u) kr[u] = bload(rk, goff[u]);
        if constexpr (SEP) {
            const __amdgpu_buffer_rsrc_t rv = rsrc(Vh + (size_t)t * kBN * d, left);
#pragma unroll
            for (int u = 0; u < C::CPT; ++u) vr[u] = bload(rv, goff[u]);
        }
    };
    bf16* lds = reinterpret_cast<bf16*>(smem) + (size_t)ksg * 2 * C::PLANES * C::TILE;
    auto lstore = [&](int buf) {
        bf16* base = lds + buf * C::PLANES * C::TILE;
#pragma unroll
        for (int u = 0; u < C::CPT; ++u) {
            *reinterpret_cast<uint4*>(base + loff[u]) = kr[u];
            if constexpr (SEP) *reinterpret_cast<uint4*>(base + C::TILE + loff[u]) = vr[u];
        }
    };

    const int ntiles = (L_loop + kBN - 1) / kBN;
    const int n_iter = (ntiles + KS - 1) / KS;   // the same in every split
    gload(ksg);
    lstore(0);
    gload(ksg + KS);
    __syncthreads();

    f32x16 dq[C::EB];
#pragma unroll
    for (int eb = 0; eb < C::EB; ++eb) dq[eb] = f32x16{};
    // transposed K read: lane l receives K[16u + 4g + t][eb*32 + l%32], t = 0..3
    const int G = lane >> 4, k16 = lane & 15;
    const int tr_row = 4 * (G >> 1) + (k16 >> 2);
    const int tr_col = 16 * (G & 1) + 4 * (k16 & 3);

    for (int it = 0; it < n_iter; ++it) {
      const int t = ksg + it * KS;
      if (t < ntiles) {
        const bf16* kb = lds + (it & 1) * C::PLANES * C::TILE;
        const bf16* vb = kb + (C::PLANES - 1) * C::TILE;
        // keys hh*32 + (r/4)*8 + 4g + r%4 of the tile, query row qcol
        f32x16 sacc[2], pacc[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) sacc[hh] = seed_s, pacc[hh] = seed_p;
#pragma unroll
        for (int k = 0; k < C::KST; ++k)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int off = (hh * 32 + l32) * C::LDK + 16 * k + 8 * g;
                const bf16x8 kf = ld8(kb + off);
                sacc[hh] = mfma32(kf, qb[k], sacc[hh]);
                pacc[hh] = mfma32(SEP ? ld8(vb + off) : kf, db[k], pacc[hh]);
            }
        // dS^T = P^T o (dP^T - D), rows past the request's memory (or past
        // the lane's prefix) masked
        // Only a request's last tile is partial (with cutoffs: any tile):
        // there the scores of masked rows become -inf, so that their weights
        // are 0 (and dP - D is finite: rows past the memory read as zeros);
        // the other tiles skip the per-score test.  The opaque copy keeps
        // the compiler from folding the tile test into per-score tests.
        const int jleft = (CUT ? cut : L) - t * kBN;
        int jl = L - t * kBN;
        asm volatile("" : "+s"(jl));
        if (CUT || jl < kBN) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) {
                    const int j = hh * 32 + (rr >> 2) * 8 + 4 * g + (rr & 3);
                    if (j >= jleft) sacc[hh][rr] = -INFINITY;
                }
        }
        bf16x8 dsb[4];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const float p = __builtin_amdgcn_exp2f(sacc[hh][rr]);
                dsb[hh * 2 + (rr >> 3)][rr & 7] = (bf16)(p * pacc[hh][rr]);
            }
        // dQ^T += K^T dS^T over the four 16-key slabs of the tile
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int eb = 0; eb < C::EB; ++eb) {
                const bf16* base = kb + (16 * u + tr_row) * C::LDK + eb * 32 + tr_col;
                dq[eb] = mfma32(cat(lds_read_tr16(base), lds_read_tr16(base + 8 * C::LDK)), dsb[u],
                                dq[eb]);
            }
      }
        if (it + 1 < n_iter) lstore((it + 1) & 1);
        gload(t + 2 * KS);
        __syncthreads();
    }
    // partial dQ of the memory splits, summed in split order (dQ is linear
    // in the memory tiles)
    if constexpr (KS > 1) {
        float* cmb = reinterpret_cast<float*>(smem);
        if (ksg > 0) {
            float* dst = cmb + (size_t)(((ksg - 1) * 2 + qblk) * C::EB * 16) * 64;
#pragma unroll
            for (int eb = 0; eb < C::EB; ++eb)
#pragma unroll
                for (int r = 0; r < 16; ++r) dst[(eb * 16 + r) * 64 + lane] = dq[eb][r];
        }
        __syncthreads();
        if (ksg > 0) return;
#pragma unroll
        for (int k = 1; k < KS; ++k) {
            const float* src = cmb + (size_t)(((k - 1) * 2 + qblk) * C::EB * 16) * 64;
#pragma unroll
            for (int eb = 0; eb < C::EB; ++eb)
#pragma unroll
                for (int r = 0; r < 16; ++r) dq[eb][r] += src[(eb * 16 + r) * 64 + lane];
        }
    }

    if (qvalid) {
        bf16* orow = static_cast<bf16*>(a.dQ) + row * d + h * DH;
#pragma unroll
        for (int eb = 0; eb < C::EB; ++eb)
#pragma unroll
            for (int b4 = 0; b4 < 4; ++b4) {
                bf16x4 v;
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) v[tt] = (bf16)(dq[eb][4 * b4 + tt] * a.scale);
                *reinterpret_cast<bf16x4*>(orow + eb * 32 + b4 * 8 + 4 * g) = v;
            }
    }
}

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
template <int DH, bool SEP>
struct DkvCfg {
    static constexpr int WK = 2, MS = 2, NW = WK * MS, NT = 64 * NW;
    static constexpr int EB = DH / 32, KST = DH / 16;
    static constexpr int LDQ = DH + 8;
    static constexpr int TILE = kBQ * LDQ;                       // elements of one row tile
    static constexpr int STAGE = 2 * TILE * 2 + 3 * kBQ * 4;     // Qs, dO tiles + lse, D, visible end
    static constexpr int STG_BYTES = MS * 2 * STAGE;             // double-buffered per split
    static constexpr int CMB_BYTES = (MS - 1) * WK * 64 * 2 * EB * 16 * 4;
    static constexpr int SMEM = STG_BYTES > CMB_BYTES ? STG_BYTES : CMB_BYTES;
    static constexpr int CPT = kBQ * DH / 8 / (64 * WK);         // 16-byte chunks per thread and tile
    static_assert(CPT >= 1 && kBQ * DH / 8 % (64 * WK) == 0, "row tile must split evenly");
};

template <int DH, bool SEP, bool CUT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(DH == 64 && !SEP ? 3 : 1)))
void bwd_dkv_kernel(BwdArgs a) {
    using C = DkvCfg<DH, SEP>;
    __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
    const int q = a.q, d = a.d, heads = a.heads;
    const int* __restrict__ kws = a.kplan;
    const int tile = blockIdx.x / heads;
    const int h = blockIdx.x - tile * heads;
    if (tile >= kws[kPlanNTiles] || kws[kPlanTileM] != 64) return;
    // memory-tile plan (the planner with the roles of memory and candidates
    // exchanged): {first candidate, candidates, first memory row, rows}
    const int4 item = reinterpret_cast<const int4*>(reinterpret_cast<const char*>(kws) +
                                                    kPlanHeaderBytes)[tile];
    const int c_lo = __builtin_amdgcn_readfirstlane(item.x);
    const int N = __builtin_amdgcn_readfirstlane(item.y);
    const int key0 = __builtin_amdgcn_readfirstlane(item.z);
    const int nk = __builtin_amdgcn_readfirstlane(item.w) & kItemNcMask;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kw = w % C::WK, ms = w / C::WK;
    const int g = lane >> 5, l32 = lane & 31;
    const int kcol = kw * 32 + l32;
    const bool kvalid = kcol < nk;
    const size_t key = (size_t)key0 + (kvalid ? kcol : nk - 1);
    const int gt = tid - ms * 64 * C::WK;   // thread index inside the split group

    // this lane's memory row (key and value), B operands for every query tile
    const bf16* __restrict__ K = static_cast<const bf16*>(a.K);
    const bf16* __restrict__ V = SEP ? static_cast<const bf16*>(a.V) : K;
    bf16x8 kb[C::KST], vb[C::KST];
#pragma unroll
    for (int k = 0; k < C::KST; ++k) {
        kb[k] = ld8(K + key * d + h * DH + 16 * k + 8 * g);
        vb[k] = SEP ? ld8(V + key * d + h * DH + 16 * k + 8 * g) : kb[k];
    }

    // the request's query rows: [row0, row0 + M), all slots of all candidates
    const int row0 = c_lo * q, M = N * q;
    const int ntq = (M + kBQ - 1) / kBQ;
    const int n_iter = (ntq + C::MS - 1) / C::MS;
    const bf16* Qh = static_cast<const bf16*>(a.Qs) + (size_t)row0 * d + h * DH;
    const bf16* dOh = static_cast<const bf16*>(a.dO) + (size_t)row0 * d + h * DH;
    int goff[C::CPT], loff[C::CPT];
#pragma unroll
    for (int u = 0; u < C::CPT; ++u) {
        const int c = gt + u * 64 * C::WK;
        const int i = c / (DH / 8), c8 = c % (DH / 8);
        goff[u] = (i * d + c8 * 8) * 2;
        loff[u] = i * C::LDQ + c8 * 8;
    }
    uint4 qr[C::CPT], dr[C::CPT];
    float sr = 0.f;   // lse (threads 0..31 of the group), D (32..63), visible end (64..95)
    auto gload = [&](int tq) {
        const long long left = (long long)(M - tq * kBQ) * d * 2;
        const __amdgpu_buffer_rsrc_t rq = rsrc(Qh + (size_t)tq * kBQ * d, left);
        const __amdgpu_buffer_rsrc_t rd = rsrc(dOh + (size_t)tq * kBQ * d, left);
#pragma unroll
        for (int u = 0; u < C::CPT; ++u) {
            qr[u] = bload(rq, goff[u]);
            dr[u] = bload(rd, goff[u]);
        }
        if (gt < (CUT ? 3 : 2) * kBQ) {
            const int i = tq * kBQ + (gt & (kBQ - 1));
            const size_t idx = ((size_t)row0 + i) * heads + h;
            // rows past the request: lse = +inf gives zero weight, D = 0
            if (gt < kBQ)
                sr = i < M ? a.lse[idx] : INFINITY;
            else if (gt < 2 * kBQ)
                sr = i < M ? a.Dsum[idx] : 0.f;
            else   // absolute end of the row's visible memory (an int in a float slot)
                sr = __builtin_bit_cast(float, i < M ? a.vis[(row0 + i) / q] : 0);
        }
    };
    char* stg = smem + ms * 2 * C::STAGE;
    auto lstore = [&](int buf) {
        bf16* qt = reinterpret_cast<bf16*>(stg + buf * C::STAGE);
        bf16* dt = qt + C::TILE;
#pragma unroll
        for (int u = 0; u < C::CPT; ++u) {
            *reinterpret_cast<uint4*>(qt + loff[u]) = qr[u];
            *reinterpret_cast<uint4*>(dt + loff[u]) = dr[u];
        }
        if (gt < (CUT ? 3 : 2) * kBQ) reinterpret_cast<float*>(dt + C::TILE)[gt] = sr;
    };

    gload(ms);
    lstore(0);
    gload(ms + C::MS);
    __syncthreads();

    f32x16 dk[C::EB], dv[C::EB];
#pragma unroll
    for (int eb = 0; eb < C::EB; ++eb) dk[eb] = f32x16{}, dv[eb] = f32x16{};
    const int G = lane >> 4, k16 = lane & 15;
    const int tr_row = 4 * (G >> 1) + (k16 >> 2);
    const int tr_col = 16 * (G & 1) + 4 * (k16 & 3);

    for (int it = 0; it < n_iter; ++it) {
        if (ms + it * C::MS < ntq) {
            const bf16* qt = reinterpret_cast<const bf16*>(stg + (it & 1) * C::STAGE);
            const bf16* dt = qt + C::TILE;
            const float* lt = reinterpret_cast<const float*>(dt + C::TILE);
            const float* Dt = lt + kBQ;
            // rows (r/4)*8 + 4g + r%4 of the tile, memory row kcol
            f32x16 sacc, pacc;
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const f32x4 l4 = *reinterpret_cast<const f32x4*>(lt + 8 * a4 + 4 * g);
                const f32x4 d4 = *reinterpret_cast<const f32x4*>(Dt + 8 * a4 + 4 * g);
#pragma unroll
                for (int b = 0; b < 4; ++b) sacc[4 * a4 + b] = -l4[b], pacc[4 * a4 + b] = -d4[b];
            }
#pragma unroll
            for (int k = 0; k < C::KST; ++k) {
                const int off = l32 * C::LDQ + 16 * k + 8 * g;
                sacc = mfma32(ld8(qt + off), kb[k], sacc);
                pacc = mfma32(ld8(dt + off), vb[k], pacc);
            }
            int vis[16];
            if constexpr (CUT) {
                const int* vt = reinterpret_cast<const int*>(Dt + kBQ);
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) {
                    const int4 v4 = *reinterpret_cast<const int4*>(vt + 8 * a4 + 4 * g);
                    vis[4 * a4] = v4.x, vis[4 * a4 + 1] = v4.y;
                    vis[4 * a4 + 2] = v4.z, vis[4 * a4 + 3] = v4.w;
                }
            }
            bf16x8 pb[2], dsb[2];
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                float p = __builtin_amdgcn_exp2f(sacc[rr]);
                if constexpr (CUT) p = (int)key < vis[rr] ? p : 0.f;   // row sees this memory row?
                pb[rr >> 3][rr & 7] = (bf16)p;
                dsb[rr >> 3][rr & 7] = (bf16)(p * pacc[rr]);
            }
            // dV^T += dO^T P and dK^T += Qs^T dS over the two 16-row slabs
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int eb = 0; eb < C::EB; ++eb) {
                    const int off = (16 * u + tr_row) * C::LDQ + eb * 32 + tr_col;
                    dv[eb] = mfma32(cat(lds_read_tr16(dt + off), lds_read_tr16(dt + off + 8 * C::LDQ)),
                                    pb[u], dv[eb]);
                    dk[eb] = mfma32(cat(lds_read_tr16(qt + off), lds_read_tr16(qt + off + 8 * C::LDQ)),
                                    dsb[u], dk[eb]);
                }
        }
        if (it + 1 < n_iter) lstore((it + 1) & 1);
        gload(ms + (it + 2) * C::MS);
        __syncthreads();
    }

    // merge the query splits in split order (the staging area is free now)
    if constexpr (C::MS > 1) {
        float* cmb = reinterpret_cast<float*>(smem);
        constexpr int PER = 2 * C::EB * 16;
        if (ms > 0) {
            float* dst = cmb + ((size_t)((ms - 1) * C::WK + kw) * PER) * 64;
#pragma unroll
            for (int eb = 0; eb < C::EB; ++eb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    dst[(eb * 16 + r) * 64 + lane] = dk[eb][r];
                    dst[((C::EB + eb) * 16 + r) * 64 + lane] = dv[eb][r];
                }
        }
        __syncthreads();
        if (ms > 0) return;
#pragma unroll
        for (int k = 1; k < C::MS; ++k) {
            const float* src = cmb + ((size_t)((k - 1) * C::WK + kw) * PER) * 64;
#pragma unroll
            for (int eb = 0; eb < C::EB; ++eb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    dk[eb][r] += src[(eb * 16 + r) * 64 + lane];
                    dv[eb][r] += src[((C::EB + eb) * 16 + r) * 64 + lane];
                }
        }
    }

    if (kvalid) {
        bf16* krow = static_cast<bf16*>(a.dK) + key * d + h * DH;
        bf16* vrow = SEP ? static_cast<bf16*>(a.dV) + key * d + h * DH : nullptr;
#pragma unroll
        for (int eb = 0; eb < C::EB; ++eb)
#pragma unroll
            for (int b4 = 0; b4 < 4; ++b4) {
                bf16x4 vk, vv;
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const float gk = dk[eb][4 * b4 + tt] * kLn2;
                    const float gv = dv[eb][4 * b4 + tt];
                    vk[tt] = (bf16)(SEP ? gk : gk + gv);
                    vv[tt] = (bf16)gv;
                }
                *reinterpret_cast<bf16x4*>(krow + eb * 32 + b4 * 8 + 4 * g) = vk;
                if constexpr (SEP) *reinterpret_cast<bf16x4*>(vrow + eb * 32 + b4 * 8 + 4 * g) = vv;
            }
    }
}

// ---------------------------------------------------------------------------
// dW_Q (split-K over candidates) and the transposed weights for dZ
// ---------------------------------------------------------------------------
constexpr int kWT = 64;     // output tile (o x i)
constexpr int kWC = 32;     // candidates per LDS stage
constexpr int kWLD = kWT + 8;

// part[ch][s][o][i] = sum over candidates c of chunk ch of dQ[c*q+s][o] Z[c*q+s][i]
__global__ __launch_bounds__(256) void bwd_dw_kernel(const bf16* __restrict__ dQ,
                                                    const bf16* __restrict__ Z, int total_cand,
                                                    int q, int d, int cpc,
                                                    float* __restrict__ part) {
    __shared__ __attribute__((aligned(16))) bf16 sa[2][kWC * kWLD];
    __shared__ __attribute__((aligned(16))) bf16 sb[2][kWC * kWLD];
    const int tpd = (d + kWT - 1) / kWT;
    int bid = blockIdx.x;
    {
        // The tpd x tpd output tiles of one (chunk, slot) read the same
        // candidate rows of dQ and Z: all of them on one XCD (work-group b
        // runs on XCD b % 8), so that those rows come from HBM once and from
        // that XCD's L2 for the other tiles.  Rounds of 8 (chunk, slot)
        // units; a last partial round keeps the plain order.
        const int G = tpd * tpd, per = 8 * G;
        if (bid < (int)gridDim.x / per * per) {
            const int x = bid % 8, k = bid / 8;
            bid = ((k / G) * 8 + x) * G + k % G;
        }
    }
    const int it = bid % tpd;
    bid /= tpd;
    const int ot = bid % tpd;
    bid /= tpd;
    const int s = bid % q;
    const int ch = bid / q;
    const int cbeg = ch * cpc;
    const int cend = min(total_cand, cbeg + cpc);
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = w >> 1, wc = w & 1;
    // staging: 32 candidates x 64 columns per operand = 256 chunks of 16 bytes
    const int srow = tid >> 3, scol = (tid & 7) * 8;
    const size_t rstride = (size_t)q * d;   // elements between a slot's rows of consecutive candidates
    // columns past d and candidates past the chunk stage zeros
    auto gload = [&](int cb, uint4& ra, uint4& rb) {
        const int c = cb + srow;
        const bool ok = c < cend;
        const size_t base = (size_t)c * rstride + (size_t)s * d;
        ra = ok && ot * kWT + scol < d ? *reinterpret_cast<const uint4*>(dQ + base + ot * kWT + scol)
                                       : uint4{};
        rb = ok && it * kWT + scol < d ? *reinterpret_cast<const uint4*>(Z + base + it * kWT + scol)
                                       : uint4{};
    };
    const int G = lane >> 4, k16 = lane & 15;
    const int tr_row = 4 * (G >> 1) + (k16 >> 2);
    const int tr_col = 16 * (G & 1) + 4 * (k16 & 3);
    f32x16 acc = f32x16{};
    uint4 ra, rb;
    gload(cbeg, ra, rb);
    int buf = 0;
    for (int cb = cbeg; cb < cend; cb += kWC) {
        *reinterpret_cast<uint4*>(&sa[buf][srow * kWLD + scol]) = ra;
        *reinterpret_cast<uint4*>(&sb[buf][srow * kWLD + scol]) = rb;
        __syncthreads();
        if (cb + kWC < cend) gload(cb + kWC, ra, rb);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int off = (16 * u + tr_row) * kWLD + tr_col;
            const bf16* pa = &sa[buf][off + wr * 32];
            const bf16* pb = &sb[buf][off + wc * 32];
            acc = mfma32(cat(lds_read_tr16(pa), lds_read_tr16(pa + 8 * kWLD)),
                         cat(lds_read_tr16(pb), lds_read_tr16(pb + 8 * kWLD)), acc);
        }
        buf ^= 1;
    }
    // acc reg r: o = ot*64 + wr*32 + (r/4)*8 + 4g + r%4, i = it*64 + wc*32 + l32
    const int g = lane >> 5, l32 = lane & 31;
    const int i = it * kWT + wc * 32 + l32;
    if (i < d) {
        float* out = part + ((size_t)ch * q + s) * d * d;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int o = ot * kWT + wr * 32 + (r >> 2) * 8 + 4 * g + (r & 3);
            if (o < d) out[(size_t)o * d + i] = acc[r];
        }
    }
}

__global__ void bwd_dw_reduce(const float* __restrict__ part, int nch, int64_t n,
                              float* __restrict__ dW) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= n) return;
    float acc = 0.f;
    for (int ch = 0; ch < nch; ++ch) acc += part[(size_t)ch * n + idx];
    dW[idx] = acc;
}

// wT[s][i][o] = wt[s][o][i]
template <typename T>
__global__ void bwd_transpose_kernel(const T* __restrict__ wt, int q, int d, T* __restrict__ wT) {
    __shared__ T tileb[32][33];
    const int s = blockIdx.z;
    const int o0 = blockIdx.y * 32, i0 = blockIdx.x * 32;
    const T* src = wt + (size_t)s * d * d;
    T* dst = wT + (size_t)s * d * d;
    for (int y = threadIdx.y; y < 32; y += blockDim.y) {
        const int o = o0 + y, i = i0 + threadIdx.x;
        if (o < d && i < d) tileb[y][threadIdx.x] = src[(size_t)o * d + i];
    }
    __syncthreads();
    for (int y = threadIdx.y; y < 32; y += blockDim.y) {
        const int i = i0 + y, o = o0 + threadIdx.x;
        if (o < d && i < d) dst[(size_t)i * d + o] = tileb[threadIdx.x][y];
    }
}

template <int DH, bool SEP, bool CUT>
hipError_t launch_dq(const BwdArgs& a, int64_t q_items, hipStream_t stream, int dq_ks) {
    // two memory splits wherever the LDS leaves room for two work-groups per
    // CU (measured faster than one on every workload, and four no better);
    // dq_ks = 1 or 2 forces either (tuning and tests)
    const int64_t wgs = q_items * a.heads;
    const int ks = dq_ks == 1 || dq_ks == 2 ? dq_ks : 2;
    const dim3 grid((unsigned)wgs);
    if constexpr (DqCfg<DH, SEP, 2>::SMEM <= 81920) {
        if (ks == 2) {
            hipLaunchKernelGGL((bwd_dq_kernel<DH, SEP, CUT, 2>), grid, dim3(256), 0, stream, a);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((bwd_dq_kernel<DH, SEP, CUT, 1>), grid, dim3(128), 0, stream, a);
    return hipGetLastError();
}

template <int DH, bool SEP, bool CUT>
hipError_t launch_bwd_variant(const BwdArgs& a, int64_t q_items, int64_t k_items,
                              hipStream_t stream, int dq_ks) {
    if (q_items > 0) {
        hipError_t e0 = launch_dq<DH, SEP, CUT>(a, q_items, stream, dq_ks);
        if (e0 != hipSuccess) return e0;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (k_items > 0)
        hipLaunchKernelGGL((bwd_dkv_kernel<DH, SEP, CUT>), dim3((unsigned)(k_items * a.heads)),
                           dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int DH>
hipError_t launch_dh_bwd(const BwdArgs& a, bool sep, int64_t q_items, int64_t k_items,
                         hipStream_t stream, int dq_ks) {
    const bool cut = a.vis != nullptr;
    if (sep)
        return cut ? launch_bwd_variant<DH, true, true>(a, q_items, k_items, stream, dq_ks)
                   : launch_bwd_variant<DH, true, false>(a, q_items, k_items, stream, dq_ks);
    return cut ? launch_bwd_variant<DH, false, true>(a, q_items, k_items, stream, dq_ks)
               : launch_bwd_variant<DH, false, false>(a, q_items, k_items, stream, dq_ks);
}

// vis[c] = cu_kv[r] + clamp(len[c], 0, L_r) for candidate c of request r
__global__ void prefix_vis_kernel(const int* __restrict__ cu_kv, const int* __restrict__ cu_cand,
                                  const int* __restrict__ len, int R, int total_cand,
                                  int* __restrict__ vis) {
    const int c = blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= total_cand) return;
    int lo = 0, hi = R - 1;   // last r with cu_cand[r] <= c
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu_cand[mid] <= c) lo = mid; else hi = mid - 1;
    }
    const int kv0 = cu_kv[lo], L = cu_kv[lo + 1] - kv0;
    const int want = len[c];
    vis[c] = kv0 + (want < 0 ? 0 : (want < L ? want : L));
}

// D[row][h] = <dO_row, O_row> over head h's features from the forward's stored
// output (the second per-row statistic of dS = P o (dP - D)), for a backward
// pass that reuses the forward's normalisers.  One thread per 8 features
// (16-byte loads of both operands); the d_h/8 threads of a head sum their
// partials in a fixed xor-tree order.  The loop bound is uniform per block, so
// every lane reaches the shuffles.
__global__ __launch_bounds__(256) void bwd_dsum_kernel(const uint4* __restrict__ dO,
                                                       const uint4* __restrict__ O, int64_t n,
                                                       int g, float* __restrict__ dsum) {
    for (int64_t i0 = (int64_t)blockIdx.x * 256; i0 < n; i0 += (int64_t)gridDim.x * 256) {
        const int64_t i = i0 + threadIdx.x;
        float acc = 0.f;
        if (i < n) {
            const uint4 a = dO[i], b = O[i];
            const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                acc = fmaf(__uint_as_float(aw[k] << 16), __uint_as_float(bw[k] << 16), acc);
                acc = fmaf(__uint_as_float(aw[k] & 0xFFFF0000u), __uint_as_float(bw[k] & 0xFFFF0000u),
                           acc);
            }
        }
        for (int off = g >> 1; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
        if (i < n && (i & (g - 1)) == 0) dsum[i / g] = acc;
    }
}

}  // namespace

hipError_t launch_bwd_dsum_bf16(const void* dO, const void* O, int64_t rows, int d, int heads,
                                float* dsum, hipStream_t stream) {
    const int g = d / heads / 8;   // 16-byte chunks per head: 4, 8 or 16
    if (g < 1 || (g & (g - 1)) != 0 || 64 % g != 0 || rows < 0) return hipErrorInvalidValue;
    const int64_t n = rows * (d / 8);
    if (n == 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(bwd_dsum_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint4*>(dO), static_cast<const uint4*>(O), n, g, dsum);
    return hipGetLastError();
}

hipError_t launch_bwd_attn_bf16(const BwdArgs& a, bool sep, int64_t q_items, int64_t k_items,
                                hipStream_t stream, int dq_ks) {
    switch (a.d / a.heads) {
        case 32: return launch_dh_bwd<32>(a, sep, q_items, k_items, stream, dq_ks);
        case 64: return launch_dh_bwd<64>(a, sep, q_items, k_items, stream, dq_ks);
        case 128: return launch_dh_bwd<128>(a, sep, q_items, k_items, stream, dq_ks);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_prefix_vis(const int* cu_kv, const int* cu_cand, const int* len, int R,
                             int total_cand, int* vis, hipStream_t stream) {
    if (total_cand <= 0) return hipSuccess;
    hipLaunchKernelGGL(prefix_vis_kernel, dim3((unsigned)((total_cand + 255) / 256)), dim3(256),
                       0, stream, cu_kv, cu_cand, len, R, total_cand, vis);
    return hipGetLastError();
}

// Chunks of the split-K weight gradient: enough for about 512 work-groups.
// Every chunk writes a full [q][d][d] fp32 partial that the reduction reads
// back, so more chunks cost HBM traffic (with 6144 query rows at d = 256,
// 1024 work-groups measured 5 % slower over the whole backward pass, 256
// about 1 % slower).  A chunk's candidates run one after the other in its
// work-group, so chunks of more than 1024 candidates are split further, up
// to about 1024 work-groups (262144 single-token candidates: 9 % faster).
int bwd_dw_chunks(int total_cand, int q, int d) {
    const int tpd = (d + kWT - 1) / kWT;
    const int64_t tiles = (int64_t)q * tpd * tpd;
    int64_t nch = (512 + tiles - 1) / tiles;
    if ((total_cand + nch - 1) / nch > 1024) nch = (1024 + tiles - 1) / tiles;
    const int64_t most = (total_cand + kWC - 1) / kWC;
    if (nch > most) nch = most;
    if (nch < 1) nch = 1;
    return (int)nch;
}

hipError_t launch_bwd_dw_bf16(const void* dQ, const void* Z, int total_cand, int q, int d,
                              float* part, int nch, float* dW, hipStream_t stream) {
    const int64_t n = (int64_t)q * d * d;
    if (total_cand <= 0) {   // no rows: a zero gradient (a fill kernel, no memset)
        hipLaunchKernelGGL(bwd_dw_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                           part, 0, n, dW);
        return hipGetLastError();
    }
    const int tpd = (d + kWT - 1) / kWT;
    int cpc = (total_cand + nch - 1) / nch;
    cpc = (cpc + kWC - 1) / kWC * kWC;
    const int64_t blocks = (int64_t)nch * q * tpd * tpd;
    hipLaunchKernelGGL(bwd_dw_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const bf16*>(dQ), static_cast<const bf16*>(Z), total_cand, q, d,
                       cpc, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_dw_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, part,
                       nch, n, dW);
    return hipGetLastError();
}

hipError_t launch_transpose_weights(const void* wt, int q, int d, bool fp32, void* wT,
                                    hipStream_t stream) {
    const dim3 grid((unsigned)((d + 31) / 32), (unsigned)((d + 31) / 32), (unsigned)q);
    if (fp32)
        hipLaunchKernelGGL((bwd_transpose_kernel<float>), grid, dim3(32, 8), 0, stream,
                           static_cast<const float*>(wt), q, d, static_cast<float*>(wT));
    else
        hipLaunchKernelGGL((bwd_transpose_kernel<bf16>), grid, dim3(32, 8), 0, stream,
                           static_cast<const bf16*>(wt), q, d, static_cast<bf16*>(wT));
    return hipGetLastError();
}

}  // namespace xattn
