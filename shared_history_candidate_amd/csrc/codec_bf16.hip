// TransX memory codec on gfx950 (TransX technical report, s.3: each key or
// value vector kept as its length plus a direction rotated into the
// eigenbasis of the directions' covariance and quantised with bits handed
// out by energy).  Per (memory row, head):
//   norm  = |x_h|                                   (fp32)
//   xr    = E_h^T (x_h / norm)                      (rotated direction)
//   code_i = clamp(floor((xr_i - m_i + a_i) / (2 a_i) * 2^b_i), 0, 2^b_i - 1)
// packed least-significant bit first into budget/32 words, coordinate 0 first
// (b_i = 0: no bits, reconstructed as m_i).  Layout, head-major:
//   codes [heads][rows][budget/32] uint32, norms [heads][rows] fp32.
//
// Attention over a coded memory never leaves the rotated basis: the key
// rotation is folded into the query weights (codec_fold_kernel: W~_Q[s] rows
// of head h = E_K,h^T W_Q[s] rows of head h), scores are q~ . k^ with
// k^ = norm * x^ (x^ the reconstructed rotated direction), the output is
// accumulated as o~ = sum_j p_j v^_j and rotated back once per query row,
// o = E_V o~ (one d_h x d_h product on the matrix cores in the epilogue).
// The reconstruction k^ = norm * (lo_i + code_i * step_i) happens while a
// memory tile is staged in LDS, so HBM carries only the codes and norms.
#include "common.h"
#include "internal.h"

namespace xattn {

namespace {

constexpr int kCBN = 64;     // memory rows per tile

__device__ __forceinline__ __amdgpu_buffer_rsrc_t crsrc(const void* p, long long bytes) {
    const uint32_t b = bytes <= 0 ? 0u : (bytes > 0xFFFFFFF0ll ? 0xFFFFFFF0u : (uint32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, b, 0x00020000);
}

// ---------------------------------------------------------------------------
// encode: one thread per (row, head)
// ---------------------------------------------------------------------------
__global__ void codec_encode_kernel(CodecBook cb, const bf16* __restrict__ X, int n, int d,
                                    int heads, uint32_t* __restrict__ codes,
                                    float* __restrict__ norms) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)n * heads) return;
    const int h = (int)(idx / n);
    const int row = (int)(idx - (int64_t)h * n);
    const int dh = d / heads, W = cb.budget / 32;
    const bf16* x = X + (size_t)row * d + h * dh;
    float n2 = 0.f;
    for (int e = 0; e < dh; ++e) {
        const float v = (float)x[e];
        n2 = fmaf(v, v, n2);
    }
    const float nrm = sqrtf(n2);
    norms[(size_t)h * n + row] = nrm;
    const float inv = nrm > 0.f ? 1.0f / nrm : 0.f;
    const float* E = cb.rot + (size_t)h * dh * dh;   // E[o][i]: column i = eigenvector i
    uint32_t* out = codes + ((size_t)h * n + row) * W;
    uint32_t word = 0;
    int wi = 0, off = 0;
    for (int i = 0; i < dh; ++i) {
        const int b = min((int)cb.bits[h * dh + i], 8);
        if (b <= 0) continue;
        float xr = 0.f;
        for (int o = 0; o < dh; ++o) xr = fmaf((float)x[o] * inv, E[o * dh + i], xr);
        const float c = cb.center[h * dh + i], a = cb.half[h * dh + i];
        const float levels = (float)(1u << b);
        const float t = floorf((xr - c + a) / (2.0f * a) * levels);
        const uint32_t code = t <= 0.f ? 0u : (t >= levels - 1.f ? (1u << b) - 1u : (uint32_t)t);
        word |= code << off;
        if (off + b >= 32) {
            if (wi < W) out[wi] = word;
            ++wi;
            word = off + b > 32 ? code >> (32 - off) : 0u;
            off = off + b - 32;
        } else {
            off += b;
        }
    }
    for (; wi < W; ++wi) {   // a bit table below the budget leaves zero words
        out[wi] = word;
        word = 0;
    }
}

// encode, block form: a work-group per head and 64-row block (grid-stride),
// the block's rows (fp32, padded pitch) and E_h staged in LDS.  The same
// fp32 operations in the same order as codec_encode_kernel: the norm as a
// running fmaf over the row, each rotated coordinate as a running fmaf over
// o of (x_o * inv) * E[o][i], then the quantiser and the packing.  Thread
// (row, quarter) forms a quarter of the row's coordinates (o outer, its
// coordinates inner, E rows read as broadcasts); one thread per row packs.
template <int DH>
__global__ __launch_bounds__(256) void codec_encode_block_kernel(CodecBook cb, const bf16* __restrict__ X,
                                                                 int n, int d,
                                                                 uint32_t* __restrict__ codes,
                                                                 float* __restrict__ norms) {
    constexpr int XP = DH + 1;   // row pitch (floats): a lane per row, no bank conflicts
    constexpr int NQ = DH / 4;   // coordinates per thread
    __shared__ float E[DH * DH];
    __shared__ float xs[64 * XP];
    __shared__ float invs[64];
    __shared__ int nbits[DH];
    __shared__ uint8_t cs[64 * DH];
    const int h = blockIdx.y, tid = threadIdx.x;
    const int W = cb.budget / 32;
    for (int idx = tid; idx < DH * DH; idx += 256) E[idx] = cb.rot[(size_t)h * DH * DH + idx];
    for (int i = tid; i < DH; i += 256) nbits[i] = min((int)cb.bits[h * DH + i], 8);
    const int nblk = (n + 63) / 64;
    for (int blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
        const int r0 = blk * 64, nr = min(64, n - r0);
        for (int idx = tid; idx < 64 * DH; idx += 256) {
            const int r = idx / DH, o = idx - r * DH;
            xs[r * XP + o] = r < nr ? (float)X[(size_t)(r0 + r) * d + h * DH + o] : 0.f;
        }
        __syncthreads();
        if (tid < 64) {
            float n2 = 0.f;
            for (int o = 0; o < DH; ++o) {
                const float v = xs[tid * XP + o];
                n2 = fmaf(v, v, n2);
            }
            const float nrm = sqrtf(n2);
            if (tid < nr) norms[(size_t)h * n + r0 + tid] = nrm;
            invs[tid] = nrm > 0.f ? 1.0f / nrm : 0.f;
        }
        __syncthreads();
        {
            const int r = tid & 63, i0 = (tid >> 6) * NQ;
            const float inv = invs[r];
            float xr[NQ];
#pragma unroll
            for (int k = 0; k < NQ; ++k) xr[k] = 0.f;
#pragma unroll 2
            for (int o = 0; o < DH; ++o) {
                const float xo = xs[r * XP + o] * inv;
                const float* eo = E + o * DH + i0;
#pragma unroll
                for (int k = 0; k < NQ; ++k) xr[k] = fmaf(xo, eo[k], xr[k]);
            }
#pragma unroll
            for (int k = 0; k < NQ; ++k) {
                const int i = i0 + k, b = nbits[i];
                uint32_t code = 0;
                if (b > 0) {
                    const float c = cb.center[h * DH + i], a = cb.half[h * DH + i];
                    const float levels = (float)(1u << b);
                    const float t = floorf((xr[k] - c + a) / (2.0f * a) * levels);
                    code = t <= 0.f ? 0u : (t >= levels - 1.f ? (1u << b) - 1u : (uint32_t)t);
                }
                cs[r * DH + i] = (uint8_t)code;
            }
        }
        __syncthreads();
        if (tid < nr) {
            uint32_t* out = codes + ((size_t)h * n + r0 + tid) * W;
            uint32_t word = 0;
            int wi = 0, off = 0;
            for (int i = 0; i < DH; ++i) {
                const int b = nbits[i];
                if (b <= 0) continue;
                const uint32_t code = cs[tid * DH + i];
                word |= code << off;
                if (off + b >= 32) {
                    if (wi < W) out[wi] = word;
                    ++wi;
                    word = off + b > 32 ? code >> (32 - off) : 0u;
                    off = off + b - 32;
                } else {
                    off += b;
                }
            }
            for (; wi < W; ++wi) {   // a bit table below the budget leaves zero words
                out[wi] = word;
                word = 0;
            }
        }
        __syncthreads();   // the block's LDS rows are free for the next block
    }
}

// W~[s][h*dh + i][c] = sum_o E_h[o][i] W[s][h*dh + o][c]  (fp32 sums, bf16 out)
__global__ void codec_fold_kernel(CodecBook cb, const bf16* __restrict__ Wq, int q, int d,
                                  int heads, bf16* __restrict__ Wr) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)q * d * d) return;
    const int c = (int)(idx % d);
    const int row = (int)((idx / d) % d);
    const int s = (int)(idx / ((int64_t)d * d));
    const int dh = d / heads, h = row / dh, i = row - h * dh;
    const float* E = cb.rot + (size_t)h * dh * dh;
    const bf16* w = Wq + ((size_t)s * d + h * dh) * d + c;
    float acc = 0.f;
    for (int o = 0; o < dh; ++o) acc = fmaf(E[o * dh + i], (float)w[(size_t)o * d], acc);
    Wr[idx] = (bf16)acc;
}

// ---------------------------------------------------------------------------
// attention over the coded memory
// ---------------------------------------------------------------------------
template <int DH, bool SEP, int QW>
struct CaCfg {
    static constexpr int NT = 64 * QW;              // QW waves x 32 query rows (tile_m = 32 QW)
    static constexpr int EB = DH / 32, KST = DH / 16;
    static constexpr int LDK = DH + 8;              // decoded tile pitch (16-byte rows)
    static constexpr int PLANES = SEP ? 2 : 1;
    static constexpr int TILE = kCBN * LDK;          // bf16 elements per decoded plane
    static constexpr int MAXW = DH / 4;              // words per row at 8 bits per coordinate
    static constexpr int RAWP = MAXW + 1;            // raw row pitch (words), one pad word
    static constexpr int RAW_WORDS = kCBN * RAWP;    // per plane
    static constexpr int RCPT = kCBN * MAXW / NT;    // raw words per thread per plane (at most)
    // LDS: decoded planes, raw codes + norms per plane, decode tables per
    // plane ({offset, bits, lo, step} per coordinate), output rotation.
    static constexpr int DEC_BYTES = PLANES * TILE * 2;
    static constexpr int RAW_BYTES = PLANES * (RAW_WORDS + kCBN) * 4;
    static constexpr int TAB_BYTES = PLANES * DH * 16;
    static constexpr int ROT_BYTES = DH * LDK * 2;
    static constexpr int SMEM = DEC_BYTES + RAW_BYTES + TAB_BYTES + ROT_BYTES;
};

template <int DH, bool SEP, int QW>
__global__ __launch_bounds__(64 * QW) void codec_attn_kernel(CodecArgs a) {
    using C = CaCfg<DH, SEP, QW>;
    __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
    bf16* dec = reinterpret_cast<bf16*>(smem);
    uint32_t* raw = reinterpret_cast<uint32_t*>(smem + C::DEC_BYTES);
    int4* tab = reinterpret_cast<int4*>(smem + C::DEC_BYTES + C::RAW_BYTES);
    bf16* rot = reinterpret_cast<bf16*>(smem + C::DEC_BYTES + C::RAW_BYTES + C::TAB_BYTES);

    const int q = a.q, d = a.d, heads = a.heads;
    const int* __restrict__ ws = a.plan;
    const int tile = blockIdx.x / heads;
    const int h = blockIdx.x - tile * heads;
    if (tile >= ws[kPlanNTiles] || ws[kPlanTileM] != 32 * QW) return;
    const int4 item = reinterpret_cast<const int4*>(reinterpret_cast<const char*>(ws) +
                                                    kPlanHeaderBytes)[tile];
    const int kv0 = __builtin_amdgcn_readfirstlane(item.x);
    const int L = __builtin_amdgcn_readfirstlane(item.y);
    const int c0 = __builtin_amdgcn_readfirstlane(item.z);
    const int iw = __builtin_amdgcn_readfirstlane(item.w);
    const int nc = iw & kItemNcMask, s = iw >> 16;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, l32 = lane & 31;
    const int qcol = w * 32 + l32;
    const bool qvalid = qcol < nc;
    const size_t row = (size_t)(qvalid ? c0 + qcol : c0 + nc - 1) * q + s;

    // decode tables {bit offset, bits, lo, step} and the output rotation E_V
#pragma unroll
    for (int p = 0; p < C::PLANES; ++p) {
        const uint8_t* bits = p == 0 ? a.kb.bits : a.vb.bits;
        const float* center = p == 0 ? a.kb.center : a.vb.center;
        const float* half = p == 0 ? a.kb.half : a.vb.half;
        for (int i = tid; i < DH; i += C::NT) {
            int off = 0;
            for (int j = 0; j < i; ++j) off += min((int)bits[h * DH + j], 8);
            const int b = min((int)bits[h * DH + i], 8);
            const float m = center[h * DH + i], hr = half[h * DH + i];
            const float step = b > 0 ? 2.0f * hr / (float)(1u << b) : 0.f;
            const float lo = b > 0 ? m - hr + 0.5f * step : m;
            tab[p * DH + i] = make_int4(off, b, __builtin_bit_cast(int, lo),
                                        __builtin_bit_cast(int, step));
        }
    }
    {
        const float* rv = SEP ? a.vb.rot : a.kb.rot;
        for (int idx = tid; idx < DH * DH; idx += C::NT) {
            const int e = idx / DH, i = idx - e * DH;
            rot[e * C::LDK + i] = (bf16)rv[((size_t)h * DH + e) * DH + i];
        }
    }

    // this lane's rotated query, scaled into exp2 units
    bf16x8 qb[C::KST];
    {
        const bf16* qr = static_cast<const bf16*>(a.Qr) + row * d + h * DH;
#pragma unroll
        for (int k = 0; k < C::KST; ++k) {
            bf16x8 v = *reinterpret_cast<const bf16x8*>(qr + 16 * k + 8 * g);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = (bf16)((float)v[e] * a.scale_log2);
            qb[k] = v;
        }
    }

    const int W = a.kb.budget / 32;
    const int nrows = a.total_kv;
    // raw codes of tile t (head h) into registers; rows past L read as zeros
    uint32_t rr_[C::PLANES][C::RCPT];
    float rn_[C::PLANES];
    auto gload = [&](int t) {
        const int r0 = kv0 + t * kCBN;
        const int left = L - t * kCBN;
        for (int p = 0; p < C::PLANES; ++p) {
            const uint32_t* cp = (p == 0 ? a.kcodes : a.vcodes) + ((size_t)h * nrows + r0) * W;
            const float* np_ = (p == 0 ? a.knorms : a.vnorms) + (size_t)h * nrows + r0;
            const __amdgpu_buffer_rsrc_t rc = crsrc(cp, (long long)left * W * 4);
            const __amdgpu_buffer_rsrc_t rn = crsrc(np_, (long long)left * 4);
#pragma unroll
            for (int u = 0; u < C::RCPT; ++u) {
                const int idx = tid + u * C::NT;
                rr_[p][u] = idx < kCBN * W ? __builtin_amdgcn_raw_buffer_load_b32(rc, idx * 4, 0, 0)
                                           : 0u;
            }
            rn_[p] = tid < kCBN ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                                rn, tid * 4, 0, 0))
                                : 0.f;
        }
    };
    auto rstore = [&]() {
        for (int p = 0; p < C::PLANES; ++p) {
            uint32_t* rp = raw + p * (C::RAW_WORDS + kCBN);
#pragma unroll
            for (int u = 0; u < C::RCPT; ++u) {
                const int idx = tid + u * C::NT;
                if (idx < kCBN * W) {
                    const int r = idx / W, ww = idx - r * W;
                    rp[r * C::RAWP + ww] = rr_[p][u];
                }
            }
            if (tid < kCBN) {
                rp[tid * C::RAWP + W] = 0u;   // pad word read by fields that end the row
                reinterpret_cast<float*>(rp + C::RAW_WORDS)[tid] = rn_[p];
            }
        }
    };
    // reconstruct the tile: thread (row tid % 64, part tid / 64) decodes
    // 1/QW of the row's coordinates in every plane; all QW query waves then
    // share the reconstructed tile
    auto decode = [&]() {
        const int r = tid & (kCBN - 1), hf = tid >> 6;
        for (int p = 0; p < C::PLANES; ++p) {
            const uint32_t* rp = raw + p * (C::RAW_WORDS + kCBN) + r * C::RAWP;
            const float nrm = reinterpret_cast<const float*>(raw + p * (C::RAW_WORDS + kCBN) +
                                                             C::RAW_WORDS)[r];
            bf16* out = dec + p * C::TILE + r * C::LDK;
#pragma unroll 4
            for (int i = hf * (DH / QW); i < (hf + 1) * (DH / QW); ++i) {
                const int4 tb = tab[p * DH + i];
                const int off = tb.x, b = tb.y;
                const uint32_t lo = rp[off >> 5], hi = rp[(off >> 5) + 1];
                const uint32_t v = __builtin_amdgcn_alignbit(hi, lo, off & 31) & ((1u << b) - 1u);
                out[i] = (bf16)(nrm * fmaf((float)v, __builtin_bit_cast(float, tb.w),
                                           __builtin_bit_cast(float, tb.z)));
            }
        }
    };

    const int ntiles = (L + kCBN - 1) / kCBN;
    f32x16 oacc[C::EB];
#pragma unroll
    for (int eb = 0; eb < C::EB; ++eb) oacc[eb] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;
    const int G = lane >> 4, k16 = lane & 15;
    const int tr_row = 4 * (G >> 1) + (k16 >> 2);
    const int tr_col = 16 * (G & 1) + 4 * (k16 & 3);

    gload(0);
    for (int t = 0; t < ntiles; ++t) {
        rstore();
        __syncthreads();   // raw tile and (first pass) tables visible
        gload(t + 1);
        decode();
        __syncthreads();   // decoded tile visible
        const bf16* kb = dec;
        const bf16* vb = dec + (C::PLANES - 1) * C::TILE;
        f32x16 sacc[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) sacc[hh] = f32x16{};
#pragma unroll
        for (int k = 0; k < C::KST; ++k)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
                sacc[hh] = mfma32(*reinterpret_cast<const bf16x8*>(
                                      kb + (hh * 32 + l32) * C::LDK + 16 * k + 8 * g),
                                  qb[k], sacc[hh]);
        const int jleft = L - t * kCBN;
        float mt = -INFINITY;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int j = hh * 32 + (r >> 2) * 8 + 4 * g + (r & 3);
                if (j >= jleft) sacc[hh][r] = -INFINITY;
                mt = fmaxf(mt, sacc[hh][r]);
            }
        const float m_new = fmaxf(m_run, fmaxf(mt, xor32(mt)));
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int eb = 0; eb < C::EB; ++eb) oacc[eb] *= alpha;
        bf16x8 pb[4];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const bf16 p = (bf16)__builtin_amdgcn_exp2f(sacc[hh][r] - m_new);
                l_run += (float)p;
                pb[hh * 2 + (r >> 3)][r & 7] = p;
            }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int eb = 0; eb < C::EB; ++eb) {
                const bf16* base = vb + (16 * u + tr_row) * C::LDK + eb * 32 + tr_col;
                oacc[eb] = mfma32(cat(lds_read_tr16(base), lds_read_tr16(base + 8 * C::LDK)),
                                  pb[u], oacc[eb]);
            }
        __syncthreads();   // tile consumed before the next one is written
    }
    if (ntiles == 0) __syncthreads();   // the tables and the rotation are staged

    // o = E_V o~ / l, rotated back on the matrix cores
    l_run += xor32(l_run);
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    bf16x8 ob[C::KST];
#pragma unroll
    for (int k = 0; k < C::KST; ++k)
#pragma unroll
        for (int t = 0; t < 8; ++t) ob[k][t] = (bf16)(oacc[k >> 1][8 * (k & 1) + t] * inv);
    bf16* orow = static_cast<bf16*>(a.O) + row * d + h * DH;
#pragma unroll
    for (int eo = 0; eo < C::EB; ++eo) {
        // every lane takes part in the products; only valid rows are stored
        f32x16 acc = f32x16{};
#pragma unroll
        for (int k = 0; k < C::KST; ++k) {
            // slot t of slice k is rotated feature 16k + 8(t/4) + 4g + t%4
            const bf16* rp = rot + (eo * 32 + l32) * C::LDK + 16 * k + 4 * g;
            acc = mfma32(cat(*reinterpret_cast<const bf16x4*>(rp),
                             *reinterpret_cast<const bf16x4*>(rp + 8)),
                         ob[k], acc);
        }
        if (qvalid) {
#pragma unroll
            for (int b4 = 0; b4 < 4; ++b4) {
                bf16x4 v;
#pragma unroll
                for (int t = 0; t < 4; ++t) v[t] = (bf16)acc[4 * b4 + t];
                *reinterpret_cast<bf16x4*>(orow + eo * 32 + b4 * 8 + 4 * g) = v;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// decode a coded memory into bf16 planes (for memories that many query tiles
// read: decoded once per call instead of once per query tile)
//   K plane: k^ = norm * x^ in the rotated basis (what the folded queries
//            score against);
//   V plane (separate mode): v = E_V (norm * x^), rotated back on the matrix
//            cores.
// In shared mode the one plane serves as key and value: attention then
// leaves its output in the rotated basis and codec_rotate_out_kernel turns
// it back.  bf16 roundings as in the attention kernels: x^ * norm to bf16,
// E_V to bf16, fp32 sums.
// ---------------------------------------------------------------------------
constexpr int kDR = 64;   // memory rows per decode block

template <int DH, bool SEP>
struct CdCfg {
    static constexpr int NT = 256;
    static constexpr int EB = DH / 32, KST = DH / 16;
    static constexpr int PLANES = SEP ? 2 : 1;       // coded planes
    static constexpr int LDK = DH + 8;               // decoded row pitch (16-byte rows)
    static constexpr int MAXW = DH / 4;              // words per row at 8 bits per coordinate
    static constexpr int RAWP = MAXW + 1;            // raw row pitch (words), one pad word
    static constexpr int TAB_BYTES = PLANES * DH * 16;
    static constexpr int ROT_BYTES = DH * LDK * 2;
    static constexpr int RAW_BYTES = PLANES * kDR * (RAWP + 1) * 4;
    static constexpr int ROW_BYTES = kDR * LDK * 2;  // one decoded 64-row plane
    static constexpr int SMEM = TAB_BYTES + (SEP ? ROT_BYTES : 0) + RAW_BYTES +
                                (PLANES + (SEP ? 1 : 0)) * ROW_BYTES;
};

template <int DH, bool SEP>
__global__ __launch_bounds__(256) void codec_decode_kernel(CodecDecodeArgs a) {
    using C = CdCfg<DH, SEP>;
    __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
    constexpr int ROT = SEP ? C::ROT_BYTES : 0;
    int4* tab = reinterpret_cast<int4*>(smem);
    bf16* rot = reinterpret_cast<bf16*>(smem + C::TAB_BYTES);
    uint32_t* raw = reinterpret_cast<uint32_t*>(smem + C::TAB_BYTES + ROT);
    bf16* xd = reinterpret_cast<bf16*>(smem + C::TAB_BYTES + ROT + C::RAW_BYTES);
    bf16* ov = xd + C::PLANES * kDR * C::LDK;

    const int h = blockIdx.y, d = a.d, n = a.total_kv;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, l32 = lane & 31;
    const int W = a.kb.budget / 32;

    // decode tables {bit offset, bits, lo, step} per plane, and E_V (bf16)
#pragma unroll
    for (int p = 0; p < C::PLANES; ++p) {
        const uint8_t* bits = p == 0 ? a.kb.bits : a.vb.bits;
        const float* center = p == 0 ? a.kb.center : a.vb.center;
        const float* half = p == 0 ? a.kb.half : a.vb.half;
        for (int i = tid; i < DH; i += C::NT) {
            int off = 0;
            for (int j = 0; j < i; ++j) off += min((int)bits[h * DH + j], 8);
            const int b = min((int)bits[h * DH + i], 8);
            const float m = center[h * DH + i], hr = half[h * DH + i];
            const float step = b > 0 ? 2.0f * hr / (float)(1u << b) : 0.f;
            const float lo = b > 0 ? m - hr + 0.5f * step : m;
            tab[p * DH + i] = make_int4(off, b, __builtin_bit_cast(int, lo),
                                        __builtin_bit_cast(int, step));
        }
    }
    if constexpr (SEP) {
        for (int idx = tid; idx < DH * DH; idx += C::NT) {
            const int e = idx / DH, i = idx - e * DH;
            rot[e * C::LDK + i] = (bf16)a.vb.rot[((size_t)h * DH + e) * DH + i];
        }
    }

    const int nblk = (n + kDR - 1) / kDR;
    for (int blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
        const int r0 = blk * kDR, nr = min(kDR, n - r0);
        // raw codes and norms of the block (rows past the memory read as zeros)
#pragma unroll
        for (int p = 0; p < C::PLANES; ++p) {
            const uint32_t* cp = (p == 0 ? a.kcodes : a.vcodes) + ((size_t)h * n + r0) * W;
            const float* np_ = (p == 0 ? a.knorms : a.vnorms) + (size_t)h * n + r0;
            uint32_t* rp = raw + p * kDR * (C::RAWP + 1);
            for (int idx = tid; idx < kDR * W; idx += C::NT) {
                const int r = idx / W, ww = idx - r * W;
                rp[r * C::RAWP + ww] = r < nr ? cp[idx] : 0u;
            }
            if (tid < kDR) {
                rp[tid * C::RAWP + W] = 0u;   // pad word read by fields that end the row
                reinterpret_cast<float*>(rp + kDR * C::RAWP)[tid] = tid < nr ? np_[tid] : 0.f;
            }
        }
        __syncthreads();
        // thread (row tid % 64, quarter tid / 64) decodes a quarter of the
        // row's coordinates in every plane
        {
            const int r = tid & (kDR - 1), part = tid >> 6;
#pragma unroll
            for (int p = 0; p < C::PLANES; ++p) {
                const uint32_t* rp = raw + p * kDR * (C::RAWP + 1) + r * C::RAWP;
                const float nrm =
                    reinterpret_cast<const float*>(raw + p * kDR * (C::RAWP + 1) + kDR * C::RAWP)[r];
                bf16* out = xd + (p * kDR + r) * C::LDK;
#pragma unroll 4
                for (int i = part * (DH / 4); i < (part + 1) * (DH / 4); ++i) {
                    const int4 tb = tab[p * DH + i];
                    const int off = tb.x, b = tb.y;
                    const uint32_t lo = rp[off >> 5], hi = rp[(off >> 5) + 1];
                    const uint32_t v = __builtin_amdgcn_alignbit(hi, lo, off & 31) & ((1u << b) - 1u);
                    out[i] = (bf16)(nrm * fmaf((float)v, __builtin_bit_cast(float, tb.w),
                                               __builtin_bit_cast(float, tb.z)));
                }
            }
        }
        __syncthreads();
        // K plane rows (rotated basis), 16-byte chunks
        for (int idx = tid; idx < kDR * (DH / 8); idx += C::NT) {
            const int r = idx / (DH / 8), c8 = idx - r * (DH / 8);
            if (r < nr)
                *reinterpret_cast<uint4*>(static_cast<bf16*>(a.Kout) + (size_t)(r0 + r) * d + h * DH + 8 * c8) =
                    *reinterpret_cast<const uint4*>(xd + r * C::LDK + 8 * c8);
        }
        if constexpr (SEP) {
        // V plane: rows x^ (32rb..) times E_V^T (features 32eb..) on the
        // matrix cores; accumulator register t holds row 32rb + (t/4)*8 +
        // 4g + t%4, feature 32eb + l32
        const bf16* xv = xd + kDR * C::LDK;
        for (int blk2 = w; blk2 < 2 * C::EB; blk2 += C::NT / 64) {
            const int rb = blk2 & 1, eb = blk2 >> 1;
            f32x16 acc = f32x16{};
#pragma unroll
            for (int kk = 0; kk < C::KST; ++kk)
                acc = mfma32(*reinterpret_cast<const bf16x8*>(xv + (32 * rb + l32) * C::LDK + 16 * kk + 8 * g),
                             *reinterpret_cast<const bf16x8*>(rot + (32 * eb + l32) * C::LDK + 16 * kk + 8 * g),
                             acc);
#pragma unroll
            for (int t = 0; t < 16; ++t)
                ov[(32 * rb + (t >> 2) * 8 + 4 * g + (t & 3)) * C::LDK + 32 * eb + l32] = (bf16)acc[t];
        }
        __syncthreads();
        for (int idx = tid; idx < kDR * (DH / 8); idx += C::NT) {
            const int r = idx / (DH / 8), c8 = idx - r * (DH / 8);
            if (r < nr)
                *reinterpret_cast<uint4*>(static_cast<bf16*>(a.Vout) + (size_t)(r0 + r) * d + h * DH + 8 * c8) =
                    *reinterpret_cast<const uint4*>(ov + r * C::LDK + 8 * c8);
        }
        }
        __syncthreads();   // the block's LDS rows are free for the next block
    }
}

// Output rows of attention over a shared-mode decoded plane are in the
// rotated basis: O_h <- E_h O_h per row and head, in place (bf16 in, fp32
// products on the matrix cores, bf16 out).
template <int DH>
__global__ __launch_bounds__(256) void codec_rotate_out_kernel(CodecBook cb, void* Ov, int rows,
                                                               int d) {
    constexpr int LDK = DH + 8, EB = DH / 32, KST = DH / 16;
    __shared__ __attribute__((aligned(16))) bf16 rot[DH * LDK];
    __shared__ __attribute__((aligned(16))) bf16 xo[2][kDR * LDK];
    bf16* O = static_cast<bf16*>(Ov);
    const int h = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, l32 = lane & 31;
    for (int idx = tid; idx < DH * DH; idx += 256) {
        const int e = idx / DH, i = idx - e * DH;
        rot[e * LDK + i] = (bf16)cb.rot[((size_t)h * DH + e) * DH + i];
    }
    const int nblk = (rows + kDR - 1) / kDR;
    for (int blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
        const int r0 = blk * kDR, nr = min(kDR, rows - r0);
        for (int idx = tid; idx < kDR * (DH / 8); idx += 256) {
            const int r = idx / (DH / 8), c8 = idx - r * (DH / 8);
            *reinterpret_cast<uint4*>(&xo[0][r * LDK + 8 * c8]) =
                r < nr ? *reinterpret_cast<const uint4*>(O + (size_t)(r0 + r) * d + h * DH + 8 * c8)
                       : uint4{};
        }
        __syncthreads();
        // rows (32rb..) times E^T (features 32eb..); register t holds row
        // 32rb + (t/4)*8 + 4g + t%4, feature 32eb + l32
        for (int b2 = w; b2 < 2 * EB; b2 += 4) {
            const int rb = b2 & 1, eb = b2 >> 1;
            f32x16 acc = f32x16{};
#pragma unroll
            for (int kk = 0; kk < KST; ++kk)
                acc = mfma32(*reinterpret_cast<const bf16x8*>(&xo[0][(32 * rb + l32) * LDK + 16 * kk + 8 * g]),
                             *reinterpret_cast<const bf16x8*>(&rot[(32 * eb + l32) * LDK + 16 * kk + 8 * g]),
                             acc);
#pragma unroll
            for (int t = 0; t < 16; ++t)
                xo[1][(32 * rb + (t >> 2) * 8 + 4 * g + (t & 3)) * LDK + 32 * eb + l32] = (bf16)acc[t];
        }
        __syncthreads();
        for (int idx = tid; idx < kDR * (DH / 8); idx += 256) {
            const int r = idx / (DH / 8), c8 = idx - r * (DH / 8);
            if (r < nr)
                *reinterpret_cast<uint4*>(O + (size_t)(r0 + r) * d + h * DH + 8 * c8) =
                    *reinterpret_cast<const uint4*>(&xo[1][r * LDK + 8 * c8]);
        }
        __syncthreads();
    }
}

template <int DH, int QW>
hipError_t launch_codec_qw(const CodecArgs& a, bool sep, int64_t items, hipStream_t stream) {
    const dim3 grid((unsigned)(items * a.heads));
    if (sep)
        hipLaunchKernelGGL((codec_attn_kernel<DH, true, QW>), grid, dim3(64 * QW), 0, stream, a);
    else
        hipLaunchKernelGGL((codec_attn_kernel<DH, false, QW>), grid, dim3(64 * QW), 0, stream, a);
    return hipGetLastError();
}

template <int DH>
hipError_t launch_codec_dh(const CodecArgs& a, bool sep, int qw, int64_t items,
                           hipStream_t stream) {
    if (items <= 0) return hipSuccess;
    switch (qw) {
        case 2: return launch_codec_qw<DH, 2>(a, sep, items, stream);
        case 4: return launch_codec_qw<DH, 4>(a, sep, items, stream);
        case 8: return launch_codec_qw<DH, 8>(a, sep, items, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_codec_encode(const CodecBook& cb, const void* X, int n, int d, int heads,
                               uint32_t* codes, float* norms, hipStream_t stream) {
    const int64_t m = (int64_t)n * heads;
    if (m <= 0) return hipSuccess;
    const int dh = d / heads;
    const int nblk = (n + 63) / 64;
    const dim3 grid((unsigned)(nblk < 512 ? nblk : 512), (unsigned)heads);
    const bf16* x = static_cast<const bf16*>(X);
    switch (dh) {
        case 32: hipLaunchKernelGGL(codec_encode_block_kernel<32>, grid, dim3(256), 0, stream, cb, x, n, d, codes, norms); break;
        case 64: hipLaunchKernelGGL(codec_encode_block_kernel<64>, grid, dim3(256), 0, stream, cb, x, n, d, codes, norms); break;
        case 128: hipLaunchKernelGGL(codec_encode_block_kernel<128>, grid, dim3(256), 0, stream, cb, x, n, d, codes, norms); break;
        default:   // other head widths: one thread per (row, head)
            hipLaunchKernelGGL(codec_encode_kernel, dim3((unsigned)((m + 127) / 128)), dim3(128), 0,
                               stream, cb, x, n, d, heads, codes, norms);
    }
    return hipGetLastError();
}

hipError_t launch_codec_fold(const CodecBook& cb, const void* Wq, int q, int d, int heads,
                             void* Wr, hipStream_t stream) {
    const int64_t m = (int64_t)q * d * d;
    if (m <= 0) return hipSuccess;
    hipLaunchKernelGGL(codec_fold_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, stream,
                       cb, static_cast<const bf16*>(Wq), q, d, heads, static_cast<bf16*>(Wr));
    return hipGetLastError();
}

hipError_t launch_codec_decode(const CodecDecodeArgs& a, bool sep, int heads, int grid_x,
                               hipStream_t stream) {
    if (a.total_kv <= 0) return hipSuccess;
    const int nblk = (a.total_kv + kDR - 1) / kDR;
    const dim3 grid((unsigned)(grid_x < nblk ? grid_x : nblk), (unsigned)heads);
#define XATTN_DEC(DH_)                                                                    \
    if (a.d / heads == DH_) {                                                            \
        if (sep)                                                                         \
            hipLaunchKernelGGL((codec_decode_kernel<DH_, true>), grid, dim3(256), 0, stream, a);  \
        else                                                                             \
            hipLaunchKernelGGL((codec_decode_kernel<DH_, false>), grid, dim3(256), 0, stream, a); \
        return hipGetLastError();                                                        \
    }
    XATTN_DEC(32)
    XATTN_DEC(64)
    XATTN_DEC(128)
#undef XATTN_DEC
    return hipErrorInvalidValue;
}

hipError_t launch_codec_rotate_out(const CodecBook& cb, void* O, int rows, int d, int heads,
                                   int grid_x, hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    const int nblk = (rows + kDR - 1) / kDR;
    const dim3 grid((unsigned)(grid_x < nblk ? grid_x : nblk), (unsigned)heads);
    switch (d / heads) {
        case 32: hipLaunchKernelGGL(codec_rotate_out_kernel<32>, grid, dim3(256), 0, stream, cb, O, rows, d); break;
        case 64: hipLaunchKernelGGL(codec_rotate_out_kernel<64>, grid, dim3(256), 0, stream, cb, O, rows, d); break;
        case 128: hipLaunchKernelGGL(codec_rotate_out_kernel<128>, grid, dim3(256), 0, stream, cb, O, rows, d); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_codec_attn(const CodecArgs& a, bool sep, int qw, int64_t items,
                             hipStream_t stream) {
    switch (a.d / a.heads) {
        case 32: return launch_codec_dh<32>(a, sep, qw, items, stream);
        case 64: return launch_codec_dh<64>(a, sep, qw, items, stream);
        case 128: return launch_codec_dh<128>(a, sep, qw, items, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace xattn
