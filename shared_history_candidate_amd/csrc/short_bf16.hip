// Short-memory cross-attention with the TSP query projection in the same
// kernel, bf16 in, fp32 accumulate, bf16 out, for gfx950 matrix cores.
//
// It computes what the projection GEMM (gemm_bf16.hip) followed by
// attn_bf16_kernel computes:
//   Q   = Z W_Q[s]                  (ReST reading note s.3.3.2, Eq. (8)),
//         rounded to bf16 once (the softmax scale log2(e)/sqrt(d_h) is
//         applied to the fp32 scores, in the same FMA that subtracts the
//         running maximum, instead of to a second bf16 copy of Q);
//   O_h = softmax(Q_h K_h^T / sqrt(d_h)) V_h
//         (ReST reading note s.3.3.1 Eq. (7); separate K and V for the
//         TransX behaviour memory, TransX report s.2)
// on a model of d = 256 features.  It is built for memories short enough
// that every head's keys and values of a request fit in LDS together (the
// TransX memory of 64 recent rows and 32 chunk summaries): up to 96 rows with
// separate K and V, 192 rows with K = V.  Longer memories are streamed
// through LDS in chunks of that many rows (correct, but without overlap).
//
// Why one kernel: with one query token per candidate and a memory of ~100
// rows, the queries are the bulk of the traffic.  A separate projection
// writes Q to HBM and the attention reads it back (2 x 2 bytes per query
// feature on top of Z in and O out); here Q lives only in LDS.
//
// Work decomposition.  A persistent grid of one 8-wave work-group per compute
// unit walks the plan's work items in order: work-group i takes items
// [i T / G, (i + 1) T / G).  The plan keeps the items of a request adjacent,
// so a request's memory is staged once per work-group that meets it.  Items
// are processed in chunks of 64 query rows:
//   1. Projection on the matrix cores.  Wave w holds rows 32w..32w+31 of
//      W_Q[s] (its 32 output features over all 256 inputs) in registers as A
//      operands, reloaded only when the slot changes; the chunk's Z rows sit
//      in LDS and every wave reads them as B operands.  The next chunk's Z
//      rows are loaded into registers meanwhile and written to LDS at the
//      end of the chunk.
//   2. The Q chunk (bf16, rows x features) overwrites the Z chunk in LDS.
//   3. Attention.  The units (head h, 32-row query block; with 128-wide
//      heads also one half of the head's output features, so that all eight
//      waves have work) are dealt to the waves round-robin.  Per 32-row
//      memory block: scores
//      S^T = K_h . Q_h^T (lane = query row), the online softmax of
//      attn_bf16_kernel (exp2 domain, maximum set by the first block and
//      moved only when a lane's weights of a block sum past 2^12), and
//      O^T += V_h^T . P^T with V^T from LDS transpose reads.
#include "common.h"
#include "internal.h"
#include "plan_device.h"

namespace xattn {

namespace {

constexpr int D = kShortD;       // model features
constexpr int NW = 8;            // waves per work-group
constexpr int NT = 64 * NW;
constexpr int QR = 64;           // query rows per chunk
constexpr int LDK = D + 8;       // LDS pitch (elements) of Z, Q, K and V rows: 16-byte rows
constexpr int MB = 32;           // memory rows per score block
constexpr int kRing = 256;       // work items held in LDS at a time
constexpr float kSumCap = 4096.0f;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int DH, bool SEP, bool CODEC>
struct SCfg {
    // a coded memory always stages two planes: keys in the rotated basis,
    // values rotated back (both decoded from the codes)
    static constexpr int PLANES = SEP || CODEC ? 2 : 1;
    static constexpr int LMAX = short_max_rows(SEP || CODEC);   // memory rows resident at once
    static constexpr int HEADS = D / DH;
    static constexpr int EB = DH / 32;                 // 32-wide feature blocks of a head
    static constexpr int KST = DH / 16;                // k-steps of the score product
    // A unit is (head, 32-row query block, part of the head's output
    // features): wide heads split their output features over two waves (both
    // compute the unit's scores) so that every wave has work.
    static constexpr int FP = 2 * (D / DH) < NW ? NW / (2 * (D / DH)) : 1;
    static constexpr int EBW = EB / FP;                // output feature blocks per unit
    static constexpr int UNITS = 2 * (D / DH) * FP;
    static constexpr int UPW = UNITS / NW;             // units per wave
    static_assert(UNITS % NW == 0, "every wave has the same number of units");
    static constexpr int KV_ELEMS = PLANES * LMAX * LDK;
    static constexpr int ZQ_OFF = KV_ELEMS * 2;        // byte offset of the Z / Q chunk
    // the plan built in the kernel (exclusive scan of the requests' item
    // counts; not with a coded memory, whose decode tables and code staging
    // take its place) and the ring of this work-group's next work items
    static constexpr int PLAN_OFF = ZQ_OFF + QR * LDK * 2;
    static constexpr int PLAN_BYTES = CODEC ? 0 : (((kPlanMaxRequests + 1 + 16 + 1) * 4 + 15) & ~15);
    static constexpr int RING_OFF = PLAN_OFF + PLAN_BYTES;
    // coded memory: {bit offset, bits, lo, step} per plane and feature, and
    // the codes + norm of one 32-row block per (row, head), with a pad word
    // read by fields that end a row
    static constexpr int TAB_OFF = RING_OFF + kRing * 16;
    static constexpr int TAB_BYTES = CODEC ? 2 * D * 16 : 0;
    static constexpr int RAWP = DH / 4 + 1;            // words per (row, head) at 8 bits per coordinate, + pad
    static constexpr int RAW_OFF = TAB_OFF + TAB_BYTES;
    static constexpr int RAW_BYTES = CODEC ? MB * HEADS * (RAWP + 1) * 4 : 0;
    static constexpr int SMEM = RAW_OFF + RAW_BYTES;
    static constexpr int KV_CPT = LMAX * (D / 8) / NT;  // 16-byte memory chunks per thread per plane
    static constexpr int Z_CPT = QR * (D / 8) / NT;     // 16-byte Z chunks per thread
    static_assert(LMAX * (D / 8) % NT == 0 && QR * (D / 8) % NT == 0, "even staging split");
    static_assert(LMAX % MB == 0, "whole score blocks");
    // memory blocks attended in one pass (unit_exact): up to three, for
    // 64-wide heads (with 32- and 128-wide heads the kernel's registers do
    // not hold their scores: the compiler spills)
    static constexpr int NBX = CODEC || DH != 64 ? 0 : (LMAX / MB < 3 ? LMAX / MB : 3);
};

// One query chunk: candidates [cb, cb + nr) of a request, slot s.
struct Chunk {
    int kv0, L, c0, nc, s;   // the work item
    int j;                   // chunk index inside the item
};

template <int DH, bool SEP, bool CODEC>
__global__ __launch_bounds__(NT) void short_bf16_kernel(AttnArgs a, ShortCodec cd) {
    using C = SCfg<DH, SEP, CODEC>;
    constexpr int LMAX = C::LMAX;
    __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
    bf16* kvs = reinterpret_cast<bf16*>(smem);                 // K rows, then V rows (SEP)
    bf16* zq = reinterpret_cast<bf16*>(smem + C::ZQ_OFF);     // Z, then Q, of one chunk
    const bf16* vsrc = kvs + (SEP || CODEC ? LMAX * LDK : 0);

    const int q = a.q;
    const float scale_log2 = a.scale_log2;
    const bf16* __restrict__ Z = static_cast<const bf16*>(a.Z);
    const bf16* __restrict__ Wq = static_cast<const bf16*>(a.Wq);
    const bf16* __restrict__ K = static_cast<const bf16*>(a.K);
    const bf16* __restrict__ V = static_cast<const bf16*>(a.V);
    bf16* __restrict__ O = static_cast<bf16*>(a.O);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, l32 = lane & 31;
    const int tile_m = a.tile_m, R = a.R;
    int* plan_pre = reinterpret_cast<int*>(smem + C::PLAN_OFF);   // [R + 1]
    int* plan_part = plan_pre + kPlanMaxRequests + 1;              // [16]
    int* plan_red = plan_part + 16;
    int4* ring = reinterpret_cast<int4*>(smem + C::RING_OFF);

    // ---------------- the work list ----------------
    // Forward (a.inplan): every work-group plans the batch itself, in request
    // order (the varlen planner of plan_device.h with rank = false: request r
    // contributes q * ceil(N_r / tile_m) items {kv0, L, c0, nc | s << 16},
    // candidate blocks ascending, slots inside a block), after checking the
    // offsets; work-group 0 writes the plan header and every work-group
    // publishes its own items, so that later calls can reuse the plan.
    // Otherwise the plan in the workspace is read (none if it failed
    // validation, T = 0, or was built for another tile size, i.e. another
    // batch shape).
    const int* __restrict__ cu_kv = a.cu_kv;
    const int* __restrict__ cu_cand = a.cu_cand;
    int* wsw = static_cast<int*>(a.ws);
    int4* tiles = reinterpret_cast<int4*>(static_cast<char*>(a.ws) + kPlanHeaderBytes);
    int T;
    if (!CODEC && a.inplan) {
        int err = 0;
        if (tid == 0) {
            if (cu_kv[0] != 0 || cu_kv[R] != a.total_kv) err |= kErrCuKv;
            if (cu_cand[0] != 0 || cu_cand[R] != a.total_cand) err |= kErrCuCand;
            *plan_red = 0;
        }
        for (int r = tid; r < R; r += NT) {
            if (cu_kv[r + 1] < cu_kv[r]) err |= kErrCuKv;
            if (cu_cand[r + 1] < cu_cand[r]) err |= kErrCuCand;
        }
        __syncthreads();
        if (err) atomicOr(plan_red, err);
        __syncthreads();
        err = *plan_red;
        T = 0;
        if (!err) {
            for (int r = tid; r < R; r += NT) {
                const int n = cu_cand[r + 1] - cu_cand[r];
                plan_pre[r] = q * ((n + tile_m - 1) / tile_m);
            }
            __syncthreads();
            T = plan_exclusive_scan<NT>(plan_pre, R, plan_part);
        }
        if (blockIdx.x == 0 && tid == 0) {
            wsw[kPlanNTiles] = T;
            wsw[kPlanError] = err;
            wsw[kPlanTileM] = tile_m;
        }
    } else {
        T = wsw[kPlanTileM] == tile_m ? wsw[kPlanNTiles] : 0;
    }
    T = __builtin_amdgcn_readfirstlane(T);
    const int G = gridDim.x;
    const int i_end = (int)((int64_t)(blockIdx.x + 1) * T / G);
    int ii = (int)((int64_t)blockIdx.x * T / G);
    if (ii >= i_end) return;

    // items [first, first + kRing) of this work-group's range into the ring
    int ring_base = ii;
    auto fill_ring = [&](int first) {
        __syncthreads();   // no wave reads the ring any more
        for (int k = tid; k < kRing && first + k < i_end; k += NT) {
            const int i = first + k;
            int4 it;
            if (!CODEC && a.inplan) {
                int lo = 0, hi = R;   // largest r with pre[r] <= i (skips empty requests)
                while (hi - lo > 1) {
                    const int mid = (lo + hi) >> 1;
                    if (plan_pre[mid] <= i) lo = mid; else hi = mid;
                }
                const int local = i - plan_pre[lo], b = local / q, sl = local - b * q;
                const int c_lo = cu_cand[lo], n = cu_cand[lo + 1] - c_lo;
                const int kv0 = cu_kv[lo];
                it = make_int4(kv0, cu_kv[lo + 1] - kv0, c_lo + b * tile_m,
                               min(tile_m, n - b * tile_m) | (sl << 16));
                tiles[i] = it;
            } else {
                it = tiles[i];
            }
            ring[k] = it;
        }
        ring_base = first;
        __syncthreads();
    };
    fill_ring(ii);

    // item i (uniform); refills the ring when i has run past it
    auto load_item = [&](int i, Chunk& c) {
        if (i - ring_base >= kRing) fill_ring(i);
        const int4 it = ring[i - ring_base];
        c.kv0 = __builtin_amdgcn_readfirstlane(it.x);
        c.L = __builtin_amdgcn_readfirstlane(it.y);
        c.c0 = __builtin_amdgcn_readfirstlane(it.z);
        const int iw = __builtin_amdgcn_readfirstlane(it.w);
        c.nc = iw & kItemNcMask;
        c.s = iw >> 16;
        c.j = 0;
    };

    // Z rows of a chunk -> registers.  Rows past the chunk's candidates lie
    // outside the descriptor and read as zeros.
    uint4 zr[C::Z_CPT];
    auto zload = [&](const Chunk& c) {
        const int cb = c.c0 + c.j * QR, nr = min(QR, c.nc - c.j * QR);
        const uint32_t bytes = (uint32_t)(((size_t)(nr - 1) * q + 1) * D * 2);
        const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(Z + ((size_t)cb * q + c.s) * D), (short)0, bytes, 0x00020000);
#pragma unroll
        for (int u = 0; u < C::Z_CPT; ++u) {
            const int idx = tid + u * NT, row = idx >> 5, col = idx & 31;
            zr[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rz, (row * q * D + col * 8) * 2, 0, 0));
        }
    };
    auto zstore = [&]() {
#pragma unroll
        for (int u = 0; u < C::Z_CPT; ++u) {
            const int idx = tid + u * NT, row = idx >> 5, col = idx & 31;
            *reinterpret_cast<uint4*>(zq + row * LDK + col * 8) = zr[u];
        }
    };

    // This wave's 32 rows of W_Q[s]: k-step kk holds inputs 16kk + 8g .. +7
    // of output feature 32w + l32.
    bf16x8 wa[D / 16];
    auto wload = [&](int s) {
        const bf16* wr = Wq + ((size_t)s * D + 32 * w + l32) * D + 8 * g;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) wa[kk] = *reinterpret_cast<const bf16x8*>(wr + 16 * kk);
    };

    // Coded memory (TransX report s.3; codec_bf16.hip): per plane (0: keys,
    // 1: values; with K = V both decode the key codes) and feature h*DH + i,
    // {bit offset, bits, lo, step} of coordinate i of head h, so that the
    // rotated coordinate is lo + code * step (the cell centre; lo = centre
    // and step = 0 for a coordinate without bits).
    if constexpr (CODEC) {
        int4* tab = reinterpret_cast<int4*>(smem + C::TAB_OFF);
        for (int idx = tid; idx < 2 * D; idx += NT) {
            const int p = idx / D, f = idx - p * D, h = f / DH, i = f - h * DH;
            const CodecBook& cb = p == 1 && SEP ? cd.vb : cd.kb;
            int off = 0;
            for (int j = 0; j < i; ++j) off += min((int)cb.bits[h * DH + j], 8);
            const int b = min((int)cb.bits[f], 8);
            const float m = cb.center[f], hr = cb.half[f];
            const float step = b > 0 ? 2.0f * hr / (float)(1u << b) : 0.f;
            const float lo = b > 0 ? m - hr + 0.5f * step : m;
            tab[idx] = make_int4(off, b, __builtin_bit_cast(int, lo), __builtin_bit_cast(int, step));
        }
        // visible to the decode behind the first staging barrier
    }

    // Memory rows [row0, row0 + nr) of K (and V) for all heads -> LDS rows
    // 0..LMAX-1; rows past nr read as zeros, so that the V rows behind a
    // partial score block are finite.
    int st_row0 = -1, st_rows = -1;
    auto kv_stage = [&](int row0, int nr) {
      if constexpr (CODEC) {
        // Decode 32-row blocks of codes, plane by plane, through LDS: the
        // key plane keeps the rotated basis (the queries come from W_Q
        // folded into it); the value plane is rotated back on the matrix
        // cores, V = norm * E x^, so that the attention needs no output
        // rotation.  Rows past nr get norm 0, i.e. zero rows.
        const int W = cd.kb.budget / 32;
        const int nkv = cd.total_kv;
        uint32_t* raw = reinterpret_cast<uint32_t*>(smem + C::RAW_OFF);
        float* rnorm = reinterpret_cast<float*>(raw + MB * C::HEADS * C::RAWP);
        const int4* tab = reinterpret_cast<const int4*>(smem + C::TAB_OFF);
        // rotated coordinate f = h*DH + i of row r of the staged block, times its norm
        auto decode = [&](int pl, int r, int f) {
            const int h = f / DH;
            const int4 tb = tab[pl * D + f];
            const uint32_t* rp = raw + (r * C::HEADS + h) * C::RAWP;
            const uint32_t v = __builtin_amdgcn_alignbit(rp[(tb.x >> 5) + 1], rp[tb.x >> 5], tb.x & 31) &
                               ((1u << tb.y) - 1u);
            return (bf16)(rnorm[r * C::HEADS + h] *
                          fmaf((float)v, __builtin_bit_cast(float, tb.w), __builtin_bit_cast(float, tb.z)));
        };
        for (int pl = 0; pl < 2; ++pl) {
            const uint32_t* codes = pl == 1 && SEP ? cd.vcodes : cd.kcodes;
            const float* norms = pl == 1 && SEP ? cd.vnorms : cd.knorms;
            for (int r0 = 0; r0 < LMAX; r0 += MB) {
                __syncthreads();   // the previous block's decode is done with the staging area
                for (int idx = tid; idx < MB * C::HEADS * W; idx += NT) {
                    const int rh = idx / W, wd = idx - rh * W, r = rh / C::HEADS, h = rh - r * C::HEADS;
                    raw[rh * C::RAWP + wd] =
                        r0 + r < nr ? codes[((size_t)h * nkv + row0 + r0 + r) * W + wd] : 0u;
                }
                for (int rh = tid; rh < MB * C::HEADS; rh += NT) {
                    const int r = rh / C::HEADS, h = rh - r * C::HEADS;
                    raw[rh * C::RAWP + W] = 0u;
                    rnorm[rh] = r0 + r < nr ? norms[(size_t)h * nkv + row0 + r0 + r] : 0.f;
                }
                __syncthreads();
                if (pl == 0) {
                    for (int e = tid; e < MB * D; e += NT) {
                        const int r = e / D, f = e - r * D;
                        kvs[(r0 + r) * LDK + f] = decode(0, r, f);
                    }
                } else {
                    // wave w: head h, output features 32eb.. of it (heads x DH/32 = 8 pairs):
                    // C[row][o] = sum_i x^[row][i] E[32eb + o][i] with x^ decoded
                    // straight into the A operand (rows = lanes' l32)
                    constexpr int EBH = DH / 32;
                    const int h = w / EBH, eb = w - h * EBH;
                    const CodecBook& cb = SEP ? cd.vb : cd.kb;
                    const float* er = cb.rot + ((size_t)h * DH + 32 * eb + l32) * DH + 8 * g;
                    f32x16 vacc = f32x16{};
#pragma unroll
                    for (int kk = 0; kk < C::KST; ++kk) {
                        bf16x8 xa, eo;
#pragma unroll
                        for (int t = 0; t < 8; ++t) {
                            xa[t] = decode(1, l32, h * DH + 16 * kk + 8 * g + t);
                            eo[t] = (bf16)er[16 * kk + t];
                        }
                        vacc = mfma32(xa, eo, vacc);
                    }
                    // vacc reg rr: row (rr/4)*8 + 4g + rr%4, output feature 32eb + l32
#pragma unroll
                    for (int rr = 0; rr < 16; ++rr)
                        kvs[(LMAX + r0 + (rr >> 2) * 8 + 4 * g + (rr & 3)) * LDK + h * DH + 32 * eb + l32] =
                            (bf16)vacc[rr];
                }
            }
        }
        __syncthreads();
        st_row0 = row0;
        st_rows = nr;
      } else {
        const uint32_t bytes = (uint32_t)nr * D * 2;
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(K + (size_t)row0 * D), (short)0, bytes, 0x00020000);
        uint4 kr[C::KV_CPT], vr[SEP ? C::KV_CPT : 1];
#pragma unroll
        for (int u = 0; u < C::KV_CPT; ++u) {
            const int idx = tid + u * NT, row = idx >> 5, col = idx & 31;
            kr[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rk, (row * D + col * 8) * 2, 0, 0));
        }
        if constexpr (SEP) {
            const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(V + (size_t)row0 * D), (short)0, bytes, 0x00020000);
#pragma unroll
            for (int u = 0; u < C::KV_CPT; ++u) {
                const int idx = tid + u * NT, row = idx >> 5, col = idx & 31;
                vr[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                      rv, (row * D + col * 8) * 2, 0, 0));
            }
        }
#pragma unroll
        for (int u = 0; u < C::KV_CPT; ++u) {
            const int idx = tid + u * NT, row = idx >> 5, col = idx & 31;
            *reinterpret_cast<uint4*>(kvs + row * LDK + col * 8) = kr[u];
            if constexpr (SEP) *reinterpret_cast<uint4*>(kvs + (LMAX + row) * LDK + col * 8) = vr[u];
        }
        st_row0 = row0;
        st_rows = nr;
      }
    };

    // transposed V read: lane l receives V[16u + 4g + t][col + l%32], t = 0..3
    const int G16 = lane >> 4, k16 = lane & 15;
    const int tr_row = 4 * (G16 >> 1) + (k16 >> 2);
    const int tr_col = 16 * (G16 & 1) + 4 * (k16 & 3);
    const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};

    // ---------------- prologue: first chunk's Z in LDS, W_Q rows in registers ----------------
    Chunk cur;
    load_item(ii, cur);
    int wslot = cur.s;
    wload(wslot);
    zload(cur);
    zstore();   // its wait covers the W_Q rows loaded before the Z rows
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) asm volatile("" : "+v"(wa[kk]));

    for (;;) {
        // the chunk after this one (possibly in the next item)
        Chunk nxt = cur;
        bool has_next = true;
        if ((cur.j + 1) * QR < cur.nc) {
            nxt.j = cur.j + 1;
        } else if (ii + 1 < i_end) {
            load_item(ii + 1, nxt);
        } else {
            has_next = false;
        }
        __syncthreads();   // Z chunk in LDS; every wave is done with the previous chunk's memory
        if (has_next) zload(nxt);
        if (cur.s != wslot) {
            // a new slot (rare): wait for its rows here, so that the
            // projection below never waits on the vector-memory counter
            // (which would also hold it for the Z rows loaded above)
            wslot = cur.s;
            wload(wslot);
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) asm volatile("" : "+v"(wa[kk]));
        }

        // ---------------- 1. projection: Q^T rows 32w.. = W_Q[s] rows 32w.. . Z^T ----------------
        f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const bf16x8 zb =
                    *reinterpret_cast<const bf16x8*>(zq + (rb * 32 + l32) * LDK + 16 * kk + 8 * g);
                acc[rb] = mfma32(wa[kk], zb, acc[rb]);
            }
        __syncthreads();   // every wave is done reading Z

        // ---------------- 2. Q chunk into LDS, the request's memory if not there ----------------
        // acc[rb] reg 4*j4 + t: feature 32w + 8*j4 + 4g + t of query row 32rb + l32
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            bf16* qrow = zq + (rb * 32 + l32) * LDK + 32 * w + 4 * g;
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) {
                bf16x4 v;
#pragma unroll
                for (int t = 0; t < 4; ++t) v[t] = (bf16)acc[rb][4 * j4 + t];
                *reinterpret_cast<bf16x4*>(qrow + 8 * j4) = v;
            }
        }
        const int rows0 = min(cur.L, LMAX);
        if (rows0 > 0 && (cur.kv0 != st_row0 || rows0 != st_rows)) kv_stage(cur.kv0, rows0);
        __syncthreads();   // Q chunk and memory visible

        // ---------------- 3. attention of this wave's units ----------------
        bf16x8 qb[C::UPW][C::KST];
#pragma unroll
        for (int k = 0; k < C::UPW; ++k) {
            const int v = ((w + NW * k) / C::FP) % (2 * (D / DH));
            const int h = v >> 1, urb = v & 1;
#pragma unroll
            for (int kk = 0; kk < C::KST; ++kk)
                qb[k][kk] = *reinterpret_cast<const bf16x8*>(zq + (urb * 32 + l32) * LDK + h * DH +
                                                             16 * kk + 8 * g);
        }
        __syncthreads();   // every wave holds its queries: the chunk buffer is free

        f32x16 oacc[C::UPW][C::EBW];
        float m_run[C::UPW], l_run[C::UPW];
        bool started[C::UPW];
#pragma unroll
        for (int k = 0; k < C::UPW; ++k) {
#pragma unroll
            for (int eb = 0; eb < C::EBW; ++eb) oacc[k][eb] = f32x16{};
            m_run[k] = -INFINITY;
            l_run[k] = 0.f;
            started[k] = false;
        }

        // One 32-row memory block (t) of the staged rows against unit k's queries.
        auto block = [&](int k, int t, int rows) {
            const int u = w + NW * k;
            const int h = (u / C::FP) >> 1, e0 = (u % C::FP) * C::EBW * 32;
            const bf16* kb = kvs + (t * MB + l32) * LDK + h * DH + 8 * g;
            bf16x8 kf[C::KST];
#pragma unroll
            for (int kk = 0; kk < C::KST; ++kk) kf[kk] = *reinterpret_cast<const bf16x8*>(kb + 16 * kk);
            // raw scores K_h . Q_h^T (fp32)
            f32x16 sacc = mfma32(kf[0], qb[k][0], f32x16{});
#pragma unroll
            for (int kk = 1; kk < C::KST; ++kk) sacc = mfma32(kf[kk], qb[k][kk], sacc);
            bf16x8 vf[2][C::EBW];
#pragma unroll
            for (int u16 = 0; u16 < 2; ++u16)
#pragma unroll
                for (int eb = 0; eb < C::EBW; ++eb) {
                    const bf16* base =
                        vsrc + (t * MB + 16 * u16 + tr_row) * LDK + h * DH + e0 + eb * 32 + tr_col;
                    vf[u16][eb] = cat(lds_read_tr16(base), lds_read_tr16(base + 8 * LDK));
                }
            // only the last block of the staged rows is partial
            int jl = rows - t * MB;
            asm volatile("" : "+s"(jl));
            if (jl < MB) {
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) {
                    const int j = (rr >> 2) * 8 + 4 * g + (rr & 3);
                    if (j >= jl) sacc[rr] = -INFINITY;
                }
            }
            // Weights 2^(score * log2(e)/sqrt(d_h) - m) against the running
            // maximum m (exp2 units).  P^T k-step u16 slot t <-> score
            // register 8*u16 + t.
            bf16x8 pb[2];
            auto weights = [&](float m) {
                float lt = 0.f;
#pragma unroll
                for (int rr = 0; rr < 16; rr += 2) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[rr], scale_log2, -m));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[rr + 1], scale_log2, -m));
                    const bf16x2 pp = {(bf16)p0, (bf16)p1};
                    lt = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, lt, false);
                    pb[rr >> 3][rr & 7] = pp[0];
                    pb[rr >> 3][(rr & 7) + 1] = pp[1];
                }
                return lt;
            };
            // the block's row maximum in exp2 units (both halves of the wave
            // agree on it; the scale is positive)
            auto block_max = [&]() {
                float mt = fmaxf(sacc[0], sacc[1]);
#pragma unroll
                for (int rr = 2; rr < 16; rr += 2) mt = fmaxf(mt, fmaxf(sacc[rr], sacc[rr + 1]));
                return fmaxf(mt, xor32(mt)) * scale_log2;
            };
            float lt;
            if (!started[k]) {
                // a unit's first block sets the running maximum (nothing to
                // rescale yet)
                m_run[k] = block_max();
                lt = weights(m_run[k]);
                started[k] = true;
            } else {
                // the maximum moves only when some weight of the block could
                // exceed kSumCap
                lt = weights(m_run[k]);
                if (__any(lt > kSumCap)) {
                    const float m_new = fmaxf(m_run[k], block_max());
                    const float alpha = __builtin_amdgcn_exp2f(m_run[k] - m_new);
                    m_run[k] = m_new;
                    l_run[k] *= alpha;
#pragma unroll
                    for (int eb = 0; eb < C::EBW; ++eb) oacc[k][eb] *= alpha;
                    lt = weights(m_new);
                }
            }
            l_run[k] += lt;
#pragma unroll
            for (int u16 = 0; u16 < 2; ++u16)
#pragma unroll
                for (int eb = 0; eb < C::EBW; ++eb) oacc[k][eb] = mfma32(vf[u16][eb], pb[u16], oacc[k][eb]);
        };

        // A memory of at most NBX blocks (the TransX memory: 96 rows) is
        // attended in one pass: the scores of all its blocks first (NBX
        // independent product chains that the matrix cores run back to
        // back), then their exact row maximum, the weights, and the PV
        // products.  No running maximum, no rescale.  Blocks past the
        // memory's rows read the zero rows staged behind them and are masked.
        auto unit_exact = [&](int k, int rows) {
            const int u = w + NW * k;
            const int h = (u / C::FP) >> 1, e0 = (u % C::FP) * C::EBW * 32;
            constexpr int NB = C::NBX > 0 ? C::NBX : 1;
            f32x16 sc[NB];
#pragma unroll
            for (int t = 0; t < NB; ++t) {
                const bf16* kb = kvs + (t * MB + l32) * LDK + h * DH + 8 * g;
                bf16x8 kf[C::KST];
#pragma unroll
                for (int kk = 0; kk < C::KST; ++kk) kf[kk] = *reinterpret_cast<const bf16x8*>(kb + 16 * kk);
                sc[t] = mfma32(kf[0], qb[k][0], f32x16{});
#pragma unroll
                for (int kk = 1; kk < C::KST; ++kk) sc[t] = mfma32(kf[kk], qb[k][kk], sc[t]);
            }
            // register rr of block t holds memory row t*MB + (rr/4)*8 + 4g + rr%4
#pragma unroll
            for (int t = 0; t < NB; ++t) {
                int jl = rows - t * MB;
                asm volatile("" : "+s"(jl));
                if (jl < MB) {
#pragma unroll
                    for (int rr = 0; rr < 16; ++rr)
                        if ((rr >> 2) * 8 + 4 * g + (rr & 3) >= jl) sc[t][rr] = -INFINITY;
                }
            }
            float mt = fmaxf(sc[0][0], sc[0][1]);
#pragma unroll
            for (int t = 0; t < NB; ++t)
#pragma unroll
                for (int rr = (t == 0 ? 2 : 0); rr < 16; rr += 2) mt = fmaxf(mt, fmaxf(sc[t][rr], sc[t][rr + 1]));
            const float m = fmaxf(mt, xor32(mt)) * scale_log2;   // row 0 is always visible: finite
            float lt[NB];
#pragma unroll
            for (int t = 0; t < NB; ++t) {
                bf16x8 pb[2];
                lt[t] = 0.f;
#pragma unroll
                for (int rr = 0; rr < 16; rr += 2) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[t][rr], scale_log2, -m));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[t][rr + 1], scale_log2, -m));
                    const bf16x2 pp = {(bf16)p0, (bf16)p1};
                    lt[t] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, lt[t], false);
                    pb[rr >> 3][rr & 7] = pp[0];
                    pb[rr >> 3][(rr & 7) + 1] = pp[1];
                }
                bf16x8 vf[2][C::EBW];
#pragma unroll
                for (int u16 = 0; u16 < 2; ++u16)
#pragma unroll
                    for (int eb = 0; eb < C::EBW; ++eb) {
                        const bf16* base =
                            vsrc + (t * MB + 16 * u16 + tr_row) * LDK + h * DH + e0 + eb * 32 + tr_col;
                        vf[u16][eb] = cat(lds_read_tr16(base), lds_read_tr16(base + 8 * LDK));
                    }
#pragma unroll
                for (int u16 = 0; u16 < 2; ++u16)
#pragma unroll
                    for (int eb = 0; eb < C::EBW; ++eb)
                        oacc[k][eb] = mfma32(vf[u16][eb], pb[u16], oacc[k][eb]);
            }
            float l = lt[0];
#pragma unroll
            for (int t = 1; t < NB; ++t) l += lt[t];
            m_run[k] = m;
            l_run[k] = l;
        };

        // memory chunks of LMAX rows; the first is staged above, later ones
        // (memories longer than LMAX) between work-group barriers here
        const int n_mc = (cur.L + LMAX - 1) / LMAX;
        if (C::NBX > 0 && cur.L > 0 && cur.L <= C::NBX * MB) {
            if constexpr (C::NBX > 0) {
#pragma unroll
                for (int k = 0; k < C::UPW; ++k) unit_exact(k, cur.L);
            }
        } else
        for (int mc = 0; mc < n_mc; ++mc) {
            const int row0 = cur.kv0 + mc * LMAX, rows = min(LMAX, cur.L - mc * LMAX);
            if (mc > 0) {
                __syncthreads();   // every wave is done with the previous memory chunk
                kv_stage(row0, rows);
                __syncthreads();
            }
            const int nb = (rows + MB - 1) / MB;
#pragma unroll
            for (int k = 0; k < C::UPW; ++k)
                for (int t = 0; t < nb; ++t) block(k, t, rows);
        }

        // Normalise and store this chunk's output rows.  Rows past the
        // chunk's candidates fall outside the descriptor and are dropped, so
        // every path issues the same stores (and the compiler's wait for the
        // next chunk's Z rows below never has to cover them).
        const int cb = cur.c0 + cur.j * QR, nr = min(QR, cur.nc - cur.j * QR);
        const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(O + ((size_t)cb * q + cur.s) * D), (short)0,
            (uint32_t)(((size_t)(nr - 1) * q + 1) * D * 2), 0x00020000);
#pragma unroll
        for (int k = 0; k < C::UPW; ++k) {
            const int u = w + NW * k;
            const int h = (u / C::FP) >> 1, urb = (u / C::FP) & 1, e0 = (u % C::FP) * C::EBW * 32;
            const float l = l_run[k] + xor32(l_run[k]);
            const float inv = l > 0.f ? 1.f / l : 0.f;
            // the row's log2 softmax normaliser (exp2 units of the scaled
            // scores), kept for a backward pass, from one lane per row
            if (a.lse && u % C::FP == 0 && g == 0 && urb * 32 + l32 < nr)
                a.lse[((size_t)(cb + urb * 32 + l32) * q + cur.s) * a.heads + h] =
                    l > 0.f ? m_run[k] + __builtin_amdgcn_logf(l) : -INFINITY;   // v_log_f32 is log2
            // Register 4*b4 + t of oacc holds feature 32eb + 8b4 + 4g + t;
            // join_runs makes one 16-byte store per (eb, bp) instead of two
            // 8-byte stores.
            const int off = ((urb * 32 + l32) * q * D + h * DH + e0 + 8 * g) * 2;
#pragma unroll
            for (int eb = 0; eb < C::EBW; ++eb)
#pragma unroll
                for (int bp = 0; bp < 2; ++bp) {
                    bf16x4 ve, vo;
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        ve[t] = (bf16)(oacc[k][eb][8 * bp + t] * inv);
                        vo[t] = (bf16)(oacc[k][eb][8 * bp + 4 + t] * inv);
                    }
                    __builtin_amdgcn_raw_buffer_store_b128(join_runs(ve, vo), ro, off + (eb * 32 + 16 * bp) * 2,
                                                           0, 0);
                }
        }
        if (!has_next) break;
        // the next chunk's Z rows, loaded a whole chunk ago, into the free
        // chunk buffer (the wait covers them and not this chunk's stores)
        zstore();
        if (nxt.j == 0) ++ii;
        cur = nxt;
    }
}

template <int DH, bool SEP, bool CODEC>
hipError_t launch_t(const AttnArgs& a, const ShortCodec& cd, int grid, hipStream_t stream) {
    AttnArgs k = a;
    k.scale_log2 = 1.4426950408889634f / sqrtf((float)DH);
    hipLaunchKernelGGL((short_bf16_kernel<DH, SEP, CODEC>), dim3((unsigned)grid), dim3(NT), 0, stream,
                       k, cd);
    return hipGetLastError();
}

template <int DH>
hipError_t launch_dh(const AttnArgs& a, int grid, hipStream_t stream) {
    const ShortCodec none{};
    return a.V ? launch_t<DH, true, false>(a, none, grid, stream)
               : launch_t<DH, false, false>(a, none, grid, stream);
}

template <int DH>
hipError_t launch_dh_codec(const AttnArgs& a, const ShortCodec& cd, bool sep, int grid,
                           hipStream_t stream) {
    return sep ? launch_t<DH, true, true>(a, cd, grid, stream)
               : launch_t<DH, false, true>(a, cd, grid, stream);
}

}  // namespace

hipError_t launch_short_bf16(const AttnArgs& a, int grid, hipStream_t stream) {
    if (a.d != kShortD || a.heads < 1 || a.d % a.heads != 0 || !a.Z || !a.Wq || a.cand_len)
        return hipErrorInvalidValue;
    if (grid <= 0) return hipSuccess;
    switch (a.d / a.heads) {
        case 32: return launch_dh<32>(a, grid, stream);
        case 64: return launch_dh<64>(a, grid, stream);
        case 128: return launch_dh<128>(a, grid, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_short_codec_bf16(const AttnArgs& a, const ShortCodec& cd, bool sep, int grid,
                                   hipStream_t stream) {
    if (a.d != kShortD || a.heads < 1 || a.d % a.heads != 0 || !a.Z || !a.Wq || a.inplan ||
        cd.kb.budget % 32 != 0 || cd.kb.budget <= 0 || (sep && cd.vb.budget != cd.kb.budget))
        return hipErrorInvalidValue;
    if (grid <= 0) return hipSuccess;
    switch (a.d / a.heads) {
        case 32: return launch_dh_codec<32>(a, cd, sep, grid, stream);
        case 64: return launch_dh_codec<64>(a, cd, sep, grid, stream);
        case 128: return launch_dh_codec<128>(a, cd, sep, grid, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace xattn
