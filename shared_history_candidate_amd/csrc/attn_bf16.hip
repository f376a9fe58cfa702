// Shared-memory cross-attention over projected queries, bf16 in, fp32
// accumulate, bf16 out, for gfx950 matrix cores.
//
// For every work item {r, s, c0, nc} of the plan and every head h:
//   O_h = softmax(Q_h K_h^T / sqrt(d_h)) V_h            (ReST reading note,
//         s.3.3.1 Eq. (7); K = V = H in projection-free mode, separate K, V
//         for the TransX behaviour memory, TransX report s.2)
// for the nc candidates c in [c0, c0+nc) of request r, query slot s, where
// Q = Z W_Q[s] comes from the projection kernel (gemm_bf16.hip).  All
// candidates of a request stream the same memory rows (shared-prefix
// serving, ReST reading note s.3.5).
//
// Work decomposition.  A work-group handles one work item and one head with
// RB x KSPLIT waves: wave w owns query block rb = w % RB (32 query columns)
// and memory split ks = w / RB (memory tiles t with t % KSPLIT == ks).  The
// waves of one split share the staged memory tiles; the KSPLIT partial
// softmax states of a query block are merged through LDS at the end.
// Head pairs (HS, 32-wide heads, K = V): HBM is read in 128-byte lines and a
// 32-wide head is half a line of each memory row, so a work-group takes the
// two heads of a line instead: its two wave groups (ks = 0, 1) attend heads
// 2p and 2p + 1 over the same staged tiles of both heads' 64 features, with
// no memory split and no merge, one register stage (four waves per SIMD),
// launched in XCD-chunked order (xcd_order.h).
//
// Products are computed transposed so that each lane holds one query row and
// the softmax reductions along the key axis stay inside the lane (plus one
// exchange between the two 32-lane halves, needed only when the running
// maximum moves):
//   scores      S^T   (64 x 32)  = K_tile (64 x d_h) . Q_h^T
//   output      O^T   (d_h x 32) += V_tile^T (d_h x 64) . P^T (64 x 32)
// The score accumulator layout is the operand layout of P^T, so the weights
// never move between lanes.  The memory is streamed in tiles of 64 rows
// through double-buffered LDS (one buffer is both K and V in projection-free
// mode) and V^T operands come from LDS transpose reads.
//
// Softmax: exp2 of log2(e)/sqrt(d_h)-scaled scores against a reference that
// the first tile of each memory split sets (its maximum) and that stays fixed:
// later weights may exceed 1, which fp32 sums and bf16 operands hold as
// exactly as weights <= 1, so the memory loop needs neither a per-tile
// maximum nor a conditional rescale of the accumulators.  A split whose tile
// weights would pass 2^50 is recomputed with a moving maximum.  Row sums
// accumulate the bf16-rounded weights that enter the PV product (v_dot2).
#include <type_traits>

#include "common.h"
#include "internal.h"
#include "lds_dma.h"
#include "plan_wave.h"
#include "xcd_order.h"

namespace xattn {

namespace {

constexpr int BN = 64;               // memory rows per tile
constexpr float kSumCap = 4096.0f;   // largest accepted per-lane weight sum of one tile (moving maximum)
// Largest per-lane weight sum the fixed reference accepts: the weights and
// their products with values below 2^47 stay finite.
constexpr float kWeightCap = 1.125899906842624e15f;   // 2^50

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Widest model the fused projection stages in LDS.
constexpr int kProjMaxD = kAttnProjMaxD;


template <int DH, int RB, int KSPLIT, bool SEP, bool PROJ, bool CUT = false, bool HS = false>
struct Cfg {
    static constexpr int NW = RB * KSPLIT;
    static constexpr int NT = 64 * NW;
    // head pairs: the KSPLIT = 2 wave groups are the pair's heads, not memory splits
    static_assert(!HS || (DH == 32 && KSPLIT == 2 && !SEP && !PROJ), "head pairs");
    static constexpr int MS = HS ? 1 : KSPLIT;       // memory splits
    static constexpr int DS = HS ? 2 * DH : DH;      // staged features per memory row
    static constexpr int SG = HS ? NW : RB;          // waves staging one tile
    static constexpr int EB = DH / 32;        // 32-wide feature blocks
    static constexpr int KST = DH / 16;       // k-steps of the score product
    // Memory tiles over caller-projected queries at head width 64 with K = V
    // are staged by direct global-to-LDS loads (no registers, no LDS store
    // instructions), NBUF buffers deep per split: the tile NBUF - 1 ahead is
    // in flight while one is computed.  Their rows are unpadded, with the
    // 16-byte chunks of row r permuted by chunk ^ ((r >> 1) & 7), which keeps
    // the score-operand and transposed value reads as free of bank conflicts
    // as the padded rows of the register-staged tiles.
    static constexpr bool DMA = !PROJ && !SEP && DH == 64;
    static constexpr int NBUF = DMA ? (KSPLIT <= 2 ? 3 : 2) : 2;
    // Row padding of the register-staged memory tile (elements).  16-byte
    // rows (8) let the score operands come in single 16-byte LDS reads; the
    // separate-K/V tiles measured faster with 8-byte rows (4).
    static constexpr int PAD = DMA ? 0 : (SEP ? 4 : 8);
    static constexpr int LDK = DS + PAD;      // memory tile pitch (elements)
    // one wave per split: a wave reads only the tiles it stored itself, so the
    // memory loop needs no work-group barrier (a wave's LDS operations retire
    // in program order)
    static constexpr bool PRIVATE = RB == 1 && !HS;
    static constexpr int PLANES = SEP ? 2 : 1;
    static constexpr int TILE = BN * LDK;     // elements per plane per buffer
    static constexpr int KV_BYTES = MS * NBUF * PLANES * TILE * 2;
    // direct loads per wave and tile: a load fills 1 KB (8 rows of 128 bytes)
    static constexpr int DPW = DMA ? BN * DH * 2 / 1024 / RB : 0;
    static constexpr int CMB_BYTES = MS > 1 ? RB * (MS - 1) * 64 * (EB * 16 + 2) * 4 : 0;
    // Fused projection (PROJ): the tile's query tokens (32*RB rows) and head
    // h's rows of W_Q[s] (DH rows) are staged in LDS (up to kProjMaxD wide,
    // aliasing the memory buffers, which are filled only afterwards); the
    // projected Q_h tile goes to its own LDS region behind both.
    static constexpr int LDS_K = kProjMaxD + 8;       // staging pitch (16-byte rows)
    static constexpr int STG_BYTES = PROJ ? (32 * RB + DH) * LDS_K * 2 : 0;
    static constexpr int ZCPT = (32 * RB * (kProjMaxD / 8) + NT - 1) / NT;   // staging chunks per thread
    static constexpr int WCPT = (DH * (kProjMaxD / 8) + NT - 1) / NT;
    static constexpr int LDQ = DH + 8;
    static constexpr int QT_OFF = KV_BYTES > STG_BYTES ? KV_BYTES : STG_BYTES;
    static constexpr int QT_BYTES = PROJ ? 32 * RB * LDQ * 2 : 0;
    static constexpr int PB = EB * RB;                 // 32x32 blocks of Q_h^T
    static constexpr int PB_PER_WAVE = (PB + NW - 1) / NW;
    static constexpr int SMEM_MAIN = PROJ ? QT_OFF + QT_BYTES : KV_BYTES;
    static constexpr int SMEM = SMEM_MAIN > CMB_BYTES ? SMEM_MAIN : CMB_BYTES;
    // the staging registers must leave room for the rest of the prologue
    static constexpr bool BUILT = !PROJ || ZCPT + WCPT <= 24;
    static constexpr int KV_CHUNKS = BN * DS / 8;                 // 16-byte chunks per plane
    static constexpr int KV_CPT = KV_CHUNKS / (64 * SG);
    static_assert(KV_CHUNKS % (64 * SG) == 0, "memory tile must split evenly over a staging group");
    // Register stages of the memory prefetch (tiles ahead of the LDS stage).
    // Per-head d_h = 32 tiles are computed quickly, so their loads get the
    // longer lead: up to 8 x 16 bytes per thread in flight (32 VGPRs), at
    // most 4 tiles ahead.  Wider heads take one stage: a second one costs a
    // wave per SIMD and measured slower.  Head pairs take one stage too:
    // their four waves share each tile's loads, and one stage leaves the
    // registers for four waves per SIMD (ragged 46.4 -> 43.2 us against
    // four stages at two waves).
    static constexpr int STAGE_REGS = KV_CPT * PLANES;
    static constexpr int P = HS || DH > 32 || STAGE_REGS >= 8 ? 1 : (8 / STAGE_REGS >= 4 ? 4 : 8 / STAGE_REGS);
    // Waves per SIMD the register allocation must leave room for: as many as
    // the LDS footprint admits, up to three (168 VGPRs per wave) with one
    // register stage, two with deeper ones; head pairs four (128 VGPRs).
    static constexpr int LDS_WAVES = (163840 / SMEM) * NW;   // per compute unit
    static constexpr int WPE = HS && LDS_WAVES >= 16 ? 4
                             : (LDS_WAVES >= 12 && P == 1 ? 3 : (LDS_WAVES >= 8 ? 2 : 1));
};

template <int DH, int RB, int KSPLIT, bool SEP, bool PROJ, bool CUT, bool HS = false>
__global__ __launch_bounds__(64 * RB * KSPLIT) __attribute__((
    amdgpu_waves_per_eu(Cfg<DH, RB, KSPLIT, SEP, PROJ, CUT, HS>::WPE))) void attn_bf16_kernel(AttnArgs a) {
    using C = Cfg<DH, RB, KSPLIT, SEP, PROJ, CUT, HS>;
    constexpr int P = C::P;
    __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
    const int q = a.q, d = a.d, heads = a.heads;
    const float scale_log2 = a.scale_log2;
    const bf16* __restrict__ K = static_cast<const bf16*>(a.K);
    const bf16* __restrict__ V = static_cast<const bf16*>(a.V);
    bf16* __restrict__ O = static_cast<bf16*>(a.O);
    int* __restrict__ ws = static_cast<int*>(a.ws);

    const int hgroups = HS ? heads / 2 : heads;   // work-groups per work item
    int tile = blockIdx.x / hgroups;
    int hw = blockIdx.x - tile * hgroups;         // head (HS: head pair)
    if constexpr (HS) xcd_pair_item(blockIdx.x, hgroups, tile, hw);   // XCD-chunked order
    int4 item;
    if (a.inplan) {
        // Small batch: every wave plans it (one lane per request) and takes
        // its work-group's item; the first wave also publishes the plan in
        // the workspace (for later calls that reuse it) or the validation
        // failure, in which case no work-group computes anything.
        const WavePlan wp = wave_plan(a.cu_kv, a.cu_cand, a.R, q, 32 * RB, a.total_cand,
                                      a.total_kv);
        if (blockIdx.x == 0 && threadIdx.x < 64) wave_plan_publish(wp, a.R, q, 32 * RB, ws, a.max_tiles);
        if (wp.err || tile >= wp.total) return;
        item = wave_plan_item(wp, tile, q, 32 * RB);
    } else {
        const int n_tiles = ws[kPlanNTiles];
        // A plan built for another tile size (another batch shape) is not
        // ours; work-groups past the plan's tiles have nothing to do.
        if (tile >= n_tiles || ws[kPlanTileM] != 32 * RB) return;
        item = reinterpret_cast<const int4*>(reinterpret_cast<const char*>(ws) +
                                             kPlanHeaderBytes)[tile];
    }
    // the item is the same in every lane: keep it in scalar registers
    const int kv0 = __builtin_amdgcn_readfirstlane(item.x);
    const int L = __builtin_amdgcn_readfirstlane(item.y);
    const int c0 = __builtin_amdgcn_readfirstlane(item.z);
    const int iw = __builtin_amdgcn_readfirstlane(item.w);
    const int nc = iw & kItemNcMask, s = iw >> 16;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // the wave index is uniform across the wave: keep it (and every tile
    // address derived from it) in scalar registers
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rb = w % RB, ksg = w / RB;     // query block, memory split (HS: head of the pair)
    const int ms = HS ? 0 : ksg;             // memory split
    const int hsel = HS ? ksg : 0;           // head within the staged features
    const int h = HS ? 2 * hw + ksg : hw;    // this wave's head
    const int g = lane >> 5, l32 = lane & 31;
    const int qcol = rb * 32 + l32;
    const bool qvalid = qcol < nc;
    const int cand = c0 + qcol;
    const int gt = HS ? tid : tid - ksg * 64 * RB;   // thread index inside the staging group

    // Per-candidate prefix cutoff (CUT; ReST reading note s.3.5, ULT): the
    // lane's query row sees memory rows [0, cut) of its request.  The tile
    // loop runs to the work-group's largest cutoff (every wave computes it
    // from all nc candidates, so all waves agree); rows past a lane's own
    // cutoff are masked.  wmin is this wave's smallest cutoff: tiles below it
    // need no mask.
    int cut = L, L_loop = L, wmin = L;
    if constexpr (CUT) {
        const int* __restrict__ cl = a.cand_len;
        auto clampL = [&](int v) { return v < 0 ? 0 : (v < L ? v : L); };
        cut = qvalid ? clampL(cl[cand]) : L;
        int mx = 0;
        for (int i = lane; i < nc; i += 64) mx = max(mx, clampL(cl[c0 + i]));
        int mn = cut;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            mx = max(mx, __shfl_xor(mx, off, 64));
            mn = min(mn, __shfl_xor(mn, off, 64));
        }
        L_loop = __builtin_amdgcn_readfirstlane(mx);
        wmin = __builtin_amdgcn_readfirstlane(mn);
    }

    // ---------------- 1. memory prefetch and this wave's Q_h^T operands ----------------
    const int ntiles_kv = (L_loop + BN - 1) / BN;
    const int n_iter = (ntiles_kv + C::MS - 1) / C::MS;
    const bf16* Kh = K + (size_t)kv0 * d + (HS ? 2 * hw : h) * DH;
    const bf16* Vh = SEP ? V + (size_t)kv0 * d + h * DH : nullptr;
    // Chunk u of this thread: tile row j_u, 16-byte column chunk c8_u.  Its
    // global byte offset inside a tile and its LDS element offset are fixed;
    // tiles differ only by the buffer base.  Buffer loads return zeros past
    // the request's last memory row (and for whole tiles past it, whose
    // descriptor covers no bytes), so partial tiles need no special case.
    int goff[C::KV_CPT], loff[C::KV_CPT];
#pragma unroll
    for (int u = 0; u < C::KV_CPT; ++u) {
        const int c = gt + u * 64 * C::SG;
        const int j = c / (C::DS / 8), c8 = c % (C::DS / 8);
        goff[u] = (j * d + c8 * 8) * 2;
        loff[u] = j * C::LDK + c8 * 8;
    }
    uint4 kreg[P][C::KV_CPT];
    uint4 vreg[P][SEP ? C::KV_CPT : 1];
    auto gload = [&](int t, uint4 (&kr)[C::KV_CPT], uint4 (&vr)[SEP ? C::KV_CPT : 1]) {
        const int row0 = t * BN;
        const int left = L_loop - row0;   // memory rows still read from this tile on
        const size_t nb = left > 0 ? (size_t)left * d * 2 : 0;
        const uint32_t bytes = nb > 0xFFFFFFF0u ? 0xFFFFFFF0u : (uint32_t)nb;
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(Kh + (size_t)row0 * d), (short)0, bytes, 0x00020000);
#pragma unroll
        for (int u = 0; u < C::KV_CPT; ++u)
            kr[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, goff[u], 0, 0));
        if constexpr (SEP) {
            const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(Vh + (size_t)row0 * d), (short)0, bytes, 0x00020000);
#pragma unroll
            for (int u = 0; u < C::KV_CPT; ++u)
                vr[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, goff[u], 0, 0));
        }
    };
    bf16* kvl = reinterpret_cast<bf16*>(smem) + (size_t)ms * C::NBUF * C::PLANES * C::TILE;
    auto lstore = [&](int buf, const uint4 (&kr)[C::KV_CPT], const uint4 (&vr)[SEP ? C::KV_CPT : 1]) {
        bf16* base = kvl + buf * C::PLANES * C::TILE;
#pragma unroll
        for (int u = 0; u < C::KV_CPT; ++u) {
            if constexpr (C::PAD % 8 == 0) {
                *reinterpret_cast<uint4*>(base + loff[u]) = kr[u];
                if constexpr (SEP) *reinterpret_cast<uint4*>(base + C::TILE + loff[u]) = vr[u];
            } else {   // rows are only 8-byte aligned
                uint2* p = reinterpret_cast<uint2*>(base + loff[u]);
                p[0] = make_uint2(kr[u].x, kr[u].y);
                p[1] = make_uint2(kr[u].z, kr[u].w);
                if constexpr (SEP) {
                    uint2* pv = reinterpret_cast<uint2*>(base + C::TILE + loff[u]);
                    pv[0] = make_uint2(vr[u].x, vr[u].y);
                    pv[1] = make_uint2(vr[u].z, vr[u].w);
                }
            }
        }
    };

    // Direct global-to-LDS staging (C::DMA): load j of this wave fills the
    // 1 KB of tile rows 8b .. 8b+7, b = rb * DPW + j, of a buffer; lane l
    // writes row 8b + l/8 at chunk position l % 8, so it loads that row's
    // global chunk (l % 8) ^ ((row >> 1) & 7).  Rows past the request's last
    // memory row (and whole tiles past it) read as zeros.
    int dgoff[C::DMA ? C::DPW : 1];
    if constexpr (C::DMA) {
#pragma unroll
        for (int j = 0; j < C::DPW; ++j) {
            const int r = 8 * (rb * C::DPW + j) + (lane >> 3);
            const int c = (lane & 7) ^ ((r >> 1) & 7);
            dgoff[j] = (r * d + c * 8) * 2;
        }
    }
    // A tile reads at most BN rows, so its descriptor covers at most BN rows
    // (32-bit arithmetic, all scalar); the LDS address of this wave's part
    // of buffer 0 is taken once.
    const uint32_t dma_lds0 = __builtin_amdgcn_readfirstlane(lds_addr_of(kvl + rb * C::DPW * 512));
    auto dma = [&](int t, int buf) {
        const int row0 = t * BN;
        const int left = L_loop - row0;
        // two scalar operations (written as a clamp, the compiler takes a
        // VALU med3 and reads its result back)
        int rows = left < BN ? left : BN;
        asm volatile("" : "+s"(rows));
        rows = rows > 0 ? rows : 0;
        const uint32_t bytes = (uint32_t)rows * (uint32_t)d * 2u;
        const size_t roff = rows > 0 ? (size_t)row0 * d : 0;
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(Kh + roff), (short)0, bytes, 0x00020000);
        const uint32_t base = dma_lds0 + (uint32_t)(buf * C::PLANES * C::TILE * 2);
#pragma unroll
        for (int j = 0; j < C::DPW; ++j) lds_dma16(rk, base + j * 1024, dgoff[j]);
    };
    // Element offsets inside a tile buffer of the fragments a lane reads: the
    // score operand of rows hh*32 + l32, k-step k (features 16k + 8g ..), and
    // the transposed value read of rows 16u + tr_row (+8) at column col.
    auto kofs = [&](int hh, int k) {
        const int r = hh * 32 + (lane & 31);
        if constexpr (C::DMA)
            return r * C::LDK + (((2 * k + (lane >> 5)) ^ ((r >> 1) & 7)) << 3);
        else
            return r * C::LDK + hsel * DH + 16 * k + 8 * (lane >> 5);
    };
    auto vofs = [&](int row, int col) {
        if constexpr (C::DMA)
            return row * C::LDK + ((((col >> 3) ^ ((row >> 1) & 7))) << 3) + (col & 7);
        else
            return row * C::LDK + hsel * DH + col;
    };

    // k-step k, half g: features 16k + 8g .. 16k + 8g + 7 of the lane's query
    // row (columns past the tile re-read its last row; their output is dropped)
    bf16x8 qb[C::KST];
    uint4 zst[PROJ ? C::ZCPT : 1], wst[PROJ ? C::WCPT : 1];
    const int cpr = d >> 3;   // 16-byte chunks per model row
    const uint32_t cmg = 0xFFFFFFFFu / (uint32_t)cpr + 1u;
    if constexpr (PROJ) {
        // Operands of the TSP projection (ReST reading note, s.3.3.2 Eq. (8)):
        // this tile's query tokens (candidates c0.., slot s; rows past nc are
        // outside the descriptor and read as zeros) and head h's rows of
        // W_Q[s], in coalesced 16-byte chunks.
        const size_t zbytes = ((size_t)(nc - 1) * q + 1) * d * 2;
        const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(static_cast<const bf16*>(a.Z) + ((size_t)c0 * q + s) * d), (short)0,
            zbytes > 0xFFFFFFF0u ? 0xFFFFFFF0u : (uint32_t)zbytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(static_cast<const bf16*>(a.Wq) + ((size_t)s * d + h * DH) * d), (short)0,
            (uint32_t)(DH * d * 2), 0x00020000);
#pragma unroll
        for (int u = 0; u < C::ZCPT; ++u) {
            const int idx = tid + u * C::NT, row = (int)__umulhi((uint32_t)idx, cmg), col = idx - row * cpr;
            zst[u] = idx < 32 * RB * cpr
                         ? __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                         rz, (row * q * d + col * 8) * 2, 0, 0))
                         : uint4{};
        }
#pragma unroll
        for (int u = 0; u < C::WCPT; ++u) {
            const int idx = tid + u * C::NT, row = (int)__umulhi((uint32_t)idx, cmg), col = idx - row * cpr;
            wst[u] = idx < DH * cpr
                         ? __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                         rw, (row * d + col * 8) * 2, 0, 0))
                         : uint4{};
        }
    } else {
        const bf16* qrow = static_cast<const bf16*>(a.Qp) +
                           ((size_t)(qvalid ? cand : c0 + nc - 1) * q + s) * d + h * DH;
#pragma unroll
        for (int k = 0; k < C::KST; ++k)
            qb[k] = *reinterpret_cast<const bf16x8*>(qrow + 16 * k + 8 * g);
    }
    // The first tiles of this split are requested right behind: P register
    // stages, or (direct staging) the NBUF - 1 buffers ahead of the computed one.
    if constexpr (C::DMA) {
#pragma unroll
        for (int j = 0; j < C::NBUF - 1; ++j) dma(ms + j * C::MS, j);
    } else {
#pragma unroll
        for (int j = 0; j < P; ++j) gload(ms + j * C::MS, kreg[j], vreg[j]);
    }
    if constexpr (PROJ) {
        bf16* zs = reinterpret_cast<bf16*>(smem);
        bf16* wsh = zs + 32 * RB * C::LDS_K;
#pragma unroll
        for (int u = 0; u < C::ZCPT; ++u) {
            const int idx = tid + u * C::NT, row = (int)__umulhi((uint32_t)idx, cmg), col = idx - row * cpr;
            if (idx < 32 * RB * cpr) *reinterpret_cast<uint4*>(zs + row * C::LDS_K + col * 8) = zst[u];
        }
#pragma unroll
        for (int u = 0; u < C::WCPT; ++u) {
            const int idx = tid + u * C::NT, row = (int)__umulhi((uint32_t)idx, cmg), col = idx - row * cpr;
            if (idx < DH * cpr) *reinterpret_cast<uint4*>(wsh + row * C::LDS_K + col * 8) = wst[u];
        }
        __syncthreads();
        // Q_h^T block (e, r) = W rows 32e.. x Z rows 32r..: fp32 over the
        // whole model width, rounded once to bf16 into the Q tile.
        bf16* qt = reinterpret_cast<bf16*>(smem + C::QT_OFF);
        const int kst = d >> 4;
#pragma unroll
        for (int u = 0; u < C::PB_PER_WAVE; ++u) {
            const int b = w + u * C::NW;
            if (b < C::PB) {
                const int e = b % C::EB, r = b / C::EB;
                const bf16* ap = wsh + (32 * e + l32) * C::LDS_K + 8 * g;
                const bf16* bp = zs + (32 * r + l32) * C::LDS_K + 8 * g;
                f32x16 acc = f32x16{};
                for (int k = 0; k < kst; ++k)
                    acc = mfma32(*reinterpret_cast<const bf16x8*>(ap + 16 * k),
                                 *reinterpret_cast<const bf16x8*>(bp + 16 * k), acc);
                // acc reg 4*j4 + t: feature 32e + 8*j4 + 4g + t of candidate row 32r + l32
                bf16* qrow = qt + (32 * r + l32) * C::LDQ + 32 * e + 4 * g;
#pragma unroll
                for (int j4 = 0; j4 < 4; ++j4) {
                    bf16x4 v;
#pragma unroll
                    for (int t = 0; t < 4; ++t) v[t] = (bf16)acc[4 * j4 + t];
                    *reinterpret_cast<bf16x4*>(qrow + 8 * j4) = v;
                }
            }
        }
        __syncthreads();
        const bf16* qrow = qt + (rb * 32 + l32) * C::LDQ;
#pragma unroll
        for (int k = 0; k < C::KST; ++k)
            qb[k] = *reinterpret_cast<const bf16x8*>(qrow + 16 * k + 8 * g);
    }
    // Fold log2(e)/sqrt(d_h) into the query operands (one more bf16 rounding
    // of Q; the scores then come out of the products in exp2 units).  This
    // also consumes the query registers before the loop: the queries are then
    // known to have arrived on entry to the memory loop, and the only loads in
    // flight across its iterations are the memory stages, which keeps the
    // compiler's wait counts inside the loop exact (no wait on a later stage).
#pragma unroll
    for (int k = 0; k < C::KST; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) qb[k][e] = (bf16)((float)qb[k][e] * scale_log2);

    if constexpr (!C::DMA) {
        lstore(0, kreg[0], vreg[0]);
        gload(ms + P * C::MS, kreg[0], vreg[0]);
        __syncthreads();
    }

    // ---------------- 2. stream this split's memory tiles ----------------
    // Softmax reference.  Every score product is seeded with -m_seed, so the
    // products deliver s*log2(e)/sqrt(d_h) - m_seed and the weights are a bare
    // exp2.  The first pass fixes m_seed at the maximum of the split's first
    // tile and never moves it: later weights may exceed 1, which fp32 sums
    // and bf16 operands hold exactly as well up to kWeightCap, and the final
    // normalisation divides the common factor out.  The memory loop then
    // carries no conditional update of the accumulators.  If some lane's
    // weights summed to more than kWeightCap, the work-group repeats the
    // split with a moving maximum (second pass, below).
    f32x16 oacc[C::EB];
#pragma unroll
    for (int eb = 0; eb < C::EB; ++eb) oacc[eb] = f32x16{};
    float m_run = -INFINITY;   // what the weights are relative to (-inf: no visible row)
    float l_run = 0.f;         // this half's share of the row sum
    float m_seed = 0.f;
    f32x16 negm = f32x16{};    // -m_seed in every register (all 16 belong to the lane's query row)

    // transposed V read: lane l receives V[16u + 4g + t][eb*32 + l%32], t = 0..3
    const int G = lane >> 4, k16 = lane & 15;
    const int tr_row = 4 * (G >> 1) + (k16 >> 2);
    const int tr_col = 16 * (G & 1) + 4 * (k16 & 3);
    const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};

    // Scores of the tile in LDS buffer buf against this wave's queries:
    // sacc[0] keys 0..31, sacc[1] keys 32..63.  All K fragments are read
    // before the first product so that the LDS latency is paid once per tile.
    f32x16 sacc[2];
    bf16x8 vf[4][C::EB];
    // (mid: issued between the K-fragment reads and the first product, in
    // the reads' latency)
    auto scores = [&](int buf, auto&& mid) {
        const bf16* kb = kvl + buf * C::PLANES * C::TILE;
        const bf16* vb = kb + (C::PLANES - 1) * C::TILE;
        bf16x8 kf[2][C::KST];
#pragma unroll
        for (int k = 0; k < C::KST; ++k) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const bf16* row = kb + kofs(hh, k);
                kf[hh][k] = cat(*reinterpret_cast<const bf16x4*>(row),
                                *reinterpret_cast<const bf16x4*>(row + 4));
            }
        }
        mid();
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) sacc[hh] = mfma32(kf[hh][0], qb[0], negm);
#pragma unroll
        for (int k = 1; k < C::KST; ++k)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) sacc[hh] = mfma32(kf[hh][k], qb[k], sacc[hh]);
        // scheduling: every K-fragment read ahead of the score products
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * C::KST, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * C::KST, 0);
        // V^T fragments for the output product, issued now so that they
        // arrive while the weights are being computed
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int eb = 0; eb < C::EB; ++eb) {
                const int row = 16 * u + tr_row, col = eb * 32 + tr_col;
                vf[u][eb] = cat(lds_read_tr16(vb + vofs(row, col)), lds_read_tr16(vb + vofs(row + 8, col)));
            }
    };
    // Only the request's last tile is partial (with cutoffs: tiles past the
    // wave's smallest cutoff).  The opaque copy keeps the compiler from
    // folding the tile-level test into the per-score tests.
    auto full_tile = [&](int t) {
        int jl = (CUT ? wmin : L) - t * BN;
        asm volatile("" : "+s"(jl));
        return jl >= BN;
    };
    // Rows past the lane's visible ones take score -inf.  Register rr of
    // sacc[hh] holds tile row hh*32 + (rr/4)*8 + 4g + rr%4: the test compares
    // the constant part with the lane's limit (no per-register row index is
    // kept across tiles).
    auto mask = [&](int t) {
        const int lim = (CUT ? cut : L) - t * BN - 4 * g;   // visible rows in the tile, minus 4g
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr)
                if (hh * 32 + (rr >> 2) * 8 + (rr & 3) >= lim) sacc[hh][rr] = -INFINITY;
    };
    // Weights 2^(score - m_seed + shift), summed per lane over the bf16
    // values that enter the PV product (two chains).
    bf16x8 pb[4];
    auto weights = [&](auto shifted, float shift) {
        float lt[2] = {0.f, 0.f};
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int rr = 0; rr < 16; rr += 2) {
                float x0 = sacc[hh][rr], x1 = sacc[hh][rr + 1];
                if constexpr (decltype(shifted)::value) x0 += shift, x1 += shift;
                const float p0 = __builtin_amdgcn_exp2f(x0);
                const float p1 = __builtin_amdgcn_exp2f(x1);
                const bf16x2 pp = {(bf16)p0, (bf16)p1};
                lt[hh] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, rr == 0 ? 0.f : lt[hh], false);
                pb[hh * 2 + (rr >> 3)][rr & 7] = pp[0];
                pb[hh * 2 + (rr >> 3)][(rr & 7) + 1] = pp[1];
            }
        return lt[0] + lt[1];
    };
    // O^T += V^T P^T over the four 16-key slabs of the tile
    auto values = [&]() {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int eb = 0; eb < C::EB; ++eb) oacc[eb] = mfma32(vf[u][eb], pb[u], oacc[eb]);
    };
    // lane maximum of the (masked) scores of the tile
    auto tile_max = [&]() {
        float mt = fmaxf(sacc[0][0], sacc[0][1]);
#pragma unroll
        for (int rr = 2; rr < 16; rr += 2) mt = fmaxf(mt, fmaxf(sacc[0][rr], sacc[0][rr + 1]));
#pragma unroll
        for (int rr = 0; rr < 16; rr += 2) mt = fmaxf(mt, fmaxf(sacc[1][rr], sacc[1][rr + 1]));
        return fmaxf(mt, xor32(mt));   // both halves' keys
    };

    // Iteration it computes this split's tile ms + it*MS from LDS buffer
    // it&1, then (advance) moves the next tile from register stage (it+1)%P
    // into the other buffer and refills that stage with the tile P iterations
    // ahead.  The refill is issued on every path (past the end it moves no
    // bytes), so the loads in flight are always the same stages in the same
    // order and the compiler's wait before each LDS store covers only the
    // stage stored.
    auto advance = [&](int it, int j) {
        const int jn = (j + 1) % P;
        if (it + 1 < n_iter) lstore((it + 1) & 1, kreg[jn], vreg[jn]);
        gload(ms + (it + 1 + P) * C::MS, kreg[jn], vreg[jn]);
        if constexpr (!C::PRIVATE) __syncthreads();
    };
    // Leading iterations whose tile is full: a loop whose body has no branch.
    const int n_fast = [&] {
        const int full = (CUT ? wmin : L) / BN;   // tiles 0 .. full-1 need no mask
        return full > ms ? (full - ms + C::MS - 1) / C::MS : 0;
    }();

    // Pacing (direct staging: the long history, three work-groups per
    // compute unit over equal memories).  A SIMD's instruction arbiter
    // favours its oldest wave, so those work-groups ran at unequal speeds
    // and finished one after another (per-work-group time stamps: 138, 168
    // and 198 us), the last one alone on the SIMDs.  Each wave starts at the
    // highest priority and steps down as it passes half, three quarters and
    // seven eighths of its tiles, so that a wave that is behind goes first
    // (steps at every quarter: 174, 186, 196 us; the finer steps near the
    // end measured 0.7 % faster still).
    // The work-groups of the first dispatch rounds (blockIdx / compute
    // units: 0 is the oldest on its compute unit) take each step earlier, by
    // 15 % of the tiles per round ahead of the third (swept 3-25 %: long
    // attention 189.3 -> 187.8 us at 15 %, same box, three runs each).
    const int round = a.ncu > 0 ? min((int)blockIdx.x / a.ncu, 2) : 2;
    const int lead = (2 - round) * n_iter * 15 / 100;
    const int q1 = (n_iter >> 1) - lead, q2 = ((3 * n_iter) >> 2) - lead, q3 = ((7 * n_iter) >> 3) - lead;
    auto pace = [&](int it) {
        if constexpr (C::DMA) {
            if (it == q1) __builtin_amdgcn_s_setprio(2);
            if (it == q2) __builtin_amdgcn_s_setprio(1);
            if (it == q3) __builtin_amdgcn_s_setprio(0);
        }
    };
    if constexpr (C::DMA) __builtin_amdgcn_s_setprio(3);
    // The epilogue's pointers, in scalar registers before the memory loop: a
    // scalar load still in flight there (the compiler issues them early)
    // would turn each wait for this tile's LDS reads into a wait for all of
    // them.
    float* const lse_out = a.lse;
    float* const dsum_out = a.Dsum;
    const bf16* const dO_in = static_cast<const bf16*>(a.dO);
    asm volatile("" ::"s"(O), "s"(lse_out), "s"(dsum_out), "s"(dO_in));

    // ---- first pass: fixed reference ----
    if constexpr (C::DMA) {
        // Direct staging: iteration it computes the tile in buffer bc (it %
        // NBUF) while the tiles up to it + PD are in flight.
        constexpr int PD = C::NBUF - 1;
        int bc = 0;
        auto begin = [&](int it) {
            pace(it);
            // this wave's loads of tile it have landed (the PD - 1 tiles behind
            // it may still be in flight) and its LDS reads of tile it - 1 are
            // done; past the barrier every wave's loads have landed and the
            // buffer of tile it - 1 takes tile it + PD
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"((PD - 1) * C::DPW) : "memory");
            if constexpr (!C::PRIVATE) __builtin_amdgcn_s_barrier();
            const int b = bc + PD < C::NBUF ? bc + PD : bc + PD - C::NBUF;
            dma(ms + (it + PD) * C::MS, b);
        };
        auto end = [&]() { bc = bc + 1 < C::NBUF ? bc + 1 : 0; };
        int it0 = 0;
        if (n_iter > 0) {
            // iteration 0: the split's first tile sets the reference
            begin(0);
            scores(bc, [] {});
            if (!full_tile(ms)) mask(ms);
            m_run = tile_max();   // -inf for a lane that sees no row of the split
            m_seed = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) negm[rr] = -m_seed;
            const float lt = weights(std::true_type{}, -m_seed);
            l_run = lt;
            values();
            end();
            it0 = 1;
        }
        // Full tiles: no mask.  With three buffers the loop runs in groups
        // of three iterations whose buffers are constants (iteration it uses
        // buffer it % 3, and the loop starts at it0 = 1), so that every LDS
        // address is a loop-invariant register plus an immediate offset; a
        // scheduling barrier ends each iteration, so that the compiler keeps
        // each tile's work in its own iteration.
        int itf = it0;
        if constexpr (C::NBUF == 3) {
            auto body = [&](int it, auto bufc) {
                constexpr int B = decltype(bufc)::value;
                pace(it);
                asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"((PD - 1) * C::DPW) : "memory");
                if constexpr (!C::PRIVATE) __builtin_amdgcn_s_barrier();
                scores(B, [&] { dma(ms + (it + PD) * C::MS, (B + PD) % C::NBUF); });
                const float lt = weights(std::false_type{}, 0.f);
                l_run += lt;
                values();
                // the row sums are materialised here (left alone, the
                // compiler sinks all three tiles' v_dot2 sums into the last
                // iteration of the group)
                asm volatile("" : "+v"(l_run));
                __builtin_amdgcn_sched_barrier(0);
            };
            if (itf == 1) {
#pragma unroll 1
                for (; itf + 3 <= n_fast; itf += 3) {
                    body(itf, std::integral_constant<int, 1>{});
                    body(itf + 1, std::integral_constant<int, 2>{});
                    body(itf + 2, std::integral_constant<int, 0>{});
                }
            }
        }
#pragma unroll 1
        for (int it = itf; it < n_fast; ++it) {
            begin(it);
            scores(bc, [] {});
            const float lt = weights(std::false_type{}, 0.f);
            l_run += lt;
            values();
            end();
        }
#pragma unroll 1
        for (int it = it0 > n_fast ? it0 : n_fast; it < n_iter; ++it) {
            const int t = ms + it * C::MS;
            begin(it);
            scores(bc, [] {});
            if (!full_tile(t)) mask(t);   // (a split past its last tile: wholly masked)
            const float lt = weights(std::false_type{}, 0.f);
            l_run += lt;
            values();
            end();
        }
        // the loads issued past the split's last tile (zeros) land before the
        // buffers are reused
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
        // iteration 0: the split's first tile sets the reference
        int it0 = 0;
        if (n_iter > 0) {
            scores(0, [] {});
            if (!full_tile(ms)) mask(ms);
            m_run = tile_max();   // -inf for a lane that sees no row of the split
            m_seed = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) negm[rr] = -m_seed;
            const float lt = weights(std::true_type{}, -m_seed);
            l_run = lt;
            values();
            advance(0, 0);
            it0 = 1;
        }
        auto fast = [&](int it) {
            scores(it & 1, [] {});
            const float lt = weights(std::false_type{}, 0.f);
            l_run += lt;
            values();
        };
        auto masked = [&](int it) {
            const int t = ms + it * C::MS;
            scores(it & 1, [] {});
            if (!full_tile(t)) mask(t);   // (a split past its last tile: wholly masked)
            const float lt = weights(std::false_type{}, 0.f);
            l_run += lt;
            values();
        };
        // Whole groups of P iterations while they end at or before n_end; the
        // register stage of every step is static (the groups start at 1, so
        // group member j is iteration it with it % P = (j + 1) % P).  Then the
        // remaining < P iterations once each.
        auto groups = [&](int& i0, int n_end, auto&& body) {
            for (; i0 + P <= n_end; i0 += P) {
#pragma unroll
                for (int j = 0; j < P; ++j) {
                    body(i0 + j);
                    advance(i0 + j, (j + 1) % P);
                }
            }
        };
        groups(it0, n_fast, fast);
        groups(it0, n_iter, masked);
#pragma unroll
        for (int j = 0; j < P - 1; ++j)
            if (it0 + j < n_iter) {
                masked(it0 + j);
                advance(it0 + j, (j + 1) % P);
            }
    }

    // ---- second pass, only if the first one saw weights past kWeightCap ----
    // The running maximum then moves with the tiles: it is set by the first
    // tile and afterwards moved (with a rescale of the accumulators) only
    // when some weight of a tile could exceed kSumCap (a lane's sum of its 32
    // non-negative weights bounds each of them).  With cutoffs a lane may
    // leave the first tile with maximum -inf (no visible row); its weights
    // then stay zero: its visible rows are a prefix of the memory, so a split
    // whose first tile shows it nothing shows it nothing later either.
    // (the lane's running sum bounds every tile's sum: testing it is the
    // stricter condition, and needs no per-tile maximum in the loop)
    if (__syncthreads_or(l_run > kWeightCap)) {
        // (rare: a plain loop, one tile at a time through LDS buffer 0)
#pragma unroll
        for (int eb = 0; eb < C::EB; ++eb) oacc[eb] = f32x16{};
        m_run = -INFINITY;
        l_run = 0.f;
        negm = f32x16{};
        bool started = false;   // m_run holds a tile maximum (wave-uniform)
#pragma unroll 1
        for (int it = 0; it < n_iter; ++it) {
            const int t = ms + it * C::MS;
            if constexpr (C::DMA) {
                dma(t, 0);
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            } else {
                gload(t, kreg[0], vreg[0]);
                lstore(0, kreg[0], vreg[0]);
            }
            __syncthreads();
            if (t < ntiles_kv) {
                scores(0, [] {});
                if (!full_tile(t)) mask(t);
                float lt = weights(std::false_type{}, 0.f);
                if (!started || __any(lt > kSumCap)) {
                    // what the scores are relative to (with cutoffs a lane
                    // may have seen no visible row yet: its maximum is still
                    // -inf, its seed 0)
                    const float m_base = m_run == -INFINITY ? 0.f : m_run;
                    const float m_new = fmaxf(m_run, m_base + tile_max());
                    // a lane without a visible row so far keeps m = -inf and zero weights
                    const bool none = CUT && m_new == -INFINITY;
                    const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
                    m_run = m_new;
                    l_run *= alpha;
#pragma unroll
                    for (int eb = 0; eb < C::EB; ++eb) oacc[eb] *= alpha;
                    lt = weights(std::true_type{}, none ? -INFINITY : m_base - m_new);
                    started = true;
#pragma unroll
                    for (int rr = 0; rr < 16; ++rr) negm[rr] = none ? 0.f : -m_new;
                }
                l_run += lt;
                values();
            }
            __syncthreads();   // buffer 0 is read by every wave before it is refilled
        }
    }
    if constexpr (C::PRIVATE) __syncthreads();   // the merge below reuses the tile buffers

    // ---------------- 3. merge the memory splits, normalise, store ----------------
    l_run += xor32(l_run);   // both halves' keys
    if constexpr (C::MS > 1) {
        float* cmb = reinterpret_cast<float*>(smem);
        constexpr int PER = C::EB * 16 + 2;
        if (ksg > 0) {
            float* dst = cmb + ((size_t)(rb * (KSPLIT - 1) + ksg - 1) * PER) * 64;
#pragma unroll
            for (int eb = 0; eb < C::EB; ++eb)
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) dst[(eb * 16 + rr) * 64 + lane] = oacc[eb][rr];
            dst[(PER - 2) * 64 + lane] = m_run;
            dst[(PER - 1) * 64 + lane] = l_run;
        }
        __syncthreads();
        if (ksg > 0) return;
#pragma unroll
        for (int k = 1; k < KSPLIT; ++k) {
            const float* src = cmb + ((size_t)(rb * (KSPLIT - 1) + k - 1) * PER) * 64;
            const float mk = src[(PER - 2) * 64 + lane];
            const float lk = src[(PER - 1) * 64 + lane];
            const float m_new = fmaxf(m_run, mk);
            // a split that saw no memory rows (m = -inf) contributes nothing
            const float a0 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
            const float a1 = mk == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mk - m_new);
            l_run = l_run * a0 + lk * a1;
#pragma unroll
            for (int eb = 0; eb < C::EB; ++eb)
#pragma unroll
                for (int rr = 0; rr < 16; ++rr)
                    oacc[eb][rr] = oacc[eb][rr] * a0 + src[(eb * 16 + rr) * 64 + lane] * a1;
            m_run = m_new;
        }
    }
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    if (lse_out) {
        // statistics for the backward pass: the row's log2 normaliser and
        // D = <dO_row, O_row> over this head's features (fp32 O)
        float dpart = 0.f;
        if (dO_in && qvalid) {
            const bf16* drow = dO_in + ((size_t)cand * q + s) * d + h * DH;
#pragma unroll
            for (int eb = 0; eb < C::EB; ++eb)
#pragma unroll
                for (int b4 = 0; b4 < 4; ++b4) {
                    const bf16x4 dv = *reinterpret_cast<const bf16x4*>(drow + eb * 32 + b4 * 8 + 4 * g);
#pragma unroll
                    for (int t = 0; t < 4; ++t) dpart += oacc[eb][4 * b4 + t] * inv * (float)dv[t];
                }
        }
        dpart += xor32(dpart);
        if (qvalid && g == 0) {
            const size_t idx = ((size_t)cand * q + s) * heads + h;
            lse_out[idx] = l_run > 0.f ? m_run + __builtin_amdgcn_logf(l_run) : -INFINITY;   // v_log_f32 is log2
            if (dsum_out) dsum_out[idx] = dpart;
        }
    }
    if (qvalid && O) {
        // (8-byte stores: the 16-byte form of join_runs costs this kernel's
        // epilogue spill slots, and its output rows are a small share of its
        // traffic)
        bf16* orow = O + ((size_t)cand * q + s) * d + h * DH;
#pragma unroll
        for (int eb = 0; eb < C::EB; ++eb) {
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

// Variants whose LDS footprint exceeds what one work-group may hold (or whose
// projection staging would need too many registers) are not built; the host
// prefers variants that leave room for two work-groups per compute unit
// (attn_bf16_variant_smem).
constexpr int kMaxSmem = 163840;

template <int DH, int RB, int KSPLIT, bool SEP, bool PROJ>
constexpr bool built() {
    using C = Cfg<DH, RB, KSPLIT, SEP, PROJ>;
    return C::SMEM <= kMaxSmem && C::BUILT;
}

template <int DH, int RB, int KSPLIT, bool SEP, bool PROJ>
hipError_t launch_one(const AttnArgs& a, hipStream_t stream) {
    if constexpr (!built<DH, RB, KSPLIT, SEP, PROJ>()) {
        return hipErrorInvalidValue;
    } else {
        if (PROJ && a.d > kProjMaxD) return hipErrorInvalidValue;
        AttnArgs k = a;
        k.scale_log2 = a.prescaled ? 1.0f : 1.4426950408889634f / sqrtf((float)DH);
        const int64_t blocks = a.max_tiles * a.heads;
        if (blocks <= 0) return hipSuccess;
        // 32-wide heads over one K = V memory (caller-projected queries, an
        // even head count, with or without cutoffs): head pairs, two wave
        // groups over each staged 128-byte line, in XCD-chunked order
        if constexpr (DH == 32 && KSPLIT == 1 && !SEP && !PROJ) {
            if (a.heads % 2 == 0) {
                // (work-groups past the last item exit)
                const int64_t grid = xcd_pair_grid(a.max_tiles, a.heads / 2);
                if (a.cand_len)
                    hipLaunchKernelGGL((attn_bf16_kernel<DH, RB, 2, false, false, true, true>),
                                       dim3((unsigned)grid), dim3(64 * RB * 2), 0, stream, k);
                else
                    hipLaunchKernelGGL((attn_bf16_kernel<DH, RB, 2, false, false, false, true>),
                                       dim3((unsigned)grid), dim3(64 * RB * 2), 0, stream, k);
                return hipGetLastError();
            }
        }
        if (a.cand_len) {
            hipLaunchKernelGGL((attn_bf16_kernel<DH, RB, KSPLIT, SEP, PROJ, true>),
                               dim3((unsigned)blocks), dim3(64 * RB * KSPLIT), 0, stream, k);
        } else {
            hipLaunchKernelGGL((attn_bf16_kernel<DH, RB, KSPLIT, SEP, PROJ, false>),
                               dim3((unsigned)blocks), dim3(64 * RB * KSPLIT), 0, stream, k);
        }
        return hipGetLastError();
    }
}

template <int DH, int RB, int KSPLIT>
hipError_t launch_mode(const AttnArgs& a, hipStream_t stream) {
    const bool sep = a.V != nullptr, proj = a.Z != nullptr;
    if (sep)
        return proj ? launch_one<DH, RB, KSPLIT, true, true>(a, stream)
                    : launch_one<DH, RB, KSPLIT, true, false>(a, stream);
    return proj ? launch_one<DH, RB, KSPLIT, false, true>(a, stream)
                : launch_one<DH, RB, KSPLIT, false, false>(a, stream);
}

template <int DH>
hipError_t launch_dh(const AttnArgs& a, int rb, int ksplit, hipStream_t stream) {
#define XATTN_CASE(R_, S_) \
    if (rb == R_ && ksplit == S_) return launch_mode<DH, R_, S_>(a, stream);
    XATTN_CASE(1, 4)
    XATTN_CASE(2, 2)
    XATTN_CASE(4, 1)
    XATTN_CASE(2, 1)
#undef XATTN_CASE
    return hipErrorInvalidValue;
}

template <int DH, int RB, int KSPLIT, bool SEP, bool PROJ>
constexpr int smem_if_built() {
    return built<DH, RB, KSPLIT, SEP, PROJ>() ? Cfg<DH, RB, KSPLIT, SEP, PROJ>::SMEM : 0;
}

template <int DH, int RB, int KSPLIT>
int smem_of(bool sep, bool proj) {
    if (sep) return proj ? smem_if_built<DH, RB, KSPLIT, true, true>()
                         : smem_if_built<DH, RB, KSPLIT, true, false>();
    return proj ? smem_if_built<DH, RB, KSPLIT, false, true>()
                : smem_if_built<DH, RB, KSPLIT, false, false>();
}

template <int DH>
int variant_smem(int rb, int ksplit, bool sep, bool proj) {
#define XATTN_FIT(R_, S_) \
    if (rb == R_ && ksplit == S_) return smem_of<DH, R_, S_>(sep, proj);
    XATTN_FIT(1, 4)
    XATTN_FIT(2, 2)
    XATTN_FIT(4, 1)
    XATTN_FIT(2, 1)
#undef XATTN_FIT
    return 0;
}

}  // namespace

int attn_bf16_variant_smem(int dh, int rb, int ksplit, bool sep, bool proj) {
    switch (dh) {
        case 32: return variant_smem<32>(rb, ksplit, sep, proj);
        case 64: return variant_smem<64>(rb, ksplit, sep, proj);
        case 128: return variant_smem<128>(rb, ksplit, sep, proj);
        default: return 0;
    }
}

hipError_t launch_attn_bf16(const AttnArgs& a, int rb, int ksplit, hipStream_t stream) {
    switch (a.d / a.heads) {
        case 32: return launch_dh<32>(a, rb, ksplit, stream);
        case 64: return launch_dh<64>(a, rb, ksplit, stream);
        case 128: return launch_dh<128>(a, rb, ksplit, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace xattn
