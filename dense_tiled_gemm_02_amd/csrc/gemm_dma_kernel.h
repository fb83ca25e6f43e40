// Tiled GEMM kernel for gfx950 with direct global -> LDS staging:  D = A x B (+ C).
// (The kernel template; gemm_dma*.hip instantiate its variants.)
//
// Same tile walk as gemm_tile.hip (K loop over BM x BN x BK slabs, grouped
// tile order, masked tails, fp32 accumulation, fp32 -> storage rounding in the
// epilogue), with the staging done the gfx950 way:
//  * global -> LDS without registers: buffer_load_dwordx4 ... lds writes each
//    lane's 16 bytes at LDS byte 16 * lane past a wave-uniform base, so one
//    wave instruction fills 1024 contiguous LDS bytes.  The LDS layout is
//    chosen by which global chunk each lane fetches (an XOR swizzle of 16-byte
//    chunks, for conflict-free operand reads).  Lanes outside the matrix (rows
//    >= M, columns >= N, k >= K) get an offset past the buffer descriptor's
//    range, which makes the hardware write zeros ("Hopper Support in Triton",
//    slides 15-16: masked loads with other = 0);
//  * an LDS ring of ST stages: the loads of K step k + ST - 1 are issued while
//    step k is contracted, one barrier per step (FlagGems "Hygon
//    optimization", section "Software pipelining"; "DCU K100 节点初探",
//    section 5.6, double buffering);
//  * each operand sits in LDS the way it sits in memory.  An operand whose k
//    index is contiguous (A row-major, TA = 0; B stored N x K, TB = 1) is kept
//    as rows of BK contiguous k and read with one 16-byte LDS read per lane
//    per fragment; an operand contiguous along its other index (A stored
//    K x M, TA = 1; B row-major, TB = 0) is kept as rows of BK k of contiguous
//    m (n) and read with the transposing 64-bit LDS read, which hands each
//    lane 4 consecutive k of one row or column: two reads make the 8 k of one
//    MFMA operand.  One shape description (OpShape) serves both operands.
// Descriptors are rebased at every K step (scalar work only), so 32-bit
// buffer offsets cover any matrix whose tile-row panel of A and of B spans
// less than 2 GiB.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "tile_order.h"

namespace dtg {
namespace {

using namespace dev;

// Swizzle of a tile kept as rows of k (CHB 16-byte chunks of contiguous m or n
// per row): physical chunk = logical chunk ^ bsw(r).  Even values keep the two
// chunks a 16-lane group reads from one row adjacent; the 4 (or 8) rows one
// transposing read touches land in distinct bank groups.
template <int CHB>
__device__ __forceinline__ int bsw(int r) {
    if constexpr (CHB >= 16) return 2 * ((r & 3) | (((r >> 3) & 1) << 2));
    else return 2 * (r & 3);
}

// Staging shape of one operand tile of E (= BM or BN) x BK elements.
//  KC: k contiguous in memory: LDS rows are the E indices, BK contiguous k
//      each, chunk swizzle swz<BK/8>(row), one 16-byte read per fragment;
//  !KC: the E index contiguous in memory: LDS rows are the BK k indices, E
//      contiguous elements each, chunk swizzle bsw<E/8>(k row), two
//      transposing reads per fragment.
// A wave instruction fills R whole LDS rows (1024 bytes).  When NW * R is a
// multiple of the swizzle's period, all of a wave's loads share one chunk
// permutation: one voffset register, the row step in the scalar offset.
template <bool KC, int E, int BK, int NW>
struct OpShape {
    static constexpr int CH = KC ? BK / 8 : E / 8;     // 16-byte chunks per LDS row
    static constexpr int R = 64 / CH;                  // LDS rows per wave instruction
    static constexpr int ROWS = KC ? E : BK;           // LDS rows per stage
    static constexpr int IW = ROWS / R / NW;           // instructions per wave per stage
    static constexpr int SZ = E * BK;                  // elements per stage
    static constexpr int PERIOD = KC ? (CH == 4 ? 8 : 16) : (CH >= 16 ? 16 : 4);
    static constexpr bool SHARED = (NW * R) % PERIOD == 0;
    static constexpr int NV = SHARED ? 1 : IW;         // voffset registers
    static_assert(KC ? (CH == 4 || CH == 8 || CH == 16) : (CH >= 8 && CH <= 64 && 64 % CH == 0), "chunks");
    static_assert(IW > 0 && ROWS % (R * NW) == 0, "load split");
    __device__ static int sw(int r) {
        if constexpr (KC) return swz<CH>(r);
        else return bsw<CH>(r);
    }
};

// Element kinds of the tile body: 16-bit floating point (fp16, bf16) with fp32
// accumulation and a 16-bit output, or 8-bit integers with int32 accumulation
// and output.  The int8 operands are staged and read as pairs of bytes (one
// 16-bit element holds two consecutive k), so the K loop is the same code;
// K, BK and the strides are in those 16-bit units.
enum { kElF16 = 0, kElBF16 = 1, kElI8 = 2 };

// Operation O of NR reads and NL loads issued in one sequence with the loads
// spread evenly: load j sits at position floor((2 j + 1) (NR + NL) / (2 NL)).
// Returns the load's number, or -(read number) - 1.
constexpr int mix_loads(int O, int NR, int NL) {
    int loads_before = 0;
    for (int j = 0; j < NL; ++j) {
        const int at = ((2 * j + 1) * (NR + NL)) / (2 * NL);
        if (at == O) return j;
        if (at < O) ++loads_before;
    }
    return -(O - loads_before) - 1;
}

// What one call of the tile body computes: output tile `tile` (grouped order)
// over its K steps [kt0, kt1), as part `part` of `nparts` (1: the whole K
// range, written out directly).  With several parts, part j's fp32 partial
// tile goes to workspace slot base + slot0 when j == 0 and base + slot1 + j
// otherwise; slots base .. base + nslots - 1 are this work's to address.
struct Work {
    int tile, kt0, kt1, part, nparts, base, slot0, slot1, nslots;
};

// The work of a data-parallel or K-sliced launch: one workgroup per (K slice,
// output tile); the XCD permutation runs over the whole grid, consecutive
// positions are consecutive tiles (grouped order) of one slice.  With one
// slice this is tile_of_workgroup.
template <int BK>
__device__ __forceinline__ Work slice_work(const KArgs& p) {
    const int ntiles = p.num_pid_m * p.num_pid_n;
    const int NS = p.splits;
    const int pos = xcd_permute<int>(blockIdx.x, ntiles * NS, p.xcds);
    const int slice = pos / ntiles;
    Work w;
    w.tile = pos - slice * ntiles;
    const int nkt_all = (p.K + BK - 1) / BK;
    const int per_slice = (nkt_all + NS - 1) / NS;
    w.kt0 = slice * per_slice;
    w.kt1 = (w.kt0 + per_slice < nkt_all) ? w.kt0 + per_slice : nkt_all;
    w.part = slice;
    w.nparts = NS;
    w.base = w.tile * NS;
    w.slot0 = w.slot1 = 0;
    w.nslots = NS;
    return w;
}

// XCH: the K-slice exchange is compiled for tiles of more than 64
// accumulators per lane too (the stream-K variants).  NTB: B is loaded
// non-temporal (the variants for a grid of one row of tiles, where each byte
// of B is read by one workgroup per K slice).
template <int BM, int BN, int BK, int WM, int WN, int MF, int ST, int EL, bool TA, bool TB, bool XCH = false,
          bool NTB = false>
__device__ __forceinline__ void dma_tile(const KArgs& p, const Work& wk) {
    constexpr bool BF16 = EL == kElBF16;
    constexpr bool I8 = EL == kElI8;
    constexpr int NW = WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / MF, FN = TN / MF;
    constexpr int KI = (MF == 16) ? 32 : 16;
    constexpr bool AKC = !TA, BKC = TB;         // operands with contiguous k
    typedef OpShape<AKC, BM, BK, NW> OA;
    typedef OpShape<BKC, BN, BK, NW> OB;
    constexpr int SA = OA::SZ, SB = OB::SZ;     // elements per stage
    constexpr int IA_W = OA::IW, IB_W = OB::IW; // loads per wave per stage
    constexpr int L = IA_W + IB_W;
    constexpr int NKS = BK / KI;                // instruction k sub-steps per K step
    static_assert(BM % (WM * MF) == 0 && BN % (WN * MF) == 0, "tile vs wave grid");
    static_assert(BK % KI == 0, "BK");
    static_assert(ST >= 2 && ST <= 5 && (ST - 1) * L < 64, "stages");
    typedef typename AccT<MF>::type acc_t;
    // accumulators per lane; above 128 (one wave per SIMD holding a
    // 128 x 128 wave tile) they live in AGPRs, placed there explicitly
    constexpr bool AGPR = FM * FN * AccT<MF>::regs > 128;
    static_assert(!(I8 && AGPR), "int8 tiles keep their accumulators in VGPRs");

    __shared__ __attribute__((aligned(1024))) uint16_t smem[ST * (SA + SB)];

    int tid = threadIdx.x;
    // Stream-K runs this body in a loop: an opaque lane index keeps the
    // compiler from hoisting lane-dependent addresses (the epilogue's among
    // them) out of that loop, where they would stay live through the K loop.
    if constexpr (XCH) asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    const int NS = wk.nparts;
    const int tile_lin = wk.tile, slice = wk.part;
    int pid_m, pid_n;
    grouped_tile<int>(tile_lin, p.num_pid_m, p.num_pid_n, p.group_m, &pid_m, &pid_n);
    const int m0 = pid_m * BM, n0 = pid_n * BN;
    const int M = p.M, N = p.N, K = p.K;

    // leading strides of the two operands as they sit in memory (elements)
    const int64_t lda = TA ? p.sak : p.lda;
    const int64_t ldb = TB ? p.sbn : p.ldb;

    // ---- per-lane load offsets (bytes, relative to the rebased descriptors).
    // Load X of an operand fills LDS rows X*NW*R + wave*R + lane/CH (its E
    // index when KC, its k index otherwise); c8 is the first element of the
    // lane's 16-byte chunk along the other index.  Bounds cost no branch:
    //  * KC operand (rows of m or n): rows past the matrix lie past the
    //    descriptor's range (it ends at the last element and the row stride is
    //    at least K); the K tail is a per-lane bit OR'd into the offset;
    //  * operand kept as rows of k: chunks past M (N) get an offset past any
    //    range once for the kernel; rows past K lie past the range (the row
    //    stride is at least M or N).
    // The planner admits only strides for which these hold.
    const int a_row0 = wave * OA::R + lane / OA::CH;
    const int b_row0 = wave * OB::R + lane / OB::CH;
    uint32_t a_voff[OA::NV], b_voff[OB::NV];
    int a_c8[OA::NV], b_c8[OB::NV];
#pragma unroll
    for (int i = 0; i < OA::NV; ++i) {
        const int row = a_row0 + i * NW * OA::R;
        const int c = (lane % OA::CH) ^ OA::sw(row);
        a_voff[i] = static_cast<uint32_t>(static_cast<int64_t>(row) * lda * 2 + c * 16);
        if (!AKC && m0 + 8 * c >= M) a_voff[i] = kOOB;
        a_c8[i] = 8 * c;
    }
#pragma unroll
    for (int i = 0; i < OB::NV; ++i) {
        const int row = b_row0 + i * NW * OB::R;
        const int c = (lane % OB::CH) ^ OB::sw(row);
        b_voff[i] = static_cast<uint32_t>(static_cast<int64_t>(row) * ldb * 2 + c * 16);
        if (!BKC && n0 + 8 * c >= N) b_voff[i] = kOOB;
        b_c8[i] = 8 * c;
    }
    const uint32_t a_step = static_cast<uint32_t>(NW * OA::R) * static_cast<uint32_t>(lda) * 2u;
    const uint32_t b_step = static_cast<uint32_t>(NW * OB::R) * static_cast<uint32_t>(ldb) * 2u;

    // LDS layout: the ST stages of A, then the ST stages of B.
    const uint32_t smem0 = lds_addr(smem);

    // Buffer descriptors of K step kt: each starts at the tile's first element
    // of that step (k0 and m0 / n0) and ends at the matrix's last element, so
    // any offset past it reads zeros.  The range is the tile's whole range
    // (64-bit, once) less the step's offset, capped in 32-bit scalar
    // arithmetic; no per-step branch.
    struct Desc {
        __amdgpu_buffer_rsrc_t ra, rb;
        int k0;
    };
    // this part's K steps: [kt0, kt1)
    const int kt0 = wk.kt0, kt1 = wk.kt1;
    const uint64_t a_full = 2u * static_cast<uint64_t>(AKC ? static_cast<int64_t>(M - 1 - m0) * lda + K
                                                           : static_cast<int64_t>(K - 1) * lda + (M - m0));
    const uint64_t b_full = 2u * static_cast<uint64_t>(BKC ? static_cast<int64_t>(N - 1 - n0) * ldb + K
                                                           : static_cast<int64_t>(K - 1) * ldb + (N - n0));
    const uint16_t* a_tile = AKC ? p.A + static_cast<int64_t>(m0) * lda : p.A + m0;
    const uint16_t* b_tile = BKC ? p.B + static_cast<int64_t>(n0) * ldb : p.B + n0;
    auto make_desc = [&](int kt) {
        Desc d;
        d.k0 = kt * BK;
        const bool live = kt < kt1;   // steps past the slice (issued only to keep the ring uniform) read nothing
        const int kb = live ? d.k0 : 0;
        const int64_t aoff = AKC ? kb : static_cast<int64_t>(kb) * lda;   // elements
        const int64_t boff = BKC ? kb : static_cast<int64_t>(kb) * ldb;
        d.ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a_tile + aoff), 0,
                                                 live ? capped_records(a_full, 2u * static_cast<uint64_t>(aoff)) : 0u,
                                                 kRsrcWord3);
        d.rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(b_tile + boff), 0,
                                                 live ? capped_records(b_full, 2u * static_cast<uint64_t>(boff)) : 0u,
                                                 kRsrcWord3);
        return d;
    };
    // Load number X (A loads first, then B) of a K step into LDS stage s.
    auto load_op = [&](auto x_tag, const Desc& d, int s) {
        constexpr int X = decltype(x_tag)::value;
        if constexpr (X < IA_W) {
            constexpr int V = OA::SHARED ? 0 : X;
            uint32_t v = a_voff[V];
            const uint32_t so = OA::SHARED ? X * a_step : 0u;
            if constexpr (AKC) v |= (d.k0 + a_c8[V] < K) ? 0u : kOOB;
            // (a non-const local: clang's host pass drops the kernel when the
            // builtin is handed a member of a const reference)
            __amdgpu_buffer_rsrc_t r = d.ra;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(smem + s * SA + (X * NW + wave) * 512), 16, v,
                                                    so, 0, 0);
        } else {
            constexpr int Y = X - IA_W;
            constexpr int V = OB::SHARED ? 0 : Y;
            uint32_t v = b_voff[V];
            const uint32_t so = OB::SHARED ? Y * b_step : 0u;
            if constexpr (BKC) v |= (d.k0 + b_c8[V] < K) ? 0u : kOOB;
            __amdgpu_buffer_rsrc_t r = d.rb;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                r, (lds_void_t*)(smem + ST * SA + s * SB + (Y * NW + wave) * 512), 16, v, so, 0,
                NTB ? kNonTemporal : 0);
        }
    };
    auto issue_tile = [&](int kt, int s) {
        const Desc d = make_desc(kt);
        static_for<L>([&](auto x_tag) { load_op(x_tag, d, s); });
    };

    acc_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < AccT<MF>::regs; ++r) acc[i][j][r] = 0.0f;

    // ---- per-lane operand read addresses (LDS bytes).  For the fragment of
    // outer index e = w*T + f*MF + lane % MF (w the wave's row or column):
    //  KC operand, sub-step ks: row e, chunk ks*KI/8 + lane / MF (swizzled);
    //     f*MF*BK*2 goes into the read's offset field: addresses per ks.
    //  !KC operand, half h: the transposing read of k rows
    //     ks*KI + 8 g + 4 h + (jq >> 2) at the 4 indices from
    //     nb + 4 (jq & 3); (ks*KI + 4 h) * E * 2 goes into the offset field:
    //     addresses per fragment.
    //  The stage offset goes there too when the 16-bit field can hold it,
    //  else each stage keeps its own addresses.
    constexpr int IMA = AKC ? (FM - 1) * MF * BK * 2 : (BK - 4) * BM * 2;
    constexpr int IMB = BKC ? (FN - 1) * MF * BK * 2 : (BK - 4) * BN * 2;
    constexpr bool AI = (ST - 1) * SA * 2 + IMA < 65536;
    constexpr bool BI = (ST - 1) * SB * 2 + IMB < 65536;
    constexpr int NAS = AI ? 1 : ST, NBS = BI ? 1 : ST;
    constexpr int NAA = AKC ? NKS : FM, NBA = BKC ? NKS : FN;
    uint32_t a_addr[NAS][NAA], b_addr[NBS][NBA];
    {
        int jq, g, col;
        if constexpr (MF == 16) { jq = lane & 15; g = lane >> 4; col = 0; }
        else { jq = lane & 15; g = lane >> 5; col = 16 * ((lane >> 4) & 1); }
        const int x_row = 8 * g + (jq >> 2);
        // one operand's addresses: KC (per ks) or transposing (per fragment)
        auto fill = [&](auto kc_tag, auto shape_tag, int w, int t, int nf, uint32_t sbase, uint32_t* out) {
            constexpr bool KCX = decltype(kc_tag)::value;
            typedef decltype(shape_tag) OS;
            if constexpr (KCX) {
                const int e_row = w * t + lane % MF;
                const int kc0 = lane / MF;
                const int sw = swz<OS::CH>(lane % MF);
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    out[ks] = sbase + (e_row * BK + (((ks * (KI / 8) + kc0) ^ sw) * 8)) * 2;
            } else {
                constexpr int EX = OS::SZ / BK;
                const int xsw = (OS::CH >= 16) ? 2 * ((jq >> 2) | ((g & 1) << 2)) : 2 * (jq >> 2);
                for (int f = 0; f < nf; ++f) {
                    const int nb = w * t + f * MF + col;
                    out[f] = sbase + (x_row * EX + (((nb >> 3) ^ xsw) << 3) + 4 * (jq & 3)) * 2;
                }
            }
        };
#pragma unroll
        for (int st = 0; st < NAS; ++st)
            fill(std::integral_constant<bool, AKC>{}, OA{}, wm, TM, FM, smem0 + st * SA * 2, a_addr[st]);
#pragma unroll
        for (int st = 0; st < NBS; ++st)
            fill(std::integral_constant<bool, BKC>{}, OB{}, wn, TN, FN, smem0 + (ST * SA + st * SB) * 2, b_addr[st]);
    }

    // Fragments, double-buffered across k sub-steps; a transposed operand's
    // two halves (k 0..3 and 4..7) are combined after their second read.
    u32x4 fa[2][FM], fb[2][FN];
    i16x4 ha[2][AKC ? 1 : FM][2], hb[2][BKC ? 1 : FN][2];
    constexpr int NRA = AKC ? FM : 2 * FM, NRB = BKC ? FN : 2 * FN;
    constexpr int NR = NRA + NRB;     // LDS reads per sub-step

    // LDS read number R of sub-step KS of stage S into slot SL: the B reads
    // first, then the A reads.
    auto read_op = [&](auto stage_tag, auto ks_tag, auto slot_tag, auto r_tag) {
        constexpr int S = decltype(stage_tag)::value;
        constexpr int KS = decltype(ks_tag)::value;
        constexpr int SL = decltype(slot_tag)::value;
        constexpr int R = decltype(r_tag)::value;
        if constexpr (R < NRB) {
            if constexpr (BKC) {
                fb[SL][R] = lds_read16<(BI ? S * SB * 2 : 0) + R * MF * BK * 2>(b_addr[BI ? 0 : S][KS]);
            } else {
                constexpr int J = R / 2, H = R % 2;
                hb[SL][J][H] =
                    lds_read_tr<(BI ? S * SB * 2 : 0) + (KS * KI + 4 * H) * BN * 2>(b_addr[BI ? 0 : S][J]);
                if constexpr (H == 1)
                    fb[SL][J] = __builtin_bit_cast(u32x4, __builtin_shufflevector(hb[SL][J][0], hb[SL][J][1],
                                                                                  0, 1, 2, 3, 4, 5, 6, 7));
            }
        } else {
            constexpr int RA2 = R - NRB;
            if constexpr (AKC) {
                fa[SL][RA2] = lds_read16<(AI ? S * SA * 2 : 0) + RA2 * MF * BK * 2>(a_addr[AI ? 0 : S][KS]);
            } else {
                constexpr int I = RA2 / 2, H = RA2 % 2;
                ha[SL][I][H] =
                    lds_read_tr<(AI ? S * SA * 2 : 0) + (KS * KI + 4 * H) * BM * 2>(a_addr[AI ? 0 : S][I]);
                if constexpr (H == 1)
                    fa[SL][I] = __builtin_bit_cast(u32x4, __builtin_shufflevector(ha[SL][I][0], ha[SL][I][1],
                                                                                  0, 1, 2, 3, 4, 5, 6, 7));
            }
        }
    };
    auto wait_frags = [&](auto slot_tag) {
        constexpr int SL = decltype(slot_tag)::value;
        lds_wait_all();
#pragma unroll
        for (int j = 0; j < FN; ++j) tie(fb[SL][j]);
#pragma unroll
        for (int i = 0; i < FM; ++i) tie(fa[SL][i]);
    };
    // MFMA number Q (row-fragment major) of a sub-step, operands in slot SL.
    // The B fragment goes in as the instruction's first operand and the A
    // fragment as its second, so each accumulator holds the transposed block:
    // a lane's registers are consecutive columns of one row of D, stored as
    // 8-byte vectors in the epilogue.
    auto mfma_op = [&](auto slot_tag, auto q_tag) {
        constexpr int SL = decltype(slot_tag)::value;
        constexpr int Q = decltype(q_tag)::value;
        constexpr int I = Q / FN, J = Q % FN;
        if constexpr (I8) acc[I][J] = mfma_i8<MF>(fb[SL][J], fa[SL][I], acc[I][J]);
        else if constexpr (AGPR) mfma_agpr<MF, BF16>(acc[I][J], fb[SL][J], fa[SL][I]);
        else acc[I][J] = mfma<MF, BF16>(fb[SL][J], fa[SL][I], acc[I][J]);
    };
    // accumulator element (i, j, r) in a VGPR, for the reduce and the epilogue
    auto acc_at = [&](int i, int j, int r) -> float {
        if constexpr (AGPR) return agpr_get(acc[i][j][r]);
        else return acc[i][j][r];
    };
    constexpr int NQ = FM * FN;       // MFMAs per sub-step

    // The MFMAs of a sub-step with NOPS memory operations spread between them:
    // operation o follows MFMA number o * SP; the last TAIL MFMAs carry none,
    // so the LDS reads have landed when the sub-step ends.  When there are
    // more operations than MFMA slots, PER of them follow each MFMA from the
    // first on (one-wave-per-SIMD tiles; the others leave the surplus after
    // the last MFMA).  Every group is fenced, so the compiler keeps exactly
    // this order.
    auto interleave = [&](auto slot_tag, auto nops_tag, auto&& op) {
        constexpr int SL = decltype(slot_tag)::value;
        constexpr int NOPS = decltype(nops_tag)::value;
        constexpr int TAIL = NQ / 4;
        constexpr int SLOTS = NQ - TAIL;
        constexpr int SP = (NOPS == 0) ? 1 : (SLOTS / NOPS > 0 ? SLOTS / NOPS : 1);
        constexpr int PER = (!AGPR || SLOTS / NOPS > 0) ? 1 : (NOPS + SLOTS - 1) / SLOTS;
        static_for<NQ>([&](auto q_tag) {
            constexpr int Q = decltype(q_tag)::value;
            mfma_op(std::integral_constant<int, SL>{}, q_tag);
            if constexpr (PER == 1) {
                if constexpr (Q % SP == 0 && Q / SP < NOPS) op(std::integral_constant<int, Q / SP>{});
            } else {
                static_for<PER>([&](auto e_tag) {
                    constexpr int O = Q * PER + decltype(e_tag)::value;
                    if constexpr (O < NOPS) op(std::integral_constant<int, O>{});
                });
            }
            __builtin_amdgcn_sched_barrier(0);
        });
        // ops left over when there are more operations than MFMA slots
        if constexpr (PER == 1 && NOPS > NQ / SP) {
            static_for<NOPS - NQ / SP>([&](auto o_tag) {
                op(std::integral_constant<int, NQ / SP + decltype(o_tag)::value>{});
            });
        }
    };

    const int nkt = kt1 > kt0 ? kt1 - kt0 : 0;   // K steps of this slice

    // One K step (tile kt) on LDS stage S = kt % ST; U is kt's position in the
    // unrolled loop, which fixes which fragment slot holds which sub-step.  On
    // entry the fragments of sub-step 0 are in slot (U * NKS) % 2.  Sub-step
    // ks runs its MFMAs with the reads of sub-step ks + 1 between them.  The
    // last sub-step first waits for tile kt + 1 (tiles up to kt + ST - 1 have
    // been issued, so ST - 2 tiles may stay in flight), passes the barrier
    // (after it every wave has read all of tile kt, so its stage may be
    // refilled), and runs its MFMAs with the reads of tile kt + 1's first
    // sub-step and the loads of tile kt + ST into this stage between them.
    // Every step does the same: tiles past the end of K are loaded from an
    // empty range (zeros, no memory access) and read but never used.
    auto step = [&](auto u_tag, int kt) {
        constexpr int U = decltype(u_tag)::value;
        constexpr int S = U % ST;
        constexpr int S1 = (S + 1) % ST;
        static_for<NKS>([&](auto ks_tag) {
            constexpr int KS = decltype(ks_tag)::value;
            constexpr int CUR = (U * NKS + KS) & 1, NXT = CUR ^ 1;
            const auto cur = std::integral_constant<int, CUR>{};
            const auto nxt = std::integral_constant<int, NXT>{};
            if constexpr (KS + 1 < NKS) {
                interleave(cur, std::integral_constant<int, NR>{}, [&](auto o_tag) {
                    read_op(std::integral_constant<int, S>{}, std::integral_constant<int, KS + 1>{}, nxt, o_tag);
                });
            } else {
                const Desc d = make_desc(kt + ST);
                wait_vm<(ST - 2) * L>();
                __builtin_amdgcn_s_barrier();
                interleave(cur, std::integral_constant<int, NR + L>{}, [&](auto o_tag) {
                    constexpr int O = decltype(o_tag)::value;
                    if constexpr (AGPR) {
                        // one wave per SIMD: the loads spread evenly among the
                        // reads (a burst of them fills the address unit's
                        // command queue and stalls the only wave)
                        constexpr int Q = mix_loads(O, NR, L);
                        if constexpr (Q >= 0)
                            load_op(std::integral_constant<int, Q>{}, d, S);
                        else
                            read_op(std::integral_constant<int, S1>{}, std::integral_constant<int, 0>{}, nxt,
                                    std::integral_constant<int, -Q - 1>{});
                    } else if constexpr (O < NR) {
                        read_op(std::integral_constant<int, S1>{}, std::integral_constant<int, 0>{}, nxt, o_tag);
                    } else {
                        load_op(std::integral_constant<int, O - NR>{}, d, S);
                    }
                });
            }
            wait_frags(nxt);
        });
    };

    // unroll so that both the stage and the fragment-slot parity repeat
    constexpr int UNROLL = ((ST * NKS) % 2 == 0) ? ST : 2 * ST;
    if (nkt > 0) {
        static_for<ST>([&](auto t_tag) { issue_tile(kt0 + decltype(t_tag)::value, decltype(t_tag)::value); });
        wait_vm<(ST - 1) * L>();
        __builtin_amdgcn_s_barrier();
        static_for<NR>([&](auto r_tag) {
            read_op(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{},
                    std::integral_constant<int, 0>{}, r_tag);
        });
        wait_frags(std::integral_constant<int, 0>{});
        if constexpr (AGPR) {
            // Whole unrolled groups only: a conditional step inside the loop
            // makes the allocator move AGPR accumulators through scratch.  A
            // step past the slice contracts the zeros its empty-range loads
            // wrote, which leaves every accumulator unchanged (an exact +0
            // added to a sum that started at +0).
            for (int j = 0; j < nkt; j += UNROLL)
                static_for<UNROLL>([&](auto u_tag) { step(u_tag, kt0 + j + decltype(u_tag)::value); });
        } else {
            for (int j = 0; j < nkt; j += UNROLL) {
                static_for<UNROLL>([&](auto u_tag) {
                    if (j + decltype(u_tag)::value < nkt) step(u_tag, kt0 + j + decltype(u_tag)::value);
                });
            }
        }
        // no load may still be writing this workgroup's LDS when it exits
        wait_vm<0>();
    }
    if constexpr (AGPR) agpr_settle();

    // ---- K slices across workgroups: publish this part's fp32 partial tile;
    // the workgroup that arrives last at the tile's counter sums the parts
    // in part order (so the result does not depend on arrival order) into
    // acc and goes on to the epilogue below; the others are done.  Partials
    // are kept in register order, [slot][wave][block][lane][4 floats], so
    // each lane writes and reads back only its own 16-byte runs, with
    // system-coherent accesses (they bypass the per-XCD L2 caches); see
    // arrive_last for the ordering.
    constexpr int NB = FM * FN * (AccT<MF>::regs / 4);   // 16-byte runs per lane
    // (two units of partials are held in registers: only tiles of at most
    // 64 accumulators per lane take K slices, or 128 in the XCH variants;
    // the planner keeps the others at 1)
    static_assert(NB > 16 || !AGPR, "K slices keep their partials in VGPRs");
    if constexpr ((NB <= 16 || (XCH && NB <= 32)) && !I8 && !AGPR) if (NS > 1) {
        constexpr int64_t WAVE_F = static_cast<int64_t>(NB) * 64 * 4;   // floats per wave per slot
        int* counters = static_cast<int*>(p.ws);
        float* parts = reinterpret_cast<float*>(static_cast<char*>(p.ws) + kCounterBytes) +
                       static_cast<int64_t>(wk.base) * NW * WAVE_F;
        const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
            parts, 0, clamp_records(static_cast<int64_t>(wk.nslots) * NW * WAVE_F * 4), kRsrcWord3);
        auto run_off = [&](int sl, int b) {   // byte offset of lane's run b of part sl
            const int slot = sl == 0 ? wk.slot0 : wk.slot1 + sl;
            return static_cast<uint32_t>(((static_cast<int64_t>(slot) * NW + wave) * WAVE_F + (b * 64 + lane) * 4) * 4);
        };
        // run b = (i * FN + j) * G + g holds registers 4g..4g+3 of acc[i][j]
        constexpr int G = AccT<MF>::regs / 4;
        auto get_run = [&](auto b_tag) {
            constexpr int B = decltype(b_tag)::value;
            constexpr int I = B / G / FN, J = (B / G) % FN, Q = B % G;
            f32x4 v;
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = acc[I][J][4 * Q + r];
            return v;
        };
        auto set_run = [&](auto b_tag, const f32x4& v) {
            constexpr int B = decltype(b_tag)::value;
            constexpr int I = B / G / FN, J = (B / G) % FN, Q = B % G;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[I][J][4 * Q + r] = v[r];
        };
        static_for<NB>([&](auto b_tag) {
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, get_run(b_tag)), pr,
                                                   run_off(slice, decltype(b_tag)::value), 0, kSysScope);
        });
        if (!arrive_last(&counters[tile_lin], NS, reinterpret_cast<int*>(smem))) return;
        // Sum the parts in order into acc (this part's own runs are read back
        // like the others: the same bits).  Loads go in units of HB runs, the
        // next unit in flight while one is added: two units of registers.
        constexpr int HB = (NB <= 8) ? NB : 8;
        constexpr int UPS = NB / HB;                  // units per slice
        f32x4 buf[2][HB];
        auto fetch = [&](int u, int bb) {
            const int sl = u / UPS, b0 = (u % UPS) * HB;
#pragma unroll
            for (int b = 0; b < HB; ++b)
                buf[bb][b] = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(pr, run_off(sl, b0 + b), 0, kSysScope));
        };
        auto add = [&](int u, int bb) {
            static_for<UPS>([&](auto h_tag) {
                constexpr int H = decltype(h_tag)::value;
                if (u % UPS == H) {
                    static_for<HB>([&](auto b_tag) {
                        constexpr int B = H * HB + decltype(b_tag)::value;
                        const f32x4 cur = (u < UPS) ? f32x4{0.0f, 0.0f, 0.0f, 0.0f}
                                                    : get_run(std::integral_constant<int, B>{});
                        set_run(std::integral_constant<int, B>{}, cur + buf[bb][decltype(b_tag)::value]);
                    });
                }
            });
        };
        const int nu = NS * UPS;
        fetch(0, 0);
        for (int u = 0; u < nu; u += 2) {
            if (u + 1 < nu) fetch(u + 1, 1);
            add(u, 0);
            if (u + 1 < nu) {
                if (u + 2 < nu) fetch(u + 2, 0);
                add(u + 1, 1);
            }
        }
        if (tid == 0) __hip_atomic_store(&counters[tile_lin], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }

    // ---- epilogue.  Lane l holds, per block (i, j), row l % MF of the block
    // and G runs of 4 consecutive columns (16x16x32: columns 4 (l / 16) +
    // 0..3; 32x32x16: run q at columns 8 q + 4 (l / 32) + 0..3).
    constexpr int G = AccT<MF>::regs / 4;

    if constexpr (I8) {
        // int32 results: the tile is staged through LDS in P8 passes of BM / P8
        // rows (16-byte chunks of 4 values at chunk position c ^ (r mod 16) of
        // their row), then each thread adds C to a 4-value row chunk and
        // writes it as one 16-byte store.  Integer sums wrap modulo 2^32, as
        // the instruction's accumulator does.
        constexpr int LDSB = ST * (SA + SB) * 2;
        constexpr int P8 = (BM * BN * 4 <= LDSB)                       ? 1
                           : (WM % 2 == 0 && BM * BN * 2 <= LDSB)     ? 2
                           : (WM % 4 == 0 && BM * BN <= LDSB)         ? 4
                                                                      : 0;
        static_assert(P8 > 0, "the int32 tile must fit the LDS in at most 4 passes");
        constexpr int PR = BM / P8, WPP = WM / P8, C4 = BN / 4, NT = 64 * NW;
        static_assert((PR * C4) % NT == 0 && C4 >= 16, "whole rounds of 4-value chunks");
        typedef uint32_t v4u __attribute__((ext_vector_type(4)));
        uint8_t* const stage = reinterpret_cast<uint8_t*>(smem);
        uint32_t* const D32 = reinterpret_cast<uint32_t*>(p.D);
        const uint32_t* const C32 = reinterpret_cast<const uint32_t*>(p.C);
        const bool has_c = p.has_c != 0;
        const bool vec4 = (p.ldd % 4 == 0) && (reinterpret_cast<uintptr_t>(p.D) % 16 == 0) &&
                          (!has_c || ((p.ldc % 4 == 0) && (reinterpret_cast<uintptr_t>(p.C) % 16 == 0)));
#pragma unroll
        for (int pass = 0; pass < P8; ++pass) {
            __syncthreads();   // operand reads (first pass) or the previous pass's reads are done
            if (wm / WPP == pass) {
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
#pragma unroll
                        for (int q = 0; q < G; ++q) {
                            const int row = (wm % WPP) * TM + i * MF + (lane % MF);
                            const int col = wn * TN + j * MF + 8 * q + 4 * (lane / MF);
                            const v4u v = {__float_as_uint(acc[i][j][4 * q]), __float_as_uint(acc[i][j][4 * q + 1]),
                                           __float_as_uint(acc[i][j][4 * q + 2]),
                                           __float_as_uint(acc[i][j][4 * q + 3])};
                            *reinterpret_cast<v4u*>(stage + row * (BN * 4) + ((col / 4) ^ (row % 16)) * 16) = v;
                        }
            }
            __syncthreads();
#pragma unroll
            for (int x0 = 0; x0 < PR * C4; x0 += NT) {
                const int x = x0 + tid;
                const int row = x / C4, c4 = x % C4;
                const int gr = m0 + pass * PR + row, gc = n0 + c4 * 4;
                if (gr < M && gc < N) {
                    v4u v = *reinterpret_cast<const v4u*>(stage + row * (BN * 4) + (c4 ^ (row % 16)) * 16);
                    uint32_t* d = D32 + static_cast<int64_t>(gr) * p.ldd + gc;
                    const uint32_t* c = has_c ? C32 + static_cast<int64_t>(gr) * p.ldc + gc : nullptr;
                    if (vec4 && gc + 4 <= N) {
                        if (has_c) v += *reinterpret_cast<const v4u*>(c);
                        typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));
                        __builtin_nontemporal_store(__builtin_bit_cast(nt_u32x4, v), reinterpret_cast<nt_u32x4*>(d));
                    } else {
                        for (int e = 0; e < 4 && gc + e < N; ++e) d[e] = v[e] + (has_c ? c[e] : 0u);
                    }
                }
            }
        }
        return;
    } else {

    // Without an addend the tile, rounded, is staged through the (now idle)
    // LDS and written out as whole 16-byte chunks of rows: a store
    // instruction then covers two or four complete tile rows instead of 16
    // rows x 32 bytes, and the output goes out at the rate of a plain fill.
    // Chunk c of tile row r sits at chunk position c ^ (r mod CPR) of the
    // row, which spreads a write instruction's rows over the banks.
    constexpr int CPR = BN / 8;                       // 16-byte chunks per tile row
    if constexpr (BM * BN <= ST * (SA + SB)) {
        if (p.has_c == 0) {
            uint8_t* const stage = reinterpret_cast<uint8_t*>(smem);
            __syncthreads();   // every wave is past its last operand read
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int q = 0; q < G; ++q) {
                        const int row = wm * TM + i * MF + (lane % MF);
                        const int col = wn * TN + j * MF + 8 * q + 4 * (lane / MF);
                        uint2 dv;
                        dv.x = static_cast<uint32_t>(narrow<BF16>(acc_at(i, j, 4 * q))) |
                               (static_cast<uint32_t>(narrow<BF16>(acc_at(i, j, 4 * q + 1))) << 16);
                        dv.y = static_cast<uint32_t>(narrow<BF16>(acc_at(i, j, 4 * q + 2))) |
                               (static_cast<uint32_t>(narrow<BF16>(acc_at(i, j, 4 * q + 3))) << 16);
                        const int pos = ((col / 8) ^ (row % CPR)) * 16 + (col % 8) * 2;
                        *reinterpret_cast<uint2*>(stage + row * (BN * 2) + pos) = dv;
                    }
            __syncthreads();
            constexpr int NT = 64 * NW;
            static_assert((BM * CPR) % NT == 0, "whole chunk rounds");
            const bool vec8 = (p.ldd % 8 == 0) && (reinterpret_cast<uintptr_t>(p.D) % 16 == 0);
#pragma unroll
            for (int x0 = 0; x0 < BM * CPR; x0 += NT) {
                const int x = x0 + tid;
                const int row = x / CPR, cc = x % CPR;
                const int gr = m0 + row, gc = n0 + cc * 8;
                if (gr < M && gc < N) {
                    const uint4 v = *reinterpret_cast<const uint4*>(stage + row * (BN * 2) + (cc ^ (row % CPR)) * 16);
                    uint16_t* d = p.D + static_cast<int64_t>(gr) * p.ldd + gc;
                    if (vec8 && gc + 8 <= N) {
                        store16_nt(d, v.x, v.y, v.z, v.w);
                    } else {
                        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
                        for (int e = 0; e < 8 && gc + e < N; ++e)
                            d[e] = static_cast<uint16_t>(u[e / 2] >> (16 * (e % 2)));
                    }
                }
            }
            return;
        }
    }

    // With an addend the fp32 tile is staged instead, in P passes of BM / P
    // rows (the waves of WM / P wave rows each), so that C is read and D
    // written as whole 16-byte row chunks: acc + C in fp32, rounded once, as
    // in the register path below.  16-byte chunks of 4 floats sit at chunk
    // position c ^ (r mod 16) of their row, which keeps a 16-lane write
    // group's 16 rows on distinct banks.
    constexpr int P = (BM * BN * 4 <= ST * (SA + SB) * 2)       ? 1
                      : (WM % 2 == 0 && BM * BN * 2 <= ST * (SA + SB) * 2) ? 2
                      : (WM % 4 == 0 && BM * BN <= ST * (SA + SB) * 2)     ? 4
                                                                           : 0;
    if constexpr (P > 0) {
        if (p.has_c != 0) {
            constexpr int PR = BM / P;                    // tile rows per pass
            constexpr int WPP = WM / P;                   // wave rows per pass
            constexpr int C32 = BN / 4;                   // fp32 chunks per tile row
            constexpr int NT = 64 * NW;
            static_assert((PR * (BN / 8)) % NT == 0, "whole rounds of 8-element runs");
            uint8_t* const stage = reinterpret_cast<uint8_t*>(smem);
            const bool vec8 = (p.ldd % 8 == 0) && (reinterpret_cast<uintptr_t>(p.D) % 16 == 0) &&
                              (p.ldc % 8 == 0) && (reinterpret_cast<uintptr_t>(p.C) % 16 == 0);
#pragma unroll
            for (int pass = 0; pass < P; ++pass) {
                __syncthreads();   // operand reads (first pass) or the previous pass's reads are done
                if (wm / WPP == pass) {
#pragma unroll
                    for (int i = 0; i < FM; ++i)
#pragma unroll
                        for (int j = 0; j < FN; ++j)
#pragma unroll
                            for (int q = 0; q < G; ++q) {
                                const int row = (wm % WPP) * TM + i * MF + (lane % MF);
                                const int col = wn * TN + j * MF + 8 * q + 4 * (lane / MF);
                                const f32x4 v = {acc_at(i, j, 4 * q), acc_at(i, j, 4 * q + 1),
                                                 acc_at(i, j, 4 * q + 2), acc_at(i, j, 4 * q + 3)};
                                *reinterpret_cast<f32x4*>(stage + row * (BN * 4) + ((col / 4) ^ (row % 16)) * 16) = v;
                            }
                }
                __syncthreads();
#pragma unroll
                for (int x0 = 0; x0 < PR * (BN / 8); x0 += NT) {
                    const int x = x0 + tid;
                    const int row = x / (BN / 8), c8 = x % (BN / 8);
                    const int gr = m0 + pass * PR + row, gc = n0 + c8 * 8;
                    if (gr < M && gc < N) {
                        const f32x4 lo = *reinterpret_cast<const f32x4*>(stage + row * (BN * 4) +
                                                                         ((2 * c8) ^ (row % 16)) * 16);
                        const f32x4 hi = *reinterpret_cast<const f32x4*>(stage + row * (BN * 4) +
                                                                         ((2 * c8 + 1) ^ (row % 16)) * 16);
                        const float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                        const uint16_t* c = p.C + static_cast<int64_t>(gr) * p.ldc + gc;
                        uint16_t* d = p.D + static_cast<int64_t>(gr) * p.ldd + gc;
                        if (vec8 && gc + 8 <= N) {
                            const uint4 cv = *reinterpret_cast<const uint4*>(c);
                            const uint32_t cu[4] = {cv.x, cv.y, cv.z, cv.w};
                            uint32_t du[4];
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const float w0 = v[2 * e] + widen<BF16>(static_cast<uint16_t>(cu[e] & 0xffffu));
                                const float w1 = v[2 * e + 1] + widen<BF16>(static_cast<uint16_t>(cu[e] >> 16));
                                du[e] = static_cast<uint32_t>(narrow<BF16>(w0)) |
                                        (static_cast<uint32_t>(narrow<BF16>(w1)) << 16);
                            }
                            store16_nt(d, du[0], du[1], du[2], du[3]);
                        } else {
                            for (int e = 0; e < 8 && gc + e < N; ++e) d[e] = narrow<BF16>(v[e] + widen<BF16>(c[e]));
                        }
                    }
                }
            }
            return;
        }
    }

    // Otherwise: + C in fp32, round once, masked store from registers.
    const bool has_c = p.has_c != 0;
    const bool dvec = (p.ldd % 4 == 0) && (reinterpret_cast<uintptr_t>(p.D) % 8 == 0);
    const bool cvec = !has_c || ((p.ldc % 4 == 0) && (reinterpret_cast<uintptr_t>(p.C) % 8 == 0));
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int row = m0 + wm * TM + i * MF + (lane % MF);
        if (row >= M) continue;
        const int64_t drow = static_cast<int64_t>(row) * p.ldd;
        const int64_t crow = static_cast<int64_t>(row) * p.ldc;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int q = 0; q < G; ++q) {
                const int col = n0 + wn * TN + j * MF + 8 * q + 4 * (lane / MF);
                float v[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = acc_at(i, j, 4 * q + r);
                if (dvec && cvec && col + 4 <= N) {
                    if (has_c) {
                        const uint2 cv = *reinterpret_cast<const uint2*>(p.C + crow + col);
                        v[0] += widen<BF16>(static_cast<uint16_t>(cv.x & 0xffffu));
                        v[1] += widen<BF16>(static_cast<uint16_t>(cv.x >> 16));
                        v[2] += widen<BF16>(static_cast<uint16_t>(cv.y & 0xffffu));
                        v[3] += widen<BF16>(static_cast<uint16_t>(cv.y >> 16));
                    }
                    uint2 dv;
                    dv.x = static_cast<uint32_t>(narrow<BF16>(v[0])) | (static_cast<uint32_t>(narrow<BF16>(v[1])) << 16);
                    dv.y = static_cast<uint32_t>(narrow<BF16>(v[2])) | (static_cast<uint32_t>(narrow<BF16>(v[3])) << 16);
                    *reinterpret_cast<uint2*>(p.D + drow + col) = dv;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if (col + r < N) {
                            float w = v[r];
                            if (has_c) w += widen<BF16>(p.C[crow + col + r]);
                            p.D[drow + col + r] = narrow<BF16>(w);
                        }
                    }
                }
            }
        }
    }
    }   // 16-bit epilogues
}

template <int BM, int BN, int BK, int WM, int WN, int MF, int ST, bool BF16, bool TA, bool TB>
__global__ __launch_bounds__(64 * WM * WN) void gemm_dma_kernel(KArgs p) {
    dma_tile<BM, BN, BK, WM, WN, MF, ST, BF16 ? kElBF16 : kElF16, TA, TB>(p, slice_work<BK>(p));
}

// One row of tiles (M <= BM: decode-like grids), row-major operands: the tile
// body with B streamed non-temporal.  The same arithmetic as gemm_dma_kernel.
template <int BM, int BN, int BK, int WM, int WN, int MF, int ST, bool BF16>
__global__ __launch_bounds__(64 * WM * WN) void gemm_dma_sb_kernel(KArgs p) {
    dma_tile<BM, BN, BK, WM, WN, MF, ST, BF16 ? kElBF16 : kElF16, false, false, false, true>(p, slice_work<BK>(p));
}

// Stream-K: the (tile, K step) iterations dealt out to the grid's workgroups
// as contiguous ranges (sk_piece, tile_order.h), positions after the XCD
// permutation so one die's workgroups hold neighbouring tiles; each piece of
// a range runs the tile body, and the tiles cut by range starts are summed
// by the K-slice exchange in part order.
template <int BM, int BN, int BK, int WM, int WN, int MF, int ST, bool BF16>
__global__ __launch_bounds__(64 * WM * WN) void gemm_dma_sk_kernel(KArgs p) {
    const uint32_t W = gridDim.x;
    const uint32_t nkt = static_cast<uint32_t>((p.K + BK - 1) / BK);
    const uint32_t total = static_cast<uint32_t>(p.num_pid_m * p.num_pid_n) * nkt;
    const uint32_t w = static_cast<uint32_t>(xcd_permute<int>(blockIdx.x, static_cast<int>(W), p.xcds));
    uint32_t it = sk_range_start(w, total, W);
    const uint32_t end = sk_range_start(w + 1, total, W);
    while (it < end) {
        const SkPiece q = sk_piece(it, end, total, nkt, W);
        Work wk;
        wk.tile = static_cast<int>(q.tile);
        wk.kt0 = static_cast<int>(q.kt0);
        wk.kt1 = static_cast<int>(q.kt1);
        wk.part = static_cast<int>(q.part);
        wk.nparts = static_cast<int>(q.nparts);
        wk.base = 0;
        wk.slot0 = static_cast<int>(q.slot0);
        wk.slot1 = static_cast<int>(q.slot1);
        wk.nslots = static_cast<int>(2 * W);
        // the previous piece's epilogue, exchange flag and LDS reads are done
        // before this piece's loads refill the LDS
        __syncthreads();
        dma_tile<BM, BN, BK, WM, WN, MF, ST, BF16 ? kElBF16 : kElF16, false, false, true>(p, wk);
        it = q.next;
    }
}

// int8 A (M x K, k contiguous) times int8 B stored N x K (k contiguous),
// int32 C and D: the tile body with the integer instruction.
template <int BM, int BN, int BK, int WM, int WN, int MF, int ST>
__global__ __launch_bounds__(64 * WM * WN) void gemm_i8_kernel(KArgs p) {
    dma_tile<BM, BN, BK, WM, WN, MF, ST, kElI8, false, true>(p, slice_work<BK>(p));
}

constexpr int kMaxDmaSplits = 64;

template <int BM, int BN, int BK, int WM, int WN, int MF, int ST, bool BF16, bool TA, bool TB>
hipError_t launch_dma(const KArgs& a, int64_t grid, hipStream_t stream) {
    hipLaunchKernelGGL((gemm_dma_kernel<BM, BN, BK, WM, WN, MF, ST, BF16, TA, TB>),
                       dim3(static_cast<unsigned>(grid)), dim3(64 * WM * WN), 0, stream, a);
    return hipGetLastError();
}

template <int BM, int BN, int BK, int WM, int WN, int MF, int ST, bool BF16>
hipError_t launch_dma_sb(const KArgs& a, int64_t grid, hipStream_t stream) {
    hipLaunchKernelGGL((gemm_dma_sb_kernel<BM, BN, BK, WM, WN, MF, ST, BF16>), dim3(static_cast<unsigned>(grid)),
                       dim3(64 * WM * WN), 0, stream, a);
    return hipGetLastError();
}

template <int BM, int BN, int BK, int WM, int WN, int MF, int ST, bool BF16>
hipError_t launch_dma_sk(const KArgs& a, int64_t grid, hipStream_t stream) {
    hipLaunchKernelGGL((gemm_dma_sk_kernel<BM, BN, BK, WM, WN, MF, ST, BF16>), dim3(static_cast<unsigned>(grid)),
                       dim3(64 * WM * WN), 0, stream, a);
    return hipGetLastError();
}

template <int BM, int BN, int BK, int WM, int WN, int MF, int ST>
hipError_t launch_i8(const KArgs& a, int64_t grid, hipStream_t stream) {
    hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, BK, WM, WN, MF, ST>), dim3(static_cast<unsigned>(grid)),
                       dim3(64 * WM * WN), 0, stream, a);
    return hipGetLastError();
}

#define DTG_STR2(x) #x
#define DTG_STR(x) DTG_STR2(x)
// LAY: bit 0 = A stored K x M (TA), bit 1 = B stored N x K (TB).
#define DMA_ENTRY(BM, BN, BK, WM, WN, MF, ST, BF, LAY)                                       \
    {KF_DMA, BM, BN, BK, ST, MF, WM, WN, ((BM / WM) * (BN / WN) / 64 <= 64 ? kMaxDmaSplits : 1), \
     BF, 1, 64 * WM * WN, static_cast<int64_t>(ST) * (BM + BN) * BK * 2,                    \
     &launch_dma<BM, BN, BK, WM, WN, MF, ST, (BF != 0), ((LAY) & 1) != 0, ((LAY) & 2) != 0>, \
     "gemm_dma_kernel<" DTG_STR(BM) "," DTG_STR(BN) "," DTG_STR(BK) "," DTG_STR(WM) ","     \
     DTG_STR(WN) "," DTG_STR(MF) "," DTG_STR(ST) "," DTG_STR(BF) ",lay" DTG_STR(LAY) ">", LAY}
#define DMA_BOTH(BM, BN, BK, WM, WN, MF, ST) \
    DMA_ENTRY(BM, BN, BK, WM, WN, MF, ST, 0, 0), DMA_ENTRY(BM, BN, BK, WM, WN, MF, ST, 1, 0)
#define DMA_LAYOUTS(BM, BN, BK, WM, WN, MF, ST)                                                 \
    DMA_ENTRY(BM, BN, BK, WM, WN, MF, ST, 0, 1), DMA_ENTRY(BM, BN, BK, WM, WN, MF, ST, 1, 1),     \
    DMA_ENTRY(BM, BN, BK, WM, WN, MF, ST, 0, 2), DMA_ENTRY(BM, BN, BK, WM, WN, MF, ST, 1, 2),     \
    DMA_ENTRY(BM, BN, BK, WM, WN, MF, ST, 0, 3), DMA_ENTRY(BM, BN, BK, WM, WN, MF, ST, 1, 3)

// Streamed-B variants (stream_b = 1): row-major A and B, K slices as gemm_dma_kernel.
#define DMA_SB_ENTRY(BM, BN, BK, WM, WN, MF, ST, BF)                                            \
    {KF_DMA, BM, BN, BK, ST, MF, WM, WN, ((BM / WM) * (BN / WN) / 64 <= 64 ? kMaxDmaSplits : 1),  \
     BF, 1, 64 * WM * WN, static_cast<int64_t>(ST) * (BM + BN) * BK * 2,                     \
     &launch_dma_sb<BM, BN, BK, WM, WN, MF, ST, (BF != 0)>,                                   \
     "gemm_dma_sb_kernel<" DTG_STR(BM) "," DTG_STR(BN) "," DTG_STR(BK) "," DTG_STR(WM) ","     \
     DTG_STR(WN) "," DTG_STR(MF) "," DTG_STR(ST) "," DTG_STR(BF) ">", 0, 1}
#define DMA_SB_BOTH(BM, BN, BK, WM, WN, MF, ST) \
    DMA_SB_ENTRY(BM, BN, BK, WM, WN, MF, ST, 0), DMA_SB_ENTRY(BM, BN, BK, WM, WN, MF, ST, 1)

// Stream-K variants: row-major A and B; the grid is the plan's workgroup count.
#define DMA_SK_ENTRY(BM, BN, BK, WM, WN, MF, ST, BF)                                           \
    {KF_DMA_SK, BM, BN, BK, ST, MF, WM, WN, 0, BF, 1, 64 * WM * WN,                            \
     static_cast<int64_t>(ST) * (BM + BN) * BK * 2, &launch_dma_sk<BM, BN, BK, WM, WN, MF, ST, (BF != 0)>, \
     "gemm_dma_sk_kernel<" DTG_STR(BM) "," DTG_STR(BN) "," DTG_STR(BK) "," DTG_STR(WM) ","      \
     DTG_STR(WN) "," DTG_STR(MF) "," DTG_STR(ST) "," DTG_STR(BF) ">", 0}
#define DMA_SK_BOTH(BM, BN, BK, WM, WN, MF, ST) \
    DMA_SK_ENTRY(BM, BN, BK, WM, WN, MF, ST, 0), DMA_SK_ENTRY(BM, BN, BK, WM, WN, MF, ST, 1)

// int8 variants: dtype 2, B stored N x K; BK in 16-bit units (2 k each); no K slices.
#define I8_ENTRY(BM, BN, BK, WM, WN, MF, ST)                                                     \
    {KF_DMA, BM, BN, BK, ST, MF, WM, WN, 1, 2, 1, 64 * WM * WN,                                  \
     static_cast<int64_t>(ST) * (BM + BN) * BK * 2, &launch_i8<BM, BN, BK, WM, WN, MF, ST>,       \
     "gemm_i8_kernel<" DTG_STR(BM) "," DTG_STR(BN) "," DTG_STR(BK) "," DTG_STR(WM) "," DTG_STR(WN) \
     "," DTG_STR(MF) "," DTG_STR(ST) ">", kLayTB}

}  // namespace
}  // namespace dtg
