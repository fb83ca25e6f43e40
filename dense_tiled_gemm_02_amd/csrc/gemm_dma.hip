// Tiled GEMM kernel for gfx950 with direct global -> LDS staging:  D = A x B (+ C).
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
//  * A is stored as rows of BK contiguous k and read with one 16-byte LDS read
//    per lane per fragment; B is stored as it is in memory (rows of BN
//    contiguous n) and read with the transposing 64-bit LDS read, which hands
//    each lane 4 consecutive k of one column: two reads make the 8 k of one
//    MFMA operand.
// Descriptors are rebased at every K step (scalar work only), so 32-bit
// buffer offsets cover any matrix whose BM rows of A and BK rows of B span
// less than 2 GiB.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "tile_order.h"

namespace dtg {
namespace {

using namespace dev;

// Swizzle of the B tile (rows of BN contiguous n, CHB 16-byte chunks per row):
// physical chunk = logical chunk ^ bsw(r).  Even values keep the two chunks a
// 16-lane group reads from one row adjacent; the 4 (or 8) rows one transposing
// read touches land in distinct bank groups.
template <int CHB>
__device__ __forceinline__ int bsw(int r) {
    if constexpr (CHB >= 16) return 2 * ((r & 3) | (((r >> 3) & 1) << 2));
    else return 2 * (r & 3);
}

// wait until at most N vector-memory operations of this wave are outstanding
template <int BM, int BN, int BK, int WM, int WN, int MF, int ST, bool BF16>
__global__ __launch_bounds__(64 * WM * WN) void gemm_dma_kernel(KArgs p) {
    constexpr int NW = WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / MF, FN = TN / MF;
    constexpr int KI = (MF == 16) ? 32 : 16;
    constexpr int CHA = BK / 8;                 // 16-byte chunks per A row
    constexpr int RA = 64 / CHA;                // A rows per wave instruction
    constexpr int IA_W = BM / RA / NW;          // A instructions per wave per stage
    constexpr int CHB = BN / 8;                 // 16-byte chunks per B row
    constexpr int RB = 64 / CHB;                // B rows per wave instruction
    constexpr int IB_W = BK / RB / NW;
    constexpr int SA = BM * BK, SB = BK * BN;   // elements per stage
    constexpr int L = IA_W + IB_W;              // loads per wave per stage
    constexpr int NKS = BK / KI;                // instruction k sub-steps per K step
    static_assert(BM % (WM * MF) == 0 && BN % (WN * MF) == 0, "tile vs wave grid");
    static_assert(BK % KI == 0 && (CHA == 4 || CHA == 8 || CHA == 16), "BK");
    static_assert(CHB >= 8 && CHB <= 64 && 64 % CHB == 0, "BN");
    static_assert((BM / RA) % NW == 0 && (BK / RB) % NW == 0 && IA_W > 0 && IB_W > 0, "load split");
    static_assert(ST >= 2 && ST <= 5 && (ST - 1) * L < 64, "stages");
    typedef typename AccT<MF>::type acc_t;

    __shared__ __attribute__((aligned(1024))) uint16_t smem[ST * (SA + SB)];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    int pid_m, pid_n;
    tile_of_workgroup<int>(blockIdx.x, p.num_pid_m, p.num_pid_n, p.group_m, p.xcds, &pid_m, &pid_n);
    const int m0 = pid_m * BM, n0 = pid_n * BN;
    const int M = p.M, N = p.N, K = p.K;
    const bool edge = (m0 + BM > M) || (n0 + BN > N);

    // ---- per-lane load offsets (bytes, relative to the rebased descriptors)
    uint32_t a_voff[IA_W];
    int a_kc[IA_W];
    bool a_ok[IA_W];
#pragma unroll
    for (int i = 0; i < IA_W; ++i) {
        const int inst = i * NW + wave;
        const int row = inst * RA + lane / CHA;
        const int c = (lane % CHA) ^ swz<CHA>(row);
        a_ok[i] = m0 + row < M;
        a_voff[i] = static_cast<uint32_t>(static_cast<int64_t>(row) * p.lda * 2 + c * 16);
        a_kc[i] = 8 * c;
    }
    uint32_t b_voff[IB_W];
    int b_kr[IB_W];
    bool b_ok[IB_W];
#pragma unroll
    for (int i = 0; i < IB_W; ++i) {
        const int inst = i * NW + wave;
        const int row = inst * RB + lane / CHB;
        const int c = (lane % CHB) ^ bsw<CHB>(row);
        b_ok[i] = n0 + 8 * c < N;
        b_voff[i] = static_cast<uint32_t>(static_cast<int64_t>(row) * p.ldb * 2 + c * 16);
        b_kr[i] = row;
    }

    auto issue = [&](auto check_tag, int kt, int s) {
        constexpr bool CHECK = decltype(check_tag)::value;
        const int k0 = kt * BK;
        const uint16_t* abase = p.A + static_cast<int64_t>(m0) * p.lda + k0;
        const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(abase), 0,
            clamp_records((static_cast<int64_t>(M - 1 - m0) * p.lda + (K - k0)) * 2), kRsrcWord3);
        const uint16_t* bbase = p.B + static_cast<int64_t>(k0) * p.ldb + n0;
        const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(bbase), 0,
            clamp_records((static_cast<int64_t>(K - 1 - k0) * p.ldb + (N - n0)) * 2), kRsrcWord3);
        uint16_t* sa = smem + s * (SA + SB);
        uint16_t* sb = sa + SA;
#pragma unroll
        for (int i = 0; i < IA_W; ++i) {
            uint32_t v = a_voff[i];
            if constexpr (CHECK) v = (a_ok[i] && k0 + a_kc[i] < K) ? v : kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t*)(sa + (i * NW + wave) * 512), 16, v, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < IB_W; ++i) {
            uint32_t v = b_voff[i];
            if constexpr (CHECK) v = (b_ok[i] && k0 + b_kr[i] < K) ? v : kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_t*)(sb + (i * NW + wave) * 512), 16, v, 0, 0, 0);
        }
    };

    acc_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < AccT<MF>::regs; ++r) acc[i][j][r] = 0.0f;

    // ---- per-lane operand read addresses (LDS bytes), for both stages
    //  A fragment (i, ks): row wm*TM + i*MF + lane % MF, chunk ks*KI/8 + lane / MF
    //  (XOR-swizzled); the i*MF*BK*2 part is an immediate offset.
    //  B fragment (j, ks), half hh: the transposing read of k rows
    //  ks*KI + 8 g + 4 hh + (jq >> 2) and 4 columns starting at
    //  nb + 4 (jq & 3); the (ks*KI + 4 hh) * BN * 2 part is an immediate offset.
    const uint32_t smem0 = lds_addr(smem);
    uint32_t a_addr[ST][NKS], b_addr[ST][FN];
    {
        const int a_row = wm * TM + lane % MF;
        const int a_kc0 = lane / MF;
        const int a_sw = swz<CHA>(lane % MF);
        int jq, g, col;
        if constexpr (MF == 16) { jq = lane & 15; g = lane >> 4; col = 0; }
        else { jq = lane & 15; g = lane >> 5; col = 16 * ((lane >> 4) & 1); }
        const int b_sw = (CHB >= 16) ? 2 * ((jq >> 2) | ((g & 1) << 2)) : 2 * (jq >> 2);
        const int b_row = 8 * g + (jq >> 2);
#pragma unroll
        for (int st = 0; st < ST; ++st) {
            const uint32_t sa = smem0 + st * (SA + SB) * 2;
            const uint32_t sb = sa + SA * 2;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                a_addr[st][ks] = sa + (a_row * BK + (((ks * (KI / 8) + a_kc0) ^ a_sw) * 8)) * 2;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int nb = wn * TN + j * MF + col;
                b_addr[st][j] = sb + (b_row * BN + (((nb >> 3) ^ b_sw) << 3) + 4 * (jq & 3)) * 2;
            }
        }
    }

    u32x4 fa[2][FM], fb[2][FN];       // fragments, double-buffered across k sub-steps

    auto read_frags = [&](auto stage_tag, auto ks_tag, auto slot_tag) {
        constexpr int S = decltype(stage_tag)::value;
        constexpr int KS = decltype(ks_tag)::value;
        constexpr int SL = decltype(slot_tag)::value;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            i16x4 h0 = lds_read_tr<(KS * KI + 0) * BN * 2>(b_addr[S][j]);
            i16x4 h1 = lds_read_tr<(KS * KI + 4) * BN * 2>(b_addr[S][j]);
            fb[SL][j] = __builtin_bit_cast(u32x4, __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
        }
        static_for<FM>([&](auto i_tag) {
            constexpr int I = decltype(i_tag)::value;
            fa[SL][I] = lds_read16<I * MF * BK * 2>(a_addr[S][KS]);
        });
    };
    auto wait_frags = [&](auto slot_tag) {
        constexpr int SL = decltype(slot_tag)::value;
        lds_wait_all();
#pragma unroll
        for (int j = 0; j < FN; ++j) tie(fb[SL][j]);
#pragma unroll
        for (int i = 0; i < FM; ++i) tie(fa[SL][i]);
    };
    auto mfmas = [&](auto slot_tag) {
        constexpr int SL = decltype(slot_tag)::value;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = mfma<MF, BF16>(fa[SL][i], fb[SL][j], acc[i][j]);
    };

    const int nkt = (K + BK - 1) / BK;
    const int nfull = K / BK;
    auto issue_tile = [&](int kt, int st) {
        if (!edge && kt < nfull) issue(Unchecked{}, kt, st);
        else issue(Checked{}, kt, st);
    };

    // Wait until tile `need` has landed: at most the tiles issued after it
    // (up to `last_issued`) may still be in flight, L loads each.
    auto wait_tile = [&](int need, int last_issued) {
        const int after = last_issued - need;
        static_for<ST>([&](auto i_tag) {
            constexpr int I = decltype(i_tag)::value;
            if (after == I) wait_vm<I * L>();
        });
    };

    // One K step (tile kt) on LDS stage S = kt % ST; U is kt's position in the
    // unrolled loop, which fixes which fragment slot holds which sub-step.  On
    // entry the fragments of sub-step 0 are in slot (U * NKS) % 2.  Sub-step ks
    // issues the reads of sub-step ks + 1 (or, at the last sub-step, waits for
    // tile kt + 1, passes the barrier, refills this stage with tile kt + ST and
    // reads tile kt + 1's first fragments), then runs its MFMAs, then waits for
    // those reads.  Tile kt + ST goes into the stage of tile kt: every wave has
    // read all of tile kt's fragments before the barrier.
    auto step = [&](auto u_tag, int kt) {
        constexpr int U = decltype(u_tag)::value;
        constexpr int S = U % ST;
        static_for<NKS>([&](auto ks_tag) {
            constexpr int KS = decltype(ks_tag)::value;
            constexpr int CUR = (U * NKS + KS) & 1, NXT = CUR ^ 1;
            bool pending = true;
            if constexpr (KS + 1 < NKS) {
                read_frags(std::integral_constant<int, S>{}, std::integral_constant<int, KS + 1>{},
                           std::integral_constant<int, NXT>{});
            } else {
                pending = kt + 1 < nkt;
                if (pending) {
                    const int last_issued = (kt + ST - 1 < nkt - 1) ? kt + ST - 1 : nkt - 1;
                    wait_tile(kt + 1, last_issued);
                    __builtin_amdgcn_s_barrier();
                    if (kt + ST < nkt) issue_tile(kt + ST, S);
                    read_frags(std::integral_constant<int, (S + 1) % ST>{}, std::integral_constant<int, 0>{},
                               std::integral_constant<int, NXT>{});
                }
            }
            mfmas(std::integral_constant<int, CUR>{});
            // keep every MFMA of this sub-step ahead of the wait
            __builtin_amdgcn_sched_barrier(0);
            if (pending) wait_frags(std::integral_constant<int, NXT>{});
        });
    };

    // unroll so that both the stage and the fragment-slot parity repeat
    constexpr int UNROLL = ((ST * NKS) % 2 == 0) ? ST : 2 * ST;
    if (nkt > 0) {
        const int first = (ST < nkt) ? ST : nkt;
        for (int t = 0; t < first; ++t) issue_tile(t, t);
        wait_tile(0, first - 1);
        __builtin_amdgcn_s_barrier();
        read_frags(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{},
                   std::integral_constant<int, 0>{});
        wait_frags(std::integral_constant<int, 0>{});
        for (int kt = 0; kt < nkt; kt += UNROLL) {
            static_for<UNROLL>([&](auto u_tag) {
                constexpr int UU = decltype(u_tag)::value;
                if (kt + UU < nkt) step(u_tag, kt + UU);
            });
        }
    }

    // ---- epilogue: + C in fp32, round, masked store
    const bool has_c = p.has_c != 0;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = n0 + wn * TN + j * MF + (lane % MF);
#pragma unroll
            for (int r = 0; r < AccT<MF>::regs; ++r) {
                int row;
                if constexpr (MF == 16) row = m0 + wm * TM + i * 16 + 4 * (lane / 16) + r;
                else row = m0 + wm * TM + i * 32 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
                if (row < M && col < N) {
                    float v = acc[i][j][r];
                    if (has_c) v += widen<BF16>(p.C[static_cast<int64_t>(row) * p.ldc + col]);
                    p.D[static_cast<int64_t>(row) * p.ldd + col] = narrow<BF16>(v);
                }
            }
        }
    }
}

template <int BM, int BN, int BK, int WM, int WN, int MF, int ST, bool BF16>
hipError_t launch_dma(const KArgs& a, int64_t grid, hipStream_t stream) {
    hipLaunchKernelGGL((gemm_dma_kernel<BM, BN, BK, WM, WN, MF, ST, BF16>),
                       dim3(static_cast<unsigned>(grid)), dim3(64 * WM * WN), 0, stream, a);
    return hipGetLastError();
}

#define DTG_STR2(x) #x
#define DTG_STR(x) DTG_STR2(x)
#define DMA_ENTRY(BM, BN, BK, WM, WN, MF, ST, BF)                                            \
    {KF_DMA, BM, BN, BK, ST, MF, WM, WN, 1, BF, 1, 64 * WM * WN,                            \
     static_cast<int64_t>(ST) * (BM + BN) * BK * 2,                                         \
     &launch_dma<BM, BN, BK, WM, WN, MF, ST, (BF != 0)>,                                    \
     "gemm_dma_kernel<" DTG_STR(BM) "," DTG_STR(BN) "," DTG_STR(BK) "," DTG_STR(WM) ","     \
     DTG_STR(WN) "," DTG_STR(MF) "," DTG_STR(ST) "," DTG_STR(BF) ">"}
#define DMA_BOTH(BM, BN, BK, WM, WN, MF, ST) \
    DMA_ENTRY(BM, BN, BK, WM, WN, MF, ST, 0), DMA_ENTRY(BM, BN, BK, WM, WN, MF, ST, 1)

const KernelEntry kDmaTable[] = {
    DMA_BOTH(256, 256, 64, 2, 4, 16, 2),
    DMA_BOTH(256, 256, 32, 2, 4, 16, 4),
    DMA_BOTH(256, 256, 64, 2, 4, 32, 2),
    DMA_BOTH(256, 256, 32, 2, 4, 32, 4),
    DMA_BOTH(256, 128, 64, 2, 2, 16, 3),
    DMA_BOTH(256, 128, 64, 2, 2, 16, 2),
    DMA_BOTH(128, 256, 64, 2, 2, 16, 2),
    DMA_BOTH(128, 128, 64, 2, 2, 16, 2),
    DMA_BOTH(128, 128, 64, 2, 2, 16, 4),
    DMA_BOTH(128, 128, 64, 2, 2, 32, 2),
};

}  // namespace

const KernelEntry* dma_kernel_table(int* count) {
    *count = static_cast<int>(sizeof(kDmaTable) / sizeof(kDmaTable[0]));
    return kDmaTable;
}

}  // namespace dtg
