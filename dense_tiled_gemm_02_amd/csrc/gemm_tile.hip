// Tiled GEMM kernel for gfx950 (CDNA4, wave64, MFMA):  D = A x B (+ C).
//
// One workgroup computes one BM x BN output tile with a K loop over BK-deep
// slabs ("Hopper Support in Triton", slide 6: fp32 accumulator, K loop of tile
// products, pointer advance by BLOCK_K).  Per K step:
//   1. global -> registers: A slab (BM x BK, K contiguous) and B slab (BK x BN,
//      N contiguous) in 16-byte vectors; edge tiles and the K tail zero-fill
//      rows >= M, columns >= N and k >= K (slides 15-16: masks with other = 0);
//   2. registers -> LDS: A as-is; B transposed in registers, 8 x 8 elements at a
//      time, so that both LDS tiles hold rows of BK contiguous k ("DCU K100
//      节点初探", section 5.8: lay the operands out so the shared-memory
//      loads are coalesced).  Rows are cut into 16-byte chunks whose position
//      is XOR-swizzled by the row index, so the MFMA operand reads and the
//      staging writes hit distinct LDS banks;
//   3. LDS -> VGPR operand reads (one 16-byte read per lane per fragment) and a
//      chain of v_mfma_f32_16x16x32 or v_mfma_f32_32x32x16 into fp32
//      accumulators that stay in registers for the whole K loop (section 5.5:
//      clear the accumulator once; section 5.8: one accumulator per 16 x 16
//      block for instruction-level parallelism).
// With two LDS stages the global loads of step k+1 are in flight while step k
// is contracted, and one barrier per step suffices (section 5.6 double buffer;
// FlagGems "Hygon optimization", section "Software pipelining").
// The epilogue adds C in fp32 once, rounds to the storage type (nearest even)
// and stores only rows < M and columns < N.
//
// Output tiles are visited in the grouped order of tile_order.h.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernels.h"
#include "tile_order.h"

namespace dtg {
namespace {

using namespace dev;

__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) {
    return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) {
    return (a >> 16) | (b & 0xffff0000u);
}

template <int BM, int BN, int BK, int WM, int WN, int MF, int ST, bool BF16, bool VEC>
__global__ __launch_bounds__(64 * WM * WN) void gemm_tile_kernel(KArgs p) {
    constexpr int NT = 64 * WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;       // wave tile
    constexpr int FM = TM / MF, FN = TN / MF;       // instruction tiles per wave
    constexpr int KI = (MF == 16) ? 32 : 16;        // k per instruction
    constexpr int CH = BK / 8;                      // 16-byte chunks per LDS row
    constexpr int A_CHUNKS = BM * CH;
    constexpr int A_PT = (A_CHUNKS + NT - 1) / NT;
    constexpr int B_BLOCKS = CH * (BN / 8);         // 8 x 8 element blocks of B
    constexpr int B_PT = (B_BLOCKS + NT - 1) / NT;
    constexpr int SA = BM * BK, SB = BN * BK;       // elements per stage
    static_assert(BM % (WM * MF) == 0 && BN % (WN * MF) == 0, "tile vs wave grid");
    static_assert(BK % KI == 0 && (CH == 4 || CH == 8 || CH == 16), "BK");
    static_assert(ST == 1 || ST == 2, "stages");
    typedef typename AccT<MF>::type acc_t;

    __shared__ __attribute__((aligned(16))) uint16_t sA[ST * SA];
    __shared__ __attribute__((aligned(16))) uint16_t sB[ST * SB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    int pid_m, pid_n;
    tile_of_workgroup<int>(blockIdx.x, p.num_pid_m, p.num_pid_n, p.group_m, p.xcds, &pid_m, &pid_n);
    const int m0 = pid_m * BM, n0 = pid_n * BN;
    const int M = p.M, N = p.N, K = p.K;
    const bool edge = (m0 + BM > M) || (n0 + BN > N);

    // ---- staging assignment (fixed over the K loop)
    // A: chunk q = tid + i*NT is row q / CH, chunk q % CH (8 lanes per 128-byte row).
    int64_t a_off[A_PT];
    int a_lds[A_PT], a_kc[A_PT];
    bool a_ok[A_PT];
#pragma unroll
    for (int i = 0; i < A_PT; ++i) {
        const int q = tid + i * NT;
        const int row = q / CH, c = q % CH;
        const bool inq = (A_CHUNKS % NT == 0) || (q < A_CHUNKS);
        a_ok[i] = inq && (m0 + row < M);
        a_off[i] = static_cast<int64_t>(a_ok[i] ? m0 + row : 0) * p.lda + 8 * c * (VEC ? 1 : p.sak);
        a_kc[i] = 8 * c;
        a_lds[i] = row * BK + ((c ^ swz<CH>(row)) * 8);
    }
    // B: block b = tid + i*NT covers k rows 8*(b % CH) + 0..7 and columns
    // n0 + 8*(b / CH) + 0..7.  Consecutive lanes take consecutive k chunks, so
    // the 8 transposed LDS rows each lane writes land on distinct banks.
    int64_t b_off[B_PT];
    int b_lds[B_PT], b_kc[B_PT], b_col[B_PT];
    bool b_in[B_PT];
#pragma unroll
    for (int i = 0; i < B_PT; ++i) {
        const int b = tid + i * NT;
        const int kc = b % CH, nb = b / CH;
        b_in[i] = (B_BLOCKS % NT == 0) || (b < B_BLOCKS);
        b_col[i] = n0 + 8 * nb;
        b_kc[i] = 8 * kc;
        b_off[i] = static_cast<int64_t>(8 * kc) * p.ldb + static_cast<int64_t>(b_in[i] ? b_col[i] : 0) * (VEC ? 1 : p.sbn);
        b_lds[i] = (8 * nb) * BK + kc * 8;   // row 8*nb (+ c added per row), chunk kc
    }

    u32x4 ra[A_PT];
    u32x4 rb[B_PT][8];

    auto gload = [&](int kt, bool check) {
        const int k0 = kt * BK;
        const uint16_t* Ak = p.A + static_cast<int64_t>(k0) * (VEC ? 1 : p.sak);
        const uint16_t* Bk = p.B + static_cast<int64_t>(k0) * p.ldb;
#pragma unroll
        for (int i = 0; i < A_PT; ++i) {
            if constexpr (VEC) {
                if (!check) {
                    if ((A_CHUNKS % NT == 0) || (tid + i * NT < A_CHUNKS))
                        ra[i] = *reinterpret_cast<const u32x4*>(Ak + a_off[i]);
                } else {
                    const bool ok = a_ok[i] && (k0 + a_kc[i] < K);
                    ra[i] = ok ? *reinterpret_cast<const u32x4*>(Ak + a_off[i]) : u32x4{0, 0, 0, 0};
                }
            } else {
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const int k = k0 + a_kc[i] + e;
                    const uint32_t x0 = (a_ok[i] && k < K) ? Ak[a_off[i] + e * p.sak] : 0u;
                    const uint32_t x1 = (a_ok[i] && k + 1 < K) ? Ak[a_off[i] + (e + 1) * p.sak] : 0u;
                    w[e / 2] = x0 | (x1 << 16);
                }
                ra[i] = u32x4{w[0], w[1], w[2], w[3]};
            }
        }
#pragma unroll
        for (int i = 0; i < B_PT; ++i) {
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const uint16_t* src = Bk + b_off[i] + static_cast<int64_t>(r) * p.ldb;
                if constexpr (VEC) {
                    if (!check) {
                        if (b_in[i]) rb[i][r] = *reinterpret_cast<const u32x4*>(src);
                    } else {
                        const bool ok = b_in[i] && (b_col[i] < N) && (k0 + b_kc[i] + r < K);
                        rb[i][r] = ok ? *reinterpret_cast<const u32x4*>(src) : u32x4{0, 0, 0, 0};
                    }
                } else {
                    const bool krow = b_in[i] && (k0 + b_kc[i] + r < K);
                    uint32_t w[4];
#pragma unroll
                    for (int e = 0; e < 8; e += 2) {
                        const uint32_t x0 = (krow && b_col[i] + e < N) ? src[e * p.sbn] : 0u;
                        const uint32_t x1 = (krow && b_col[i] + e + 1 < N) ? src[(e + 1) * p.sbn] : 0u;
                        w[e / 2] = x0 | (x1 << 16);
                    }
                    rb[i][r] = u32x4{w[0], w[1], w[2], w[3]};
                }
            }
        }
    };

    auto lds_store = [&](int s) {
        uint16_t* As = sA + s * SA;
        uint16_t* Bs = sB + s * SB;
#pragma unroll
        for (int i = 0; i < A_PT; ++i)
            if ((A_CHUNKS % NT == 0) || (tid + i * NT < A_CHUNKS))
                *reinterpret_cast<u32x4*>(As + a_lds[i]) = ra[i];
#pragma unroll
        for (int i = 0; i < B_PT; ++i) {
            if (!b_in[i]) continue;
            // rb[i][r] holds k row r, columns c = 0..7 (two per dword).  Column c
            // of the block becomes LDS row 8*nb + c holding k = 0..7.
            const int kc = b_kc[i] / 8;
            const int row0 = b_lds[i] / BK;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const int d = c >> 1;
                u32x4 v;
                if (c & 1) {
                    v = u32x4{hi_pair(rb[i][0][d], rb[i][1][d]), hi_pair(rb[i][2][d], rb[i][3][d]),
                              hi_pair(rb[i][4][d], rb[i][5][d]), hi_pair(rb[i][6][d], rb[i][7][d])};
                } else {
                    v = u32x4{lo_pair(rb[i][0][d], rb[i][1][d]), lo_pair(rb[i][2][d], rb[i][3][d]),
                              lo_pair(rb[i][4][d], rb[i][5][d]), lo_pair(rb[i][6][d], rb[i][7][d])};
                }
                const int row = row0 + c;
                *reinterpret_cast<u32x4*>(Bs + row * BK + ((kc ^ swz<CH>(row)) * 8)) = v;
            }
        }
    };

    acc_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < AccT<MF>::regs; ++r) acc[i][j][r] = 0.0f;

    // operand read offsets (elements, within a stage); the swizzle is a
    // per-lane constant because fragment rows start at multiples of 16
    const int frag_row = lane % MF;
    const int frag_kc = lane / MF;                  // chunk within one instruction's k
    const int fsw = swz<CH>(frag_row);

    auto compute = [&](int s) {
        const uint16_t* As = sA + s * SA;
        const uint16_t* Bs = sB + s * SB;
#pragma unroll
        for (int ks = 0; ks < BK / KI; ++ks) {
            const int c = ks * (KI / 8) + frag_kc;
            const int coff = ((c ^ fsw) * 8);
            u32x4 af[FM], bfr[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = *reinterpret_cast<const u32x4*>(As + (wm * TM + i * MF + frag_row) * BK + coff);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bfr[j] = *reinterpret_cast<const u32x4*>(Bs + (wn * TN + j * MF + frag_row) * BK + coff);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma<MF, BF16>(af[i], bfr[j], acc[i][j]);
        }
    };

    const int nkt = (K + BK - 1) / BK;
    const int nfull = K / BK;
    if (nkt > 0) gload(0, edge || nfull < 1 || !VEC);
    for (int kt = 0; kt < nkt; ++kt) {
        const int s = (ST == 1) ? 0 : (kt & 1);
        if (ST == 1 && kt > 0) __syncthreads();
        lds_store(s);
        if (kt + 1 < nkt) gload(kt + 1, edge || kt + 1 >= nfull || !VEC);
        __syncthreads();
        compute(s);
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

template <int BM, int BN, int BK, int WM, int WN, int MF, int ST, bool BF16, bool VEC>
hipError_t launch_tile(const KArgs& a, int64_t grid, hipStream_t stream) {
    hipLaunchKernelGGL((gemm_tile_kernel<BM, BN, BK, WM, WN, MF, ST, BF16, VEC>),
                       dim3(static_cast<unsigned>(grid)), dim3(64 * WM * WN), 0, stream, a);
    return hipGetLastError();
}

#define DTG_STR2(x) #x
#define DTG_STR(x) DTG_STR2(x)
#define TILE_ENTRY(BM, BN, BK, WM, WN, MF, ST, BF, VEC)                                      \
    {KF_TILE, BM, BN, BK, ST, MF, WM, WN, 1, BF, VEC, 64 * WM * WN,                           \
     static_cast<int64_t>(ST) * (BM + BN) * BK * 2,                                          \
     &launch_tile<BM, BN, BK, WM, WN, MF, ST, (BF != 0), (VEC != 0)>,                        \
     "gemm_tile_kernel<" DTG_STR(BM) "," DTG_STR(BN) "," DTG_STR(BK) "," DTG_STR(WM) ","     \
     DTG_STR(WN) "," DTG_STR(MF) "," DTG_STR(ST) "," DTG_STR(BF) "," DTG_STR(VEC) ">", (VEC) ? 0 : -1}

#define TILE_BOTH(BM, BN, BK, WM, WN, MF, ST, VEC) \
    TILE_ENTRY(BM, BN, BK, WM, WN, MF, ST, 0, VEC), TILE_ENTRY(BM, BN, BK, WM, WN, MF, ST, 1, VEC)

const KernelEntry kTileTable[] = {
    TILE_BOTH(256, 256, 64, 2, 4, 32, 2, 1),
    TILE_BOTH(256, 128, 64, 2, 2, 16, 2, 1),
    TILE_BOTH(256, 128, 64, 2, 2, 32, 2, 1),
    TILE_BOTH(128, 256, 64, 2, 2, 16, 2, 1),
    TILE_BOTH(128, 128, 64, 2, 2, 16, 2, 1),
    TILE_BOTH(128, 128, 64, 2, 2, 32, 2, 1),
    TILE_BOTH(128, 128, 64, 2, 2, 16, 1, 1),
    TILE_BOTH(128, 128, 32, 2, 2, 16, 2, 1),
    TILE_BOTH(64, 64, 64, 2, 2, 16, 2, 1),
    TILE_BOTH(64, 64, 32, 2, 2, 16, 2, 1),
    TILE_BOTH(64, 64, 32, 2, 2, 16, 1, 1),
    TILE_BOTH(32, 32, 32, 2, 2, 16, 2, 1),
    TILE_BOTH(16, 64, 64, 1, 4, 16, 2, 1),
    TILE_BOTH(64, 64, 32, 2, 2, 16, 2, 0),
};

}  // namespace

const KernelEntry* tile_kernel_table(int* count) {
    *count = static_cast<int>(sizeof(kTileTable) / sizeof(kTileTable[0]));
    return kTileTable;
}

}  // namespace dtg
