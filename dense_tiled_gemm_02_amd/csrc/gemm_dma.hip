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

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

typedef std::integral_constant<bool, true> T;    // checked loads (edges, K tail)
typedef std::integral_constant<bool, false> F;   // interior loads

constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw buffer of dwords
constexpr uint32_t kOOB = 0x80000000u;         // offset past any descriptor range
constexpr int64_t kMaxRecords = 0x7ffffff0;

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
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Transposing 64-bit LDS read (ds_read_b64_tr_b16) at LDS byte address
// `addr`: within each 16-lane group the 16 addressed 8-byte pieces, in lane
// order, form a 4 x 16 matrix of halfwords (lanes 4i..4i+3 give row i); lane t
// receives column t.  Issued as inline asm so the compiler does not guard it
// with a wait for every outstanding global -> LDS load; the caller waits with
// lds_wait() before using the result.
__device__ __forceinline__ i16x4 lds_read_tr(uint32_t addr) {
    i16x4 v;
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(addr));
    return v;
}

// Wait for every LDS read of this wave, and make the values in `regs` depend
// on that wait so no use of them is scheduled before it.
template <int NR>
__device__ __forceinline__ void lds_wait(u32x4 (&regs)[NR]) {
    static_assert(NR >= 1 && NR <= 8, "lds_wait");
    if constexpr (NR == 1) asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(regs[0]));
    else if constexpr (NR == 2) asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(regs[0]), "+v"(regs[1]));
    else if constexpr (NR == 4)
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(regs[0]), "+v"(regs[1]), "+v"(regs[2]), "+v"(regs[3]));
    else if constexpr (NR == 8)
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(regs[0]), "+v"(regs[1]), "+v"(regs[2]), "+v"(regs[3]), "+v"(regs[4]),
                       "+v"(regs[5]), "+v"(regs[6]), "+v"(regs[7]));
    else static_assert(NR == 1 || NR == 2 || NR == 4 || NR == 8, "lds_wait");
}

__device__ __forceinline__ uint32_t lds_addr(const uint16_t* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint16_t*)p));
}

__device__ __forceinline__ uint32_t clamp_records(int64_t bytes) {
    return static_cast<uint32_t>(bytes < kMaxRecords ? bytes : kMaxRecords);
}

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
    static_assert(BM % (WM * MF) == 0 && BN % (WN * MF) == 0, "tile vs wave grid");
    static_assert(BK % KI == 0 && (CHA == 4 || CHA == 8 || CHA == 16), "BK");
    static_assert(CHB >= 8 && CHB <= 64 && 64 % CHB == 0, "BN");
    static_assert((BM / RA) % NW == 0 && (BK / RB) % NW == 0 && IA_W > 0 && IB_W > 0, "load split");
    static_assert(ST >= 2 && (ST - 2) * L < 64, "stages");
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

    // per-lane operand read geometry
    const int a_row = lane % MF;
    const int a_kc0 = lane / MF;
    const int a_sw = swz<CHA>(a_row);
    int b_jq, b_g, b_col;                       // see the two cases below
    if constexpr (MF == 16) {
        b_jq = lane & 15;                       // column within the fragment
        b_g = lane >> 4;                        // k group: k = 8 g + 0..7
        b_col = 0;
    } else {
        b_jq = lane & 15;                       // column within a 16-column half
        b_g = lane >> 5;                        // k group: k = 8 g + 0..7
        b_col = 16 * ((lane >> 4) & 1);         // which 16-column half
    }
    const int b_sw = (CHB >= 16) ? 2 * ((b_jq >> 2) | ((b_g & 1) << 2)) : 2 * (b_jq >> 2);

    auto compute = [&](int s) {
        const uint16_t* As = smem + s * (SA + SB);
        const uint16_t* Bs = As + SA;
#pragma unroll
        for (int ks = 0; ks < BK / KI; ++ks) {
            u32x4 af[FM], bv[FN];
            const int coff = (((ks * (KI / 8) + a_kc0) ^ a_sw) * 8);
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = *reinterpret_cast<const u32x4*>(As + (wm * TM + i * MF + a_row) * BK + coff);
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int nb = wn * TN + j * MF + b_col;
                i16x4 h[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int r = ks * KI + 8 * b_g + 4 * hh + (b_jq >> 2);
                    const uint16_t* src = Bs + r * BN + (((nb >> 3) ^ b_sw) << 3) + 4 * (b_jq & 3);
                    h[hh] = lds_read_tr(lds_addr(src));
                }
                bv[j] = __builtin_bit_cast(u32x4, __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7));
            }
            lds_wait(bv);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma<MF, BF16>(af[i], bv[j], acc[i][j]);
        }
    };

    const int nkt = (K + BK - 1) / BK;
    const int nfull = K / BK;
#pragma unroll
    for (int s = 0; s < ST - 1; ++s) {
        if (s < nkt) {
            if (!edge && s < nfull) issue(F{}, s, s);
            else issue(T{}, s, s);
        }
    }
    for (int kt = 0; kt < nkt; ++kt) {
        // tile kt is complete once at most min(ST - 2, tiles issued after it)
        // stages of loads are still in flight
        const int after = (nkt - 1 - kt < ST - 2) ? (nkt - 1 - kt) : (ST - 2);
        if constexpr (ST == 2) {
            wait_vm<0>();
        } else if constexpr (ST == 3) {
            if (after >= 1) wait_vm<L>(); else wait_vm<0>();
        } else {
            static_assert(ST <= 4, "stages");
            if (after >= 2) wait_vm<2 * L>(); else if (after == 1) wait_vm<L>(); else wait_vm<0>();
        }
        __builtin_amdgcn_s_barrier();
        const int nt = kt + ST - 1;
        if (nt < nkt) {
            if (!edge && nt < nfull) issue(F{}, nt, nt % ST);
            else issue(T{}, nt, nt % ST);
        }
        compute(kt % ST);
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
    DMA_BOTH(256, 256, 32, 2, 4, 16, 3),
    DMA_BOTH(256, 256, 32, 2, 4, 16, 4),
    DMA_BOTH(256, 256, 64, 2, 4, 32, 2),
    DMA_BOTH(256, 128, 64, 2, 2, 16, 2),
    DMA_BOTH(256, 128, 64, 2, 2, 16, 3),
    DMA_BOTH(128, 128, 64, 2, 2, 16, 2),
    DMA_BOTH(128, 128, 64, 2, 2, 16, 3),
    DMA_BOTH(128, 128, 64, 2, 2, 32, 2),
};

}  // namespace

const KernelEntry* dma_kernel_table(int* count) {
    *count = static_cast<int>(sizeof(kDmaTable) / sizeof(kDmaTable[0]));
    return kDmaTable;
}

}  // namespace dtg
