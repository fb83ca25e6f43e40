// The block-scaled (MX) tile kernel for gfx950, shared by the variant tables
// of gemm_mx.hip (pairs of one width: 8-bit with 8-bit, E2M1 with E2M1) and
// gemm_mx_pairs.hip (the other pairs).
//
// D = A x B (+ C), where A and B hold FP8 (E4M3, E5M2), FP6 (E2M3, E3M2) or
// FP4 (E2M1) elements, chosen per operand, and every 32 consecutive k of a row
// of A (of a column of B) share one E8M0 power-of-two scale.  The scaled
// matrix instruction of gfx950 (v_mfma_scale_f32_32x32x64_f8f6f4) applies the
// scales inside the contraction and takes the two operands' formats
// separately ("Tuning Triton kernels", section 6: the gfx950 instruction set
// adds a scaled MFMA as the way to the microscaled types; the FP4 x FP4 kernel
// of the same section runs on it), so the kernel is the direct-to-LDS tile
// kernel of gemm_dma_kernel.h with narrower elements and a scale pipeline
// beside the operand pipeline:
//
//  * both operands are k-contiguous (A row-major M x K, B stored N x K, the
//    block runs along k in both), kept in LDS as rows of one K step's k: 256
//    k for E2M1 with E2M1, else 128 k, i.e. rows of 128 (8-bit), 96 (6-bit)
//    or 64 (4-bit) bytes, each operand its own width; 16-byte chunks placed by
//    a swizzle of the row (XOR for 8 and 4 chunks, a rotation for 6), filled
//    by direct global -> LDS loads (masked lanes read zeros);
//  * the scales of a K step (4 or 8 per row) are loaded the same way, 4 bytes
//    per lane, into an LDS scale tile [row][block] per stage;
//  * operand lane layouts of the 32x32x64 instruction (pinned by the probe
//    tests): lane l = r + 32 g holds row (column) r; an 8-bit operand holds
//    k = 16 g .. 16 g + 15 in its first 16 bytes and k = 32 + 16 g .. in the
//    next 16, a 6-bit operand k = 32 g .. 32 g + 31 in its first 24 bytes (one
//    little-endian bit string), a 4-bit operand k = 32 g .. 32 g + 31 in its
//    first 16; the scale of row r and of the instruction's 32-k block b is
//    taken from byte `opsel` of lane r + 32 b's scale register.  The kernel
//    feeds the instruction of k step m (of NKI per K step) block b = 0, 1 from
//    the K step's block b * NKI + m, for every width, so lane g's scales for
//    the NKI instructions are NKI consecutive bytes of its row: one 2- or
//    4-byte LDS read per fragment per K step, instruction m selecting byte m.
//    A sub-step covers 64 k (one instruction per accumulator), or 128 k of
//    E2M1 with E2M1 (two);
//  * scales of blocks past ceil(K / 32) (the end of the last K step) are
//    replaced in registers: by 1.0, where every element past K is a zero from
//    a masked load, and by 0 (2^-127) where an FP6 block past K can share a
//    16-byte chunk with the last one inside K (every FP6 and FP4 code is
//    finite, so the 2^-254 product scale takes it to zero); either way no
//    scale byte read past the blocks can inject a NaN.
//
// The operand order is swapped (B fragment first) so each accumulator holds
// the transposed block and a lane's registers are 4 consecutive columns of one
// output row.  K steps past the end of K are loaded from an empty range, so
// every step of the software pipeline is uniform.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "kernels_mx.h"
#include "tile_order.h"

namespace dtg {
namespace {

using namespace dev;

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// One scaled 32x32x64 instruction: c += (x scaled by sx) x (y scaled by sy)^T,
// formats FX / FY, scale bytes OPS of sx and sy.
template <int FX, int FY, int OPS>
__device__ __forceinline__ f32x16 mfma_mx(i32x8 x, i32x8 y, int sx, int sy, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, c, FX, FY, OPS, sx, OPS, sy);
}

// Element bits of a format code, and the k of one K step of a pair: 256 for
// E2M1 with E2M1 (128-byte rows), else 128 (rows of 128, 96 or 64 bytes).
template <int F>
constexpr int mx_bits() { return F <= kMxE5M2 ? 8 : (F == kMxE2M1 ? 4 : 6); }
template <int FA, int FB>
constexpr int mx_bke() { return (FA == kMxE2M1 && FB == kMxE2M1) ? 256 : 128; }

// Physical 16-byte chunk of logical chunk c of LDS row r for rows of CH
// chunks: the XOR swizzles of 8 and 4 chunks, and for the 6 chunks of a 96-byte
// FP6 row a rotation by (r mod 16) / 4, which keeps the 8-byte operand reads
// of 16 consecutive rows within two-way bank conflicts (the 8-byte half of a
// read within its chunk is fixed by the 24-byte element blocks, so no
// permutation of whole chunks does better).
template <int CH>
__device__ __forceinline__ int mx_phys(int c, int r) {
    if constexpr (CH == 6) return (c + ((r >> 2) & 3)) % 6;
    else return c ^ swz<CH>(r);
}
template <int CH>
__device__ __forceinline__ int mx_logical(int pc, int r) {
    if constexpr (CH == 6) return (pc + 6 - ((r >> 2) & 3)) % 6;
    else return pc ^ swz<CH>(r);
}

// Operand registers of one 32-row fragment for one sub-step (MPS instruction
// k steps of 64 k), filled by NR LDS reads:
//  - 8 bits: two 16-byte reads, bytes 0-15 and 16-31 of one instruction's operand;
//  - 4 bits, two instructions per sub-step: one 16-byte read per instruction;
//  - 4 bits, one instruction: one 16-byte read (register dwords 4-7 unused);
//  - 6 bits: the 24 bytes of one 32-k block (dwords 6-7 unused) as a 16-byte
//    and an 8-byte read: a block of even index starts a 16-byte chunk (a whole
//    chunk, then the first half of the next), one of odd index starts in the
//    middle of one (its second half, then the next chunk whole).  P is the
//    block parity, that of the sub-step.
// The operand tuple is assembled where the instruction uses it, after the
// reads have been waited for (the reads are asm whose results the compiler
// takes as ready at once, so no copy of them may come earlier).
template <int BITS, int MPS>
struct MxFrag {
    static constexpr int NR = BITS == 4 && MPS == 1 ? 1 : 2;
    u32x4 w[BITS == 6 ? 1 : NR];
    u32x2 n;   // 6 bits: the 8-byte half
    template <int R, int OFF, int P>
    __device__ __forceinline__ void read(uint32_t addr) {
        if constexpr (BITS != 6) w[R] = lds_read16_any<OFF>(addr);
        else if constexpr (R == 1 - P) n = lds_read8_any<OFF>(addr);
        else w[0] = lds_read16_any<OFF>(addr);
    }
    __device__ __forceinline__ void tie_all() {
#pragma unroll
        for (int r = 0; r < (BITS == 6 ? 1 : NR); ++r) tie(w[r]);
        if constexpr (BITS == 6) tie(n);
    }
    // operand of instruction H of the sub-step
    template <int H, int P>
    __device__ __forceinline__ i32x8 operand() const {
        if constexpr (BITS == 8) {
            return __builtin_shufflevector(__builtin_bit_cast(i32x4, w[0]), __builtin_bit_cast(i32x4, w[1]), 0, 1,
                                           2, 3, 4, 5, 6, 7);
        } else if constexpr (BITS == 4) {
            const i32x4 v = __builtin_bit_cast(i32x4, w[MPS == 2 ? H : 0]);
            return __builtin_shufflevector(v, v, 0, 1, 2, 3, -1, -1, -1, -1);
        } else {
            const i32x4 v = __builtin_bit_cast(i32x4, w[0]);
            const i32x4 h = __builtin_bit_cast(i32x4, __builtin_shufflevector(n, n, 0, 1, -1, -1));
            if constexpr (P == 0) return __builtin_shufflevector(v, h, 0, 1, 2, 3, 4, 5, -1, -1);
            else return __builtin_shufflevector(h, v, 0, 1, 4, 5, 6, 7, -1, -1);
        }
    }
};

template <bool BF16>
__device__ __forceinline__ void store4_16(uint16_t* d, const uint16_t* c, bool vec, int n_ok, const float (&v)[4]) {
    float w[4] = {v[0], v[1], v[2], v[3]};
    if (vec) {
        if (c) {
            const uint2 cv = *reinterpret_cast<const uint2*>(c);
            w[0] += widen<BF16>(static_cast<uint16_t>(cv.x & 0xffffu));
            w[1] += widen<BF16>(static_cast<uint16_t>(cv.x >> 16));
            w[2] += widen<BF16>(static_cast<uint16_t>(cv.y & 0xffffu));
            w[3] += widen<BF16>(static_cast<uint16_t>(cv.y >> 16));
        }
        uint2 dv;
        dv.x = static_cast<uint32_t>(narrow<BF16>(w[0])) | (static_cast<uint32_t>(narrow<BF16>(w[1])) << 16);
        dv.y = static_cast<uint32_t>(narrow<BF16>(w[2])) | (static_cast<uint32_t>(narrow<BF16>(w[3])) << 16);
        *reinterpret_cast<uint2*>(d) = dv;
    } else {
        for (int r = 0; r < 4; ++r)
            if (r < n_ok) d[r] = narrow<BF16>(c ? w[r] + widen<BF16>(c[r]) : w[r]);
    }
}

// Four fp32 values rounded to 16 bits, packed little-end first.
template <bool BF16>
__device__ __forceinline__ uint2 pack4(const float (&w)[4]) {
    uint2 dv;
    dv.x = static_cast<uint32_t>(narrow<BF16>(w[0])) | (static_cast<uint32_t>(narrow<BF16>(w[1])) << 16);
    dv.y = static_cast<uint32_t>(narrow<BF16>(w[2])) | (static_cast<uint32_t>(narrow<BF16>(w[3])) << 16);
    return dv;
}

__device__ __forceinline__ void store4_32(float* d, const float* c, bool vec, int n_ok, const float (&v)[4]) {
    if (vec) {
        f32x4 w = {v[0], v[1], v[2], v[3]};
        if (c) w += *reinterpret_cast<const f32x4*>(c);
        *reinterpret_cast<f32x4*>(d) = w;
    } else {
        for (int r = 0; r < 4; ++r)
            if (r < n_ok) d[r] = c ? v[r] + c[r] : v[r];
    }
}

// LDS bytes of a tile kernel: operand stages (rows of BKE k of each
// operand's width), scale stages (each operand's region a whole number of
// 256-byte load instructions), a 256-byte and (with FP6 rows) a 1024-byte
// scratch slot for loads that have no rows; at least what the epilogue of a
// 16-bit output stages (the tile's rows padded by 16 bytes).
constexpr int64_t mx_lds(int bm, int bn, int st, int fa, int fb) {
    const int bits_a = fa <= kMxE5M2 ? 8 : (fa == kMxE2M1 ? 4 : 6);
    const int bits_b = fb <= kMxE5M2 ? 8 : (fb == kMxE2M1 ? 4 : 6);
    const int bke = (fa == kMxE2M1 && fb == kMxE2M1) ? 256 : 128;
    const int nblk = bke / 32;
    const int64_t oper = static_cast<int64_t>(st) * (bm * bke * bits_a / 8 + bn * bke * bits_b / 8) +
                         static_cast<int64_t>(st) * 256 * ((bm * nblk + 255) / 256 + (bn * nblk + 255) / 256) + 256 +
                         ((bits_a == 6 || bits_b == 6) ? 1024 : 0);
    const bool legacy = (bits_a == 8 && bits_b == 8) || (bits_a == 4 && bits_b == 4);
    const int64_t epi = static_cast<int64_t>(bm) * (bn * 2 + 16);
    return legacy || oper >= epi ? oper : epi;
}

template <int BM, int BN, int WM, int WN, int ST, int FA, int FB>
__global__ __launch_bounds__(64 * WM * WN) void gemm_mx_kernel(MxArgs p) {
    constexpr int NW = WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int EBA = mx_bits<FA>(), EBB = mx_bits<FB>();   // element bits of A and of B
    constexpr int BKE = mx_bke<FA, FB>();              // k per K step
    constexpr int ROWA = BKE * EBA / 8, ROWBB = BKE * EBB / 8;  // bytes of k per row and K step
    constexpr int CHA = ROWA / 16, CHB = ROWBB / 16;   // 16-byte chunks per row (8, 6 or 4)
    constexpr int NKI = BKE / 64;                      // instruction k steps per K step
    constexpr int MPS = (BKE == 256) ? 2 : 1;          // instruction k steps per sub-step
    constexpr int NKS = NKI / MPS;                     // sub-steps per K step (2)
    constexpr int NBLK = BKE / 32;                     // scale blocks per K step
    typedef MxFrag<EBA, MPS> FragA;
    typedef MxFrag<EBB, MPS> FragB;
    constexpr int RA = FragA::NR, RB = FragB::NR;      // LDS reads per fragment per sub-step
    // operand load instructions per stage (1024 bytes each) and per wave; the
    // last round of a 96-byte-row operand may leave waves without a load
    constexpr int NIA = BM * CHA / 64, NIB = BN * CHB / 64;
    constexpr int IA_W = (NIA + NW - 1) / NW, IB_W = (NIB + NW - 1) / NW;
    static_assert((BM * CHA) % 64 == 0 && (BN * CHB) % 64 == 0, "whole load instructions per stage");
    static_assert(CHA == 6 || NIA % NW == 0, "uniform load rounds for 8- and 4-bit rows");
    static_assert(CHB == 6 || NIB % NW == 0, "uniform load rounds for 8- and 4-bit rows");
    static_assert(TM % 32 == 0 && TN % 32 == 0, "tile vs wave grid");
    // scale loads: 64 lanes x 4 bytes = 256 bytes of [row][NBLK] per instruction
    constexpr int SRPI = 256 / NBLK;                   // scale rows per instruction
    // instructions per stage for A's and B's scales; a tile of fewer rows than
    // one instruction covers pads its scale region to the instruction's 256 bytes
    constexpr int SIA = (BM + SRPI - 1) / SRPI, SIB = (BN + SRPI - 1) / SRPI;
    constexpr int NSA = (SIA + NW - 1) / NW, NSB = (SIB + NW - 1) / NW;   // per wave (some may be empty)
    constexpr int NSL = NSA + NSB;
    constexpr int L = IA_W + IB_W + NSL;               // loads per wave per K step
    constexpr int LA = IA_W + IB_W;                    // operand loads (load numbers 0 .. LA - 1)
    static_assert(ST >= 2 && ST <= 8 && (ST - 1) * L < 64, "stages");

    constexpr int SA_B = BM * ROWA, SB_B = BN * ROWBB; // bytes per stage
    constexpr int SSA_B = SIA * 256, SSB_B = SIB * 256;
    constexpr int OFF_B = ST * SA_B;
    constexpr int OFF_S = ST * (SA_B + SB_B);
    constexpr int OFF_SB = OFF_S + ST * SSA_B;
    constexpr int OFF_DUMMY = OFF_SB + ST * SSB_B;     // 256 bytes: scale loads with no rows
    constexpr int OFF_DUMMY_OP = OFF_DUMMY + 256;      // 1024 bytes: operand loads with no rows
    constexpr int LDS_BYTES = static_cast<int>(mx_lds(BM, BN, ST, FA, FB));
    static_assert(LDS_BYTES >= OFF_DUMMY + 256, "LDS layout");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    // Workgroup -> (K slice, output tile): the XCD permutation runs over the
    // whole grid, consecutive positions are consecutive tiles (grouped order)
    // of one slice.  With one slice this is tile_of_workgroup.
    const int ntiles = p.num_pid_m * p.num_pid_n;
    const int NS = p.splits;
    int pid_m, pid_n, tile_lin, slice;
    {
        const int pos = xcd_permute<int>(blockIdx.x, ntiles * NS, p.xcds);
        slice = pos / ntiles;
        tile_lin = pos - slice * ntiles;
        grouped_tile<int>(tile_lin, p.num_pid_m, p.num_pid_n, p.group_m, &pid_m, &pid_n);
    }
    const int m0 = pid_m * BM, n0 = pid_n * BN;
    const int M = p.M, N = p.N, K = p.K;
    const int kbytes_a = K * EBA / 8, kbytes_b = K * EBB / 8;   // bytes of k of a row
    const int nblocks = (K + 31) / 32;

    // ---- per-lane operand load offsets: load Y of an operand fills LDS rows
    // Y*NW*R + wave*R + lane/8 with the lane's 16-byte chunk lane % 8 of the
    // row; the lane fetches the chunk that the swizzle puts there, at byte
    // offset vo0 + Y * (NW*R rows).  Rows past the matrix need no mask: the
    // descriptor's range ends K's bytes into the last row, and the next row
    // starts a row stride (>= K's bytes) after that row.  The K tail is a
    // per-lane bit OR'd in at each step.  One base offset per operand (not
    // one per load) keeps the 8-bit 256 x 256 tile clear of register spills,
    // whose reloads would drain the load ring; masking is arithmetic, so the
    // loop has no data-dependent branches.
    // Rows of 8 or 4 chunks: a load instruction fills 64 / CH whole rows and
    // every wave's loads share one chunk permutation (the swizzle depends on
    // the row mod 16), so one base offset and a row stride per operand.  Rows
    // of 6 chunks (FP6): instruction Y of wave w fills the tile's chunks
    // (Y NW + w) 64 .. + 63 in row order, so each load has its own offset and
    // chunk (and a wave past the last instruction loads nothing).
    const int ld_row_a = wave * (64 / (CHA == 6 ? 8 : CHA)) + lane / (CHA == 6 ? 8 : CHA);
    const int ld_row_b = wave * (64 / (CHB == 6 ? 8 : CHB)) + lane / (CHB == 6 ? 8 : CHB);
    const int ld_chunk_a = mx_logical<CHA == 6 ? 8 : CHA>(lane % (CHA == 6 ? 8 : CHA), ld_row_a);
    const int ld_chunk_b = mx_logical<CHB == 6 ? 8 : CHB>(lane % (CHB == 6 ? 8 : CHB), ld_row_b);
    const uint32_t a_vo0 = static_cast<uint32_t>(static_cast<int64_t>(ld_row_a) * p.lda + ld_chunk_a * 16);
    const uint32_t b_vo0 = static_cast<uint32_t>(static_cast<int64_t>(ld_row_b) * p.ldb + ld_chunk_b * 16);
    const uint32_t a_ys = static_cast<uint32_t>(NW * (64 / (CHA == 6 ? 8 : CHA)) * p.lda);
    const uint32_t b_ys = static_cast<uint32_t>(NW * (64 / (CHB == 6 ? 8 : CHB)) * p.ldb);
    uint32_t a6_vo[CHA == 6 ? IA_W : 1], b6_vo[CHB == 6 ? IB_W : 1];
    int a6_c[CHA == 6 ? IA_W : 1], b6_c[CHB == 6 ? IB_W : 1];
    auto six = [&](int y, int ni, int64_t ld, uint32_t* vo, int* c) {
        const int ins = y * NW + wave;
        const int q = ins * 64 + lane;
        const int row = q / 6;
        const int lc = mx_logical<6>(q % 6, row);
        *vo = ins < ni ? static_cast<uint32_t>(static_cast<int64_t>(row) * ld + lc * 16) : kOOB;
        *c = lc;
    };
    if constexpr (CHA == 6) {
#pragma unroll
        for (int y = 0; y < IA_W; ++y) six(y, NIA, p.lda, &a6_vo[y], &a6_c[y]);
    }
    if constexpr (CHB == 6) {
#pragma unroll
        for (int y = 0; y < IB_W; ++y) six(y, NIB, p.ldb, &b6_vo[y], &b6_c[y]);
    }
    // scale loads: A's instruction X of a wave is number si = X * NW + wave of
    // the stage (SRPI rows of the scale tile), B's likewise.  A wave whose si is
    // past the tile loads nothing (offset past the range) into a scratch slot;
    // lanes past the matrix's rows read zeros.  Per-lane offsets, LDS
    // destinations and their stage strides are fixed for the whole kernel, so
    // the loop holds no wave-dependent control flow.
    constexpr int DPR = NBLK / 4;                      // dwords per scale row
    uint32_t s_voff[NSL];
    int s_dst[NSL], s_stage[NSL];
#pragma unroll
    for (int x = 0; x < NSL; ++x) {
        const bool is_a = x < NSA;
        const int si = (is_a ? x : x - NSA) * NW + wave;
        const bool valid = si < (is_a ? SIA : SIB);
        const int rr = si * SRPI + lane / DPR;
        const bool in_rows = rr < (is_a ? BM : BN) && (is_a ? m0 + rr < M : n0 + rr < N);
        s_voff[x] = (valid && in_rows)
                        ? static_cast<uint32_t>(static_cast<int64_t>(rr) * (is_a ? p.ldsa : p.ldsb) + 4 * (lane % DPR))
                        : kOOB;
        s_dst[x] = valid ? (is_a ? OFF_S : OFF_SB) + si * 256 : OFF_DUMMY;
        s_stage[x] = valid ? (is_a ? SSA_B : SSB_B) : 0;
    }

    const uint32_t smem0 = lds_addr(reinterpret_cast<const uint16_t*>(smem));

    // A's and B's rows alike with one chunk per lane: one K-tail mask for both
    constexpr bool SAME = CHA == CHB && EBA == EBB && CHA != 6;
    constexpr int NKA = CHA == 6 ? IA_W : 1, NKB = SAME ? 1 : (CHB == 6 ? IB_W : 1);
    struct Desc {
        __amdgpu_buffer_rsrc_t ra, rb, rsa, rsb;
        // kOOB for a lane's chunk when it is past K, else 0 (per load for FP6 rows)
        uint32_t kmask_a[NKA], kmask_b[NKB];
    };
    // this slice's K steps: [kt0, kt1)
    const int nkt_all = (K + BKE - 1) / BKE;
    const int per_slice = (nkt_all + NS - 1) / NS;
    const int kt0 = slice * per_slice;
    const int kt1 = kt0 + per_slice < nkt_all ? kt0 + per_slice : nkt_all;
    const int nkt = kt1 > kt0 ? kt1 - kt0 : 0;
    // Descriptor ranges, clamped once: each step's descriptor starts at the
    // step's first byte of k, so its range is the tile's range less that
    // offset (the planner keeps 256 rows plus K bytes under 2^31, so a clamped
    // range still covers every offset a step uses); scale rows are read whole
    // up to their row stride (a multiple of 4).  Per step this is 32-bit
    // scalar arithmetic only.
    const uint8_t* a_base = p.A + static_cast<int64_t>(m0) * p.lda;
    const uint8_t* b_base = p.B + static_cast<int64_t>(n0) * p.ldb;
    const uint8_t* sa_base = p.SA + static_cast<int64_t>(m0) * p.ldsa;
    const uint8_t* sb_base = p.SB + static_cast<int64_t>(n0) * p.ldsb;
    const uint32_t a_rec = clamp_records(static_cast<int64_t>(M - 1 - m0) * p.lda + kbytes_a);
    const uint32_t b_rec = clamp_records(static_cast<int64_t>(N - 1 - n0) * p.ldb + kbytes_b);
    const uint32_t sa_rec = clamp_records(static_cast<int64_t>(M - m0) * p.ldsa);
    const uint32_t sb_rec = clamp_records(static_cast<int64_t>(N - n0) * p.ldsb);
    auto make_desc = [&](int kt) {
        Desc d;
        const int kba0 = kt * ROWA, kbb0 = kt * ROWBB;
        const bool live = kt < kt1;   // steps past the slice (kept for a uniform ring) read nothing
        const uint32_t kba = live ? static_cast<uint32_t>(kba0) : 0u;
        const uint32_t kbb = live ? static_cast<uint32_t>(kbb0) : 0u;
        const uint32_t sb = live ? static_cast<uint32_t>(kt * NBLK) : 0u;
        d.ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a_base + kba), 0, live ? a_rec - kba : 0u,
                                                 kRsrcWord3);
        d.rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(b_base + kbb), 0, live ? b_rec - kbb : 0u,
                                                 kRsrcWord3);
        d.rsa = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(sa_base + sb), 0, live ? sa_rec - sb : 0u,
                                                  kRsrcWord3);
        d.rsb = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(sb_base + sb), 0, live ? sb_rec - sb : 0u,
                                                  kRsrcWord3);
        // opaque to the compiler, so it cannot fold the K-tail bit into
        // per-load offsets hoisted out of the loop (one register per load)
#pragma unroll
        for (int y = 0; y < NKA; ++y) {
            d.kmask_a[y] = kba0 + (CHA == 6 ? a6_c[y] : ld_chunk_a) * 16 < kbytes_a ? 0u : kOOB;
            tie(d.kmask_a[y]);
        }
        if constexpr (!SAME) {
#pragma unroll
            for (int y = 0; y < NKB; ++y) {
                d.kmask_b[y] = kbb0 + (CHB == 6 ? b6_c[y] : ld_chunk_b) * 16 < kbytes_b ? 0u : kOOB;
                tie(d.kmask_b[y]);
            }
        }
        return d;
    };
    // Load number X of a K step into stage s: A's operand loads, B's, then the scale loads.
    auto load_op = [&](auto x_tag, const Desc& d, int s) {
        constexpr int X = decltype(x_tag)::value;
        if constexpr (X < IA_W + IB_W) {
            constexpr bool IS_A = X < IA_W;
            constexpr int Y = IS_A ? X : X - IA_W;
            constexpr int CH = IS_A ? CHA : CHB;
            const uint32_t km = IS_A ? d.kmask_a[CH == 6 ? Y : 0] : (SAME ? d.kmask_a[0] : d.kmask_b[CH == 6 ? Y : 0]);
            uint32_t v;
            int dst;
            if constexpr (CH == 6) {
                // the offset of a wave past the last instruction is kOOB already
                v = (IS_A ? a6_vo[Y] : b6_vo[Y]) | km;
                dst = (Y * NW + wave) < (IS_A ? NIA : NIB)
                          ? (IS_A ? s * SA_B : OFF_B + s * SB_B) + (Y * NW + wave) * 1024
                          : OFF_DUMMY_OP;
            } else {
                // Y * stride < 2^31 (the planner bounds a tile's rows), so
                // OR-ing the K-tail bit adds it; the sum stays below 2^32
                v = (IS_A ? a_vo0 : b_vo0) + ((Y * (IS_A ? a_ys : b_ys)) | km);
                dst = (IS_A ? s * SA_B : OFF_B + s * SB_B) + (Y * NW + wave) * 1024;
            }
            // (a non-const local: clang's host pass drops the kernel when the
            // builtin is handed a member of a const reference)
            __amdgpu_buffer_rsrc_t r = IS_A ? d.ra : d.rb;
            // the decode slab (BM <= 32: one row of tiles) reads each byte of B
            // exactly once: non-temporal loads; square tiles share B panels
            // between rows of tiles through the L2 and keep the default policy
            constexpr int AUX = (!IS_A && BM <= 32) ? kNonTemporal : 0;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(smem + dst), 16, v, 0, 0, AUX);
        } else {
            constexpr int S = X - IA_W - IB_W;
            __amdgpu_buffer_rsrc_t r = (S < NSA) ? d.rsa : d.rsb;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(smem + s_dst[S] + s * s_stage[S]), 4, s_voff[S],
                                                    0, 0, 0);
        }
    };
    auto issue_tile = [&](int kt, int s) {
        const Desc d = make_desc(kt);
        static_for<L>([&](auto x_tag) { load_op(x_tag, d, s); });
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // ---- per-lane read addresses.  Fragment f of a wave covers rows
    // w*T + 32 f .. + 31 (its offset 32 f * 128 bytes goes into the read's
    // offset field, with the stage offset); lane l reads row l % 32 at the
    // chunk of sub-step ks and half h: 8-bit: block h*NKS + ks, bytes
    // 16 g .. 16 g + 15 of it (chunk 2 (h NKS + ks) + g), the two halves one
    // instruction's operand; 4-bit: block g NKI + 2 ks + h (chunk likewise),
    // half h the operand of instruction k step 2 ks + h.
    // A 6-bit operand reads the 24 bytes of block g NKI + ks as three 8-byte
    // pieces (byte 24 blk + 8 j: chunk / 16, its half / 8 within the chunk).
    const int g = lane / 32;
    const int fr = lane % 32;
    auto frag_addr = [&](auto bits_tag, auto ch_tag, int rowb, int base, int ks, int r) -> uint32_t {
        constexpr int BITS = decltype(bits_tag)::value;
        constexpr int CH = decltype(ch_tag)::value;
        int c, half = 0;
        if constexpr (BITS == 8) {
            c = 2 * (r * NKS + ks) + g;
        } else if constexpr (BITS == 4) {
            c = g * NKI + MPS * ks + r;
        } else {
            // block g NKI + ks (of parity ks & 1): read r of it (see MxFrag)
            const int c0 = 3 * ((g * NKI + ks) >> 1);
            if ((ks & 1) == 0) {
                c = c0 + r;                 // chunk c0 whole, then the first half of c0 + 1
            } else {
                c = c0 + 1 + r;             // the second half of c0 + 1, then c0 + 2 whole
                half = r == 0 ? 1 : 0;
            }
        }
        return smem0 + base + fr * rowb + mx_phys<CH>(c, fr) * 16 + 8 * half;
    };
    uint32_t a_addr[NKS][RA], b_addr[NKS][RB];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int r = 0; r < RA; ++r)
            a_addr[ks][r] = frag_addr(std::integral_constant<int, EBA>{}, std::integral_constant<int, CHA>{}, ROWA,
                                      wm * TM * ROWA, ks, r);
#pragma unroll
        for (int r = 0; r < RB; ++r)
            b_addr[ks][r] = frag_addr(std::integral_constant<int, EBB>{}, std::integral_constant<int, CHB>{}, ROWBB,
                                      OFF_B + wn * TN * ROWBB, ks, r);
    }
    const uint32_t sa_addr = smem0 + OFF_S + (wm * TM + fr) * NBLK + g * NKI;
    const uint32_t sb_addr = smem0 + OFF_SB + (wn * TN + fr) * NBLK + g * NKI;

    FragA fa[2][FM];
    FragB fb[2][FN];
    uint32_t ssa[2][FM], ssb[2][FN];
    constexpr int NRF = FM * RA + FN * RB;            // operand reads per sub-step
    constexpr int NRS = FM + FN;                      // scale reads per K step

    // LDS read R of sub-step KS of stage S into fragment slot SL (scales: tile slot TS).
    auto read_op = [&](auto stage_tag, auto ks_tag, auto slot_tag, auto ts_tag, auto r_tag) {
        constexpr int S = decltype(stage_tag)::value;
        constexpr int KS = decltype(ks_tag)::value;
        constexpr int SL = decltype(slot_tag)::value;
        constexpr int TS = decltype(ts_tag)::value;
        constexpr int RR = decltype(r_tag)::value;
        if constexpr (RR < FN * RB) {
            constexpr int J = RR / RB, H = RR % RB;
            fb[SL][J].template read<H, S * SB_B + J * 32 * ROWBB, (KS & 1)>(b_addr[KS][H]);
        } else if constexpr (RR < NRF) {
            constexpr int I = (RR - FN * RB) / RA, H = (RR - FN * RB) % RA;
            fa[SL][I].template read<H, S * SA_B + I * 32 * ROWA, (KS & 1)>(a_addr[KS][H]);
        } else if constexpr (RR - NRF < FN) {
            constexpr int J = RR - NRF;
            if constexpr (NKI == 2) ssb[TS][J] = lds_read_u16<S * SSB_B + J * 32 * NBLK>(sb_addr);
            else ssb[TS][J] = lds_read_b32<S * SSB_B + J * 32 * NBLK>(sb_addr);
        } else {
            constexpr int I = RR - NRF - FN;
            if constexpr (NKI == 2) ssa[TS][I] = lds_read_u16<S * SSA_B + I * 32 * NBLK>(sa_addr);
            else ssa[TS][I] = lds_read_b32<S * SSA_B + I * 32 * NBLK>(sa_addr);
        }
    };
    auto wait_frags = [&](auto slot_tag) {
        constexpr int SL = decltype(slot_tag)::value;
        lds_wait_all();
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[SL][j].tie_all();
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[SL][i].tie_all();
    };
    // Scales of tile kt (slot TS), after their reads landed: bytes of blocks
    // at or past ceil(K / 32) become 127 (2^0); their elements are zeros.  With
    // an FP6 operand they become 0 (2^-127) instead: a 24-byte block can end
    // inside a 16-byte chunk, whose remaining bytes (the next block's, past
    // K) are loaded as they are, and FP6 and FP4 codes are finite, so a
    // 2^-254 product scale takes them to zero.
    constexpr uint32_t FILL = (EBA == 6 || EBB == 6) ? 0u : 0x7f7f7f7fu;
    auto mask_scales = [&](auto ts_tag, int kt) {
        constexpr int TS = decltype(ts_tag)::value;
        const int v = nblocks - kt * NBLK - g * NKI;    // valid bytes of this lane's NKI
        const uint32_t keep = v >= NKI ? 0xffffffffu : v <= 0 ? 0u : (1u << (8 * v)) - 1u;
        const uint32_t fill = FILL & ~keep;
#pragma unroll
        for (int j = 0; j < FN; ++j) { tie(ssb[TS][j]); ssb[TS][j] = (ssb[TS][j] & keep) | fill; }
#pragma unroll
        for (int i = 0; i < FM; ++i) { tie(ssa[TS][i]); ssa[TS][i] = (ssa[TS][i] & keep) | fill; }
    };
    auto mfma_op = [&](auto slot_tag, auto ts_tag, auto ks_tag, auto q_tag) {
        constexpr int SL = decltype(slot_tag)::value;
        constexpr int TS = decltype(ts_tag)::value;
        constexpr int KS = decltype(ks_tag)::value;
        constexpr int Q = decltype(q_tag)::value;
        if constexpr (MPS == 1) {
            constexpr int I = Q / FN, J = Q % FN;
            acc[I][J] = mfma_mx<FB, FA, KS>(fb[SL][J].template operand<0, (KS & 1)>(),
                                            fa[SL][I].template operand<0, (KS & 1)>(),
                                            static_cast<int>(ssb[TS][J]), static_cast<int>(ssa[TS][I]), acc[I][J]);
        } else {
            // all blocks of half 0, then of half 1: an accumulator's two
            // instructions are FM * FN instructions apart
            constexpr int H = Q / (FM * FN), I = (Q % (FM * FN)) / FN, J = Q % FN;
            acc[I][J] = mfma_mx<FB, FA, MPS * KS + H>(fb[SL][J].template operand<H, 0>(),
                                                      fa[SL][I].template operand<H, 0>(), static_cast<int>(ssb[TS][J]),
                                                      static_cast<int>(ssa[TS][I]), acc[I][J]);
        }
    };
    constexpr int NQ = FM * FN * MPS;                 // instructions per sub-step

    // The MFMAs of a sub-step with NOPS memory operations between them,
    // ceil(NOPS / NQ) after each MFMA from the first on, so the loads and
    // reads of the sub-step are all in flight early.
    auto interleave = [&](auto slot_tag, auto ts_tag, auto ks_tag, auto nops_tag, auto&& op) {
        constexpr int NOPS = decltype(nops_tag)::value;
        constexpr int PER = (NOPS + NQ - 1) / NQ;
        static_for<NQ>([&](auto q_tag) {
            constexpr int Q = decltype(q_tag)::value;
            mfma_op(slot_tag, ts_tag, ks_tag, q_tag);
            static_for<NOPS>([&](auto o_tag) {
                if constexpr (decltype(o_tag)::value / PER == Q) op(o_tag);
            });
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    // One K step (tile kt) on stage S = U % ST, tile slot U % 2; sub-step ks
    // uses fragment slot (U NKS + ks) % 2.  The last sub-step waits for tile
    // kt + 1, passes the barrier, and runs its MFMAs with the operand loads of
    // tile kt + ST into this stage and the reads of tile kt + 1 (its first
    // sub-step's fragments and its scales) between them.  The scale loads of
    // a tile follow one sub-step later, in the first sub-step of the next K
    // step (their stage is free since the same barrier): measured against
    // issuing all loads together, E4M3 4096^3 65.8 -> 63.6 us, E2M1 41.6 ->
    // 41.1 us, E2M1 16 x 8192 x 8192 11.07 -> 10.80 us, bitwise-identical.
    auto step = [&](auto u_tag, int kt) {
        constexpr int U = decltype(u_tag)::value;
        constexpr int S = U % ST, S1 = (U + 1) % ST;
        constexpr int TS = U % 2, TS1 = (U + 1) % 2;
        static_for<NKS>([&](auto ks_tag) {
            constexpr int KS = decltype(ks_tag)::value;
            constexpr int CUR = (U * NKS + KS) & 1, NXT = CUR ^ 1;
            const auto cur = std::integral_constant<int, CUR>{};
            const auto nxt = std::integral_constant<int, NXT>{};
            const auto ts = std::integral_constant<int, TS>{};
            if constexpr (KS + 1 < NKS) {
                // (KS == 0: the scale loads of tile kt + ST - 1, into its stage)
                constexpr int LS = (KS == 0) ? L - LA : 0;
                const Desc ds = make_desc(kt + ST - 1);
                interleave(cur, ts, ks_tag, std::integral_constant<int, LS + NRF>{}, [&](auto o_tag) {
                    constexpr int O = decltype(o_tag)::value;
                    if constexpr (O < LS)
                        load_op(std::integral_constant<int, LA + O>{}, ds, (S + ST - 1) % ST);
                    else
                        read_op(std::integral_constant<int, S>{}, std::integral_constant<int, KS + 1>{}, nxt, ts,
                                std::integral_constant<int, O - LS>{});
                });
                wait_frags(nxt);
            } else {
                const Desc d = make_desc(kt + ST);
                wait_vm<(ST - 2) * L>();
                __builtin_amdgcn_s_barrier();
                // the loads first: from here to the same point of the next
                // step (one K step) is the time they have to land
                interleave(cur, ts, ks_tag, std::integral_constant<int, NRF + NRS + LA>{}, [&](auto o_tag) {
                    constexpr int O = decltype(o_tag)::value;
                    if constexpr (O < LA)
                        load_op(std::integral_constant<int, O>{}, d, S);
                    else
                        read_op(std::integral_constant<int, S1>{}, std::integral_constant<int, 0>{}, nxt,
                                std::integral_constant<int, TS1>{}, std::integral_constant<int, O - LA>{});
                });
                wait_frags(nxt);
                mask_scales(std::integral_constant<int, TS1>{}, kt + 1);
            }
        });
    };

    constexpr int UNROLL = (ST % 2 == 0) ? ST : 2 * ST;   // stage, fragment and tile slots repeat
    if (nkt > 0) {
        // tiles kt0 .. kt0 + ST - 2 whole, tile kt0 + ST - 1 without its
        // scales (the first step loads them); then wait for tile kt0
        static_for<ST - 1>([&](auto t_tag) { issue_tile(kt0 + decltype(t_tag)::value, decltype(t_tag)::value); });
        {
            const Desc d = make_desc(kt0 + ST - 1);
            static_for<LA>([&](auto x_tag) { load_op(x_tag, d, ST - 1); });
        }
        wait_vm<(ST - 2) * L + LA>();
        __builtin_amdgcn_s_barrier();
        static_for<NRF + NRS>([&](auto r_tag) {
            read_op(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{},
                    std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, r_tag);
        });
        wait_frags(std::integral_constant<int, 0>{});
        mask_scales(std::integral_constant<int, 0>{}, kt0);
        for (int j = 0; j < nkt; j += UNROLL) {
            static_for<UNROLL>([&](auto u_tag) {
                if (j + decltype(u_tag)::value < nkt) step(u_tag, kt0 + j + decltype(u_tag)::value);
            });
        }
        // no load may still be writing this workgroup's LDS when it exits
        wait_vm<0>();
    }

    // ---- K slices across workgroups: each slice publishes its fp32 partial
    // tile in register order, [tile][slice][wave][block][lane][4 floats]; the
    // workgroup that arrives last at the tile's counter adds the slices in
    // slice order (so the result does not depend on arrival order) into acc
    // and goes on to the epilogue; the others are done.  Partials move with
    // system-scope accesses (past the per-XCD L2 caches).
    constexpr int NB = FM * FN * 4;                   // 16-byte runs per lane
    if constexpr (NB <= 16) if (NS > 1) {
        constexpr int64_t WAVE_F = static_cast<int64_t>(NB) * 64 * 4;   // floats per wave per slice
        int* counters = static_cast<int*>(p.ws);
        float* tile_part = reinterpret_cast<float*>(static_cast<char*>(p.ws) + kCounterBytes) +
                           static_cast<int64_t>(tile_lin) * NS * NW * WAVE_F;
        const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
            tile_part, 0, clamp_records(static_cast<int64_t>(NS) * NW * WAVE_F * 4), kRsrcWord3);
        auto run_off = [&](int sl, int b) {
            return static_cast<uint32_t>(((static_cast<int64_t>(sl) * NW + wave) * WAVE_F + (b * 64 + lane) * 4) * 4);
        };
        // run b = (i * FN + j) * 4 + q holds registers 4q..4q+3 of acc[i][j]
        auto get_run = [&](auto b_tag) {
            constexpr int B = decltype(b_tag)::value;
            constexpr int I = B / 4 / FN, J = (B / 4) % FN, Q = B % 4;
            f32x4 v;
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = acc[I][J][4 * Q + r];
            return v;
        };
        auto set_run = [&](auto b_tag, const f32x4& v) {
            constexpr int B = decltype(b_tag)::value;
            constexpr int I = B / 4 / FN, J = (B / 4) % FN, Q = B % 4;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[I][J][4 * Q + r] = v[r];
        };
        static_for<NB>([&](auto b_tag) {
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, get_run(b_tag)), pr,
                                                   run_off(slice, decltype(b_tag)::value), 0, kSysScope);
        });
        if (!arrive_last(&counters[tile_lin], NS, reinterpret_cast<int*>(smem))) return;
        // slices in order into acc, in units of HB runs, the next unit in
        // flight while one is added (two units of registers)
        constexpr int HB = (NB <= 8) ? NB : NB / 2;
        constexpr int UPS = NB / HB;
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

    // ---- epilogue, 16-bit output without an addend: the tile, rounded, is
    // staged through the (now idle) LDS and written out as whole 16-byte
    // chunks of rows, a wave covering two 512-byte rows per store.  The
    // register layout would write 32 rows x 16 bytes per store instruction;
    // staged, the 32 MB output of a 4096^3 product goes out ~2x faster.  Rows
    // are padded by 16 bytes so the 8-byte LDS writes of a wave's 32 rows
    // spread over the banks.
    constexpr int OPITCH = BN * 2 + 16;
    if constexpr (BM * OPITCH <= LDS_BYTES) {
        if (p.has_c == 0 && p.out != 2) {
            const bool bf = p.out == 1;
            __syncthreads();   // every wave is past its last operand read
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float w[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                            acc[i][j][4 * q + 3]};
                        const int row = wm * TM + i * 32 + fr, col = wn * TN + j * 32 + 8 * q + 4 * g;
                        *reinterpret_cast<uint2*>(smem + row * OPITCH + col * 2) = bf ? pack4<true>(w)
                                                                                      : pack4<false>(w);
                    }
            __syncthreads();
            constexpr int CPR = BN / 8;                   // 16-byte chunks per tile row
            constexpr int NT = 64 * NW;
            static_assert((BM * CPR) % NT == 0, "whole chunk rounds");
            const bool dvec = (p.ldd % 8 == 0) && (reinterpret_cast<uintptr_t>(p.D) % 16 == 0);
            uint16_t* const D = static_cast<uint16_t*>(p.D);
#pragma unroll
            for (int x0 = 0; x0 < BM * CPR; x0 += NT) {
                const int x = x0 + tid;
                const int row = x / CPR, cc = x % CPR;
                const int gr = m0 + row, gc = n0 + cc * 8;
                if (gr < M && gc < N) {
                    const uint4 v = *reinterpret_cast<const uint4*>(smem + row * OPITCH + cc * 16);
                    uint16_t* d = D + static_cast<int64_t>(gr) * p.ldd + gc;
                    if (dvec && gc + 8 <= N) {
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

    // ---- epilogue with an addend or an fp32 output: the fp32 tile is staged
    // in P passes of BM / P rows (the waves of WM / P wave rows each); C is
    // read and D written as runs of 8 elements of a row (16- or 32-byte
    // accesses), acc + C added in fp32 and rounded once, as in the register
    // path below.  16-byte chunks of 4 floats sit at chunk position
    // c ^ (r mod SW) of their row, SW = min(32, chunks per row).
    constexpr int P32 = (BM * BN * 4 <= LDS_BYTES)                     ? 1
                        : (WM % 2 == 0 && BM * BN * 2 <= LDS_BYTES) ? 2
                        : (WM % 4 == 0 && BM * BN <= LDS_BYTES)     ? 4
                                                                    : 0;
    if constexpr (P32 > 0) {
        constexpr int PR = BM / P32, WPP = WM / P32;
        constexpr int C32 = BN / 4;                       // fp32 chunks per tile row
        constexpr int SW = C32 < 32 ? C32 : 32;
        constexpr int NT = 64 * NW;
        static_assert((PR * (BN / 8)) % NT == 0, "whole rounds of 8-element runs");
        const bool has_c = p.has_c != 0;
        const int out = p.out;
        const int esz = out == 2 ? 4 : 2;
        const bool vec = (p.ldd % 8 == 0) && (reinterpret_cast<uintptr_t>(p.D) % (8 * esz) == 0) &&
                         (!has_c || ((p.ldc % 8 == 0) && (reinterpret_cast<uintptr_t>(p.C) % (8 * esz) == 0)));
#pragma unroll
        for (int pass = 0; pass < P32; ++pass) {
            __syncthreads();   // operand reads (first pass) or the previous pass's reads are done
            if (wm / WPP == pass) {
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int row = (wm % WPP) * TM + i * 32 + fr;
                            const int col = wn * TN + j * 32 + 8 * q + 4 * g;
                            const f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                             acc[i][j][4 * q + 3]};
                            *reinterpret_cast<f32x4*>(smem + row * (BN * 4) + ((col / 4) ^ (row % SW)) * 16) = v;
                        }
            }
            __syncthreads();
#pragma unroll
            for (int x0 = 0; x0 < PR * (BN / 8); x0 += NT) {
                const int x = x0 + tid;
                const int row = x / (BN / 8), c8 = x % (BN / 8);
                const int gr = m0 + pass * PR + row, gc = n0 + c8 * 8;
                if (gr < M && gc < N) {
                    const f32x4 lo = *reinterpret_cast<const f32x4*>(smem + row * (BN * 4) + ((2 * c8) ^ (row % SW)) * 16);
                    const f32x4 hi =
                        *reinterpret_cast<const f32x4*>(smem + row * (BN * 4) + ((2 * c8 + 1) ^ (row % SW)) * 16);
                    float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    const int64_t doff = static_cast<int64_t>(gr) * p.ldd + gc;
                    const int64_t coff = static_cast<int64_t>(gr) * p.ldc + gc;
                    const int n_ok = N - gc;
                    if (out == 2) {
                        float* d = static_cast<float*>(p.D) + doff;
                        const float* c = has_c ? static_cast<const float*>(p.C) + coff : nullptr;
                        if (vec && n_ok >= 8) {
                            f32x4 w0 = lo, w1 = hi;
                            if (c) {
                                w0 += *reinterpret_cast<const f32x4*>(c);
                                w1 += *reinterpret_cast<const f32x4*>(c + 4);
                            }
                            store16_nt(d, w0);
                            store16_nt(d + 4, w1);
                        } else {
                            for (int e = 0; e < 8 && e < n_ok; ++e) d[e] = c ? v[e] + c[e] : v[e];
                        }
                    } else {
                        uint16_t* d = static_cast<uint16_t*>(p.D) + doff;
                        const uint16_t* c = has_c ? static_cast<const uint16_t*>(p.C) + coff : nullptr;
                        const bool bf = out == 1;
                        if (vec && n_ok >= 8) {
                            if (c) {
                                const uint4 cv = *reinterpret_cast<const uint4*>(c);
                                const uint32_t cu[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
                                for (int e = 0; e < 4; ++e) {
                                    const uint16_t c0 = static_cast<uint16_t>(cu[e] & 0xffffu);
                                    const uint16_t c1 = static_cast<uint16_t>(cu[e] >> 16);
                                    v[2 * e] += bf ? widen<true>(c0) : widen<false>(c0);
                                    v[2 * e + 1] += bf ? widen<true>(c1) : widen<false>(c1);
                                }
                            }
                            const float w0[4] = {v[0], v[1], v[2], v[3]}, w1[4] = {v[4], v[5], v[6], v[7]};
                            const uint2 a = bf ? pack4<true>(w0) : pack4<false>(w0);
                            const uint2 b = bf ? pack4<true>(w1) : pack4<false>(w1);
                            store16_nt(d, a.x, a.y, b.x, b.y);
                        } else {
                            for (int e = 0; e < 8 && e < n_ok; ++e) {
                                float w = v[e];
                                if (c) w += bf ? widen<true>(c[e]) : widen<false>(c[e]);
                                d[e] = bf ? narrow<true>(w) : narrow<false>(w);
                            }
                        }
                    }
                }
            }
        }
        return;
    }

    // ---- otherwise: + C in fp32, round to the output type, masked store.
    // Lane l holds, per block (i, j), row l % 32 and, for q = 0..3, columns
    // 8 q + 4 (l / 32) + 0..3 in registers 4 q .. 4 q + 3.
    const bool has_c = p.has_c != 0;
    const int out = p.out;
    const int esz = out == 2 ? 4 : 2;
    const int vq = out == 2 ? 4 : 4;   // elements per vector store
    const bool dvec = (p.ldd % vq == 0) && (reinterpret_cast<uintptr_t>(p.D) % (vq * esz) == 0);
    const bool cvec = !has_c || ((p.ldc % vq == 0) && (reinterpret_cast<uintptr_t>(p.C) % (vq * esz) == 0));
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int row = m0 + wm * TM + i * 32 + fr;
        if (row >= M) continue;
        const int64_t drow = static_cast<int64_t>(row) * p.ldd;
        const int64_t crow = static_cast<int64_t>(row) * p.ldc;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int col = n0 + wn * TN + j * 32 + 8 * q + 4 * g;
                if (col >= N) continue;
                float v[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = acc[i][j][4 * q + r];
                const bool vec = dvec && cvec && col + 4 <= N;
                const int n_ok = N - col;
                if (out == 2) {
                    store4_32(static_cast<float*>(p.D) + drow + col,
                              has_c ? static_cast<const float*>(p.C) + crow + col : nullptr, vec, n_ok, v);
                } else if (out == 1) {
                    store4_16<true>(static_cast<uint16_t*>(p.D) + drow + col,
                                    has_c ? static_cast<const uint16_t*>(p.C) + crow + col : nullptr, vec, n_ok, v);
                } else {
                    store4_16<false>(static_cast<uint16_t*>(p.D) + drow + col,
                                     has_c ? static_cast<const uint16_t*>(p.C) + crow + col : nullptr, vec, n_ok, v);
                }
            }
        }
    }
}

template <int BM, int BN, int WM, int WN, int ST, int FA, int FB>
hipError_t launch_mx(const MxArgs& a, int64_t grid, hipStream_t stream) {
    hipLaunchKernelGGL((gemm_mx_kernel<BM, BN, WM, WN, ST, FA, FB>), dim3(static_cast<unsigned>(grid)),
                       dim3(64 * WM * WN), 0, stream, a);
    return hipGetLastError();
}

constexpr int kMaxMxSplits = 64;

#define DTG_STR2(x) #x
#define DTG_STR(x) DTG_STR2(x)
#define MX_ENTRY(BM, BN, WM, WN, ST, FA, FB)                                                                    \
    {BM, BN, mx_bke<FA, FB>(), ST, 32, WM, WN, FA, FB,                                                         \
     ((BM / WM / 32) * (BN / WN / 32) * 4 <= 16 ? kMaxMxSplits : 1), 64 * WM * WN, mx_lds(BM, BN, ST, FA, FB), \
     &launch_mx<BM, BN, WM, WN, ST, FA, FB>,                                                                   \
     "gemm_mx_kernel<" DTG_STR(BM) "," DTG_STR(BN) "," DTG_STR(WM) "," DTG_STR(WN) "," DTG_STR(ST) ","        \
     DTG_STR(FA) "," DTG_STR(FB) ">", kMxKernelTile}
}  // namespace
}  // namespace dtg
