// Block-scaled (MX) GEMM for every pair of element formats, register-direct:
// D = A x B (+ C) with A and B of FP8 (E4M3, E5M2), FP6 (E2M3, E3M2) or FP4
// (E2M1) elements, each 32 consecutive k sharing one E8M0 scale, on gfx950's
// scaled matrix instruction v_mfma_scale_f32_32x32x64_f8f6f4, which takes the
// two operands' formats separately ("Tuning Triton kernels", section 6: the
// gfx950 instruction set adds a scaled MFMA as the way to the microscaled
// types).  The LDS-staged kernel of gemm_mx.hip runs the pairs of one width
// (8-bit with 8-bit, E2M1 with E2M1); this one runs the rest: FP6 elements
// (24 bytes per 32 k, which the 128-byte staging rows of that kernel do not
// divide) and operands of different widths.
//
// Each lane loads its operand registers straight from memory: the
// instruction's lane l = r + 32 g holds row (column) r and, in its operand
// registers,
//   - 8-bit: k = 16 g .. 16 g + 15 in bytes 0-15, k = 32 + 16 g .. + 15 in
//     bytes 16-31 (two 16-byte loads);
//   - 6-bit: k = 32 g .. 32 g + 31 as one little-endian bit string in bytes
//     0-23 (a 16-byte and an 8-byte load: the 24 bytes the row stores them in);
//   - 4-bit: k = 32 g .. 32 g + 31, two per byte, in bytes 0-15;
// and the scale of row r and 32-k block g in byte 0 of its scale register
// (opsel 0) - the layouts the probe tests pin.  A workgroup of 2 x 2 waves
// computes a 128 x 128 tile, each wave 64 x 64 (2 x 2 instructions per 64 k),
// with the next 64 k loaded while the current ones are contracted.  Rows past
// M or N and k past K are loaded from offsets past the buffer's range, which
// returns zeros (and scale 0, i.e. 2^-127, never a NaN code); steps past K
// add exact zeros.
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

typedef int i32x8 __attribute__((ext_vector_type(8)));

template <int F>
constexpr int elem_bits() { return F <= kMxE5M2 ? 8 : (F == kMxE2M1 ? 4 : 6); }

// Operand registers of lane group g for the 64 k starting at k0, of a row at
// byte offset row_off of the buffer (masked rows pass ok = false).
template <int BITS>
__device__ __forceinline__ i32x8 load_operand(__amdgpu_buffer_rsrc_t r, uint32_t row_off, bool ok, int k0, int K,
                                              int g) {
    i32x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
    if constexpr (BITS == 8) {
        const int ka = k0 + 16 * g, kb = k0 + 32 + 16 * g;
        const uint32_t oa = (ok && ka < K) ? row_off + static_cast<uint32_t>(ka) : kOOB;
        const uint32_t ob = (ok && kb < K) ? row_off + static_cast<uint32_t>(kb) : kOOB;
        const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, oa, 0, 0));
        const u32x4 b = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, ob, 0, 0));
        v = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
    } else {
        const int kk = k0 + 32 * g;
        const uint32_t o = (ok && kk < K) ? row_off + static_cast<uint32_t>(kk * BITS / 8) : kOOB;
        const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, 0));
        v[0] = (int)a[0];
        v[1] = (int)a[1];
        v[2] = (int)a[2];
        v[3] = (int)a[3];
        if constexpr (BITS == 6) {
            const u32x2 b = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, o + 16u, 0, 0));
            v[4] = (int)b[0];
            v[5] = (int)b[1];
        }
    }
    return v;
}

// Four fp32 values of one output row, + C (same type as D), rounded and stored.
__device__ __forceinline__ void store_run(const MxArgs& p, int row, int col, int n_ok, const float (&v)[4]) {
    const int64_t dofs = static_cast<int64_t>(row) * p.ldd + col;
    const int64_t cofs = static_cast<int64_t>(row) * p.ldc + col;
    if (p.out == 2) {
        float* d = static_cast<float*>(p.D) + dofs;
        const float* c = p.has_c ? static_cast<const float*>(p.C) + cofs : nullptr;
        for (int e = 0; e < 4; ++e)
            if (e < n_ok) d[e] = c ? v[e] + c[e] : v[e];
        return;
    }
    uint16_t* d = static_cast<uint16_t*>(p.D) + dofs;
    const uint16_t* c = p.has_c ? static_cast<const uint16_t*>(p.C) + cofs : nullptr;
    for (int e = 0; e < 4; ++e) {
        if (e >= n_ok) break;
        if (p.out == 1) d[e] = narrow<true>(c ? v[e] + widen<true>(c[e]) : v[e]);
        else d[e] = narrow<false>(c ? v[e] + widen<false>(c[e]) : v[e]);
    }
}

template <int FA, int FB>
__global__ __launch_bounds__(256) void gemm_mx_direct_kernel(MxArgs p) {
    constexpr int BA = elem_bits<FA>(), BB = elem_bits<FB>();
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    int pid_m, pid_n;
    tile_of_workgroup<int>(blockIdx.x, p.num_pid_m, p.num_pid_n, p.group_m, p.xcds, &pid_m, &pid_n);
    const int M = p.M, N = p.N, K = p.K;
    const int m0 = pid_m * 128, n0 = pid_n * 128;
    const int r = lane & 31, g = lane >> 5;

    // Buffers start at the tile's first row (32-bit offsets cover its 128
    // rows plus K's bytes: the planner bounds the row strides).
    const int64_t arow_bytes = static_cast<int64_t>(K) * BA / 8, brow_bytes = static_cast<int64_t>(K) * BB / 8;
    const int nblk = (K + 31) / 32;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(p.A + static_cast<int64_t>(m0) * p.lda), 0,
        clamp_records(static_cast<int64_t>(M - 1 - m0) * p.lda + arow_bytes), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(p.B + static_cast<int64_t>(n0) * p.ldb), 0,
        clamp_records(static_cast<int64_t>(N - 1 - n0) * p.ldb + brow_bytes), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(p.SA + static_cast<int64_t>(m0) * p.ldsa), 0,
        clamp_records(static_cast<int64_t>(M - 1 - m0) * p.ldsa + nblk), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(p.SB + static_cast<int64_t>(n0) * p.ldsb), 0,
        clamp_records(static_cast<int64_t>(N - 1 - n0) * p.ldsb + nblk), kRsrcWord3);

    // this lane's rows: A rows wm*64 + 32 i + r, B rows (columns) wn*64 + 32 j + r
    uint32_t a_off[2], b_off[2], sa_off[2], sb_off[2];
    bool a_ok[2], b_ok[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int ra_row = wm * 64 + 32 * i + r, rb_row = wn * 64 + 32 * i + r;
        a_ok[i] = m0 + ra_row < M;
        b_ok[i] = n0 + rb_row < N;
        a_off[i] = static_cast<uint32_t>(static_cast<int64_t>(ra_row) * p.lda);
        b_off[i] = static_cast<uint32_t>(static_cast<int64_t>(rb_row) * p.ldb);
        sa_off[i] = static_cast<uint32_t>(static_cast<int64_t>(ra_row) * p.ldsa);
        sb_off[i] = static_cast<uint32_t>(static_cast<int64_t>(rb_row) * p.ldsb);
    }

    i32x8 fa[2][2], fb[2][2];
    int sa[2][2], sb[2][2];
    auto load = [&](auto slot_tag, int kt) {
        constexpr int S = decltype(slot_tag)::value;
        const int k0 = kt * 64;
        const int blk = kt * 2 + g;
        const bool kin = k0 + 32 * g < K;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            fa[S][i] = load_operand<BA>(ra, a_off[i], a_ok[i], k0, K, g);
            fb[S][i] = load_operand<BB>(rb, b_off[i], b_ok[i], k0, K, g);
            sa[S][i] = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b8(
                rsa, (a_ok[i] && kin) ? sa_off[i] + static_cast<uint32_t>(blk) : kOOB, 0, 0));
            sb[S][i] = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b8(
                rsb, (b_ok[i] && kin) ? sb_off[i] + static_cast<uint32_t>(blk) : kOOB, 0, 0));
        }
    };
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    // B's fragment is the instruction's first operand, so each accumulator
    // holds the transposed block: lane (r, g) owns row r of the A fragment and
    // runs of 4 consecutive columns.
    auto contract = [&](auto slot_tag) {
        constexpr int S = decltype(slot_tag)::value;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[S][j], fa[S][i], acc[i][j], FB, FA,
                                                                              0, sb[S][j], 0, sa[S][i]);
    };
    const int nkt = (K + 63) / 64;
    if (nkt > 0) load(std::integral_constant<int, 0>{}, 0);
    for (int kt = 0; kt < nkt; kt += 2) {
        load(std::integral_constant<int, 1>{}, kt + 1);     // past K: zeros, scale 2^-127
        contract(std::integral_constant<int, 0>{});
        load(std::integral_constant<int, 0>{}, kt + 2);
        contract(std::integral_constant<int, 1>{});
    }

    // Element e of acc[i][j] (q = e / 4) is row m0 + wm*64 + 32 i + r,
    // column n0 + wn*64 + 32 j + 8 q + 4 g + e % 4.
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = m0 + wm * 64 + 32 * i + r;
        if (row >= M) continue;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int col = n0 + wn * 64 + 32 * j + 8 * q + 4 * g;
                if (col >= N) continue;
                const float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                    acc[i][j][4 * q + 3]};
                store_run(p, row, col, N - col, v);
            }
    }
}

template <int FA, int FB>
hipError_t launch_direct(const MxArgs& a, int64_t grid, hipStream_t stream) {
    hipLaunchKernelGGL((gemm_mx_direct_kernel<FA, FB>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

#define DTG_STR2(x) #x
#define DTG_STR(x) DTG_STR2(x)
#define DIRECT_ENTRY(FA, FB)                                                                               \
    {128, 128, 64, 1, 32, 2, 2, FA, FB, 1, 256, 0, &launch_direct<FA, FB>,                                 \
     "gemm_mx_direct_kernel<" DTG_STR(FA) "," DTG_STR(FB) ">", kMxKernelDirect}
#define DIRECT_ROW(FA) DIRECT_ENTRY(FA, 0), DIRECT_ENTRY(FA, 1), DIRECT_ENTRY(FA, 2), DIRECT_ENTRY(FA, 3), \
                       DIRECT_ENTRY(FA, 4)

const MxEntry kDirectTable[] = {DIRECT_ROW(0), DIRECT_ROW(1), DIRECT_ROW(2), DIRECT_ROW(3), DIRECT_ROW(4)};

}  // namespace

const MxEntry* mx_direct_kernel_table(int* count) {
    *count = static_cast<int>(sizeof(kDirectTable) / sizeof(kDirectTable[0]));
    return kDirectTable;
}

}  // namespace dtg
