// Single-instruction probe kernels: test infrastructure, built into
// tests/gpu_probes/libgemm_probe.so by tests/gpu_probes/build.py (never part
// of the GEMM library).  They pin the lane layouts the kernels assume.
//
// probe_mfma runs ONE matrix instruction in one wavefront with the operand and
// result lane layouts the tile kernel assumes, on a small A (rows x k) and
// B (k x cols) given in row-major order, and writes the rows x cols result in
// row-major order.  A test with exact integer inputs then pins those layouts
// (the single-instruction kernel of "DCU K100 节点初探", section 5.4, used as a
// layout check).
//
// probe_lds_dma records where the direct global -> LDS loads put each lane's
// 16 bytes, and that the buffer form writes zeros for offsets past the
// descriptor's range.
//
// probe_lds_read_tr fills 1024 bytes of LDS from `in` and has every lane run one
// transposing 64-bit LDS read at byte address 8 * lane; the 4 halfwords each
// lane receives are written to out[4 * lane + 0..3].  It reports the lane
// mapping of that instruction; every address is inside the 1024 bytes.
//
// probe_mfma_rate times back-to-back independent matrix instructions (no
// memory access in the loop) over the whole chip: the throughput a kernel's
// instruction stream can reach, against which the kernels' fractions of the
// nominal peaks can be read.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

template <int MF, bool BF16>
__global__ __launch_bounds__(64) void probe_mfma_kernel(const uint16_t* A, const uint16_t* B, float* D) {
    constexpr int KI = (MF == 16) ? 32 : 16;
    const int l = threadIdx.x;
    const int rc = l % MF, g = l / MF;
    uint16_t a[8], b[8];
    for (int t = 0; t < 8; ++t) {
        a[t] = A[rc * KI + 8 * g + t];       // A row rc, k = 8g + t
        b[t] = B[(8 * g + t) * MF + rc];     // B column rc, k = 8g + t
    }
    u32x4 av, bv;
    for (int d = 0; d < 4; ++d) {
        av[d] = a[2 * d] | (static_cast<uint32_t>(a[2 * d + 1]) << 16);
        bv[d] = b[2 * d] | (static_cast<uint32_t>(b[2 * d + 1]) << 16);
    }
    if constexpr (MF == 16) {
        f32x4 c = {0, 0, 0, 0};
        if constexpr (BF16)
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                        __builtin_bit_cast(bf16x8, bv), c, 0, 0, 0);
        else
            c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, av),
                                                       __builtin_bit_cast(f16x8, bv), c, 0, 0, 0);
        for (int r = 0; r < 4; ++r) D[(4 * g + r) * 16 + rc] = c[r];
    } else {
        f32x16 c = {};
        if constexpr (BF16)
            c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                        __builtin_bit_cast(bf16x8, bv), c, 0, 0, 0);
        else
            c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, av),
                                                       __builtin_bit_cast(f16x8, bv), c, 0, 0, 0);
        for (int r = 0; r < 16; ++r) D[(8 * (r / 4) + 4 * g + (r % 4)) * 32 + rc] = c[r];
    }
}

// One integer matrix instruction (v_mfma_i32_16x16x64_i8 or 32x32x32_i8) in
// one wavefront with the lane layouts the int8 tile kernel assumes: lane l
// holds row / column l % MF and the 16 consecutive k 16 (l / MF) .. + 15 of A
// (rows x k, row-major int8) and of B (k x cols, row-major int8); the int32
// result goes out in row-major order with the floating-point instructions'
// result layout.
template <int MF>
__global__ __launch_bounds__(64) void probe_mfma_i8_kernel(const int8_t* A, const int8_t* B, int* D) {
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    typedef int i32x16 __attribute__((ext_vector_type(16)));
    constexpr int KI = (MF == 16) ? 64 : 32;
    const int l = threadIdx.x;
    const int rc = l % MF, g = l / MF;
    uint32_t a[4] = {0, 0, 0, 0}, b[4] = {0, 0, 0, 0};
    for (int t = 0; t < 16; ++t) {
        a[t / 4] |= static_cast<uint32_t>(static_cast<uint8_t>(A[rc * KI + 16 * g + t])) << (8 * (t % 4));
        b[t / 4] |= static_cast<uint32_t>(static_cast<uint8_t>(B[(16 * g + t) * MF + rc])) << (8 * (t % 4));
    }
    const i32x4 av = {static_cast<int>(a[0]), static_cast<int>(a[1]), static_cast<int>(a[2]), static_cast<int>(a[3])};
    const i32x4 bv = {static_cast<int>(b[0]), static_cast<int>(b[1]), static_cast<int>(b[2]), static_cast<int>(b[3])};
    if constexpr (MF == 16) {
        i32x4 c = {0, 0, 0, 0};
        c = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, c, 0, 0, 0);
        for (int r = 0; r < 4; ++r) D[(4 * g + r) * 16 + rc] = c[r];
    } else {
        i32x16 c = {};
        c = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, bv, c, 0, 0, 0);
        for (int r = 0; r < 16; ++r) D[(8 * (r / 4) + 4 * g + (r % 4)) * 32 + rc] = c[r];
    }
}

// One scaled matrix instruction (v_mfma_scale_f32_{16x16x128,32x32x64}_f8f6f4)
// on raw per-lane registers: lane l supplies a[8l..8l+7] and b[8l..8l+7] as
// its A and B operand registers (only the first 4 dwords are used for the
// 4-bit format, the first 6 for the 6-bit ones), sa[l] and sb[l] as its
// scale registers, of which the byte
// selected by OSA / OSB is the scale; the accumulator starts at zero and
// lane l's result registers go to out[R l .. R l + R - 1] (R = 4 or 16).
// Format codes FA / FB: 0 E4M3, 1 E5M2, 2 E2M3, 3 E3M2, 4 E2M1.
template <int MF, int FA, int FB, int OSA, int OSB>
__global__ __launch_bounds__(64) void probe_mfma_scaled_kernel(const uint32_t* a, const uint32_t* b,
                                                               const uint32_t* sa, const uint32_t* sb, float* out) {
    typedef int i32x8 __attribute__((ext_vector_type(8)));
    const int l = threadIdx.x;
    i32x8 av, bv;
    for (int d = 0; d < 8; ++d) {
        av[d] = static_cast<int>(a[8 * l + d]);
        bv[d] = static_cast<int>(b[8 * l + d]);
    }
    const int s_a = static_cast<int>(sa[l]), s_b = static_cast<int>(sb[l]);
    if constexpr (MF == 16) {
        f32x4 c = {0, 0, 0, 0};
        c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, FA, FB, OSA, s_a, OSB, s_b);
        for (int r = 0; r < 4; ++r) out[4 * l + r] = c[r];
    } else {
        f32x16 c = {};
        c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, FA, FB, OSA, s_a, OSB, s_b);
        for (int r = 0; r < 16; ++r) out[16 * l + r] = c[r];
    }
}

__global__ __launch_bounds__(64) void probe_lds_read_tr_kernel(const uint16_t* in, uint16_t* out) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[512];
    const int l = threadIdx.x;
    for (int i = l; i < 512; i += 64) lds[i] = in[i];
    __syncthreads();
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds + 4 * l));
    for (int i = 0; i < 4; ++i) out[4 * l + i] = static_cast<uint16_t>(v[i]);
}

// 64 lanes, one 16-byte load each, straight into LDS.  LDS halfwords
// [0, 512): buffer loads through a descriptor covering the first num_records
// bytes of `in`; lane l < 48 fetches 16-byte chunk (7 l) mod 64, lanes 48..55
// use offset 0x80000000 and lanes 56..63 offsets num_records + 16 (l - 56),
// both past num_records (the descriptor's range check must return zeros).
// LDS halfwords [512, 1024): plain global loads, lane l fetches chunk (5 l)
// mod 64.  LDS starts filled with 0xFFFF; all of it is copied to out.
// `in` must hold at least num_records + 128 bytes and num_records >= 1024.
__global__ __launch_bounds__(64) void probe_lds_dma_kernel(const uint16_t* in, uint16_t* out,
                                                           int num_records) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[1024];
    const int l = threadIdx.x;
    for (int i = l; i < 1024; i += 64) lds[i] = 0xFFFF;
    __syncthreads();
    __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)in, 0, num_records, 0x00020000);
    const unsigned voff = (l < 48) ? ((l * 7) % 64) * 16
                        : (l < 56) ? 0x80000000u : static_cast<unsigned>(num_records + 16 * (l - 56));
    typedef __attribute__((address_space(3))) void lds_void;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, 0, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)(in + 8 * ((l * 5) % 64)), (lds_void*)(lds + 512), 16, 0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int i = l; i < 1024; i += 64) out[i] = lds[i];
}

// Rate kernels: NACC independent accumulators per wave, `iters` rounds; each
// thread writes one sum (so nothing is optimized away) to out[global id].
typedef int i32x8 __attribute__((ext_vector_type(8)));

template <int FX, int FY, int NACC>
__global__ __launch_bounds__(512) void rate_scaled_kernel(float* out, int iters) {
    i32x8 x, y;
    for (int i = 0; i < 8; ++i) {
        x[i] = static_cast<int>((threadIdx.x * 7u + i) & 0x11111111u);
        y[i] = static_cast<int>((threadIdx.x * 3u + i) & 0x22222222u);
    }
    f32x16 acc[NACC];
    for (int a = 0; a < NACC; ++a)
        for (int r = 0; r < 16; ++r) acc[a][r] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int a = 0; a < NACC; ++a)
            acc[a] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, acc[a], FX, FY, 0, 127, 0, 127);
    }
    float sum = 0.0f;
    for (int a = 0; a < NACC; ++a)
        for (int r = 0; r < 16; ++r) sum += acc[a][r];
    out[blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

template <int NACC>
__global__ __launch_bounds__(512) void rate_bf16_kernel(float* out, int iters) {
    bf16x8 x, y;
    for (int i = 0; i < 8; ++i) {
        x[i] = static_cast<__bf16>(static_cast<float>((threadIdx.x + i) & 3));
        y[i] = static_cast<__bf16>(static_cast<float>(i & 1));
    }
    f32x4 acc[NACC];
    for (int a = 0; a < NACC; ++a)
        for (int r = 0; r < 4; ++r) acc[a][r] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int a = 0; a < NACC; ++a) acc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, acc[a], 0, 0, 0);
    }
    float sum = 0.0f;
    for (int a = 0; a < NACC; ++a)
        for (int r = 0; r < 4; ++r) sum += acc[a][r];
    out[blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

}  // namespace

extern "C" {

// kind: 0 bf16 16x16x32 (8 accumulators), 1 E4M3, 2 E2M1, 3 E2M3 (FP6),
// 4 E4M3 x E2M1 (scaled 32x32x64, 4 accumulators).  grid workgroups of
// 64 * waves threads (waves 4 or 8), `iters` rounds; out: device floats,
// at least grid * 64 * waves.  *ms gets the timed launch's duration (one
// untimed launch first); *flop the flops it performed.  Returns a hipError_t.
int probe_mfma_rate(int kind, int grid, int waves, int iters, float* out, void* stream, float* ms, double* flop) {
    if (grid < 1 || (waves != 4 && waves != 8) || iters < 1 || kind < 0 || kind > 4 || !out || !ms || !flop)
        return static_cast<int>(hipErrorInvalidValue);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 g(static_cast<unsigned>(grid)), b(static_cast<unsigned>(64 * waves));
    auto launch = [&](int n) {
        switch (kind) {
            case 0: hipLaunchKernelGGL(rate_bf16_kernel<8>, g, b, 0, s, out, n); break;
            case 1: hipLaunchKernelGGL((rate_scaled_kernel<0, 0, 4>), g, b, 0, s, out, n); break;
            case 2: hipLaunchKernelGGL((rate_scaled_kernel<4, 4, 4>), g, b, 0, s, out, n); break;
            case 3: hipLaunchKernelGGL((rate_scaled_kernel<2, 2, 4>), g, b, 0, s, out, n); break;
            default: hipLaunchKernelGGL((rate_scaled_kernel<0, 4, 4>), g, b, 0, s, out, n); break;
        }
    };
    hipEvent_t e0, e1;
    hipError_t err = hipEventCreate(&e0);
    if (err != hipSuccess) return static_cast<int>(err);
    err = hipEventCreate(&e1);
    if (err != hipSuccess) {
        hipEventDestroy(e0);
        return static_cast<int>(err);
    }
    launch(iters);
    hipEventRecord(e0, s);
    launch(iters);
    hipEventRecord(e1, s);
    err = hipEventSynchronize(e1);
    if (err == hipSuccess) err = hipEventElapsedTime(ms, e0, e1);
    if (err == hipSuccess) err = hipGetLastError();
    hipEventDestroy(e0);
    hipEventDestroy(e1);
    const double per = kind == 0 ? 8.0 * 2 * 16 * 16 * 32 : 4.0 * 2 * 32 * 32 * 64;
    *flop = per * static_cast<double>(grid) * waves * iters;
    return static_cast<int>(err);
}

// in: >= num_records + 128 bytes, out: 1024 halfwords (device pointers).
int probe_lds_dma(const uint16_t* in, uint16_t* out, int num_records, void* stream) {
    if (num_records < 1024) return static_cast<int>(hipErrorInvalidValue);
    hipLaunchKernelGGL(probe_lds_dma_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), in, out,
                       num_records);
    return static_cast<int>(hipGetLastError());
}

// mf: 16 (A 16x32, B 32x16, D 16x16) or 32 (A 32x16, B 16x32, D 32x32).
// dtype: 0 fp16, 1 bf16.  All pointers are device pointers.  Returns a
// hipError_t value (0 = success); the kernel runs on `stream`.
int probe_mfma(int mf, int dtype, const uint16_t* A, const uint16_t* B, float* D, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (mf == 16 && dtype == 1) hipLaunchKernelGGL((probe_mfma_kernel<16, true>), dim3(1), dim3(64), 0, s, A, B, D);
    else if (mf == 16 && dtype == 0) hipLaunchKernelGGL((probe_mfma_kernel<16, false>), dim3(1), dim3(64), 0, s, A, B, D);
    else if (mf == 32 && dtype == 1) hipLaunchKernelGGL((probe_mfma_kernel<32, true>), dim3(1), dim3(64), 0, s, A, B, D);
    else if (mf == 32 && dtype == 0) hipLaunchKernelGGL((probe_mfma_kernel<32, false>), dim3(1), dim3(64), 0, s, A, B, D);
    else return static_cast<int>(hipErrorInvalidValue);
    return static_cast<int>(hipGetLastError());
}

// Scaled matrix instruction on raw lane registers (probe_mfma_scaled_kernel).
// mf 16 or 32; (fa, fb, osa, osb) one of the instantiated combinations below.
// a, b: 512 dwords; sa, sb: 64 dwords; out: 64 * (mf == 16 ? 4 : 16) floats
// (device pointers).  Returns a hipError_t value.
int probe_mfma_scaled(int mf, int fa, int fb, int osa, int osb, const uint32_t* a, const uint32_t* b,
                      const uint32_t* sa, const uint32_t* sb, float* out, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
#define PROBE_SC(MF_, FA_, FB_, OA_, OB_)                                                                  \
    if (mf == MF_ && fa == FA_ && fb == FB_ && osa == OA_ && osb == OB_) {                                \
        hipLaunchKernelGGL((probe_mfma_scaled_kernel<MF_, FA_, FB_, OA_, OB_>), dim3(1), dim3(64), 0, s, a, b, \
                           sa, sb, out);                                                                   \
        return static_cast<int>(hipGetLastError());                                                        \
    }
#define PROBE_SC_MF(MF_)                                                                     \
    PROBE_SC(MF_, 0, 0, 0, 0) PROBE_SC(MF_, 1, 1, 0, 0) PROBE_SC(MF_, 4, 4, 0, 0)            \
    PROBE_SC(MF_, 0, 1, 0, 0) PROBE_SC(MF_, 0, 0, 1, 2) PROBE_SC(MF_, 0, 0, 3, 1)            \
    PROBE_SC(MF_, 4, 4, 2, 3) PROBE_SC(MF_, 2, 2, 0, 0) PROBE_SC(MF_, 3, 3, 0, 0)            \
    PROBE_SC(MF_, 2, 3, 0, 0) PROBE_SC(MF_, 0, 4, 0, 0) PROBE_SC(MF_, 4, 0, 0, 0)            \
    PROBE_SC(MF_, 2, 4, 0, 0) PROBE_SC(MF_, 4, 3, 0, 0) PROBE_SC(MF_, 1, 2, 0, 0)
    PROBE_SC_MF(16)
    PROBE_SC_MF(32)
#undef PROBE_SC_MF
#undef PROBE_SC
    return static_cast<int>(hipErrorInvalidValue);
}

// mf: 16 (A 16x64, B 64x16, D 16x16) or 32 (A 32x32, B 32x32, D 32x32); int8
// A and B, int32 D (device pointers).  Returns a hipError_t value.
int probe_mfma_i8(int mf, const int8_t* A, const int8_t* B, int* D, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (mf == 16) hipLaunchKernelGGL(probe_mfma_i8_kernel<16>, dim3(1), dim3(64), 0, s, A, B, D);
    else if (mf == 32) hipLaunchKernelGGL(probe_mfma_i8_kernel<32>, dim3(1), dim3(64), 0, s, A, B, D);
    else return static_cast<int>(hipErrorInvalidValue);
    return static_cast<int>(hipGetLastError());
}

// in: 512 halfwords, out: 256 halfwords (device pointers).
int probe_lds_read_tr(const uint16_t* in, uint16_t* out, void* stream) {
    hipLaunchKernelGGL(probe_lds_read_tr_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), in, out);
    return static_cast<int>(hipGetLastError());
}

}  // extern "C"
