// Single-instruction probe kernels (test support, built into libgemm_probe.so).
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

// One scaled matrix instruction (v_mfma_scale_f32_{16x16x128,32x32x64}_f8f6f4)
// on raw per-lane registers: lane l supplies a[8l..8l+7] and b[8l..8l+7] as
// its A and B operand registers (only the first 4 dwords are used for the
// 4-bit format), sa[l] and sb[l] as its scale registers, of which the byte
// selected by OSA / OSB is the scale; the accumulator starts at zero and
// lane l's result registers go to out[R l .. R l + R - 1] (R = 4 or 16).
// Format codes FA / FB: 0 E4M3, 1 E5M2, 4 E2M1.
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

// Streaming reads of `bytes` bytes (a multiple of 16) for a read-bandwidth
// reference: every thread walks the buffer in a grid-stride loop of 16-byte
// loads, U loads in flight per thread; the XOR of all loaded words goes to
// out[blockIdx.x] so the loads are not dead.  Every address is < bytes.
template <int U>
__global__ __launch_bounds__(256) void probe_stream_read_kernel(const u32x4* in, uint64_t n16, uint32_t* out) {
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * 256;
    uint64_t i = static_cast<uint64_t>(blockIdx.x) * 256 + threadIdx.x;
    u32x4 acc = {0, 0, 0, 0};
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(in + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u];
    }
    for (; i < n16; i += stride) acc ^= in[i];
    uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
    __shared__ uint32_t red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

// Band reads: the buffer is `rows` rows of `row_bytes`; workgroup w reads the
// column band [band * (w % nbands), band * (w % nbands + 1)) of rows
// [rows_per * (w / nbands), rows_per * (w / nbands + 1)), 16 bytes per lane,
// each wave instruction covering 1024 / band consecutive rows.  Reports the
// bandwidth of a column-slab access pattern.  Every address is inside
// rows * row_bytes (band divides row_bytes, rows_per divides rows).
__global__ __launch_bounds__(256) void probe_band_read_kernel(const uint8_t* in, int rows, int row_bytes,
                                                              int band, int rows_per, uint32_t* out) {
    const int nbands = row_bytes / band;
    const int b = blockIdx.x % nbands, slice = blockIdx.x / nbands;
    const int lanes_per_row = band / 16;
    const int rows_per_iter = 256 / lanes_per_row;
    const int t = threadIdx.x;
    const int r_in = t / lanes_per_row, c = (t % lanes_per_row) * 16;
    u32x4 acc = {0, 0, 0, 0};
    const int r0 = slice * rows_per;
    for (int r = r0 + r_in; r < r0 + rows_per; r += 4 * rows_per_iter) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int rr = r + u * rows_per_iter;
            v[u] = rr < r0 + rows_per
                       ? *reinterpret_cast<const u32x4*>(in + static_cast<int64_t>(rr) * row_bytes + b * band + c)
                       : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) acc ^= v[u];
    }
    uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
    __shared__ uint32_t red[4];
    if ((t & 63) == 0) red[t >> 6] = x;
    __syncthreads();
    if (t == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

// Band reads straight into LDS: same geometry as probe_band_read_kernel, but
// each wave issues 16-byte buffer loads into an 8-slot LDS ring of its own
// (1 KB per slot), keeping at most 7 loads in flight before reusing a slot.
// Nothing reads the LDS; out gets one word per workgroup.  Every global offset
// is < rows * row_bytes; LDS use is 4 waves x 8 KB.
__global__ __launch_bounds__(256) void probe_band_read_lds_kernel(const uint8_t* in, int rows, int row_bytes,
                                                                  int band, int rows_per, uint32_t* out) {
    __shared__ __attribute__((aligned(1024))) uint8_t ring[4 * 8 * 1024];
    const int nbands = row_bytes / band;
    const int b = blockIdx.x % nbands, slice = blockIdx.x / nbands;
    const int lanes_per_row = band / 16;
    const int rows_per_inst = 64 / lanes_per_row;             // rows one wave instruction covers
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r_in = lane / lanes_per_row, c = (lane % lanes_per_row) * 16;
    const int r0 = slice * rows_per;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(in), 0, 0x7ffffff0, 0x00020000);
    typedef __attribute__((address_space(3))) void lds_void;
    int it = 0;
    for (int r = r0 + wave * rows_per_inst; r < r0 + rows_per; r += 4 * rows_per_inst, ++it) {
        const int rr = r + r_in;
        const int64_t off = static_cast<int64_t>(rr) * row_bytes + b * band + c;
        // offsets within the 2 GiB descriptor range (the probe uses < 2 GiB)
        const uint32_t v = rr < r0 + rows_per ? static_cast<uint32_t>(off) : 0x80000000u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(ring + (wave * 8 + (it & 7)) * 1024), 16, v,
                                                 0, 0, 0);
        __builtin_amdgcn_s_waitcnt((7 & 15) | (7 << 4) | (15 << 8));        // vmcnt(7)
    }
    __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8));            // vmcnt(0)
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = ring[blockIdx.x & 1023];
}

// LDS read patterns, one kernel per pattern so counters separate them.  Four
// waves, 64 KiB of LDS; wave w works in its own 8 KiB window at 8192 w + the
// offsets below (all < 8192).  Each wave runs `iters` reads and XORs the data
// into out[threadIdx.x + 256 blockIdx.x].
//  0: 16-byte reads, lane l at 16 l (+ 1 KiB per iteration mod 4 KiB)
//  1: 16-byte reads, operand layout of A (rows of 128 bytes, lane l: row
//     l % 16 + 16 (it % 4), logical chunk l / 16 + 4 (it % 2), XOR swizzle)
//  2: as 1 without the swizzle
//  3: transposing 8-byte reads, operand layout of B (rows of 512 bytes, lane
//     group g = l / 16, j = l % 16: row 8 g + 4 (it % 2) + j / 4, columns
//     16 (it / 2 % 16) + 4 (j % 4), chunk-pair XOR swizzle)
//  4: as 3 without the swizzle
//  5: transposing 8-byte reads, lane l at 8 l
//  6: 8-byte reads, lane l at 8 l
template <int P>
__global__ __launch_bounds__(256) void probe_lds_pattern_kernel(uint32_t* out, int iters) {
    __shared__ __attribute__((aligned(1024))) uint32_t lds[16384];
    for (int i = threadIdx.x; i < 16384; i += 256) lds[i] = i * 2654435761u;
    __syncthreads();
    const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
                              (const __attribute__((address_space(3))) uint32_t*)lds)) + w * 8192;
    u32x4 acc = {0, 0, 0, 0};
    for (int it = 0; it < iters; ++it) {
        uint32_t a;
        if constexpr (P == 0) {
            a = 16 * l + 1024 * (it & 3);
        } else if constexpr (P == 1 || P == 2) {
            const int row = (l & 15) + 16 * (it & 3), chunk = (l >> 4) + 4 * ((it >> 2) & 1);
            const int sw = (P == 1) ? ((row & 7) ^ ((row >> 3) & 1)) : 0;
            a = row * 128 + ((chunk ^ sw) * 16);
        } else if constexpr (P == 3 || P == 4) {
            const int g = l >> 4, j = l & 15, h = it & 1;
            const int r = 8 * g + 4 * h + (j >> 2);
            const int nb = 16 * ((it >> 1) & 15);
            const int f = (P == 3) ? 2 * ((r & 3) | (((r >> 3) & 1) << 2)) : 0;
            a = r * 512 + ((((nb >> 3) ^ f)) << 4) + 8 * (j & 3);
        } else {
            a = 8 * l + 512 * (it & 7);
        }
        if constexpr (P <= 2) {
            u32x4 v;
            asm volatile("ds_read_b128 %0, %1\n s_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(base + a));
            acc ^= v;
        } else if constexpr (P <= 5) {
            i16x4 v;
            asm volatile("ds_read_b64_tr_b16 %0, %1\n s_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(base + a));
            acc[0] ^= __builtin_bit_cast(uint64_t, v) & 0xffffffffu;
        } else {
            i16x4 v;
            asm volatile("ds_read_b64 %0, %1\n s_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(base + a));
            acc[0] ^= __builtin_bit_cast(uint64_t, v) & 0xffffffffu;
        }
    }
    out[threadIdx.x + 256 * blockIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// Lane-pair LDS probe: every lane reads 16 bytes at 16 l (no conflicts),
// except lane j, which reads at 16 i + 4096 (same banks as lane i under any
// bank period dividing 4096).  The bank-conflict counter of a dispatch then
// tells whether lanes i and j are served in the same LDS cycle.  One wave per
// workgroup, 8 KiB of LDS; all addresses < 8192.
__global__ __launch_bounds__(64) void probe_lds_pair_kernel(uint32_t* out, int i, int j, int iters) {
    __shared__ __attribute__((aligned(1024))) uint32_t lds[2048];
    for (int k = threadIdx.x; k < 2048; k += 64) lds[k] = k;
    __syncthreads();
    const int l = threadIdx.x;
    const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (const __attribute__((address_space(3))) uint32_t*)lds));
    const uint32_t a = base + ((l == j) ? 16 * i + 4096 : 16 * l);
    u32x4 acc = {0, 0, 0, 0};
    for (int it = 0; it < iters; ++it) {
        u32x4 v;
        asm volatile("ds_read_b128 %0, %1\n s_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a));
        acc ^= v;
    }
    out[threadIdx.x + 64 * blockIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// Swizzle-candidate probe: the 16-byte operand reads of an A tile with
// 128-byte rows, physical chunk = logical chunk ^ table[row % 16].
// mf = 16: lane l reads row l % 16 + 16 (it % 4), logical chunk l / 16 + 4 (it / 4 % 2);
// mf = 32: lane l reads row l % 32 + 32 (it % 2), logical chunk l / 32 + 2 (it / 2 % 4).
// table (16 ints, each 0..7) is passed by value.  One wave per workgroup,
// 8 KiB of LDS; all addresses < 8192.
struct SwzTable { int v[16]; };
__global__ __launch_bounds__(64) void probe_lds_swizzle_kernel(uint32_t* out, SwzTable t, int mf, int iters) {
    __shared__ __attribute__((aligned(1024))) uint32_t lds[2048];
    for (int k = threadIdx.x; k < 2048; k += 64) lds[k] = k;
    __syncthreads();
    const int l = threadIdx.x;
    const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (const __attribute__((address_space(3))) uint32_t*)lds));
    u32x4 acc = {0, 0, 0, 0};
    for (int it = 0; it < iters; ++it) {
        int row, chunk;
        if (mf == 16) { row = (l & 15) + 16 * (it & 3); chunk = (l >> 4) + 4 * ((it >> 2) & 1); }
        else { row = (l & 31) + 32 * (it & 1); chunk = (l >> 5) + 2 * ((it >> 1) & 3); }
        const uint32_t a = base + row * 128 + ((chunk ^ (t.v[row & 15] & 7)) * 16);
        u32x4 v;
        asm volatile("ds_read_b128 %0, %1\n s_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a));
        acc ^= v;
    }
    out[threadIdx.x + 64 * blockIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}


// probe_mfma_rate: every wave of a workgroup of up to 8 waves issues `iters`
// rounds of matrix instructions on register operands (16x16x32: 32
// independent accumulators per round; 32x32x16: 8 accumulators, each used
// twice), 524288 flop per wave per round either way.  Wave 0 of each
// workgroup records the shader-clock count (s_memtime) and the 100 MHz
// constant-rate count (s_memrealtime) across its loop into clk[2 * block];
// the host derives the sustained matrix rate and the clock under that load.
template <int MF>
__global__ __launch_bounds__(512) void probe_mfma_rate_kernel(int iters, float* out, uint64_t* clk) {
    const int l = threadIdx.x & 63;
    u32x4 av, bv;
    for (int d = 0; d < 4; ++d) {
        av[d] = 0x3f803f80u ^ static_cast<uint32_t>((l * 7 + d) & 3);
        bv[d] = 0x3c003c00u ^ static_cast<uint32_t>((l * 5 + d) & 3);
    }
    const bf16x8 a = __builtin_bit_cast(bf16x8, av), b = __builtin_bit_cast(bf16x8, bv);
    const uint64_t t0 = __builtin_readcyclecounter();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    float sum = 0.0f;
    if constexpr (MF == 16) {
        f32x4 acc[32];
        for (int i = 0; i < 32; ++i) acc[i] = f32x4{static_cast<float>(i), 0, 0, 0};
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int i = 0; i < 32; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[i], 0, 0, 0);
        for (int i = 0; i < 32; ++i) sum += acc[i][0] + acc[i][3];
    } else {
        f32x16 acc[8];
        for (int i = 0; i < 8; ++i) { acc[i] = f32x16{}; acc[i][0] = static_cast<float>(i); }
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i & 7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i & 7], 0, 0, 0);
        for (int i = 0; i < 8; ++i) sum += acc[i][0] + acc[i][15];
    }
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    const uint64_t t1 = __builtin_readcyclecounter();
    out[blockIdx.x * blockDim.x + threadIdx.x] = sum;
    if (threadIdx.x == 0) {
        clk[2 * blockIdx.x] = t1 - t0;
        clk[2 * blockIdx.x + 1] = r1 - r0;
    }
}

// Register-only loop of scaled matrix instructions (v_mfma_scale_f32_*_f8f6f4,
// element format FMT for both operands, scale 1.0): the issue rate of the
// block-scaled contraction with no memory traffic.  Same clocks as
// probe_mfma_rate_kernel.
template <int MF, int FMT>
__global__ __launch_bounds__(512) void probe_mfma_scaled_rate_kernel(int iters, float* out, uint64_t* clk) {
    typedef int i32x8 __attribute__((ext_vector_type(8)));
    const int l = threadIdx.x & 63;
    i32x8 a, b;
    for (int d = 0; d < 8; ++d) {
        a[d] = static_cast<int>(0x38383838u ^ static_cast<uint32_t>((l * 7 + d) & 3));
        b[d] = static_cast<int>(0x30303030u ^ static_cast<uint32_t>((l * 5 + d) & 3));
    }
    const int sc = 0x7f7f7f7f;
    const uint64_t t0 = __builtin_readcyclecounter();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    float sum = 0.0f;
    if constexpr (MF == 16) {
        f32x4 acc[32];
        for (int i = 0; i < 32; ++i) acc[i] = f32x4{static_cast<float>(i), 0, 0, 0};
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int i = 0; i < 32; ++i)
                acc[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[i], FMT, FMT, 0, sc, 0, sc);
        for (int i = 0; i < 32; ++i) sum += acc[i][0] + acc[i][3];
    } else {
        f32x16 acc[8];
        for (int i = 0; i < 8; ++i) { acc[i] = f32x16{}; acc[i][0] = static_cast<float>(i); }
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                acc[i & 7] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i & 7], FMT, FMT, 0, sc, 0, sc);
        for (int i = 0; i < 8; ++i) sum += acc[i][0] + acc[i][15];
    }
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    const uint64_t t1 = __builtin_readcyclecounter();
    out[blockIdx.x * blockDim.x + threadIdx.x] = sum;
    if (threadIdx.x == 0) {
        clk[2 * blockIdx.x] = t1 - t0;
        clk[2 * blockIdx.x + 1] = r1 - r0;
    }
}

// probe_lds_fill_rate: each 8-wave workgroup owns 64 KiB of `src` (its block
// index selects the slice; the slices stay in L2 after the first pass) and
// fills its 64 KiB of LDS from it `iters` times; every wave moves 8 KiB per
// pass, in 1 KiB instructions.  Modes:
//   0  direct global -> LDS loads (buffer_load_dwordx4 ... lds)
//   1  as 0, plus 24 16-byte LDS reads per wave per pass (the operand-read
//      traffic of a 256 x 256 x 64 GEMM step)
//   2  only the 24 LDS reads per wave per pass
//   3  global -> VGPR loads (buffer_load_dwordx4) then 16-byte LDS writes
//   4  as 3, plus the 24 LDS reads
// Wave 0 records the shader-clock cycles of its loop in cyc[block]; every
// access stays inside the workgroup's 64 KiB of src and of LDS.
template <int MODE>
__global__ __launch_bounds__(512) void probe_lds_fill_rate_kernel(const uint16_t* src, int iters, uint32_t* cyc,
                                                                  uint32_t* sink) {
    typedef __attribute__((address_space(3))) void lds_void;
    __shared__ __attribute__((aligned(1024))) uint16_t lds[32768];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint16_t* base = src + static_cast<int64_t>(blockIdx.x) * 32768;
    __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, 65536, 0x00020000);
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (const __attribute__((address_space(3))) uint16_t*)lds));
    u32x4 acc = {0, 0, 0, 0};
    __syncthreads();
    const uint64_t t0 = __builtin_readcyclecounter();
    for (int it = 0; it < iters; ++it) {
        if constexpr (MODE == 0 || MODE == 1) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(lds + (wave * 8 + i) * 512), 16,
                                                        (wave * 8 + i) * 1024 + lane * 16, 0, 0, 0);
        }
        if constexpr (MODE == 3 || MODE == 4) {
            u32x4 v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                    r, (wave * 8 + i) * 1024 + lane * 16, 0, 0));
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t a = lds0 + (wave * 8 + i) * 1024 + lane * 16;
                asm volatile("ds_write_b128 %0, %1" : : "v"(a), "v"(v[i]) : "memory");
            }
        }
        if constexpr (MODE == 1 || MODE == 2 || MODE == 4) {
#pragma unroll
            for (int j = 0; j < 24; ++j) {
                u32x4 v;
                const uint32_t a = lds0 + (((wave * 24 + j) * 1024 + lane * 16) & 65535);
                asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(a));
                acc ^= v;
            }
        }
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __syncthreads();
    }
    const uint64_t t1 = __builtin_readcyclecounter();
    if (threadIdx.x == 0) cyc[blockIdx.x] = static_cast<uint32_t>(t1 - t0);
    if (acc[0] == 0x9e3779b9u && acc[1] == 0x7f4a7c15u) sink[threadIdx.x] = acc[2] + lds[threadIdx.x];
}

template <typename Fn, int... I>
__device__ __forceinline__ void static_for32_impl(Fn&& fn, std::integer_sequence<int, I...>) {
    (fn(std::integral_constant<int, I>{}), ...);
}
template <typename Fn>
__device__ __forceinline__ void static_for32(Fn&& fn) {
    static_for32_impl(fn, std::make_integer_sequence<int, 32>{});
}

// probe_mfma_mix: every wave of an 8-wave workgroup runs `iters` rounds of 32
// independent 16x16x32 MFMAs on register operands; after every 32 / NL of
// them it issues one memory instruction of 1 KiB (NL per round), inside the
// workgroup's own 64 KiB of src and of LDS:
//   MODE 0  direct global -> LDS load       MODE 1  global -> VGPR load + LDS write
//   MODE 2  16-byte LDS read                MODE 3  global -> VGPR load only
// and waits for them at the end of the round.  Wave 0 records the
// shader-clock cycles of its loop in cyc[block]: with NL = 0 the pure
// matrix-core time, otherwise how the memory traffic slows it.
template <int MODE, int NL>
__global__ __launch_bounds__(512) void probe_mfma_mix_kernel(const uint16_t* src, int iters, uint32_t* cyc,
                                                             float* out) {
    typedef __attribute__((address_space(3))) void lds_void;
    __shared__ __attribute__((aligned(1024))) uint16_t lds[32768];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint16_t* base = src + static_cast<int64_t>(blockIdx.x) * 32768;
    __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, 65536, 0x00020000);
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (const __attribute__((address_space(3))) uint16_t*)lds));
    u32x4 av, bv;
    for (int d = 0; d < 4; ++d) {
        av[d] = 0x3f803f80u ^ static_cast<uint32_t>((lane * 7 + d) & 3);
        bv[d] = 0x3c003c00u ^ static_cast<uint32_t>((lane * 5 + d) & 3);
    }
    const bf16x8 a = __builtin_bit_cast(bf16x8, av), b = __builtin_bit_cast(bf16x8, bv);
    f32x4 acc[32];
    for (int i = 0; i < 32; ++i) acc[i] = f32x4{static_cast<float>(i), 0, 0, 0};
    u32x4 keep = {0, 0, 0, 0};
    __syncthreads();
    const uint64_t t0 = __builtin_readcyclecounter();
    for (int it = 0; it < iters; ++it) {
        static_for32([&](auto q_tag) {
            constexpr int Q = decltype(q_tag)::value;
            acc[Q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[Q], 0, 0, 0);
            if constexpr (NL > 0 && Q % (32 / (NL > 0 ? NL : 1)) == 0) {
                constexpr int X = Q / (32 / (NL > 0 ? NL : 1));
                const int slot = (wave * 8 + ((it * NL + X) & 7));
                if constexpr (MODE == 0) {
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(lds + slot * 512), 16, slot * 1024 + lane * 16,
                                                            0, 0, 0);
                } else if constexpr (MODE == 1 || MODE == 3) {
                    u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                        r, slot * 1024 + lane * 16, 0, 0));
                    if constexpr (MODE == 1) {
                        const uint32_t ad = lds0 + slot * 1024 + lane * 16;
                        asm volatile("ds_write_b128 %0, %1" : : "v"(ad), "v"(v) : "memory");
                    } else {
                        keep ^= v;
                    }
                } else {
                    u32x4 v;
                    const uint32_t ad = lds0 + slot * 1024 + lane * 16;
                    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(ad));
                    keep ^= v;
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        });
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    }
    const uint64_t t1 = __builtin_readcyclecounter();
    if (threadIdx.x == 0) cyc[blockIdx.x] = static_cast<uint32_t>(t1 - t0);
    float sum = static_cast<float>(keep[0] ^ keep[1] ^ keep[2] ^ keep[3]) * 1e-30f;
    for (int i = 0; i < 32; ++i) sum += acc[i][0] + acc[i][3];
    out[blockIdx.x * 512 + threadIdx.x] = sum;
}

}  // namespace

extern "C" {

// Swizzle probe: table = 16 ints in host memory (each masked to 0..7).
int probe_lds_swizzle(const int* table, int mf, uint32_t* out, int grid, int iters, void* stream) {
    if (mf != 16 && mf != 32) return static_cast<int>(hipErrorInvalidValue);
    SwzTable t;
    for (int k = 0; k < 16; ++k) t.v[k] = table[k] & 7;
    hipLaunchKernelGGL(probe_lds_swizzle_kernel, dim3(grid), dim3(64), 0, static_cast<hipStream_t>(stream), out, t,
                       mf, iters);
    return static_cast<int>(hipGetLastError());
}

// Lane-pair probe: `grid` one-wave workgroups; out needs 64 * grid words;
// 0 <= i, j < 64.
int probe_lds_pair(int i, int j, uint32_t* out, int grid, int iters, void* stream) {
    if (i < 0 || i > 63 || j < 0 || j > 63) return static_cast<int>(hipErrorInvalidValue);
    hipLaunchKernelGGL(probe_lds_pair_kernel, dim3(grid), dim3(64), 0, static_cast<hipStream_t>(stream), out, i,
                       j, iters);
    return static_cast<int>(hipGetLastError());
}

// LDS pattern probe: `grid` workgroups of 256 threads; out needs 256 * grid words.
int probe_lds_pattern(int pattern, uint32_t* out, int grid, int iters, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (pattern) {
        case 0: hipLaunchKernelGGL(probe_lds_pattern_kernel<0>, dim3(grid), dim3(256), 0, s, out, iters); break;
        case 1: hipLaunchKernelGGL(probe_lds_pattern_kernel<1>, dim3(grid), dim3(256), 0, s, out, iters); break;
        case 2: hipLaunchKernelGGL(probe_lds_pattern_kernel<2>, dim3(grid), dim3(256), 0, s, out, iters); break;
        case 3: hipLaunchKernelGGL(probe_lds_pattern_kernel<3>, dim3(grid), dim3(256), 0, s, out, iters); break;
        case 4: hipLaunchKernelGGL(probe_lds_pattern_kernel<4>, dim3(grid), dim3(256), 0, s, out, iters); break;
        case 5: hipLaunchKernelGGL(probe_lds_pattern_kernel<5>, dim3(grid), dim3(256), 0, s, out, iters); break;
        case 6: hipLaunchKernelGGL(probe_lds_pattern_kernel<6>, dim3(grid), dim3(256), 0, s, out, iters); break;
        default: return static_cast<int>(hipErrorInvalidValue);
    }
    return static_cast<int>(hipGetLastError());
}

// Band-read-into-LDS probe; same arguments and limits as probe_band_read,
// plus rows * row_bytes < 2 GiB.
int probe_band_read_lds(const void* in, int rows, int row_bytes, int band, int rows_per, uint32_t* out,
                        void* stream) {
    if (band < 16 || band > 1024 || band % 16 || row_bytes % band || rows_per <= 0 || rows % rows_per ||
        64 % (band / 16) || static_cast<int64_t>(rows) * row_bytes >= (int64_t(1) << 31))
        return static_cast<int>(hipErrorInvalidValue);
    const int grid = (row_bytes / band) * (rows / rows_per);
    hipLaunchKernelGGL(probe_band_read_lds_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint8_t*>(in), rows, row_bytes, band, rows_per, out);
    return static_cast<int>(hipGetLastError());
}

// Band-read probe (see the kernel); grid = (row_bytes / band) * (rows / rows_per).
int probe_band_read(const void* in, int rows, int row_bytes, int band, int rows_per, uint32_t* out,
                    void* stream) {
    if (band < 16 || band > 4096 || band % 16 || row_bytes % band || rows_per <= 0 || rows % rows_per ||
        256 % (band / 16))
        return static_cast<int>(hipErrorInvalidValue);
    const int grid = (row_bytes / band) * (rows / rows_per);
    hipLaunchKernelGGL(probe_band_read_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint8_t*>(in), rows, row_bytes, band, rows_per, out);
    return static_cast<int>(hipGetLastError());
}

// Streaming-read probe: reads `bytes` (multiple of 16) bytes of `in` with
// `grid` workgroups of 256 threads; out needs `grid` words.  unroll: 4 or 8.
int probe_stream_read(const void* in, uint64_t bytes, uint32_t* out, int grid, int unroll, void* stream) {
    if (bytes % 16 || grid <= 0) return static_cast<int>(hipErrorInvalidValue);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const u32x4* p = static_cast<const u32x4*>(in);
    if (unroll == 8) hipLaunchKernelGGL(probe_stream_read_kernel<8>, dim3(grid), dim3(256), 0, s, p, bytes / 16, out);
    else if (unroll == 4) hipLaunchKernelGGL(probe_stream_read_kernel<4>, dim3(grid), dim3(256), 0, s, p, bytes / 16, out);
    else return static_cast<int>(hipErrorInvalidValue);
    return static_cast<int>(hipGetLastError());
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
    PROBE_SC(MF_, 4, 4, 2, 3)
    PROBE_SC_MF(16)
    PROBE_SC_MF(32)
#undef PROBE_SC_MF
#undef PROBE_SC
    return static_cast<int>(hipErrorInvalidValue);
}

// in: 512 halfwords, out: 256 halfwords (device pointers).
int probe_lds_read_tr(const uint16_t* in, uint16_t* out, void* stream) {
    hipLaunchKernelGGL(probe_lds_read_tr_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), in, out);
    return static_cast<int>(hipGetLastError());
}

// mf 16 or 32, waves per workgroup 1..8; out: grid * 64 * waves floats,
// clk: 2 * grid uint64 (device pointers).  Returns a hipError_t value.
int probe_mfma_rate(int mf, int waves, int iters, int grid, float* out, uint64_t* clk, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (waves < 1 || waves > 8 || grid < 1 || iters < 0) return static_cast<int>(hipErrorInvalidValue);
    if (mf == 16) hipLaunchKernelGGL(probe_mfma_rate_kernel<16>, dim3(grid), dim3(64 * waves), 0, s, iters, out, clk);
    else if (mf == 32) hipLaunchKernelGGL(probe_mfma_rate_kernel<32>, dim3(grid), dim3(64 * waves), 0, s, iters, out, clk);
    else return static_cast<int>(hipErrorInvalidValue);
    return static_cast<int>(hipGetLastError());
}

// Scaled-instruction rate: mf 16 or 32, fmt 0 (E4M3) or 4 (E2M1), waves 1..8;
// out: grid * 64 * waves floats, clk: 2 * grid uint64.  Returns a hipError_t value.
int probe_mfma_scaled_rate(int mf, int fmt, int waves, int iters, int grid, float* out, uint64_t* clk,
                           void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (waves < 1 || waves > 8 || grid < 1 || iters < 0) return static_cast<int>(hipErrorInvalidValue);
    const dim3 g(grid), b(64 * waves);
    if (mf == 16 && fmt == 0) hipLaunchKernelGGL((probe_mfma_scaled_rate_kernel<16, 0>), g, b, 0, s, iters, out, clk);
    else if (mf == 16 && fmt == 4) hipLaunchKernelGGL((probe_mfma_scaled_rate_kernel<16, 4>), g, b, 0, s, iters, out, clk);
    else if (mf == 32 && fmt == 0) hipLaunchKernelGGL((probe_mfma_scaled_rate_kernel<32, 0>), g, b, 0, s, iters, out, clk);
    else if (mf == 32 && fmt == 4) hipLaunchKernelGGL((probe_mfma_scaled_rate_kernel<32, 4>), g, b, 0, s, iters, out, clk);
    else return static_cast<int>(hipErrorInvalidValue);
    return static_cast<int>(hipGetLastError());
}

// src: at least grid * 64 KiB readable bytes; cyc: grid uint32; sink: 512
// uint32 (written only if a data-dependent test passes).  Device pointers.
int probe_lds_fill_rate(int mode, const uint16_t* src, int64_t src_bytes, int grid, int iters, uint32_t* cyc,
                        uint32_t* sink, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (grid < 1 || iters < 1 || src_bytes < static_cast<int64_t>(grid) * 65536)
        return static_cast<int>(hipErrorInvalidValue);
    switch (mode) {
        case 0: hipLaunchKernelGGL(probe_lds_fill_rate_kernel<0>, dim3(grid), dim3(512), 0, s, src, iters, cyc, sink); break;
        case 1: hipLaunchKernelGGL(probe_lds_fill_rate_kernel<1>, dim3(grid), dim3(512), 0, s, src, iters, cyc, sink); break;
        case 2: hipLaunchKernelGGL(probe_lds_fill_rate_kernel<2>, dim3(grid), dim3(512), 0, s, src, iters, cyc, sink); break;
        case 3: hipLaunchKernelGGL(probe_lds_fill_rate_kernel<3>, dim3(grid), dim3(512), 0, s, src, iters, cyc, sink); break;
        case 4: hipLaunchKernelGGL(probe_lds_fill_rate_kernel<4>, dim3(grid), dim3(512), 0, s, src, iters, cyc, sink); break;
        default: return static_cast<int>(hipErrorInvalidValue);
    }
    return static_cast<int>(hipGetLastError());
}

// mode 0..3, nl in {0, 1, 2, 4, 8}; src: at least grid * 64 KiB readable bytes;
// cyc: grid uint32; out: grid * 512 floats.  Device pointers.
int probe_mfma_mix(int mode, int nl, const uint16_t* src, int64_t src_bytes, int grid, int iters, uint32_t* cyc,
                   float* out, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (grid < 1 || iters < 1 || src_bytes < static_cast<int64_t>(grid) * 65536)
        return static_cast<int>(hipErrorInvalidValue);
#define DTG_MIX(M, NLV) \
    if (mode == M && nl == NLV) { hipLaunchKernelGGL((probe_mfma_mix_kernel<M, NLV>), dim3(grid), dim3(512), 0, s, src, iters, cyc, out); return static_cast<int>(hipGetLastError()); }
#define DTG_MIX_ALL(M) DTG_MIX(M, 1) DTG_MIX(M, 2) DTG_MIX(M, 4) DTG_MIX(M, 8)
    DTG_MIX(0, 0)
    DTG_MIX_ALL(0) DTG_MIX_ALL(1) DTG_MIX_ALL(2) DTG_MIX_ALL(3)
#undef DTG_MIX_ALL
#undef DTG_MIX
    return static_cast<int>(hipErrorInvalidValue);
}

}  // extern "C"
