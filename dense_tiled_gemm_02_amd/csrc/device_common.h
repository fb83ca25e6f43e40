// Device helpers shared by the GEMM kernels (gfx950): matrix-instruction
// wrappers, conversions, LDS swizzles, buffer-descriptor constants, explicit
// wait helpers and inline-asm LDS reads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace dtg {
namespace dev {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int MF> struct AccT;
template <> struct AccT<16> { typedef f32x4 type; static constexpr int regs = 4; };
template <> struct AccT<32> { typedef f32x16 type; static constexpr int regs = 16; };

// acc += a x b for one instruction tile.  Operand lane layouts (gfx950):
//  16x16x32: lane l holds row/column l % 16, k = 8 * (l / 16) + 0..7;
//            the result element r of lane l is (row 4 * (l / 16) + r, column l % 16).
//  32x32x16: lane l holds row/column l % 32, k = 8 * (l / 32) + 0..7;
//            result element r is (row 8 * (r / 4) + 4 * (l / 32) + r % 4, column l % 32).
template <int MF, bool BF16>
__device__ __forceinline__ typename AccT<MF>::type mfma(u32x4 a, u32x4 b,
                                                        typename AccT<MF>::type c) {
    if constexpr (MF == 16) {
        if constexpr (BF16)
            return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                           __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
        else
            return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                          __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    } else {
        if constexpr (BF16)
            return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                           __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
        else
            return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                          __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
}

// acc += a x b on 8-bit integers (each 16-byte operand register set holds 16
// consecutive k): v_mfma_i32_16x16x64_i8 / 32x32x32_i8, int32 accumulation
// that wraps modulo 2^32.  The accumulator is carried in float vectors as
// raw bits, like the floating-point tiles' (zero bits are integer zero).
template <int MF>
__device__ __forceinline__ typename AccT<MF>::type mfma_i8(u32x4 a, u32x4 b, typename AccT<MF>::type c) {
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    typedef int i32x16 __attribute__((ext_vector_type(16)));
    if constexpr (MF == 16)
        return __builtin_bit_cast(f32x4, __builtin_amdgcn_mfma_i32_16x16x64_i8(
                                             __builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b),
                                             __builtin_bit_cast(i32x4, c), 0, 0, 0));
    else
        return __builtin_bit_cast(f32x16, __builtin_amdgcn_mfma_i32_32x32x32_i8(
                                              __builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b),
                                              __builtin_bit_cast(i32x16, c), 0, 0, 0));
}

// The same contraction with the accumulator held in AGPRs ("+a"), for tiles
// whose accumulators fill the whole AGPR file (256 per lane at one wave per
// SIMD): left to itself the register allocator splits such an accumulator
// between VGPRs and AGPRs and spills.  The operands come from LDS reads that
// the kernel waits for explicitly; the caller pads the hazard between the
// last instruction and the first read of the result (agpr_settle).
template <int MF, bool BF16>
__device__ __forceinline__ void mfma_agpr(typename AccT<MF>::type& c, u32x4 a, u32x4 b) {
    if constexpr (MF == 32) {
        if constexpr (BF16) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
        else asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    } else {
        if constexpr (BF16) asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
        else asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    }
}

// Wait states between the last matrix instruction writing an AGPR
// accumulator and the first VALU read of it: the compiler does not see into
// the asm above, so the longest required gap (below 32) is padded by hand.
__device__ __forceinline__ void agpr_settle() {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// Element of an AGPR-held accumulator, moved to a VGPR here and not earlier
// (the allocator would otherwise copy the whole tile out at once and spill).
__device__ __forceinline__ float agpr_get(float a) {
    float v;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
    return v;
}

template <bool BF16>
__device__ __forceinline__ float widen(uint16_t h) {
    if constexpr (BF16) return __uint_as_float(static_cast<uint32_t>(h) << 16);
    else return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// fp32 -> storage type, round to nearest even.
template <bool BF16>
__device__ __forceinline__ uint16_t narrow(float v) {
    if constexpr (BF16) return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
    else return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
}

// Physical 16-byte chunk of logical chunk c in LDS row r is c ^ swz(r).  The
// XOR pattern depends only on r % 16, so it is a per-lane constant for the
// MFMA operand reads (fragment rows start at multiples of 16).  For 128-byte
// rows (CH = 8) the pattern was chosen by measurement: of the 4096 linear XOR
// maps of the row bits, this one reads both instruction shapes' operand
// layouts (16 rows x one chunk per 16 lanes, 32 rows x one chunk per 32 lanes)
// without a single bank-conflict cycle, whereas e.g. r & 7 or
// (r & 7) ^ (r >> 3 & 1) each conflict on one of the two.
template <int CH>
__device__ __forceinline__ int swz(int r) {
    if constexpr (CH == 4) return ((r >> 2) ^ (r >> 1)) & 3;
    else if constexpr (CH == 8) return ((r >> 1) & 7) ^ (r & 1);
    else return r & 15;
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

typedef std::integral_constant<bool, true> Checked;     // loads with edge / K-tail masks
typedef std::integral_constant<bool, false> Unchecked;  // interior loads

constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw buffer of dwords
constexpr uint32_t kOOB = 0x80000000u;         // offset past any descriptor range
// cache-policy bits of a buffer access at system scope (sc0 | sc1): the
// access goes past the per-XCD L2 caches, like a system-scope atomic
constexpr int kSysScope = 1 | 16;
// cache-policy bit of a buffer load marking it non-temporal (nt): for data
// read exactly once, such as a weight matrix streamed by the decode kernels
constexpr int kNonTemporal = 2;
constexpr int64_t kMaxRecords = 0x7ffffff0;

template <int N, typename Fn>
__device__ __forceinline__ void static_for(Fn&& fn) {
    if constexpr (N > 0) {
        static_for<N - 1>(fn);
        fn(std::integral_constant<int, N - 1>{});
    }
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// LDS operand reads are issued as inline asm: the compiler then neither
// guards them with waits for every outstanding global -> LDS load (it cannot
// tell which stage a read touches) nor moves them; the kernel waits for them
// explicitly with lds_wait_all() + tie() before the MFMAs that use them.
//
// 16-byte read at LDS byte address addr + OFF.
template <int OFF>
__device__ __forceinline__ u32x4 lds_read16(uint32_t addr) {
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}

// lds_read16 for any non-negative offset: whole multiples of 64 KiB (past
// the instruction's 16-bit offset field) are added to the address.
template <int OFF>
__device__ __forceinline__ u32x4 lds_read16_any(uint32_t addr) {
    if constexpr (OFF < 65536)
        return lds_read16<OFF>(addr);
    else
        return lds_read16<OFF % 65536>(addr + static_cast<uint32_t>(OFF / 65536) * 65536u);
}

// 8-byte read at LDS byte address addr + OFF (addr + OFF a multiple of 8),
// and the same for any non-negative offset.
template <int OFF>
__device__ __forceinline__ u32x2 lds_read8(uint32_t addr) {
    u32x2 v;
    asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}
template <int OFF>
__device__ __forceinline__ u32x2 lds_read8_any(uint32_t addr) {
    if constexpr (OFF < 65536)
        return lds_read8<OFF>(addr);
    else
        return lds_read8<OFF % 65536>(addr + static_cast<uint32_t>(OFF / 65536) * 65536u);
}

// Transposing 64-bit read (ds_read_b64_tr_b16) at addr + OFF: within each
// 16-lane group the 16 addressed 8-byte pieces, in lane order, form a 4 x 16
// matrix of halfwords (lanes 4i..4i+3 give row i); lane t receives column t.
template <int OFF>
__device__ __forceinline__ i16x4 lds_read_tr(uint32_t addr) {
    i16x4 v;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}

// 16-byte global store marked non-temporal (streamed out; an output written
// once is not worth keeping in the caches): ~0.8 us less for a 32 MB output.
__device__ __forceinline__ void store16_nt(void* p, uint32_t x, uint32_t y, uint32_t z, uint32_t w) {
    typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));
    const nt_u32x4 v = {x, y, z, w};
    __builtin_nontemporal_store(v, static_cast<nt_u32x4*>(p));
}
// The same for four floats (the whole vector is reinterpreted: a bit cast of
// one element of a vector reads the vector's first element).
__device__ __forceinline__ void store16_nt(void* p, const f32x4& v) {
    typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(__builtin_bit_cast(nt_u32x4, v), static_cast<nt_u32x4*>(p));
}

// 2-byte (zero-extended) and 4-byte reads at addr + OFF.
template <int OFF>
__device__ __forceinline__ uint32_t lds_read_u16(uint32_t addr) {
    uint32_t v;
    asm volatile("ds_read_u16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}
template <int OFF>
__device__ __forceinline__ uint32_t lds_read_b32(uint32_t addr) {
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}

// Arrival of one K slice at its output tile's (or slab's) counter; true on
// the last arriver.  The partials are written and read with system-coherent
// accesses (SC0 SC1: stores are written through the per-XCD L2 caches to
// memory, loads miss them), and every wave waits until its stores are
// acknowledged before the barrier that precedes the count: when the count
// reaches `slices`, every partial is in memory, and the last arriver's loads
// read memory.  The HIP memory model orders such an exchange only with an
// agent-scope release / acquire pair; on gfx950 the release is an L2
// write-back, which measured +7.8 us on the 30 us bf16 16 x 8192 x 8192
// product with one per workgroup (3.3x with one per wave) and changes
// nothing these accesses see, so the count stays relaxed.  flag is a word of
// LDS.
__device__ __forceinline__ bool arrive_last(int* counter, int slices, int* flag) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0)
        *flag = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) == slices - 1;
    __syncthreads();
    return *flag != 0;
}

__device__ __forceinline__ void lds_wait_all() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Make `v` depend on the preceding lds_wait_all() (volatile asm keeps its
// order), so no use of v is scheduled before the wait.
__device__ __forceinline__ void tie(u32x4& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void tie(i16x4& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void tie(u32x2& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void tie(uint32_t& v) { asm volatile("" : "+v"(v)); }

__device__ __forceinline__ uint32_t lds_addr(const uint16_t* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint16_t*)p));
}

__device__ __forceinline__ uint32_t clamp_records(int64_t bytes) {
    return static_cast<uint32_t>(bytes < kMaxRecords ? bytes : kMaxRecords);
}

// Range of a descriptor that starts `off` bytes into a region of `full` bytes
// (off <= full), capped at kMaxRecords, in 32-bit operations: with uniform
// arguments it stays on the scalar unit, with no branch.  A capped range is
// still inside the region, and covers every offset below the cap.
__device__ __forceinline__ uint32_t capped_records(uint64_t full, uint64_t off) {
    const uint64_t r = full - off;
    const uint32_t hi = static_cast<uint32_t>(r >> 32), lo = static_cast<uint32_t>(r);
    const uint32_t cap = static_cast<uint32_t>(kMaxRecords);
    return hi != 0u ? cap : (lo < cap ? lo : cap);
}

}  // namespace dev
}  // namespace dtg
