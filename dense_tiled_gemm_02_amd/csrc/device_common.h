// Device helpers shared by the GEMM kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dtg {
namespace dev {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
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
// MFMA operand reads (fragment rows start at multiples of 16).  Chosen so that
// the 16 rows read by one 16-lane group fall on distinct banks.
template <int CH>
__device__ __forceinline__ int swz(int r) {
    if constexpr (CH == 4) return ((r >> 2) ^ (r >> 1)) & 3;
    else if constexpr (CH == 8) return (r & 7) ^ ((r >> 3) & 1);
    else return r & 15;
}

}  // namespace dev
}  // namespace dtg
