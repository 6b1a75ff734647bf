// kv_types.hpp - element types of the paged K/V cache and their exact conversions (gfx950 device code).
//
// f32 and bf16 caches hold keys and values as they are; an fp8 cache holds 8-bit E4M3 codes (the OCP
// 8-bit floating-point format, FN variant).  Every finite E4M3 value is a bf16 value (3 mantissa bits,
// exponents 2^-9 .. 2^8), so a code converts to bf16, and on to fp32, without rounding: kernels load the
// codes, convert them in registers and run the bf16 path from there.  Queries and min/max metadata of an
// fp8 cache are bf16.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace prr {

enum KvType { kKtF32 = 0, kKtBf16 = 1, kKtFp8 = 2 };

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// Codes in bytes 2 HI and 2 HI + 1 of x as two bf16 values (element 0 from the lower byte): gfx950's
// packed E4M3 -> bf16 conversion with a unit scale, which is exact.
template <bool HI>
__device__ __forceinline__ bf16x2v fp8x2_to_bf16(uint32_t x) {
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, HI);
}

// The four codes of x as floats, byte i -> f[i].
__device__ __forceinline__ void fp8x4_to_f32(uint32_t x, float (&f)[4]) {
    const bf16x2v a = fp8x2_to_bf16<false>(x), b = fp8x2_to_bf16<true>(x);
    f[0] = (float)a[0];
    f[1] = (float)a[1];
    f[2] = (float)b[0];
    f[3] = (float)b[1];
}

// One code as a float.
__device__ __forceinline__ float fp8_to_f32(uint8_t x) { return (float)fp8x2_to_bf16<false>((uint32_t)x)[0]; }

}  // namespace prr
