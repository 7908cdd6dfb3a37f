// Exact E4M3 quantization of one bf16 value on the device, shared by the static
// quantizer and the fused K/V producer.
//
// Rounding contract: the code is the correctly rounded E4M3 value of the exact
// quotient x / descale (nearest, ties to even, saturating at +-448, NaN kept).
// The value is multiplied by r = 1/descale in fp32, which can be off by up to
// ~3 ulp, then rounded with integer bit operations. Only when the fp32 quotient
// lies within 16 ulp of an E4M3 rounding boundary M can that differ from the exact
// result; there the sign of x - M*descale is taken in fp64, where M*descale
// (5 + 24 significant bits) and the difference are exact.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {
namespace dev {

// One bf16 (bits in the low 16 bits) divided by descale d (r ~ 1/d) to an E4M3 code.
__device__ __forceinline__ uint32_t quant_one(uint32_t xb, float d, float r) {
  const uint32_t sign = (xb >> 8) & 0x80u;
  const uint32_t xa = (xb & 0x7FFFu) << 16;  // |x| as fp32 bits
  if (xa > 0x7F800000u) return 0x7Fu | sign;  // NaN
  const float ax = __uint_as_float(xa);
  const float qf = ax * r;
  const uint32_t a = __float_as_uint(qf);
  if (a > 0x43E00000u) return 0x7Eu | sign;  // > 448 (also +Inf): saturate, no boundary nearby
  uint32_t lower;  // code of the E4M3 value just below (or at) qf
  bool up, near;
  float mid;       // the rounding boundary above `lower`
  if (a >= 0x3C800000u) {  // >= 2^-6: normal E4M3 range
    lower = (a >> 20) - (120u << 3);
    const uint32_t low = a & 0xFFFFFu;
    up = low > 0x80000u;
    near = (low > 0x80000u ? low - 0x80000u : 0x80000u - low) <= 16u;
    mid = __uint_as_float((a & ~0xFFFFFu) | 0x80000u);
  } else {  // subnormal E4M3: multiples of 2^-9
    const float t = qf * 512.0f;  // exact
    const float n = floorf(t);
    const float f = t - n;        // exact
    lower = static_cast<uint32_t>(n);
    up = f > 0.5f;
    near = fabsf(f - 0.5f) <= 0x1p-17f;
    mid = (n + 0.5f) * 0x1p-9f;  // exact
  }
  if (near) {
    // exact side of the boundary: sign of |x| - mid * d, computed exactly in fp64
    const double diff = static_cast<double>(ax) - static_cast<double>(mid) * static_cast<double>(d);
    up = diff > 0.0 || (diff == 0.0 && (lower & 1u));
  }
  return (lower + (up ? 1u : 0u)) | sign;
}

// Codes of 16 bf16 values divided by d (r = 1/d); w[i] holds elements 2i (low half) and
// 2i+1 (high half); byte k of the result is the code of element k.
__device__ __forceinline__ uint4 quant16(const uint32_t (&w)[8], float d, float r) {
  uint32_t out[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t w0 = w[2 * k], w1 = w[2 * k + 1];
    out[k] = quant_one(w0 & 0xFFFFu, d, r) | (quant_one(w0 >> 16, d, r) << 8) |
             (quant_one(w1 & 0xFFFFu, d, r) << 16) | (quant_one(w1 >> 16, d, r) << 24);
  }
  return make_uint4(out[0], out[1], out[2], out[3]);
}

}  // namespace dev
}  // namespace mla
