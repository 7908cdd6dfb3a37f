// Exact E4M3 quantization of one bf16 value on the device, and code tables built from it,
// shared by the static quantizer and the fused K/V producer.
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

// Code tables. For a descale d in [2^E, 2^(E+1)), a bf16 magnitude below binade
// e_lo = E + 117 is under 2^(E-10), so its quotient is under 2^-10 (half the smallest
// subnormal): code 0. From binade e_lo + 20 = E + 137 up it is at least 2^(E+10), so the
// quotient exceeds 512: saturated (0x7E). The 20 binades between hold every other code.
// Table entry 0 is 0, entry 1 + ((e - e_lo) << 7 | mantissa) the code of that magnitude
// (from quant_one, so every lookup equals it), entry 1 + 20 * 128 is 0x7E; the index is
// the magnitude minus (e_lo << 7), clamped to [-1, 20 * 128], plus one. Tables are for
// descales in [2^-126, 2^126] (table_ok); NaN inputs lie above the window and take
// quant_one itself.
constexpr int kTabRows = 20;
constexpr int kTabEntries = kTabRows * 128 + 2;
constexpr int kTabBytes = (kTabEntries + 15) / 16 * 16;

__device__ __forceinline__ bool table_ok(float d) { return d >= 0x1p-126f && d <= 0x1p126f; }

// e_lo of descale d (d within table_ok)
__device__ __forceinline__ int table_elo(float d) { return ilogbf(d) + 117; }

// Entry j of the code table of descale d (r = 1/d, e_lo = table_elo(d))
__device__ __forceinline__ uint8_t table_entry(int j, float d, float r, int e_lo) {
  const int e = e_lo + ((j - 1) >> 7);
  uint32_t code = 0;
  if (j == kTabEntries - 1)
    code = 0x7Eu;
  else if (j > 0 && e >= 0 && e <= 255)
    code = quant_one(static_cast<uint32_t>((e << 7) | ((j - 1) & 127)), d, r);
  return static_cast<uint8_t>(code);
}

// Codes of 16 bf16 values (w[i] holds elements 2i and 2i+1) through the table of descale
// d (base = e_lo << 7, r = 1/d); byte k of the result is the code of element k. A group
// holding a NaN anywhere in the wave takes quant16.
__device__ __forceinline__ uint4 quant16_tab(const uint32_t (&w)[8], const uint8_t* tab,
                                             int base, float d, float r) {
  uint32_t mx = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) mx = max(mx, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  if (__builtin_expect(__any(mx > 0x7F80u), 0)) return quant16(w, d, r);
  auto look = [&](uint32_t mag) {
    const int idx = min(max(static_cast<int>(mag) - base, -1), kTabRows * 128) + 1;
    return static_cast<uint32_t>(tab[idx]);
  };
  uint32_t out[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t w0 = w[2 * k], w1 = w[2 * k + 1];
    const uint32_t c = look(w0 & 0x7FFFu) | (look((w0 >> 16) & 0x7FFFu) << 8) |
                       (look(w1 & 0x7FFFu) << 16) | (look((w1 >> 16) & 0x7FFFu) << 24);
    // the sign bits: the high byte of each bf16 element
    out[k] = c | (__builtin_amdgcn_perm(w1, w0, 0x07050301u) & 0x80808080u);
  }
  return make_uint4(out[0], out[1], out[2], out[3]);
}

}  // namespace dev
}  // namespace mla
