// Internal helpers shared by the libmla_fp8 sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_fp8.h"

namespace mla {

// Records a thread-local error text and returns `status`.
int fail(int status, const char* fmt, ...);
// Clears the thread-local error text and returns MLA_OK.
int ok();
// Maps the last HIP launch error to a status.
int check_launch(const char* what);
// Compute units of the current device (queried once per device; 256 if the query fails).
int cu_count();

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Unsigned 32-bit division by a runtime constant d >= 1 (round-up method with a
// 33-bit magic): q = (umulhi(n, magic) + n) >> shift, valid for n < 2^31.
struct FastDiv {
  uint32_t d;
  uint32_t magic;
  uint32_t shift;
};

inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  f.shift = s;
  // magic = floor(2^32 * (2^s - d) / d) + 1
  f.magic = static_cast<uint32_t>(((1ull << 32) * ((1ull << s) - d)) / d + 1);
  return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
  uint32_t hi = __umulhi(n, f.magic);
  return (hi + n) >> f.shift;
}

// bf16 (round to nearest even) of a finite or infinite fp32 value; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  uint32_t b = __float_as_uint(x);
  uint32_t r = (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
  return (x != x) ? ((b >> 16) | 0x40u) : r;
}

// One prefill launch. cu_q/cu_k may be NULL: then batch must be 1 and the
// sequence spans total_q queries and total_k keys. Head dims are 192/128.
struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* cu_q;
  const int32_t* cu_k;
  int32_t batch;
  int32_t max_seqlen_q;
  int64_t total_q;
  int64_t total_k;
  int32_t n_heads;
  const float* dq;
  const float* dk;
  const float* dv;
  float softmax_scale;
  int32_t causal;
  void* out;        // bf16 [total_q, n_heads, 128], or fp32 when out_f32 = 1
  int32_t out_f32;
  float* lse;
  int64_t lse_stride;
  // multi-segment launches only: the partials' LSE row stride, and the arrival counters
  // of the fused merge (NULL: no merge; else ceil(max_seqlen_q / 256) * n_heads zeroed
  // ints, left zeroed); with the merge, out / lse / lse_stride above receive the merged
  // bf16 result
  int64_t seg_lse_stride = 0;
  int32_t* counters = nullptr;
  // the caller's max_seqlen_k with cu_seqlens over several sequences (0: not given)
  int32_t max_seqlen_k = 0;
};

// One context segment of a multi-segment launch: the same query rows attend keys
// [k0, k0 + lk) of the launch's K/V (causal: bottom-right within the segment) and write
// their own partial out (fp32 when the launch has out_f32) and LSE.
constexpr int kMaxPrefillSegments = 64;
struct PrefillSegment {
  int64_t k0;
  int32_t lk;
  int32_t causal;
  void* out;
  float* lse;
};
int prefill_launch(const PrefillArgs& a, hipStream_t stream);
// the same launch on 4-wave workgroups of 128 rows (the library's second prefill build)
int prefill_launch_small(const PrefillArgs& a, hipStream_t stream);
// one launch over n segments for the query rows of a (a.batch == 1, no cu_seqlens; a.k/a.v
// hold all keys, a.total_k of them; a.causal is ignored; a.out and a.lse are the merged
// result when a.counters is set, else ignored)
int prefill_launch_segments(const PrefillArgs& a, const PrefillSegment* segs, int n,
                            hipStream_t stream);
// query rows per workgroup of the FP8 prefill (the tile of the merge counters)
int prefill_rows_per_block();
// zero n ints on the stream (a fill kernel, so that the call can be graph-captured)
int zero_ints(int32_t* p, int64_t n, hipStream_t stream);

// LSE merge launch with validated arguments; partials are bf16 or (in_f32) fp32.
int merge_launch(int32_t n_segments, const void* const* outs, int32_t in_f32,
                 const float* const* lses, int64_t lse_in_stride, int64_t total_q,
                 int32_t n_heads, void* out, float* lse_out, int64_t lse_out_stride,
                 hipStream_t stream);
int prefill_check_common(int32_t n_heads, int32_t head_dim_qk, int32_t head_dim_v,
                         float softmax_scale, int32_t causal);

}  // namespace mla
