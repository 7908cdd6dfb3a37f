// Log-sum-exp merge of per-segment attention partials.
//
// "[ROCm][MLA] Add guarded gfx942 FP8 context prefill" (vLLM #51551), "What
// this PR does": long contexts are attended segment by segment with one
// quantized Q; each segment yields (out_s, lse_s) and the partials are
// combined by the softmax-over-a-union identity
//   L = ln sum_s exp(L_s),   out = sum_s exp(L_s - L) * out_s.
//
// HBM-bound: per (token, head) it reads n * (128 bf16 + 1 fp32) and writes
// 128 bf16 + 1 fp32. 16 lanes share one (token, head) row, each owning 8
// dims (one 16-byte load per segment, one 16-byte store). The 16 lanes of a
// row sit in one wavefront, so every lane reads the segment LSEs before any
// lane writes the merged LSE (in-place merges are safe).
#include "mla_internal.h"

namespace {

constexpr int kMergeThreads = 256;
constexpr int kMaxSegments = 64;

struct MergeParams {
  const void* outs[kMaxSegments];
  const float* lses[kMaxSegments];
  uint16_t* out;
  float* lse_out;
  int64_t lse_in_stride;
  int64_t lse_out_stride;
  uint32_t n_rows;  // total_q * n_heads
  int32_t n_seg;
  mla::FastDiv heads;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// 8 consecutive partial values of segment s as fp32
template <bool kF32>
__device__ __forceinline__ void load8(const void* base, int64_t eo, float v[8]) {
  if (kF32) {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + eo);
    const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + eo + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + eo);
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
  }
}

template <bool kF32>
__global__ __launch_bounds__(kMergeThreads) void merge_lse_kernel(MergeParams p) {
  const uint64_t n_threads = static_cast<uint64_t>(p.n_rows) * 16u;
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kMergeThreads;
  for (uint64_t g = static_cast<uint64_t>(blockIdx.x) * kMergeThreads + threadIdx.x; g < n_threads;
       g += stride) {
    const uint32_t row = static_cast<uint32_t>(g >> 4);
    const uint32_t col = static_cast<uint32_t>(g & 15u);
    const uint32_t t = mla::fdiv(row, p.heads);
    const uint32_t h = row - t * p.heads.d;
    const int64_t li = static_cast<int64_t>(h) * p.lse_in_stride + t;
    float m = -INFINITY;
    for (int s = 0; s < p.n_seg; ++s) m = fmaxf(m, p.lses[s][li]);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float tot = 0.f;
    const int64_t eo = static_cast<int64_t>(row) * 128 + col * 8;
    if (m != -INFINITY) {
      for (int s = 0; s < p.n_seg; ++s) {
        const float w = __expf(p.lses[s][li] - m);  // exp(-inf) = 0 for empty segments
        tot += w;
        float v[8];
        load8<kF32>(p.outs[s], eo, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += w * v[i];
      }
    }
    const float inv = (m != -INFINITY) ? 1.0f / tot : 0.0f;
    uint4 o;
    o.x = mla::f32_to_bf16_rne(acc[0] * inv) | (mla::f32_to_bf16_rne(acc[1] * inv) << 16);
    o.y = mla::f32_to_bf16_rne(acc[2] * inv) | (mla::f32_to_bf16_rne(acc[3] * inv) << 16);
    o.z = mla::f32_to_bf16_rne(acc[4] * inv) | (mla::f32_to_bf16_rne(acc[5] * inv) << 16);
    o.w = mla::f32_to_bf16_rne(acc[6] * inv) | (mla::f32_to_bf16_rne(acc[7] * inv) << 16);
    *reinterpret_cast<uint4*>(p.out + eo) = o;
    if (col == 0 && p.lse_out != nullptr)
      p.lse_out[static_cast<int64_t>(h) * p.lse_out_stride + t] =
          (m != -INFINITY) ? m + __logf(tot) : -INFINITY;
  }
}

}  // namespace

namespace mla {

int merge_launch(int32_t n_segments, const void* const* outs, int32_t in_f32,
                 const float* const* lses, int64_t lse_in_stride, int64_t total_q,
                 int32_t n_heads, void* out, float* lse_out, int64_t lse_out_stride,
                 hipStream_t stream) {
  const uint64_t rows = static_cast<uint64_t>(total_q) * static_cast<uint64_t>(n_heads);
  if (rows == 0) return ok();
  MergeParams p{};
  for (int s = 0; s < n_segments; ++s) {
    p.outs[s] = outs[s];
    p.lses[s] = lses[s];
  }
  p.out = static_cast<uint16_t*>(out);
  p.lse_out = lse_out;
  p.lse_in_stride = lse_in_stride;
  p.lse_out_stride = lse_out_stride;
  p.n_rows = static_cast<uint32_t>(rows);
  p.n_seg = n_segments;
  p.heads = make_fastdiv(static_cast<uint32_t>(n_heads));
  uint64_t blocks = (rows * 16 + kMergeThreads - 1) / kMergeThreads;
  if (blocks > 256ull * 16ull) blocks = 256ull * 16ull;
  if (in_f32)
    hipLaunchKernelGGL(merge_lse_kernel<true>, dim3(static_cast<unsigned>(blocks)),
                       dim3(kMergeThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(merge_lse_kernel<false>, dim3(static_cast<unsigned>(blocks)),
                       dim3(kMergeThreads), 0, stream, p);
  return check_launch("merge_lse_kernel");
}

}  // namespace mla

extern "C" int mla_merge_lse(int32_t n_segments, const void* const* outs, const float* const* lses,
                             int64_t lse_in_stride, int64_t total_q, int32_t n_heads,
                             int32_t head_dim_v, void* out, float* lse_out,
                             int64_t lse_out_stride, void* stream) {
  if (n_segments < 1 || n_segments > kMaxSegments)
    return mla::fail(MLA_ERR_INVALID_ARGUMENT, "n_segments = %d not in 1..64", n_segments);
  if (head_dim_v != 128)
    return mla::fail(MLA_ERR_UNSUPPORTED, "head_dim_v = %d is not 128", head_dim_v);
  if (n_heads < 1) return mla::fail(MLA_ERR_INVALID_ARGUMENT, "n_heads = %d < 1", n_heads);
  if (total_q < 0) return mla::fail(MLA_ERR_INVALID_ARGUMENT, "total_q < 0");
  if (outs == nullptr || lses == nullptr)
    return mla::fail(MLA_ERR_INVALID_ARGUMENT, "outs or lses is NULL");
  if (total_q == 0) return mla::ok();
  if (out == nullptr || !mla::aligned16(out))
    return mla::fail(MLA_ERR_INVALID_ARGUMENT, "out is NULL or not 16-byte aligned");
  if (lse_in_stride < total_q)
    return mla::fail(MLA_ERR_INVALID_ARGUMENT, "lse_in_stride < total_q");
  if (lse_out != nullptr && lse_out_stride < total_q)
    return mla::fail(MLA_ERR_INVALID_ARGUMENT, "lse_out_stride < total_q");
  const uint64_t rows = static_cast<uint64_t>(total_q) * static_cast<uint64_t>(n_heads);
  if (rows >= (1ull << 31)) return mla::fail(MLA_ERR_UNSUPPORTED, "total_q * n_heads >= 2^31");
  for (int s = 0; s < n_segments; ++s) {
    if (outs[s] == nullptr || lses[s] == nullptr || !mla::aligned16(outs[s]))
      return mla::fail(MLA_ERR_INVALID_ARGUMENT, "segment %d: NULL or misaligned pointer", s);
    if (lse_out != nullptr && lses[s] == lse_out && lse_out_stride != lse_in_stride)
      return mla::fail(MLA_ERR_INVALID_ARGUMENT, "in-place LSE merge needs equal strides");
  }
  return mla::merge_launch(n_segments, outs, 0, lses, lse_in_stride, total_q, n_heads, out,
                           lse_out, lse_out_stride, static_cast<hipStream_t>(stream));
}
