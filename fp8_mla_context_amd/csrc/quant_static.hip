// Static per-head FP8 (OCP E4M3FN) quantizer and per-head amax calibration.
//
// "[ROCm][MLA] Add guarded gfx942 FP8 context prefill" (vLLM #51551), Summary
// and "What this PR does": static per-head scales replace the runtime amax
// reduction, and one kernel quantizes the attention inputs. Here one launch
// covers up to three tensors (Q, K, V) with their own head dims and descales.
//
// Rounding contract: the code is the correctly rounded E4M3 value of the exact
// quotient x / descale (nearest, ties to even, saturating at +-448, NaN kept); see
// quant16 and quant_one for how the device reaches it.
//
// HBM-bound: 2 bytes read + 1 byte written per element. One workgroup takes 256 tokens
// of one (tensor, head), heads fastest over the grid so that neighbouring heads of the
// same tokens are read together; it first fills the head's code table (see
// e4m3_quant.h) in LDS with the exact routine, then each thread handles 16 consecutive
// elements of a (token, head) row at a time: two 16-byte loads, table lookups, one
// 16-byte store. With the exact routine on every element instead, the kernel was
// arithmetic-bound (the same loads and stores alone ran 1.6x as fast).
#include "mla_internal.h"
#include "e4m3_quant.h"

namespace {

constexpr int kQuantThreads = 256;
constexpr int kMaxJobs = 3;

struct QuantJobDev {
  const uint16_t* x;
  uint8_t* y;
  const float* descale;  // fp32 descales, or (from_amax) the fp32 bit patterns of the amax
  int64_t stride_token;
  int64_t stride_head;
  int64_t n_tokens;
  uint32_t block_begin;  // first workgroup of this job
  int32_t head_dim;
  int32_t vec;        // 1: 16-byte loads are aligned
  int32_t from_amax;  // 1: descale = descale_of_amax(descale[h])
};

struct QuantParams {
  QuantJobDev job[kMaxJobs];
  int32_t n_jobs;
  uint32_t total_blocks;
  mla::FastDiv heads;
};

constexpr int kTileTokens = 256;  // tokens of one (tensor, head) per quantizer workgroup

// Dynamic scales: descale = RN_fp32(amax / 448) floored at 2^-126 (1/descale stays
// finite), or 1 when the head is all zeros (any positive descale gives the same codes).
__device__ __forceinline__ float descale_of_amax(float amax) {
  if (!(amax > 0.f)) return 1.f;
  return fmaxf(__fdiv_rn(amax, 448.f), 0x1p-126f);
}

// Chunk c (16 consecutive elements) of a token tile whose (token 0, head) row starts at
// src0: its inputs in w, elements 2i and 2i+1 in w[i]. Returns the chunk's token in the tile
// (chunks of a row: 12 for head dim 192, else 8) and its column in *col.
__device__ __forceinline__ int load_tile_chunk(const QuantJobDev& jb, const uint16_t* src0,
                                               bool wide, int c, uint32_t (&w)[8],
                                               int* col = nullptr) {
  const int t = wide ? c / 12 : c >> 3;
  const int cc = c - t * (wide ? 12 : 8);
  if (col != nullptr) *col = cc;
  const uint16_t* src = src0 + t * jb.stride_token + cc * 16;
  if (jb.vec) {
    const uint4 a = *reinterpret_cast<const uint4*>(src);
    const uint4 b = *reinterpret_cast<const uint4*>(src + 8);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      w[i] = static_cast<uint32_t>(src[2 * i]) | (static_cast<uint32_t>(src[2 * i + 1]) << 16);
  }
  return t;
}

// Workgroup b: its job (blocks [job.block_begin, next job's)), then token tile and head,
// heads fastest. The (job, head) descale comes from the caller, or (dynamic path) from the
// amax; descales outside the tables' range round every element with quant16.
__global__ __launch_bounds__(kQuantThreads) void quant_static_kernel(QuantParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t tab[mla::dev::kTabBytes];
  const uint32_t b = blockIdx.x;
  int j = 0;
  if (p.n_jobs > 1 && b >= p.job[1].block_begin) j = 1;
  if (p.n_jobs > 2 && b >= p.job[2].block_begin) j = 2;
  const QuantJobDev& jb = p.job[j];
  const uint32_t local = b - jb.block_begin;
  const uint32_t tile = mla::fdiv(local, p.heads);
  const uint32_t h = local - tile * p.heads.d;
  const float d = jb.from_amax ? descale_of_amax(jb.descale[h]) : jb.descale[h];
  const float r = 1.0f / d;
  const bool use_tab = mla::dev::table_ok(d);  // uniform over the workgroup
  const int e_lo = use_tab ? mla::dev::table_elo(d) : 0;
  if (use_tab)
    for (int i = threadIdx.x; i < mla::dev::kTabEntries; i += kQuantThreads)
      tab[i] = mla::dev::table_entry(i, d, r, e_lo);
  __syncthreads();
  const int64_t t0 = static_cast<int64_t>(tile) * kTileTokens;
  const int n_tok = static_cast<int>(min<int64_t>(kTileTokens, jb.n_tokens - t0));
  const bool wide = jb.head_dim == 192;  // 12 chunks of 16 per row, else 8
  const int n_chunks = n_tok * (wide ? 12 : 8);
  const uint16_t* src0 = jb.x + t0 * jb.stride_token + static_cast<int64_t>(h) * jb.stride_head;
  uint8_t* dst0 = jb.y + (t0 * p.heads.d + h) * jb.head_dim;
  const int64_t dst_rs = static_cast<int64_t>(p.heads.d) * jb.head_dim;
  // chunk c of the tile: its 16 inputs in w (elements 2i, 2i+1 in w[i]), its codes' address
  auto load = [&](int c, uint32_t (&w)[8]) {
    int col;
    const int t = load_tile_chunk(jb, src0, wide, c, w, &col);
    return dst0 + t * dst_rs + col * 16;
  };
  auto codes = [&](const uint32_t (&w)[8]) {
    return use_tab ? mla::dev::quant16_tab(w, tab, e_lo << 7, d, r) : mla::dev::quant16(w, d, r);
  };
  int c = threadIdx.x;
  // two chunks per iteration: both chunks' loads are in flight before either is rounded
  for (; c + kQuantThreads < n_chunks; c += 2 * kQuantThreads) {
    uint32_t w0[8], w1[8];
    uint8_t* d0 = load(c, w0);
    uint8_t* d1 = load(c + kQuantThreads, w1);
    *reinterpret_cast<uint4*>(d0) = codes(w0);
    *reinterpret_cast<uint4*>(d1) = codes(w1);
  }
  if (c < n_chunks) {
    uint32_t w[8];
    uint8_t* d0 = load(c, w);
    *reinterpret_cast<uint4*>(d0) = codes(w);
  }
}

// ---------------------------------------------------------------------------
// amax per head: max |x| over tokens and dims. Float bits of |x| order like
// unsigned integers, so an integer atomic max is exact and order-independent.
// NaN inputs (bits above +Inf) win the max and surface as a non-finite amax.
//
// Same 16-element chunks as the quantizer (two 16-byte loads per thread), for up
// to three tensors in one launch; each workgroup keeps per-(tensor, head) maxima
// in LDS and publishes them with one global atomic each at the end.

__global__ __launch_bounds__(kQuantThreads) void zero_words_kernel(uint32_t* p, int n) {
  int i = blockIdx.x * kQuantThreads + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// amax_bits[j * H + h] receives the max of job j, head h (the jobs' descale field is
// not read). Workgroup b covers the (job, token tile, head) of the quantizer's workgroup
// b: a running max per thread, a reduction over the workgroup, one global atomic.
__global__ __launch_bounds__(kQuantThreads) void amax_chunks_kernel(QuantParams p,
                                                                    uint32_t* amax_bits) {
  __shared__ uint32_t wave_max[kQuantThreads / 64];
  const uint32_t b = blockIdx.x;
  int j = 0;
  if (p.n_jobs > 1 && b >= p.job[1].block_begin) j = 1;
  if (p.n_jobs > 2 && b >= p.job[2].block_begin) j = 2;
  const QuantJobDev& jb = p.job[j];
  const uint32_t local = b - jb.block_begin;
  const uint32_t tile = mla::fdiv(local, p.heads);
  const uint32_t h = local - tile * p.heads.d;
  const int64_t t0 = static_cast<int64_t>(tile) * kTileTokens;
  const int n_tok = static_cast<int>(min<int64_t>(kTileTokens, jb.n_tokens - t0));
  const bool wide = jb.head_dim == 192;
  const int n_chunks = n_tok * (wide ? 12 : 8);
  const uint16_t* src0 = jb.x + t0 * jb.stride_token + static_cast<int64_t>(h) * jb.stride_head;
  auto chunk_max = [&](int c) {
    uint32_t w[8];
    load_tile_chunk(jb, src0, wide, c, w);
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = max(m, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
    return m;
  };
  uint32_t m = 0;
  int c = threadIdx.x;
  for (; c + kQuantThreads < n_chunks; c += 2 * kQuantThreads)
    m = max(m, max(chunk_max(c), chunk_max(c + kQuantThreads)));
  if (c < n_chunks) m = max(m, chunk_max(c));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), off)));
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kQuantThreads / 64; ++w) m = max(m, wave_max[w]);
    if (m != 0u) atomicMax(amax_bits + j * static_cast<int>(p.heads.d) + h, m << 16);
  }
}

// in place: amax bit patterns -> dynamic descales
__global__ __launch_bounds__(kQuantThreads) void descale_of_amax_kernel(float* v, int n) {
  int i = blockIdx.x * kQuantThreads + threadIdx.x;
  if (i < n) v[i] = descale_of_amax(v[i]);
}

// Validate the jobs and fill the launch parameters. need_y: the job writes codes;
// need_descale: the job reads caller descales. Returns MLA_OK with *total chunks.
int build_params(const mla_quant_job* jobs, int32_t n_jobs, int32_t n_heads, bool need_y,
                 bool need_descale, QuantParams& p, uint64_t& total) {
  if (jobs == nullptr) return mla::fail(MLA_ERR_INVALID_ARGUMENT, "jobs is NULL");
  if (n_jobs < 1 || n_jobs > kMaxJobs)
    return mla::fail(MLA_ERR_INVALID_ARGUMENT, "n_jobs = %d not in 1..3", n_jobs);
  if (n_heads < 1) return mla::fail(MLA_ERR_INVALID_ARGUMENT, "n_heads = %d < 1", n_heads);
  p = QuantParams{};
  p.n_jobs = n_jobs;
  total = 0;
  uint64_t blocks = 0;
  for (int j = 0; j < n_jobs; ++j) {
    const mla_quant_job& s = jobs[j];
    if (s.head_dim != 192 && s.head_dim != 128)
      return mla::fail(MLA_ERR_UNSUPPORTED, "job %d: head_dim %d is not 192 or 128", j, s.head_dim);
    if (s.n_tokens < 0) return mla::fail(MLA_ERR_INVALID_ARGUMENT, "job %d: n_tokens < 0", j);
    if (s.n_tokens > 0 && (s.x == nullptr || (need_y && s.y == nullptr) ||
                           (need_descale && s.descale == nullptr)))
      return mla::fail(MLA_ERR_INVALID_ARGUMENT, "job %d: NULL pointer", j);
    if (s.stride_token < 0 || s.stride_head < 0)
      return mla::fail(MLA_ERR_INVALID_ARGUMENT, "job %d: negative stride", j);
    if (need_y && s.n_tokens > 0 && !mla::aligned16(s.y))
      return mla::fail(MLA_ERR_INVALID_ARGUMENT, "job %d: y is not 16-byte aligned", j);
    if ((reinterpret_cast<uintptr_t>(s.x) & 1u) != 0)
      return mla::fail(MLA_ERR_INVALID_ARGUMENT, "job %d: x is not 2-byte aligned", j);
    const uint64_t rows = static_cast<uint64_t>(s.n_tokens) * static_cast<uint64_t>(n_heads);
    const uint64_t chunks = rows * static_cast<uint64_t>(s.head_dim / 16);
    if (rows >= (1ull << 31))
      return mla::fail(MLA_ERR_UNSUPPORTED, "job %d: n_tokens * n_heads >= 2^31", j);
    QuantJobDev& d = p.job[j];
    d.x = static_cast<const uint16_t*>(s.x);
    d.y = static_cast<uint8_t*>(s.y);
    d.descale = s.descale;
    d.stride_token = s.stride_token;
    d.stride_head = s.stride_head;
    d.head_dim = s.head_dim;
    d.n_tokens = s.n_tokens;
    d.block_begin = static_cast<uint32_t>(blocks);
    blocks += static_cast<uint64_t>((s.n_tokens + kTileTokens - 1) / kTileTokens) *
              static_cast<uint64_t>(n_heads);
    if (blocks >= (1ull << 31))
      return mla::fail(MLA_ERR_UNSUPPORTED, "more than 2^31 quantizer workgroups");
    d.vec = (mla::aligned16(s.x) && (s.stride_token % 8) == 0 && (s.stride_head % 8) == 0) ? 1 : 0;
    d.from_amax = 0;
    total += chunks;
    if (total >= (1ull << 31))
      return mla::fail(MLA_ERR_UNSUPPORTED, "more than 2^35 elements in one launch");
  }
  p.total_blocks = static_cast<uint32_t>(blocks);
  p.heads = mla::make_fastdiv(static_cast<uint32_t>(n_heads));
  return MLA_OK;
}

// zero the n amax words, then the per-(job, head) maxima of the jobs' inputs
int launch_amax(const QuantParams& p, uint64_t total, uint32_t* amax_bits, int n, hipStream_t st) {
  hipLaunchKernelGGL(zero_words_kernel, dim3((n + kQuantThreads - 1) / kQuantThreads),
                     dim3(kQuantThreads), 0, st, amax_bits, n);
  int s = mla::check_launch("zero_words_kernel");
  if (s != MLA_OK || total == 0) return s;
  hipLaunchKernelGGL(amax_chunks_kernel, dim3(p.total_blocks), dim3(kQuantThreads), 0, st, p,
                     amax_bits);
  return mla::check_launch("amax_chunks_kernel");
}

}  // namespace

extern "C" int mla_fp8_quant_static(const mla_quant_job* jobs, int32_t n_jobs, int32_t n_heads,
                                    void* stream) {
  QuantParams p;
  uint64_t total = 0;
  const int st = build_params(jobs, n_jobs, n_heads, true, true, p, total);
  if (st != MLA_OK) return st;
  if (total == 0) return mla::ok();
  hipLaunchKernelGGL(quant_static_kernel, dim3(p.total_blocks), dim3(kQuantThreads), 0,
                     static_cast<hipStream_t>(stream), p);
  return mla::check_launch("quant_static_kernel");
}

extern "C" int mla_fp8_quant_dynamic(const mla_quant_job* jobs, int32_t n_jobs, int32_t n_heads,
                                     float* descale_out, void* stream) {
  if (descale_out == nullptr) return mla::fail(MLA_ERR_INVALID_ARGUMENT, "descale_out is NULL");
  QuantParams p;
  uint64_t total = 0;
  int st = build_params(jobs, n_jobs, n_heads, true, false, p, total);
  if (st != MLA_OK) return st;
  if (static_cast<int64_t>(n_jobs) * n_heads >= (1ll << 31))
    return mla::fail(MLA_ERR_UNSUPPORTED, "n_jobs * n_heads too large");
  const int n = n_jobs * n_heads;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  uint32_t* bits = reinterpret_cast<uint32_t*>(descale_out);
  st = launch_amax(p, total, bits, n, hs);
  if (st != MLA_OK) return st;
  if (total > 0) {
    for (int j = 0; j < n_jobs; ++j) {
      p.job[j].descale = descale_out + static_cast<int64_t>(j) * n_heads;
      p.job[j].from_amax = 1;
    }
    hipLaunchKernelGGL(quant_static_kernel, dim3(p.total_blocks), dim3(kQuantThreads), 0, hs, p);
    st = mla::check_launch("quant_static_kernel");
    if (st != MLA_OK) return st;
  }
  hipLaunchKernelGGL(descale_of_amax_kernel, dim3((n + kQuantThreads - 1) / kQuantThreads),
                     dim3(kQuantThreads), 0, hs, descale_out, n);
  return mla::check_launch("descale_of_amax_kernel");
}

extern "C" int mla_fp8_amax_per_head(const void* x, int64_t stride_token, int64_t stride_head,
                                     int64_t n_tokens, int32_t n_heads, int32_t head_dim,
                                     float* amax, void* stream) {
  if (amax == nullptr) return mla::fail(MLA_ERR_INVALID_ARGUMENT, "amax is NULL");
  if (n_tokens > 0 && x == nullptr) return mla::fail(MLA_ERR_INVALID_ARGUMENT, "x is NULL");
  mla_quant_job job{x, stride_token, stride_head, n_tokens, head_dim, nullptr, nullptr};
  QuantParams p;
  uint64_t total = 0;
  const int st = build_params(&job, 1, n_heads, false, false, p, total);
  if (st != MLA_OK) return st;
  return launch_amax(p, total, reinterpret_cast<uint32_t*>(amax), n_heads,
                     static_cast<hipStream_t>(stream));
}
