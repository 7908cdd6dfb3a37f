// Chunked-context prefill driver: one sequence, context attended segment by
// segment with one quantized Q, partials merged by log-sum-exp.
//
// "[ROCm][MLA] Add guarded gfx942 FP8 context prefill" (vLLM #51551), "What
// this PR does": Q is quantized once per context pass and its per-head scale
// is reused across context segments; each segment writes into a per-chunk
// output buffer. The segmentation itself is not written on the pages; the
// plan used here, for Lq queries that are the last Lq of Lk keys
// (off = Lk - Lq, bottom-right causal alignment):
//   * queries are processed in chunks of seg rows;
//   * keys [0, off) are cached context in segments of seg keys, visible in full
//     to every query (non-causal calls);
//   * for query chunk [r0, r1), the sequence's own keys [off, off + r0) come in
//     segments of seg keys seen in full, and [off + r0, off + r1) is the
//     diagonal (a causal call with Lq = Lk = r1 - r0); later keys are invisible;
//   * non-causal requests split every query chunk over all key segments.
// The host walks the plan: each query chunk's parts run as ONE prefill launch over
// all its segments (a segment table in the kernel arguments) on the caller's stream;
// the launch merges its own partials: the last workgroup of each (query tile, head) to
// finish combines the segments' fp32 partials into `out`. Adjacent non-causal segments
// of a query chunk are attended as one range when the launch keeps at least four
// workgroups per CU that way (the LSE merge is associative, so this equals merging their
// partials): fewer fp32 partials are written and merged, and the workspace the plan needs
// is an upper bound. Partials are kept in fp32 in a caller-provided workspace, so the
// output is rounded to bf16 once, by the merge; a query chunk with a single part is
// written straight into `out`. The workspace ends in the merge's arrival counters,
// zeroed once per call (each launch leaves them zero).
#include <mutex>
#include <vector>

#include "mla_internal.h"

// Device scratch of mla_fp8_prefill_chunked_noalloc (partials, LSEs and merge counters of
// its launches); each GPU the library runs on holds one copy until the process ends.
static constexpr int64_t kScratchBytes = MLA_FP8_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxParts = 64;  // the merge kernel's segment limit
constexpr int64_t kAlign = 256;
// Launch size below which adjacent non-causal segments stay separate: four workgroups
// per CU of a 256-CU MI355X, with the prefill's default 256 query rows per workgroup.
#ifndef MLA_CHUNK_GROUP_MIN_BLOCKS
#define MLA_CHUNK_GROUP_MIN_BLOCKS (4 * 256)
#endif
constexpr int64_t kMinBlocks = MLA_CHUNK_GROUP_MIN_BLOCKS;
constexpr int64_t kPrefillRows = 256;

struct Part {
  int64_t k0, k1;
  int32_t causal;
};

int64_t align_up(int64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Parts of query chunk [r0, r1). Returns false if the plan is not defined.
bool chunk_parts(int64_t lq, int64_t lk, int64_t seg, int32_t causal, int64_t r0, int64_t r1,
                 std::vector<Part>& parts) {
  parts.clear();
  if (!causal) {
    for (int64_t k0 = 0; k0 < lk; k0 += seg) parts.push_back({k0, std::min(lk, k0 + seg), 0});
    if (parts.empty()) parts.push_back({0, 0, 0});  // no keys: zeros and -inf
    return true;
  }
  const int64_t off = lk - lq;
  if (off < 0) return false;
  for (int64_t k0 = 0; k0 < off; k0 += seg) parts.push_back({k0, std::min(off, k0 + seg), 0});
  for (int64_t c0 = 0; c0 < r0; c0 += seg)
    parts.push_back({off + c0, off + std::min(r0, c0 + seg), 0});
  parts.push_back({off + r0, off + r1, 1});
  return true;
}

// Coalesce the leading n_nc non-causal parts (contiguous key ranges) into as few groups
// of near-equal size as keep (groups + other parts) x blocks_per_part >= kMinBlocks.
void group_parts(std::vector<Part>& parts, int64_t blocks_per_part) {
  const int64_t n = static_cast<int64_t>(parts.size());
  int64_t n_nc = 0;
  while (n_nc < n && !parts[n_nc].causal) ++n_nc;
  if (n_nc < 2) return;
  int64_t ng = 1;
  while (ng < n_nc && (ng + n - n_nc) * blocks_per_part < kMinBlocks) ++ng;
  if (ng == n_nc) return;
  std::vector<Part> out;
  for (int64_t gi = 0, i = 0; gi < ng; ++gi) {
    const int64_t cnt = n_nc / ng + (gi < n_nc % ng ? 1 : 0);
    out.push_back({parts[i].k0, parts[i + cnt - 1].k1, 0});
    i += cnt;
  }
  for (int64_t i = n_nc; i < n; ++i) out.push_back(parts[i]);
  parts.swap(out);
}

// arrival counters of the fused merge: one int per (query tile, head) of a query chunk
int64_t counter_bytes(int64_t rows, int32_t n_heads) {
  const int64_t bm = mla::prefill_rows_per_block();
  return align_up((rows + bm - 1) / bm * n_heads * 4);
}

int64_t max_parts(int64_t lq, int64_t lk, int64_t seg, int32_t causal) {
  if (!causal) return std::max<int64_t>(1, (lk + seg - 1) / seg);
  const int64_t off = lk - lq;
  // the last chunk has the most parts
  const int64_t last_r0 = lq > 0 ? ((lq - 1) / seg) * seg : 0;
  return (off + seg - 1) / seg + (last_r0 + seg - 1) / seg + 1;
}

// Workspace layout for launches of up to `rows` query rows and n parts: n fp32 partial
// outputs, n partial LSEs, then the merge counters.
int64_t layout_bytes(int64_t n, int64_t rows, int32_t n_heads) {
  if (n <= 1) return 0;
  return n * (align_up(rows * n_heads * 128 * 4) + align_up(rows * n_heads * 4)) +
         counter_bytes(rows, n_heads);
}

// Checks shared by the entry points; n_max = the plan's most parts per query chunk.
int check_plan(int64_t lq, int64_t lk, int32_t n_heads, int32_t seg_len, int32_t causal,
               int64_t* n_max) {
  if (lq < 0 || lk < 0 || n_heads < 1 || seg_len < 1 || (causal != 0 && causal != 1))
    return mla::fail(MLA_ERR_INVALID_ARGUMENT, "bad size, head count, segment length or causal");
  if (causal && lk < lq)
    return mla::fail(MLA_ERR_INVALID_ARGUMENT, "causal chunked prefill needs Lk >= Lq");
  *n_max = max_parts(lq, lk, seg_len, causal);
  if (*n_max > kMaxParts)
    return mla::fail(MLA_ERR_UNSUPPORTED, "%lld parts per query chunk exceed %d",
                     static_cast<long long>(*n_max), kMaxParts);
  return MLA_OK;
}

int check_call(const void* q, const void* k, const void* v, int64_t lq, int64_t lk,
               int32_t n_heads, const float* descale_q, const float* descale_k,
               const float* descale_v, float softmax_scale, int32_t seg_len, int32_t causal,
               void* out, float* lse, int64_t lse_stride, int64_t* n_max) {
  int st = mla::prefill_check_common(n_heads, 192, 128, softmax_scale, causal);
  if (st != MLA_OK) return st;
  st = check_plan(lq, lk, n_heads, seg_len, causal, n_max);
  if (st != MLA_OK) return st;
  if (lq >= (1ll << 31) || lk >= (1ll << 31))
    return mla::fail(MLA_ERR_UNSUPPORTED, "Lq and Lk must be < 2^31");
  if (lq == 0) return MLA_OK;
  if (q == nullptr || out == nullptr || descale_q == nullptr || descale_k == nullptr ||
      descale_v == nullptr || (lk > 0 && (k == nullptr || v == nullptr)))
    return mla::fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (!mla::aligned16(q) || !mla::aligned16(k) || !mla::aligned16(v) || !mla::aligned16(out))
    return mla::fail(MLA_ERR_INVALID_ARGUMENT, "q, k, v and out must be 16-byte aligned");
  if (lse != nullptr && lse_stride < lq)
    return mla::fail(MLA_ERR_INVALID_ARGUMENT, "lse_stride < Lq");
  return MLA_OK;
}

// Walk the plan with launches of at most rows_per_launch query rows (the whole query chunk,
// or a multiple of the prefill's row tile): the rows [a, b) of query chunk [r0, r1) attend
// the chunk's parts, with the causal diagonal cut to keys [off + r0, off + b) (bottom-right
// alignment keeps every row's visible keys). ws holds layout_bytes(n_max, rows_per_launch).
int run_plan(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, int64_t lq, int64_t lk,
             int32_t n_heads, const float* descale_q, const float* descale_k,
             const float* descale_v, float softmax_scale, int64_t seg, int32_t causal,
             uint8_t* out8, float* lse, int64_t lse_stride, uint8_t* ws, int64_t n_max,
             int64_t rows_per_launch, hipStream_t s) {
  const int64_t out_part = align_up(rows_per_launch * n_heads * 128 * 4);
  const int64_t lse_part = align_up(rows_per_launch * n_heads * 4);
  uint8_t* lse_ws = ws + n_max * out_part;
  int32_t* counters = reinterpret_cast<int32_t*>(lse_ws + n_max * lse_part);
  bool counters_zeroed = false;
  const int64_t qrow = static_cast<int64_t>(n_heads) * 192;
  const int64_t vrow = static_cast<int64_t>(n_heads) * 128;
  const int64_t orow = static_cast<int64_t>(n_heads) * 128 * 2;
  const int64_t off = lk - lq;
  std::vector<Part> chunk, parts;
  int st = MLA_OK;
  for (int64_t r0 = 0; r0 < lq; r0 += seg) {
    const int64_t r1 = std::min(lq, r0 + seg);
    if (!chunk_parts(lq, lk, seg, causal, r0, r1, chunk))
      return mla::fail(MLA_ERR_INVALID_ARGUMENT, "no chunk plan");
    for (int64_t a = r0; a < r1; a += rows_per_launch) {
      const int64_t b = std::min(r1, a + rows_per_launch);
      const int64_t rows = b - a;
      parts = chunk;
      if (causal) parts.back().k1 = off + b;  // the diagonal is the plan's last part
      group_parts(parts, (rows + kPrefillRows - 1) / kPrefillRows * n_heads);
      const int n = static_cast<int>(parts.size());
      if (n == 1) {
        // a single part is written straight into the output rows
        const Part& pt = parts[0];
        mla::PrefillArgs pa{q8 + a * qrow, k8 + pt.k0 * qrow, v8 + pt.k0 * vrow, nullptr, nullptr,
                            1, static_cast<int32_t>(rows), rows, pt.k1 - pt.k0, n_heads, descale_q,
                            descale_k, descale_v, softmax_scale, pt.causal, out8 + a * orow, 0,
                            lse ? lse + a : nullptr, lse_stride};
        st = mla::prefill_launch(pa, s);
        if (st != MLA_OK) return st;
        continue;
      }
      // all parts of these rows in ONE launch (fp32 partials in the workspace), non-causal
      // segments first (the plan lists the causal diagonal last), merged by the launch
      // itself into the output rows
      if (!counters_zeroed) {
        st = mla::zero_ints(counters, counter_bytes(rows_per_launch, n_heads) / 4, s);
        if (st != MLA_OK) return st;
        counters_zeroed = true;
      }
      mla::PrefillSegment segs[kMaxParts];
      for (int i = 0; i < n; ++i) {
        const Part& pt = parts[i];
        segs[i] = mla::PrefillSegment{pt.k0, static_cast<int32_t>(pt.k1 - pt.k0), pt.causal,
                                      ws + i * out_part,
                                      reinterpret_cast<float*>(lse_ws + i * lse_part)};
      }
      mla::PrefillArgs pa{q8 + a * qrow, k8, v8, nullptr, nullptr, 1, static_cast<int32_t>(rows),
                          rows, lk, n_heads, descale_q, descale_k, descale_v, softmax_scale, 0,
                          out8 + a * orow, 1, lse ? lse + a : nullptr, lse_stride, rows,
                          counters};
      st = mla::prefill_launch_segments(pa, segs, n, s);
      if (st != MLA_OK) return st;
    }
  }
  return mla::ok();
}

// Scratch of the entry point that allocates nothing: one copy per GPU, resolved with
// hipGetSymbolAddress on the first call on each device (in host code `scratch` names a
// host-side stand-in, never the device memory itself).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
uint8_t* g_scratch_ptr[kMaxDevices] = {};

int scratch_of_current_device(uint8_t** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return mla::fail(MLA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return mla::fail(MLA_ERR_UNSUPPORTED, "device %d beyond the %d this library tracks", dev,
                     kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return mla::fail(MLA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = static_cast<uint8_t*>(p);
  }
  *ptr = g_scratch_ptr[dev];
  return MLA_OK;
}

}  // namespace

extern "C" int mla_fp8_chunked_workspace_size(int64_t lq, int64_t lk, int32_t n_heads,
                                              int32_t seg_len, int32_t causal, uint64_t* bytes) {
  if (bytes == nullptr) return mla::fail(MLA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  int64_t n = 0;
  const int st = check_plan(lq, lk, n_heads, seg_len, causal, &n);
  if (st != MLA_OK) return st;
  *bytes = static_cast<uint64_t>(layout_bytes(n, std::min<int64_t>(seg_len, lq), n_heads));
  return mla::ok();
}

extern "C" int mla_fp8_prefill_chunked(const void* q, const void* k, const void* v, int64_t lq,
                                       int64_t lk, int32_t n_heads, const float* descale_q,
                                       const float* descale_k, const float* descale_v,
                                       float softmax_scale, int32_t seg_len, int32_t causal,
                                       void* out, float* lse, int64_t lse_stride, void* workspace,
                                       uint64_t workspace_bytes, void* stream) {
  int64_t n_max = 0;
  int st = check_call(q, k, v, lq, lk, n_heads, descale_q, descale_k, descale_v, softmax_scale,
                      seg_len, causal, out, lse, lse_stride, &n_max);
  if (st != MLA_OK || lq == 0) return st == MLA_OK ? mla::ok() : st;
  const int64_t rows = std::min<int64_t>(seg_len, lq);
  const uint64_t need = static_cast<uint64_t>(layout_bytes(n_max, rows, n_heads));
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !mla::aligned16(workspace)))
    return mla::fail(MLA_ERR_INVALID_ARGUMENT,
                     "workspace must be 16-byte aligned and hold %llu bytes",
                     static_cast<unsigned long long>(need));
  return run_plan(static_cast<const uint8_t*>(q), static_cast<const uint8_t*>(k),
                  static_cast<const uint8_t*>(v), lq, lk, n_heads, descale_q, descale_k, descale_v,
                  softmax_scale, seg_len, causal, static_cast<uint8_t*>(out), lse, lse_stride,
                  static_cast<uint8_t*>(workspace), n_max, rows, static_cast<hipStream_t>(stream));
}

extern "C" int mla_fp8_prefill_chunked_noalloc(const void* q, const void* k, const void* v,
                                               int64_t lq, int64_t lk, int32_t n_heads,
                                               const float* descale_q, const float* descale_k,
                                               const float* descale_v, float softmax_scale,
                                               int32_t seg_len, int32_t causal, void* out,
                                               float* lse, int64_t lse_stride, void* stream) {
  int64_t n_max = 0;
  int st = check_call(q, k, v, lq, lk, n_heads, descale_q, descale_k, descale_v, softmax_scale,
                      seg_len, causal, out, lse, lse_stride, &n_max);
  if (st != MLA_OK || lq == 0) return st == MLA_OK ? mla::ok() : st;
  // the most query rows per launch whose partials fit the scratch: the whole query chunk,
  // else a multiple of the prefill's row tile
  const int64_t chunk = std::min<int64_t>(seg_len, lq);
  int64_t rows = chunk;
  if (layout_bytes(n_max, rows, n_heads) > kScratchBytes) {
    const int64_t tile = mla::prefill_rows_per_block();
    rows = (chunk - 1) / tile * tile;
    while (rows > 0 && layout_bytes(n_max, rows, n_heads) > kScratchBytes) rows -= tile;
    if (rows <= 0)
      return mla::fail(MLA_ERR_UNSUPPORTED,
                       "%lld parts of %lld rows x %d heads need %lld bytes of partials; the "
                       "scratch holds %lld",
                       static_cast<long long>(n_max), static_cast<long long>(std::min(chunk, tile)),
                       n_heads, static_cast<long long>(layout_bytes(n_max, std::min(chunk, tile),
                                                                    n_heads)),
                       static_cast<long long>(kScratchBytes));
  }
  uint8_t* ws = nullptr;
  if (layout_bytes(n_max, rows, n_heads) > 0) {
    st = scratch_of_current_device(&ws);
    if (st != MLA_OK) return st;
  }
  return run_plan(static_cast<const uint8_t*>(q), static_cast<const uint8_t*>(k),
                  static_cast<const uint8_t*>(v), lq, lk, n_heads, descale_q, descale_k, descale_v,
                  softmax_scale, seg_len, causal, static_cast<uint8_t*>(out), lse, lse_stride, ws,
                  n_max, rows, static_cast<hipStream_t>(stream));
}
