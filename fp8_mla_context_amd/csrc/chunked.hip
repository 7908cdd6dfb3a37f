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
#include <vector>

#include "mla_internal.h"

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

}  // namespace

extern "C" int mla_fp8_chunked_workspace_size(int64_t lq, int64_t lk, int32_t n_heads,
                                              int32_t seg_len, int32_t causal, uint64_t* bytes) {
  if (bytes == nullptr) return mla::fail(MLA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (lq < 0 || lk < 0 || n_heads < 1 || seg_len < 1 || (causal != 0 && causal != 1))
    return mla::fail(MLA_ERR_INVALID_ARGUMENT, "bad size, head count, segment length or causal");
  if (causal && lk < lq)
    return mla::fail(MLA_ERR_INVALID_ARGUMENT, "causal chunked prefill needs Lk >= Lq");
  const int64_t n = max_parts(lq, lk, seg_len, causal);
  if (n > kMaxParts)
    return mla::fail(MLA_ERR_UNSUPPORTED, "%lld parts per query chunk exceed %d",
                     static_cast<long long>(n), kMaxParts);
  const int64_t rows = std::min<int64_t>(seg_len, lq);
  const int64_t out_part = align_up(rows * n_heads * 128 * 4);
  const int64_t lse_part = align_up(rows * n_heads * 4);
  *bytes = (n > 1) ? static_cast<uint64_t>(n * (out_part + lse_part) + counter_bytes(rows, n_heads))
                   : 0u;
  return mla::ok();
}

extern "C" int mla_fp8_prefill_chunked(const void* q, const void* k, const void* v, int64_t lq,
                                       int64_t lk, int32_t n_heads, const float* descale_q,
                                       const float* descale_k, const float* descale_v,
                                       float softmax_scale, int32_t seg_len, int32_t causal,
                                       void* out, float* lse, int64_t lse_stride, void* workspace,
                                       uint64_t workspace_bytes, void* stream) {
  int st = mla::prefill_check_common(n_heads, 192, 128, softmax_scale, causal);
  if (st != MLA_OK) return st;
  uint64_t need = 0;
  st = mla_fp8_chunked_workspace_size(lq, lk, n_heads, seg_len, causal, &need);
  if (st != MLA_OK) return st;
  if (lq >= (1ll << 31) || lk >= (1ll << 31))
    return mla::fail(MLA_ERR_UNSUPPORTED, "Lq and Lk must be < 2^31");
  if (lq == 0) return mla::ok();
  if (q == nullptr || out == nullptr || descale_q == nullptr || descale_k == nullptr ||
      descale_v == nullptr || (lk > 0 && (k == nullptr || v == nullptr)))
    return mla::fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (!mla::aligned16(q) || !mla::aligned16(k) || !mla::aligned16(v) || !mla::aligned16(out))
    return mla::fail(MLA_ERR_INVALID_ARGUMENT, "q, k, v and out must be 16-byte aligned");
  if (lse != nullptr && lse_stride < lq)
    return mla::fail(MLA_ERR_INVALID_ARGUMENT, "lse_stride < Lq");
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !mla::aligned16(workspace)))
    return mla::fail(MLA_ERR_INVALID_ARGUMENT,
                     "workspace must be 16-byte aligned and hold %llu bytes",
                     static_cast<unsigned long long>(need));

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t seg = seg_len;
  const int64_t rows_max = std::min<int64_t>(seg, lq);
  const int64_t out_part = align_up(rows_max * n_heads * 128 * 4);
  const int64_t lse_part = align_up(rows_max * n_heads * 4);
  const int64_t n_max = max_parts(lq, lk, seg, causal);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint8_t* lse_ws = ws + n_max * out_part;
  int32_t* counters = reinterpret_cast<int32_t*>(lse_ws + n_max * lse_part);
  bool counters_zeroed = false;
  const uint8_t* q8 = static_cast<const uint8_t*>(q);
  const uint8_t* k8 = static_cast<const uint8_t*>(k);
  const uint8_t* v8 = static_cast<const uint8_t*>(v);
  uint8_t* out8 = static_cast<uint8_t*>(out);
  const int64_t qrow = static_cast<int64_t>(n_heads) * 192;
  const int64_t vrow = static_cast<int64_t>(n_heads) * 128;
  const int64_t orow = static_cast<int64_t>(n_heads) * 128 * 2;

  std::vector<Part> parts;
  for (int64_t r0 = 0; r0 < lq; r0 += seg) {
    const int64_t r1 = std::min(lq, r0 + seg);
    const int64_t rows = r1 - r0;
    if (!chunk_parts(lq, lk, seg, causal, r0, r1, parts))
      return mla::fail(MLA_ERR_INVALID_ARGUMENT, "no chunk plan");
    group_parts(parts, (rows + kPrefillRows - 1) / kPrefillRows * n_heads);
    const int n = static_cast<int>(parts.size());
    if (n == 1) {
      // a single part is written straight into the output rows
      const Part& pt = parts[0];
      mla::PrefillArgs a{q8 + r0 * qrow, k8 + pt.k0 * qrow, v8 + pt.k0 * vrow, nullptr, nullptr,
                         1, static_cast<int32_t>(rows), rows, pt.k1 - pt.k0, n_heads, descale_q,
                         descale_k, descale_v, softmax_scale, pt.causal, out8 + r0 * orow, 0,
                         lse ? lse + r0 : nullptr, lse_stride};
      st = mla::prefill_launch(a, s);
      if (st != MLA_OK) return st;
      continue;
    }
    // all parts of this query chunk in ONE launch (fp32 partials in the workspace),
    // non-causal segments first (the plan lists the causal diagonal last), merged by the
    // launch itself into the chunk's output rows
    if (!counters_zeroed) {
      st = mla::zero_ints(counters, counter_bytes(rows_max, n_heads) / 4, s);
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
    mla::PrefillArgs a{q8 + r0 * qrow, k8, v8, nullptr, nullptr, 1, static_cast<int32_t>(rows),
                       rows, lk, n_heads, descale_q, descale_k, descale_v, softmax_scale, 0,
                       out8 + r0 * orow, 1, lse ? lse + r0 : nullptr, lse_stride, rows, counters};
    st = mla::prefill_launch_segments(a, segs, n, s);
    if (st != MLA_OK) return st;
  }
  return mla::ok();
}
