// FP8 varlen context-prefill attention for MLA shapes (Q/K 192, V 128) on gfx950.
//
// "[ROCm][MLA] Add guarded gfx942 FP8 context prefill" (vLLM #51551):
// Background (a packed variable-length kernel for D192 Q/K and D128 V with
// per-head static FP8 quantization) and "What this PR does" (12 heads, FP8
// Q/K/V); the close comment separates causal and non-causal shapes.
//
// Design (gfx950, wave64):
//  * One workgroup = 8 waves = 256 query rows of one (sequence, head); each wave owns
//    32 rows; one workgroup per CU, two waves per SIMD, so one wave's VALU work fills the
//    other's MFMA time. Every K/V tile a workgroup loads and converts serves 256 rows
//    (4-wave workgroups of 128 rows, two per CU, are a second build of this source: 5 %
//    slower on the 32K causal prefill, faster on grids that leave CUs idle or are mostly
//    padding, which prefill_launch hands to it). Workgroups are ordered heaviest first:
//    the flattened block index walks query tiles from the last (most keys under a causal
//    mask) to the first, with heads and sequences fastest.
//  * 64-key K tiles and FP8 V tiles live in two LDS buffers each, filled by
//    global->LDS DMA (global_load_lds_dwordx4, no register staging). K rows are padded to
//    208 bytes; V rows are 128 bytes with XOR-swizzled 16-byte chunks (see v_swizzle).
//    Iteration t issues the S MFMAs of tile t+1 with the row max of tile t and the
//    conversion of V tile t to bf16 V^T (two V^T buffers) between them, then the loads of
//    K(t+2) and V(t+1), then the PV MFMAs of tile t-1 with the exponentials of tile t
//    between them (exponentials co-issue with bf16 MFMAs, hardly with FP8 ones);
//    one barrier per tile.
//  * S^T = K * Q^T on v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3 -> fp32): the Q fragment
//    (32 rows x 192) stays in registers as the B operand, K rows are read from LDS as
//    the A operand. In the 32x32 accumulator layout every lane holds one query row
//    (lane % 32) and 32 of the tile's keys, so a row max needs one cross-lane step
//    (lane ^ 32) and row sums stay per lane until the end.
//  * Online softmax in base 2: c = dq*dk*softmax_scale*log2(e) > 0, so the tile max is
//    taken on raw logits and scaled once; P = 2^(c*s - m) is one FMA and one v_exp_f32
//    per element. The reference max m moves only when a row's max exceeds it by more
//    than kRescaleSlack (a rare wave-uniform branch rescales l, and O once the previous
//    tile's PV has been added).
//  * O^T = V^T * P^T on v_mfma_f32_32x32x16_bf16 with P rounded to bf16 (one term: an
//    E4M3 P carries up to 2^-4 relative error per weight, more than the output tolerance
//    allows on diffuse heads, and two E4M3 terms cost more VALU work than this path).
//    Registers 8 ck .. 8 ck + 7 of an S accumulator are one P^T B operand (16 keys). V
//    stays FP8 in HBM and LDS: the waves read 32-dim blocks of the tile with
//    ds_read_b64_tr_b8 (within each 16-lane group, output lane i receives byte i % 8 of
//    the 8-byte windows addressed by lanes 2b + i/8, so lane i gets dim d0 + i of 8 keys
//    in the key order of the P operand), convert them exactly to bf16
//    (v_cvt_scalef32_pk_bf16_fp8) and store them as V^T rows; the keys a lane converts
//    are exactly those its own PV A operands need, so every A operand is one 16-byte
//    read. The conversion is shared by the workgroup: waves w and w + 4 convert the two
//    key halves of dim block w % 4, 8 conversions per lane per tile.
//  * Causal (bottom-right aligned: key j visible to row i iff j <= i + Lk - Lq):
//    a wave skips tiles past its last visible key; only tiles that cross the
//    diagonal or the ragged end are masked element-wise.
//  * Epilogue: out = O * dv / l in bf16 (fp32 for the partials of a chunked pass),
//    lse = ln2 * (m + log2 l). A launch over several key segments merges its own
//    partials: the last workgroup of each (query tile, head) to finish combines them
//    (merge_on_last_arrival).
#include <stdlib.h>

#include <algorithm>

#include "mla_internal.h"
#include "device_common.h"

namespace {

using namespace mla::dev;

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int kDqk = 192;
constexpr int kDv = 128;
// The library holds this source twice: the default 8-wave build, and a 4-wave build
// (MLA_PREFILL_SMALL_GRID) that exports only mla::prefill_launch_small, to which the
// default build hands grids that would leave CUs idle or are mostly padding (see
// prefill_launch).
#ifndef MLA_PREFILL_WAVES
#define MLA_PREFILL_WAVES 8
#endif
constexpr int kWaves = MLA_PREFILL_WAVES;  // waves per workgroup
constexpr int kWgPerCu = 8 / kWaves;       // resident workgroups per CU (2 waves per SIMD)
static_assert(kWaves == 4 || kWaves == 8, "4 or 8 waves per workgroup");
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // query rows per workgroup
constexpr int kBN = 64;           // keys per tile
constexpr int kKStride = 208;     // LDS bytes per K row: 192 + 16 (8 consecutive rows hit distinct banks)
constexpr int kVStride = 128;     // LDS bytes per V row, 16-byte chunks XOR-swizzled by key
constexpr int kKTile = kBN * kKStride;
constexpr int kVTile = kBN * kVStride;
// bf16 V^T of one tile: one row per dim, 64 keys (two halves of 32, see the header) + pad;
// rows 144 bytes apart, so the 16-byte reads of 16 consecutive dims hit distinct banks
constexpr int kVtStride = 144;
constexpr int kVtBytes = kDv * kVtStride;
// PV arithmetic, a build option: 0 (default) P rounded once to bf16 and V converted to
// bf16 in LDS, on v_mfma_f32_32x32x16_bf16; 1: P' = 2^8 P rounded once to E4M3 (one
// term) and V used as its FP8 codes, on the FP8 MFMA; 2: P' in two E4M3 terms
// (hi + lo, both summed into O) on the FP8 MFMA.
#ifndef MLA_PV_MODE
#define MLA_PV_MODE 0
#endif
constexpr int kPvMode = MLA_PV_MODE;
static_assert(kPvMode >= 0 && kPvMode <= 2, "MLA_PV_MODE is 0, 1 or 2");
constexpr bool kPvFp8 = kPvMode != 0;
constexpr int kLdsBytes =  // bf16 PV: 79872 (two workgroups per CU)
    kPvFp8 ? 2 * (kKTile + kVTile) : 2 * (kKTile + kVTile + kVtBytes);
constexpr float kLn2 = 0.69314718055994530942f;
// P = 2^(logit*log2e - m) <= 2^kRescaleSlack. As a bf16 operand the slack only bounds O;
// the E4M3 operand is P' = 2^8 P <= 2^8.75 < 448, and small weights stay clear of the
// E4M3 subnormals.
constexpr float kRescaleSlack = kPvFp8 ? 0.75f : 8.0f;

struct PrefillParams {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const float* dq;
  const float* dk;
  const float* dv;
  void* out;
  float* lse;
  int64_t lse_stride;
  int64_t total_q;
  int64_t total_k;
  int32_t batch;
  int32_t n_heads;
  int32_t n_m_tiles;
  int32_t causal;
  int32_t out_f32;  // 1: out is fp32 (partials of a chunked pass), 0: bf16
  int32_t xcd_order;  // 1: XCD-aware block order (one sequence, H % 4 == 0, even tile count)
  float scale_log2;
  // multi-segment launches: row stride of the segments' partial LSEs, and (if not null)
  // one arrival counter per (query tile, head), all zero at launch: the last workgroup of
  // a tile to finish merges the segments' fp32 partials into out (bf16) and lse
  // (lse_stride) and sets the counter back to zero
  int64_t seg_lse_stride;
  int32_t* counters;
};

// Context segments of a multi-segment launch (see mla::PrefillSegment); N = 1 for the
// ordinary launch, whose table is unused.
struct SegDev {
  int64_t k0;
  int32_t lk;
  int32_t causal;
  void* out;
  float* lse;
};
template <int N>
struct SegTable {
  int32_t n;
  SegDev e[N];
};

__device__ __forceinline__ v16f mfma_f8(const v8i& a, const v8i& b, const v16f& c) {
  // cbsz = blgp = 0: both operands E4M3; zero scales select the unscaled instruction
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v16f mfma_bf16(const v8bf& a, const v8bf& b, const v16f& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v8i load32(const uint8_t* p) {
  const v4i a = *reinterpret_cast<const v4i*>(p);
  const v4i b = *reinterpret_cast<const v4i*>(p + 16);
  return v8i{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
}

__device__ __forceinline__ v2i read_tr8(const uint8_t* lds_ptr) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) v2i*)(lds_ptr));
}

// Partials of a launch that merges its own segments are exchanged between workgroups on
// different XCDs, whose L2 caches are not coherent with each other. They are written and
// read with agent-coherent accesses (the sc1 form the compiler gives agent-scope atomic
// loads and stores), so neither side needs a whole-L2 write-back or invalidate.
__device__ __forceinline__ void store16_agent(float* ptr, float4 v) {
  typedef float v4f __attribute__((ext_vector_type(4)));
  const v4f d = {v.x, v.y, v.z, v.w};
  asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(ptr), "v"(d) : "memory");
}
__device__ __forceinline__ float load_agent(const float* ptr) {
  return __hip_atomic_load(ptr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// eight consecutive floats (32-byte aligned) as four agent-coherent 8-byte loads
__device__ __forceinline__ void load8_agent(const float* ptr, float (&x)[8]) {
  const uint64_t* q = reinterpret_cast<const uint64_t*>(ptr);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint64_t v = __hip_atomic_load(q + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    x[2 * i] = __uint_as_float(static_cast<uint32_t>(v));
    x[2 * i + 1] = __uint_as_float(static_cast<uint32_t>(v >> 32));
  }
}

// S^T block for one tile: two 32-key blocks, K-dim 192 = 3 x 64
__device__ __forceinline__ void qk_tile(const uint8_t* kl, int col, int g, const v8i qf[3],
                                        v16f s[2]) {
#pragma unroll
  for (int b2 = 0; b2 < 2; ++b2) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[b2][r] = 0.f;
#pragma unroll
    for (int kb = 0; kb < 3; ++kb) {
      const v8i a = load32(kl + (32 * b2 + col) * kKStride + 64 * kb + 32 * g);
      s[b2] = mfma_f8(a, qf[kb], s[b2]);
    }
  }
}

// V tiles are stored with unpadded 128-byte rows; the 16-byte chunk c of key row k sits at
// position c ^ v_swizzle(k). For the transposed reads (8 keys x two 16-byte halves of a
// 32-dim block per 16 lanes) this spreads every group of 16 or 32 lanes over distinct
// banks, with 32 or with 64 four-byte banks.
__device__ __forceinline__ int v_swizzle(int key) { return (key & 3) | (((key >> 3) & 1) << 2); }

// Fused LSE merge of a multi-segment launch. Every workgroup of query tile m_tile and
// head h has written its segment's fp32 partial out and LSE (agent-coherent stores, all
// completed before the workgroup's barrier); the last of the st.n workgroups of that
// tile to count its arrival combines them for the tile's rows [row0, row0 + rows):
//   L = ln sum_s exp(L_s),  out = sum_s exp(L_s - L) * out_s   (all L_s = -inf: 0, -inf)
// with the arithmetic of the separate merge kernel (same order over s), reading the
// partials with agent-coherent loads issued after the counter returned.
constexpr int kMergeBatch = 4;  // segments whose partials a merge loads at once

template <int kNSeg>
__device__ __forceinline__ void merge_on_last_arrival(const PrefillParams& p,
                                                      const SegTable<kNSeg>& st, int h, int m_tile,
                                                      int row0, int rows) {
  __shared__ int last;
  const int tid = threadIdx.x;
  int32_t* counter = p.counters + static_cast<int64_t>(m_tile) * p.n_heads + h;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's partial stores are done
  __syncthreads();                                  // ... and every other wave's
  if (tid == 0)
    last = (__hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
            st.n - 1) ? 1 : 0;
  __syncthreads();
  if (!last) return;
  if (tid == 0)  // ready for the next launch on this stream
    __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int H = p.n_heads;
  const int n = st.n;
  for (int item = tid; item < rows * 16; item += kThreads) {
    const int64_t row = row0 + (item >> 4);
    const int c8 = item & 15;
    const int64_t li = static_cast<int64_t>(h) * p.seg_lse_stride + row;
    const int64_t eo = (row * H + h) * kDv + 8 * c8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float tot = 0.f;
    float m = -INFINITY;
    // The loads of up to kMergeBatch segments are issued together, so that a row waits
    // for memory once when its segments fit one batch, else twice per batch (the LSEs for
    // the maximum, then LSEs and partials), rather than twice per segment; the arithmetic
    // and its order over s are unchanged.
    if (n <= kMergeBatch) {
      float lv[kMergeBatch], x[kMergeBatch][8];
#pragma unroll
      for (int j = 0; j < kMergeBatch; ++j) {
        lv[j] = -INFINITY;
        if (j < n) {
          lv[j] = load_agent(st.e[j].lse + li);
          load8_agent(static_cast<const float*>(st.e[j].out) + eo, x[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < kMergeBatch; ++j)
        if (j < n) m = fmaxf(m, lv[j]);
      if (m != -INFINITY) {
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) {
          if (j < n) {
            const float w = __expf(lv[j] - m);  // 0 for an empty segment
            tot += w;
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] += w * x[j][i];
          }
        }
      }
    } else {
      for (int s0 = 0; s0 < n; s0 += kMergeBatch) {
        float lv[kMergeBatch];
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j)
          lv[j] = (s0 + j < n) ? load_agent(st.e[s0 + j].lse + li) : -INFINITY;
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j)
          if (s0 + j < n) m = fmaxf(m, lv[j]);
      }
      if (m != -INFINITY) {
        for (int s0 = 0; s0 < n; s0 += kMergeBatch) {
          float lv[kMergeBatch], x[kMergeBatch][8];
#pragma unroll
          for (int j = 0; j < kMergeBatch; ++j) {
            lv[j] = -INFINITY;
            if (s0 + j < n) {
              lv[j] = load_agent(st.e[s0 + j].lse + li);
              load8_agent(static_cast<const float*>(st.e[s0 + j].out) + eo, x[j]);
            }
          }
#pragma unroll
          for (int j = 0; j < kMergeBatch; ++j) {
            if (s0 + j < n) {
              const float w = __expf(lv[j] - m);  // 0 for an empty segment
              tot += w;
#pragma unroll
              for (int i = 0; i < 8; ++i) acc[i] += w * x[j][i];
            }
          }
        }
      }
    }
    const float inv = (m != -INFINITY) ? 1.0f / tot : 0.0f;
    uint4 o;
    o.x = mla::f32_to_bf16_rne(acc[0] * inv) | (mla::f32_to_bf16_rne(acc[1] * inv) << 16);
    o.y = mla::f32_to_bf16_rne(acc[2] * inv) | (mla::f32_to_bf16_rne(acc[3] * inv) << 16);
    o.z = mla::f32_to_bf16_rne(acc[4] * inv) | (mla::f32_to_bf16_rne(acc[5] * inv) << 16);
    o.w = mla::f32_to_bf16_rne(acc[6] * inv) | (mla::f32_to_bf16_rne(acc[7] * inv) << 16);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.out) + eo) = o;
    if (c8 == 0 && p.lse != nullptr)
      p.lse[static_cast<int64_t>(h) * p.lse_stride + row] =
          (m != -INFINITY) ? m + __logf(tot) : -INFINITY;
  }
}

// kPv (= MLA_PV_MODE) only names the build variant, so that kernel traces keep them apart
template <int kNSeg, int kPv>
#ifdef MLA_PREFILL_SMALL_GRID
#define prefill_fp8_kernel prefill_fp8_4w_kernel  // its own name in kernel traces
#endif
__global__ __launch_bounds__(kThreads, kWgPerCu) void prefill_fp8_kernel(PrefillParams p,
                                                                        SegTable<kNSeg> st) {
  static_assert(kPv == kPvMode, "the PV arithmetic is chosen at build time");
  // K tile t, FP8 V tile t and bf16 V^T of tile t each in buffer t % 2 of their kind
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int H = p.n_heads;

  int h, b = 0, m_tile;
  int64_t q0 = 0, q1 = p.total_q, k0 = 0, k1 = p.total_k;
  bool causal = p.causal != 0;
  void* out_ptr = p.out;
  float* lse_ptr = p.lse;
  if constexpr (kNSeg > 1) {
    // multi-segment launch: segments in the host's order (heaviest first); within a
    // segment the XCD-aware order of the single-sequence launch below (its block range
    // starts at a multiple of 8, so block % 8 is still the XCD), else query tiles from the
    // last, heads fastest
    const int per_seg = p.n_m_tiles * H;
    const int e = blockIdx.x / per_seg;
    const int local = blockIdx.x - e * per_seg;
    if (p.xcd_order) {
      const int hp = H >> 2;
      const int slot = local >> 3;
      const int half = hp * (local & 7) + slot % hp;
      h = half >> 1;
      m_tile = p.n_m_tiles - 2 + (half & 1) - 2 * (slot / hp);
    } else {
      h = local % H;
      m_tile = p.n_m_tiles - 1 - local / H;
    }
    const SegDev& sg = st.e[e];
    k0 = min(max(sg.k0, (int64_t)0), p.total_k);
    k1 = min(k0 + sg.lk, p.total_k);
    causal = sg.causal != 0;
    out_ptr = sg.out;
    lse_ptr = sg.lse;
  } else if (p.xcd_order) {
    // One sequence: workgroups are dealt round-robin to the 8 XCDs (block % 8). Each
    // head's query tiles are split into an even and an odd half (equal causal work) and
    // each XCD takes H/4 consecutive half-heads, heaviest tile first, so its L2 serves
    // the K/V of about H/8 heads instead of H/4 spread over all XCDs. (A bijection of
    // the grid whatever the dispatch order.)
    const int hp = H >> 2;                 // half-heads per XCD
    const int xcd = blockIdx.x & 7;
    const int slot = blockIdx.x >> 3;
    const int half = hp * xcd + slot % hp;  // 0 .. 2H-1
    const int rank = slot / hp;             // 0 .. n_m/2 - 1
    h = half >> 1;
    m_tile = p.n_m_tiles - 2 + (half & 1) - 2 * rank;
  } else {
    // heaviest query tiles first; within a tile index, the (sequence, head) pairs with
    // heads fastest, rotated by 3 per tile index: blocks go to XCD block % 8, and with a
    // multiple of 8 pairs per tile index an unrotated order would give each XCD the same
    // pairs at every tile index (sequences of unequal length: unequal XCD loads; measured
    // on 8 packed sequences of 808-3946 tokens, 6 % faster rotated)
    const int pairs = H * p.batch;
    const int mi = blockIdx.x / pairs;
    const int pr = (blockIdx.x - mi * pairs + 3 * mi) % pairs;
    h = pr % H;
    b = pr / H;
    m_tile = p.n_m_tiles - 1 - mi;
  }

  // packed sequences from cu_seqlens, or one sequence spanning all tokens
  if (kNSeg == 1 && p.cu_q != nullptr) {
    q0 = p.cu_q[b];
    q1 = p.cu_q[b + 1];
    k0 = p.cu_k[b];
    k1 = p.cu_k[b + 1];
  }
  q0 = min(max(q0, (int64_t)0), p.total_q);
  q1 = min(max(q1, q0), p.total_q);
  k0 = min(max(k0, (int64_t)0), p.total_k);
  k1 = min(max(k1, k0), p.total_k);
  const int Lq = static_cast<int>(q1 - q0);
  const int Lk = static_cast<int>(k1 - k0);
  const int row0 = m_tile * kBM;
  if (row0 >= Lq) return;  // uniform over the workgroup
  const int off = Lk - Lq;
  int kend = Lk;
  if (causal) kend = min(Lk, max(0, min(Lq, row0 + kBM) + off));
  const int n_tiles = (kend + kBN - 1) / kBN;

  const int g = lane >> 5;
  const int col = lane & 31;
  const int wrow0 = row0 + wave * 32;
  const int my_row = wrow0 + col;
  const bool row_ok = my_row < Lq;
  // tiles this wave computes: [0, wave_tiles)
  int wave_kend = (wrow0 < Lq) ? kend : 0;
  if (causal && wrow0 < Lq) wave_kend = min(Lk, max(0, min(Lq, wrow0 + 32) + off));
  const int wave_tiles = (wave_kend + kBN - 1) / kBN;
  const int wave_iters = wave_tiles > 0 ? wave_tiles + 1 : 0;  // + the trailing PV

  const int64_t q_rs = static_cast<int64_t>(H) * kDqk;
  const int64_t k_rs = static_cast<int64_t>(H) * kDqk;
  const int64_t v_rs = static_cast<int64_t>(H) * kDv;

  // Q fragment (B operand): row my_row, dims [64*kb + 32*g, +32)
  v8i qf[3];
  if (row_ok) {
    const uint8_t* qp = p.q + (q0 + my_row) * q_rs + h * kDqk + 32 * g;
#pragma unroll
    for (int kb = 0; kb < 3; ++kb) qf[kb] = load32(qp + 64 * kb);
  } else {
#pragma unroll
    for (int kb = 0; kb < 3; ++kb) qf[kb] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  }

  const float c = p.dq[h] * p.dk[h] * p.scale_log2;
  float m_run = -INFINITY;
  float l_run = 0.f;  // this lane's part of the row sum (its 32 keys of every tile)
  v16f o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;

  const uint8_t* kbase = uniform_ptr(p.k + k0 * k_rs + h * kDqk);
  const uint8_t* vbase = uniform_ptr(p.v + k0 * v_rs + h * kDv);

  // Tile fill by direct global->LDS loads (global_load_lds_dwordx4): one wave
  // instruction writes 64 consecutive 16-byte LDS slots, lane l to slot l, from any
  // per-lane global address. A K tile is 64 rows x 13 slots (12 data + 1 pad), a V tile
  // 64 rows x 8 slots (chunks swizzled); the 13 K and the 8 V instructions of a tile are
  // dealt round-robin to the waves. Pad slots load a duplicate chunk; rows past the
  // sequence load its last row (K logits there are masked to -inf and their P is 0, so
  // the duplicate never contributes, and no uninitialised bytes are ever read).
  //
  // Schedule: K, V and V^T of tile t live in buffer t % 2 of their kind. Iteration t
  // reads K(t+1) (S of the next tile), V(t) (converted to V^T) and the V^T of tile t-1
  // (PV of the previous tile), and issues K(t+2) and V(t+1) after its S MFMAs, into the
  // buffers that K(t) and V(t-1) left at the previous barrier; they land before the
  // iteration's closing barrier.
  constexpr int kKInstr = kBN * (kKStride / 16) / 64;  // 13
  constexpr int kVInstr = kBN * (kVStride / 16) / 64;  // 8
  constexpr int kPerK = (kKInstr + kWaves - 1) / kWaves;
  constexpr int kPerV = (kVInstr + kWaves - 1) / kWaves;
  // Slot j of a K (V) tile (instruction i = wave + j * kWaves): this lane's tile row and
  // the byte offset of its chunk within the row. Full tiles use a wave-uniform 64-bit tile
  // base plus row * row_stride + chunk (< 64 * H * 192 < 2^31, checked on the host); the
  // ragged last tile clamps rows.
  auto dma_row = [&](int j, bool is_k) {
    const int slot = (wave + j * kWaves) * 64 + lane;
    if (is_k) {
      const int row = slot / 13;
      const int chunk = min(slot - 13 * row, 11);  // pad slot -> last data chunk
      return make_int2(row, 16 * chunk);
    }
    const int row = slot >> 3;  // V: LDS position slot & 7 holds chunk position ^ swizzle
    return make_int2(row, 16 * ((slot & 7) ^ v_swizzle(row)));
  };
  const uint32_t k_rs32 = static_cast<uint32_t>(k_rs), v_rs32 = static_cast<uint32_t>(v_rs);
  uint32_t dma_off_k[kPerK], dma_off_v[kPerV];
#pragma unroll
  for (int j = 0; j < kPerK; ++j) {
    const int2 rc = dma_row(j, true);
    dma_off_k[j] = static_cast<uint32_t>(rc.x) * k_rs32 + static_cast<uint32_t>(rc.y);
  }
#pragma unroll
  for (int j = 0; j < kPerV; ++j) {
    const int2 rc = dma_row(j, false);
    dma_off_v[j] = static_cast<uint32_t>(rc.x) * v_rs32 + static_cast<uint32_t>(rc.y);
  }
  auto kbuf = [&](int t) { return lds + (t & 1) * kKTile; };
  auto vbuf = [&](int t) { return lds + 2 * kKTile + (t & 1) * kVTile; };
  auto vtbuf = [&](int t) { return lds + 2 * (kKTile + kVTile) + (t & 1) * kVtBytes; };
  // issue this wave's loads of the K (is_k) or V part of tile t
  auto issue = [&](int t, bool is_k) {
    const int kt = t * kBN;
    const int64_t rs = is_k ? k_rs : v_rs;
    const uint32_t rs32 = is_k ? k_rs32 : v_rs32;
    const uint8_t* base = uniform_ptr((is_k ? kbase : vbase) + static_cast<int64_t>(kt) * rs);
    const uint32_t dst0 = lds_address(is_k ? kbuf(t) : vbuf(t));
    const int n_instr = is_k ? kKInstr : kVInstr;
    const bool full = kt + kBN <= Lk;
#pragma unroll
    for (int j = 0; j < (is_k ? kPerK : kPerV); ++j) {
      const int i = wave + j * kWaves;  // wave-uniform
      if (i < n_instr) {
        uint32_t off = is_k ? dma_off_k[j] : dma_off_v[j < kPerV ? j : 0];
        if (!full) {  // ragged last tile: rows past the sequence re-read its last row
          const int2 rc = dma_row(j, is_k);
          off = static_cast<uint32_t>(min(rc.x, Lk - 1 - kt)) * rs32 + static_cast<uint32_t>(rc.y);
        }
        dma_load16(base, off, dst0 + 1024u * static_cast<uint32_t>(i));
      }
    }
  };

  // transposed-read addresses (see the header): lane -> (16-lane group, source slot)
  const int grp = lane >> 4, slot = lane & 15;
  const int tb = slot >> 1, tp = slot & 1;
  // key of read r (r = 0..3) is 16 r + key0; the 16 r part is an immediate offset
  // (keys vt_key0 + 16 r share the swizzle; block db of 32 dims flips address bits 5..6)
  const int vt_key0 = 8 * (tb >> 2) + 4 * (grp >> 1) + (tb & 3);
  const int vt_off = vt_key0 * kVStride + 16 * ((grp & 1) ^ v_swizzle(vt_key0)) + 8 * tp;

  // prologue: K(0), V(0), K(1) in LDS, S of tile 0 computed, the V^T buffer that
  // iteration 0 reads zeroed (it multiplies a zero P: no uninitialised LDS reaches an MFMA)
  if constexpr (kPvFp8) {
    // FP8 PV reads the FP8 V tile of the previous iteration: V buffer 1 stands for tile -1
    for (int i = tid; i < kVTile / 16; i += kThreads)
      reinterpret_cast<uint4*>(vbuf(1))[i] = make_uint4(0, 0, 0, 0);
    if (n_tiles > 0) issue(0, true);
  } else {
    for (int i = tid; i < kVtBytes / 16; i += kThreads)
      reinterpret_cast<uint4*>(vtbuf(1))[i] = make_uint4(0, 0, 0, 0);
    if (n_tiles > 0) { issue(0, true); issue(0, false); }
  }
  if (n_tiles > 1) issue(1, true);
  wait_vmcnt(0);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the zero stores have landed
  // retire the Q-fragment loads here on every path (an empty asm that reads the
  // registers), so that no compiler-inserted memory wait is left inside the loop
#pragma unroll
  for (int kb = 0; kb < 3; ++kb) asm volatile("" ::"v"(qf[kb]));
  block_barrier();
  v16f s_cur[2];
  if (wave_tiles > 0) qk_tile(kbuf(0), col, g, qf, s_cur);
  block_barrier();  // K(0) is read: iteration 0 may load K(2) into its buffer

  static_assert(kWaves == 4 || kWaves == 8, "the waves split the V conversion evenly");
  // V conversion: wave w converts dim block w & 3; with 4 waves both key halves of it,
  // with 8 waves the half w >> 2
  const int conv_db = wave & 3;
  const v2bf ones2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  // Softmax of two keys: S block b2, accumulator registers 8 ck + 2 i and 8 ck + 2 i + 1.
  // P = 2^(c*s + nbias) rounded to bf16 (nearest even) fills elements 2 i, 2 i + 1 of the
  // B operand of one bf16 PV MFMA (registers 8 ck .. 8 ck + 7 of S block b2 make one
  // operand: MFMA k-index 8 g + i stands for key 32 b2 + 16 ck + 8 (i / 4) + 4 g + i % 4);
  // the row sum adds the rounded weights.
  auto softmax_pair = [&](const v16f(&sc)[2], float nbias, int b2, int ck, int i, v8bf& pb) {
    const float e0 = __builtin_amdgcn_exp2f(fmaf(sc[b2][8 * ck + 2 * i], c, nbias));
    const float e1 = __builtin_amdgcn_exp2f(fmaf(sc[b2][8 * ck + 2 * i + 1], c, nbias));
    const v2bf pr = __builtin_convertvector(v2f{e0, e1}, v2bf);
    l_run = __builtin_amdgcn_fdot2_f32_bf16(pr, ones2, l_run, false);
    pb[2 * i] = pr[0];
    pb[2 * i + 1] = pr[1];
    // pin the pair here: its result is only read in the next iteration, and the compiler
    // would otherwise sink it below the MFMAs it is meant to overlap
    asm volatile("" ::"v"(pr), "v"(l_run));
  };
  // The transposed reads give lane (g, col) dim 32 db + col of the 32 keys
  // 32 b2 + 8 q + 4 g + i at byte 16 b2 + 4 q + i (b2, q, i = 0..1, 0..3, 0..3).
  // Wave w converts dims 32 w .. 32 w + 31 of FP8 V tile t to the bf16 V^T buffer: row
  // 32 w + col, bytes 64 g .. 64 g + 63 hold the lane's 32 keys in the order above. The
  // keys that lane (g, col) converts are exactly those its PV A operands need, so PV
  // operand (db, b2, ck) is the 16 bytes at 64 g + 32 b2 + 16 ck of row 32 db + col.
  // The conversion in two parts, so that each fills a gap between FP8 MFMAs: the
  // transposed reads of key half `half` (the keys of S block b2 = half), then the
  // conversion and the two V^T stores.
  auto conv_read = [&](int t, int half) {
    const uint8_t* vp = vbuf(t) + (vt_off ^ (conv_db << 5)) + 32 * half * kVStride;
    const v2i r0 = read_tr8(vp);
    const v2i r1 = read_tr8(vp + 16 * kVStride);
    return v4i{r0.x, r0.y, r1.x, r1.y};
  };
  auto conv_write = [&](int t, int half, const v4i& raw) {
    uint8_t* dst = vtbuf(t) + (32 * conv_db + col) * kVtStride + 64 * g + 32 * half;
    uint32_t cv[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      cv[2 * w] = __builtin_bit_cast(
          uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[w], 1.0f, false));
      cv[2 * w + 1] = __builtin_bit_cast(
          uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[w], 1.0f, true));
    }
    *reinterpret_cast<uint4*>(dst) = make_uint4(cv[0], cv[1], cv[2], cv[3]);
    *reinterpret_cast<uint4*>(dst + 16) = make_uint4(cv[4], cv[5], cv[6], cv[7]);
  };
  auto convert_half = [&](int t, int half) { conv_write(t, half, conv_read(t, half)); };
  auto vt_read = [&](const uint8_t* vt, int db, int b2, int ck) {
    return *reinterpret_cast<const v8bf*>(vt + (32 * db + col) * kVtStride + 64 * g + 32 * b2 +
                                          16 * ck);
  };
  // K operand of S MFMA k (k = 0..5 alternates the two 32-key blocks: consecutive MFMAs
  // write different accumulators)
  auto k_operand = [&](const uint8_t* kl, int k) {
    const int b2 = k & 1, kb = k >> 1;
    return load32(kl + (32 * b2 + col) * kKStride + 64 * kb + 32 * g);
  };
  // One software-pipelined iteration. S of tile it is in s_c, the bf16 P of tile it-1 in
  // pb_p and its V^T in V^T buffer (it-1) % 2 (on iteration 0: zero P and a zeroed
  // buffer). It first issues the 6 S MFMAs of tile it+1 with the VALU work that needs no
  // exponentials spread between them (mask and row max of S block 0; row max of block 1;
  // rescale test; transposed reads of V tile it; their conversion to V^T buffer it % 2),
  // then the loads of K(it+2) and V(it+1) into the buffers that K(it) and V(it-1) left at
  // the previous barrier, then the 16 PV MFMAs of tile it-1 with
  // one softmax pair of tile it (P to pb_c) after each: exponentials overlap bf16 MFMAs
  // well and FP8 MFMAs poorly. LDS operands are read three PV MFMAs (V^T) or one S MFMA
  // (K) ahead of use. A wave runs wave_tiles + 1 active iterations: the last one is a
  // fully masked tile that only completes the PV of its last tile. Every wave takes part
  // in every conversion. One barrier per iteration; all loads land before it.
  auto step = [&](int it, v16f(&s_c)[2], v16f(&s_n)[2], const v8bf(&pb_p)[4], v8bf(&pb_c)[4]) {
    const bool active = it < wave_iters;
    const bool convert = it < n_tiles;
    const uint8_t* kl = kbuf(it + 1);
    const uint8_t* vt = vtbuf(it - 1);
    v8bf va[3];
    v8i ka;
    if (active) {
      va[0] = vt_read(vt, 0, 0, 0);
      va[1] = vt_read(vt, 1, 0, 0);
      va[2] = vt_read(vt, 2, 0, 0);
      ka = k_operand(kl, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (!active) {
      if (it + 2 < n_tiles) issue(it + 2, true);
      if (it + 1 < n_tiles) issue(it + 1, false);
    }

    if (active) {
      const int kt = it * kBN;
      const bool need_mask =
          it >= wave_tiles || (kt + kBN > Lk) || (causal && kt + kBN - 1 > wrow0 + off);
      // S MFMA k writes accumulator k & 1 with Q fragment k >> 1; the first two start from 0
      const v16f zero = {};
      s_n[0] = mfma_f8(ka, qf[0], zero);
      ka = k_operand(kl, 1);
      __builtin_amdgcn_sched_barrier(0);
      if (need_mask) {
        // side-effect barrier: keeps this rare block a real branch (the compiler would
        // otherwise if-convert it into selects executed on every tile)
        asm volatile("" ::: "memory");
        const bool all = it >= wave_tiles;  // the trailing tile: nothing visible
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kt + 32 * b2 + 8 * (r >> 2) + 4 * g + (r & 3);
            if (all || key >= Lk || (causal && key > my_row + off)) s_c[b2][r] = -INFINITY;
          }
      }
      // the row max of S block 0, S MFMA 1, that of block 1, S MFMA 2
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = vmax3(mx, s_c[0][r], s_c[0][r + 1]);
      __builtin_amdgcn_sched_barrier(0);
      s_n[1] = mfma_f8(ka, qf[0], zero);
      ka = k_operand(kl, 2);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = vmax3(mx, s_c[1][r], s_c[1][r + 1]);
      __builtin_amdgcn_sched_barrier(0);
      s_n[0] = mfma_f8(ka, qf[1], s_n[0]);
      ka = k_operand(kl, 3);
      __builtin_amdgcn_sched_barrier(0);
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                         false, false);
        mx = __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      const float m_tile = mx * c;  // c > 0; -inf stays -inf
      // Lazy rescale: keep the reference max m_run unless some row's max exceeds it by
      // more than kRescaleSlack. The row sum is rescaled now; O after the PV of the
      // previous tile (computed against the old reference) has been added.
      const bool rescale = __any(m_tile > m_run + kRescaleSlack);
      float alpha = 1.f;
      if (rescale) {
        asm volatile("" ::: "memory");  // keep the rescale a real branch (see above)
        const float m_new = fmaxf(m_run, m_tile);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        alpha = __builtin_amdgcn_exp2f(m_run - m_use);  // 0 while m_run is -inf
        l_run *= alpha;
        m_run = m_new;
      }
      const float nbias = (m_run == -INFINITY) ? 0.f : -m_run;

      // S MFMA 3, the transposed V reads, S MFMA 4, the conversion, S MFMA 5
      __builtin_amdgcn_sched_barrier(0);
      s_n[1] = mfma_f8(ka, qf[1], s_n[1]);
      ka = k_operand(kl, 4);
      __builtin_amdgcn_sched_barrier(0);
      v4i craw0, craw1;
      if (convert) {
        craw0 = conv_read(it, kWaves == 4 ? 0 : wave >> 2);
        if constexpr (kWaves == 4) craw1 = conv_read(it, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      s_n[0] = mfma_f8(ka, qf[2], s_n[0]);
      ka = k_operand(kl, 5);
      __builtin_amdgcn_sched_barrier(0);
      if (convert) {
        conv_write(it, kWaves == 4 ? 0 : wave >> 2, craw0);
        if constexpr (kWaves == 4) conv_write(it, 1, craw1);
      }
      __builtin_amdgcn_sched_barrier(0);
      s_n[1] = mfma_f8(ka, qf[2], s_n[1]);
      // the loads of K(it+2) and V(it+1), issued once the S MFMAs are under way (at the
      // top of the iteration, before the operand reads had landed, 1-2 % slower; spread
      // over the S and PV MFMAs wave by wave, 4-5 % slower)
      if (it + 2 < n_tiles) issue(it + 2, true);
      if (it + 1 < n_tiles) issue(it + 1, false);
      __builtin_amdgcn_sched_barrier(0);
      // PV MFMA j covers dims 32 (j & 3) .. + 31 and key chunk q = j >> 2 (b2 = q >> 1,
      // ck = q & 1); softmax pair j & 3 of chunk q follows it
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        o[j & 3] = mfma_bf16(va[j % 3], pb_p[j >> 2], o[j & 3]);
        if (j + 3 < 16) va[j % 3] = vt_read(vt, (j + 3) & 3, (j + 3) >> 3, ((j + 3) >> 2) & 1);
        __builtin_amdgcn_sched_barrier(0);
        softmax_pair(s_c, nbias, j >> 3, (j >> 2) & 1, j & 3, pb_c[j >> 2]);
        __builtin_amdgcn_sched_barrier(0);
      }

      if (rescale) {
        // alpha passes through an opaque asm so that the multiplies stay in this rare
        // branch (alpha is 1 on the other path, which would let them be speculated)
        asm volatile("" : "+v"(alpha)::"memory");
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      }
    } else if (convert) {
      if constexpr (kWaves == 4) {
        convert_half(it, 0);
        convert_half(it, 1);
      } else {
        convert_half(it, wave >> 2);
      }
    }
    wait_vmcnt(0);  // K(it+2) and V(it+1) have landed
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // so have the V^T stores
    block_barrier();
  };

  // ---- FP8 PV (build option). The 32-byte A operand of dim block db is read with four
  // transposed reads from the FP8 V tile; its byte j = 16 b2 + 4 q + i is key
  // 32 b2 + 8 q + 4 g + i, which is also the key of byte 4 w + i (w = 4 b2 + q) of the
  // lane's P operand: registers 4 q .. 4 q + 3 of S block b2.
  auto vt_operand = [&](const uint8_t* vl, int db) {
    const uint8_t* vp = vl + (vt_off ^ (db << 5));
    const v2i r0 = read_tr8(vp);
    const v2i r1 = read_tr8(vp + 16 * kVStride);
    const v2i r2 = read_tr8(vp + 32 * kVStride);
    const v2i r3 = read_tr8(vp + 48 * kVStride);
    return v8i{r0.x, r0.y, r1.x, r1.y, r2.x, r2.y, r3.x, r3.y};
  };
  // Softmax of group w (4 keys) into E4M3 operand bytes 4 w .. 4 w + 3.
  //  one term:  P' = 2^(c s - m + 8), rounded to E4M3 (nearest even); the row sum adds
  //             the fp32 P'.
  //  two terms: P = 2^(c s - m) rounded toward zero to f16. The f16 bit pattern of P read
  //             at bits 7..14 is the E4M3 code of 256 P with its mantissa truncated to 3
  //             bits (the exponent biases differ by 8 and f16 subnormals map onto E4M3
  //             subnormals): the hi term is a shift and a byte permute. lo = P - hi is
  //             exact in f16 and is rounded to 3 mantissa bits (half away from zero) by
  //             adding 2^6 at bit 0 before the same extraction, so hi + lo is 256 P within
  //             2^-7 relative. The row sum adds the f16 P (scaled by 256 at the end).
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 ones_h2 = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
  auto softmax_group = [&](const v16f(&sc)[2], float nb, int w, v8i& phi, v8i& plo) {
    const int b2 = w >> 2, r = 4 * (w & 3);
    const float e0 = __builtin_amdgcn_exp2f(fmaf(sc[b2][r], c, nb));
    const float e1 = __builtin_amdgcn_exp2f(fmaf(sc[b2][r + 1], c, nb));
    const float e2 = __builtin_amdgcn_exp2f(fmaf(sc[b2][r + 2], c, nb));
    const float e3 = __builtin_amdgcn_exp2f(fmaf(sc[b2][r + 3], c, nb));
    if constexpr (kPvMode == 1) {
      l_run += (e0 + e1) + (e2 + e3);
      int v = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, 0, false);
      v = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, v, true);
      phi[w] = v;
      asm volatile("" ::"v"(phi[w]), "v"(l_run));
    } else {
      const h2 p01 = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(e0, e1));
      const h2 p23 = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(e2, e3));
      l_run = __builtin_amdgcn_fdot2(p01, ones_h2, l_run, false);
      l_run = __builtin_amdgcn_fdot2(p23, ones_h2, l_run, false);
      const uint32_t u01 = __builtin_bit_cast(uint32_t, p01);
      const uint32_t u23 = __builtin_bit_cast(uint32_t, p23);
      // (u << 1) moves bits 7..14 of each half to bytes 1 and 3
      phi[w] = static_cast<int>(__builtin_amdgcn_perm(u23 << 1, u01 << 1, 0x07050301u));
      const h2 lo01 = p01 - __builtin_bit_cast(h2, u01 & 0xFF80FF80u);
      const h2 lo23 = p23 - __builtin_bit_cast(h2, u23 & 0xFF80FF80u);
      const uint32_t q01 = (__builtin_bit_cast(uint32_t, lo01) << 1) + 0x00800080u;
      const uint32_t q23 = (__builtin_bit_cast(uint32_t, lo23) << 1) + 0x00800080u;
      plo[w] = static_cast<int>(__builtin_amdgcn_perm(q23, q01, 0x07050301u));
      asm volatile("" ::"v"(phi[w]), "v"(plo[w]), "v"(l_run));
    }
  };
  // One iteration with FP8 PV: K(it+2) and V(it) are loaded (V(it) into the buffer that
  // V(it-2) left; PV of tile it-1 reads V(it-1) as FP8 codes, V buffer 1 zeroed for
  // tile -1). The 6 S MFMAs of tile it+1 with the mask and row max of tile it between
  // them, then the PV MFMAs of tile it-1 (4 dim blocks, one or two terms) with the
  // softmax groups of tile it between them.
  auto step_fp8 = [&](int it, v16f(&s_c)[2], v16f(&s_n)[2], const v8i& phi_p, const v8i& plo_p,
                      v8i& phi_c, v8i& plo_c) {
    const bool active = it < wave_iters;
    const uint8_t* kl = kbuf(it + 1);
    const uint8_t* vl = vbuf(it - 1);
    v8i va[4];
    v8i ka;
    if (active) {
      va[0] = vt_operand(vl, 0);
      va[1] = vt_operand(vl, 1);
      ka = k_operand(kl, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (it + 2 < n_tiles) issue(it + 2, true);
    if (it < n_tiles) issue(it, false);

    if (active) {
      const int kt = it * kBN;
      const bool need_mask =
          it >= wave_tiles || (kt + kBN > Lk) || (causal && kt + kBN - 1 > wrow0 + off);
      const v16f zero = {};
      s_n[0] = mfma_f8(ka, qf[0], zero);
      ka = k_operand(kl, 1);
      __builtin_amdgcn_sched_barrier(0);
      if (need_mask) {
        asm volatile("" ::: "memory");
        const bool all = it >= wave_tiles;
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kt + 32 * b2 + 8 * (r >> 2) + 4 * g + (r & 3);
            if (all || key >= Lk || (causal && key > my_row + off)) s_c[b2][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = vmax3(mx, s_c[0][r], s_c[0][r + 1]);
      __builtin_amdgcn_sched_barrier(0);
      s_n[1] = mfma_f8(ka, qf[0], zero);
      ka = k_operand(kl, 2);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = vmax3(mx, s_c[1][r], s_c[1][r + 1]);
      __builtin_amdgcn_sched_barrier(0);
      s_n[0] = mfma_f8(ka, qf[1], s_n[0]);
      ka = k_operand(kl, 3);
      __builtin_amdgcn_sched_barrier(0);
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                         false, false);
        mx = __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      const float m_tile = mx * c;
      const bool rescale = __any(m_tile > m_run + kRescaleSlack);
      float alpha = 1.f;
      if (rescale) {
        asm volatile("" ::: "memory");
        const float m_new = fmaxf(m_run, m_tile);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        l_run *= alpha;
        m_run = m_new;
      }
      // one term: P' = 2^8 P directly from the exponent
      const float nb = ((m_run == -INFINITY) ? 0.f : -m_run) + (kPvMode == 1 ? 8.f : 0.f);
      __builtin_amdgcn_sched_barrier(0);
      s_n[1] = mfma_f8(ka, qf[1], s_n[1]);
      ka = k_operand(kl, 4);
      va[2] = vt_operand(vl, 2);
      __builtin_amdgcn_sched_barrier(0);
      s_n[0] = mfma_f8(ka, qf[2], s_n[0]);
      ka = k_operand(kl, 5);
      va[3] = vt_operand(vl, 3);
      __builtin_amdgcn_sched_barrier(0);
      s_n[1] = mfma_f8(ka, qf[2], s_n[1]);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kPvMode == 1) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          o[db] = mfma_f8(va[db], phi_p, o[db]);
          __builtin_amdgcn_sched_barrier(0);
          softmax_group(s_c, nb, 2 * db, phi_c, plo_c);
          softmax_group(s_c, nb, 2 * db + 1, phi_c, plo_c);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        // hi and lo terms alternate between dim blocks: consecutive MFMAs write
        // different accumulators
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int db = 2 * (j >> 2) + (j & 1);
          o[db] = mfma_f8(va[db], (j & 2) ? plo_p : phi_p, o[db]);
          __builtin_amdgcn_sched_barrier(0);
          softmax_group(s_c, nb, j, phi_c, plo_c);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (rescale) {
        asm volatile("" : "+v"(alpha)::"memory");
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      }
    }
    wait_vmcnt(0);  // K(it+2) and V(it) have landed
    block_barrier();
  };

  v16f s_alt[2];
  if constexpr (kPvFp8) {
    v8i phi_a = {}, plo_a = {}, phi_b = {}, plo_b = {};
    for (int it = 0; it <= n_tiles; it += 2) {
      step_fp8(it, s_cur, s_alt, phi_a, plo_a, phi_b, plo_b);
      if (it + 1 <= n_tiles) step_fp8(it + 1, s_alt, s_cur, phi_b, plo_b, phi_a, plo_a);
    }
    l_run *= (kPvMode == 2) ? 256.f : 1.f;  // l in units of P' = 2^8 P
  } else {
    v8bf pb_a[4] = {v8bf{}, v8bf{}, v8bf{}, v8bf{}};
    v8bf pb_b[4] = {v8bf{}, v8bf{}, v8bf{}, v8bf{}};
    for (int it = 0; it <= n_tiles; it += 2) {
      step(it, s_cur, s_alt, pb_a, pb_b);
      if (it + 1 <= n_tiles) step(it + 1, s_alt, s_cur, pb_b, pb_a);
    }
  }

  // epilogue: this lane holds row my_row, dims 32*db + 8*(r/4) + 4*g + r%4
  float l_tot;
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run),
                                                     false, false);
    l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  if (row_ok) {
    // O holds sum P v with v the decoded V codes (their descale is applied here)
    const float inv = (l_tot > 0.f) ? p.dv[h] / l_tot : 0.f;
    const int64_t obase = (q0 + my_row) * (static_cast<int64_t>(H) * kDv) + h * kDv;
    if (p.out_f32) {
      float* op = static_cast<float*>(out_ptr) + obase;
      const bool coherent = kNSeg > 1 && p.counters != nullptr;  // read by another workgroup
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int grp4 = 0; grp4 < 4; ++grp4) {
          const float4 v = make_float4(o[db][4 * grp4 + 0] * inv, o[db][4 * grp4 + 1] * inv,
                                       o[db][4 * grp4 + 2] * inv, o[db][4 * grp4 + 3] * inv);
          float* dst = op + 32 * db + 8 * grp4 + 4 * g;
          if (coherent)
            store16_agent(dst, v);
          else
            *reinterpret_cast<float4*>(dst) = v;
        }
    } else {
      uint16_t* op = static_cast<uint16_t*>(out_ptr) + obase;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int grp4 = 0; grp4 < 4; ++grp4) {
          const uint32_t e0 = mla::f32_to_bf16_rne(o[db][4 * grp4 + 0] * inv);
          const uint32_t e1 = mla::f32_to_bf16_rne(o[db][4 * grp4 + 1] * inv);
          const uint32_t e2 = mla::f32_to_bf16_rne(o[db][4 * grp4 + 2] * inv);
          const uint32_t e3 = mla::f32_to_bf16_rne(o[db][4 * grp4 + 3] * inv);
          *reinterpret_cast<uint2*>(op + 32 * db + 8 * grp4 + 4 * g) =
              make_uint2(e0 | (e1 << 16), e2 | (e3 << 16));
        }
    }
    if (g == 0 && lse_ptr != nullptr) {
      float* lp = lse_ptr + static_cast<int64_t>(h) * (kNSeg > 1 ? p.seg_lse_stride : p.lse_stride) +
                  q0 + my_row;
      const float lv =
          (l_tot > 0.f) ? (m_run + __log2f(l_tot) - (kPvFp8 ? 8.f : 0.f)) * kLn2 : -INFINITY;
      if (kNSeg > 1 && p.counters != nullptr)
        __hip_atomic_store(lp, lv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        *lp = lv;
    }
  }
  if constexpr (kNSeg > 1) {
    if (p.counters != nullptr) merge_on_last_arrival(p, st, h, m_tile, row0, min(kBM, Lq - row0));
  }
}

}  // namespace

namespace mla {

namespace {

// common checks and parameters of both launch forms; returns the number of query tiles
int prefill_params(const PrefillArgs& a, PrefillParams& prm, int64_t& n_m) {
  // per-lane DMA offsets within one 64-key tile are 32-bit; tile bases are 64-bit
  if (static_cast<int64_t>(a.n_heads) * kDqk * kBN >= (1ll << 31))
    return fail(MLA_ERR_UNSUPPORTED, "n_heads * 192 * 64 must be < 2^31");
  n_m = (static_cast<int64_t>(a.max_seqlen_q) + kBM - 1) / kBM;
  prm = PrefillParams{};
  prm.q = static_cast<const uint8_t*>(a.q);
  prm.k = static_cast<const uint8_t*>(a.k);
  prm.v = static_cast<const uint8_t*>(a.v);
  prm.cu_q = a.cu_q;
  prm.cu_k = a.cu_k;
  prm.dq = a.dq;
  prm.dk = a.dk;
  prm.dv = a.dv;
  prm.out = a.out;
  prm.out_f32 = a.out_f32;
  prm.lse = a.lse;
  prm.lse_stride = a.lse_stride;
  prm.total_q = a.total_q;
  prm.total_k = a.total_k;
  prm.batch = a.batch;
  prm.n_heads = a.n_heads;
  prm.n_m_tiles = static_cast<int32_t>(n_m);
  prm.causal = a.causal;
  prm.scale_log2 = a.softmax_scale * 1.44269504088896340736f;
  prm.seg_lse_stride = a.seg_lse_stride;
  prm.counters = a.counters;
  return MLA_OK;
}

__global__ void zero_ints_kernel(int32_t* p, int64_t n) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = 0;
}

}  // namespace

#ifdef MLA_PREFILL_SMALL_GRID

int prefill_launch_small(const PrefillArgs& a, hipStream_t stream) {
  if (a.total_q == 0 || a.batch == 0 || a.max_seqlen_q == 0) return ok();
  PrefillParams prm;
  int64_t n_m = 0;
  const int st = prefill_params(a, prm, n_m);
  if (st != MLA_OK) return st;
  const int64_t blocks = n_m * a.batch * a.n_heads;
  if (blocks >= (1ll << 31)) return fail(MLA_ERR_UNSUPPORTED, "grid too large");
  prm.xcd_order = (a.batch == 1 && a.n_heads % 4 == 0 && n_m % 2 == 0) ? 1 : 0;
  SegTable<1> none{};
  hipLaunchKernelGGL((prefill_fp8_kernel<1, kPvMode>), dim3(static_cast<unsigned>(blocks)),
                     dim3(kThreads), 0, stream, prm, none);
  return check_launch("prefill_fp8_4w_kernel");
}

#else  // the default build

int prefill_rows_per_block() { return kBM; }

int zero_ints(int32_t* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return ok();
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(zero_ints_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, p,
                     n);
  return check_launch("zero_ints_kernel");
}

int prefill_launch(const PrefillArgs& a, hipStream_t stream) {
  if (a.total_q == 0 || a.batch == 0 || a.max_seqlen_q == 0) return ok();
  PrefillParams prm;
  int64_t n_m = 0;
  const int st = prefill_params(a, prm, n_m);
  if (st != MLA_OK) return st;
  const int64_t blocks = n_m * a.batch * a.n_heads;
  if (blocks >= (1ll << 31)) return fail(MLA_ERR_UNSUPPORTED, "grid too large");
#if MLA_PV_MODE == 0
  // Grids that leave CUs idle, or whose workgroups differ much in length, run as 4-wave
  // workgroups of 128 rows (twice the workgroups, bit-identical results) where that
  // measured faster: (a) at most one workgroup per two CUs, so that every 4-wave workgroup
  // has a CU to itself (1K-2.5K queries at 12 heads, causal or not, and short query chunks
  // over long contexts: 14-19 % faster); (b) at most one workgroup per CU in a causal call
  // whose first query tile sees at most half the keys of the last, where the heaviest
  // workgroup sets the time and 128-row workgroups halve it (single sequences of 1K-5K
  // tokens: 6-17 %); (c) packed sequences of unequal lengths, estimated from the grid
  // being more than a quarter padding (query tiles past a shorter sequence's end), where
  // the smaller workgroups balance the CUs better (2-10 %; the 8-sequence C2 mix 5 %).
  // Beyond these the 8-wave kernel is faster: 4K queries at the end of a 69K-token
  // context 11 %, 3K-4K non-causal queries 7-8 %, full grids of equal sequences up to 8 %.
  // MLA_FP8_PREFILL_SMALL_GRID in the environment: 0 keeps every call on the 8-wave
  // kernel, 1 also sends every grid of at most one workgroup per CU to the 4-wave kernel.
  {
    const char* env = getenv("MLA_FP8_PREFILL_SMALL_GRID");
    if (env == nullptr || env[0] != '0') {
      const int cus = cu_count();
      bool small = false;
      if (blocks <= cus) {
        // one sequence (the call's totals), or the longest sequences of a packed batch
        const int64_t lq = a.batch > 1 ? a.max_seqlen_q : a.total_q;
        const int64_t lk = a.batch > 1 ? a.max_seqlen_k : a.total_k;
        const int64_t first = std::min<int64_t>(  // keys of the first query tile
            lk, std::max<int64_t>(0, std::min<int64_t>(lq, kBM) + lk - lq));
        small = (env != nullptr && env[0] == '1') || 2 * blocks <= cus ||
                (a.causal != 0 && lk > 0 && lk >= 2 * first);
      }
      // workgroups with rows: about (total_q / 256 + batch / 2) per head; the 128-row grid
      // must stay within the launch limit
      if (!small && a.batch > 1 && 2 * blocks < (1ll << 31))
        small = (a.total_q + static_cast<int64_t>(kBM / 2) * a.batch) * a.n_heads <
                static_cast<int64_t>(kBM) * 3 / 4 * blocks;
      if (small) return prefill_launch_small(a, stream);
    }
  }
#endif
  prm.xcd_order = (a.batch == 1 && a.n_heads % 4 == 0 && n_m % 2 == 0) ? 1 : 0;
  SegTable<1> none{};
  hipLaunchKernelGGL((prefill_fp8_kernel<1, kPvMode>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads),
                     0, stream, prm, none);
  return check_launch("prefill_fp8_kernel");
}

int prefill_launch_segments(const PrefillArgs& a, const PrefillSegment* segs, int n,
                            hipStream_t stream) {
  if (n < 1 || n > kMaxPrefillSegments)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%d segments not in 1..%d", n, kMaxPrefillSegments);
  if (a.batch != 1 || a.cu_q != nullptr)
    return fail(MLA_ERR_INVALID_ARGUMENT, "segments need one sequence without cu_seqlens");
  if (a.counters != nullptr &&
      (a.out_f32 != 1 || a.out == nullptr || !aligned16(a.out) || a.seg_lse_stride < a.total_q ||
       (a.lse != nullptr && a.lse_stride < a.total_q)))
    return fail(MLA_ERR_INVALID_ARGUMENT, "fused merge needs fp32 partials and a bf16 output");
  if (a.total_q == 0 || a.max_seqlen_q == 0) return ok();
  PrefillParams prm;
  int64_t n_m = 0;
  const int st = prefill_params(a, prm, n_m);
  if (st != MLA_OK) return st;
  SegTable<kMaxPrefillSegments> tab{};
  tab.n = n;
  for (int i = 0; i < n; ++i) {
    if (segs[i].k0 < 0 || segs[i].lk < 0 || segs[i].k0 + segs[i].lk > a.total_k)
      return fail(MLA_ERR_INVALID_ARGUMENT, "segment %d outside the keys", i);
    tab.e[i] = SegDev{segs[i].k0, segs[i].lk, segs[i].causal, segs[i].out, segs[i].lse};
  }
  const int64_t blocks = n_m * n * a.n_heads;
  if (blocks >= (1ll << 31)) return fail(MLA_ERR_UNSUPPORTED, "grid too large");
  // XCD-aware order within each segment (measured: the 16,384-row chunks of a
  // 131,072-token context 1.1-1.3 % faster, 4,096-row chunks unchanged)
  prm.xcd_order = (a.n_heads % 4 == 0 && n_m % 2 == 0) ? 1 : 0;
  hipLaunchKernelGGL((prefill_fp8_kernel<kMaxPrefillSegments, kPvMode>), dim3(static_cast<unsigned>(blocks)),
                     dim3(kThreads), 0, stream, prm, tab);
  return check_launch("prefill_fp8_kernel");
}

int prefill_check_common(int32_t n_heads, int32_t head_dim_qk, int32_t head_dim_v,
                         float softmax_scale, int32_t causal) {
  if (head_dim_qk != kDqk || head_dim_v != kDv)
    return fail(MLA_ERR_UNSUPPORTED, "head dims %d/%d: only 192/128 are implemented", head_dim_qk,
                head_dim_v);
  if (n_heads < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "n_heads = %d < 1", n_heads);
  if (causal != 0 && causal != 1)
    return fail(MLA_ERR_INVALID_ARGUMENT, "causal = %d is not 0 or 1", causal);
  if (!(softmax_scale > 0.f) || !(softmax_scale <= 3.4028234663852886e38f))
    return fail(MLA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and positive");
  return MLA_OK;
}

#endif  // MLA_PREFILL_SMALL_GRID

}  // namespace mla

#ifndef MLA_PREFILL_SMALL_GRID

extern "C" int mla_fp8_prefill_varlen(const void* q, const void* k, const void* v,
                                      const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                      int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                      int64_t total_q, int64_t total_k, int32_t n_heads,
                                      int32_t head_dim_qk, int32_t head_dim_v,
                                      const float* descale_q, const float* descale_k,
                                      const float* descale_v, float softmax_scale, int32_t causal,
                                      void* out, float* lse, int64_t lse_stride, void* stream) {
  int st = mla::prefill_check_common(n_heads, head_dim_qk, head_dim_v, softmax_scale, causal);
  if (st != MLA_OK) return st;
  if (batch < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || total_q < 0 || total_k < 0)
    return mla::fail(MLA_ERR_INVALID_ARGUMENT, "negative size");
  if (total_q >= (1ll << 31) || total_k >= (1ll << 31))
    return mla::fail(MLA_ERR_UNSUPPORTED, "total_q and total_k must be < 2^31");
  if (total_q == 0 || batch == 0 || max_seqlen_q == 0) return mla::ok();
  if (q == nullptr || out == nullptr || cu_seqlens_q == nullptr || cu_seqlens_k == nullptr ||
      descale_q == nullptr || descale_k == nullptr || descale_v == nullptr)
    return mla::fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (total_k > 0 && (k == nullptr || v == nullptr))
    return mla::fail(MLA_ERR_INVALID_ARGUMENT, "k or v is NULL");
  if (!mla::aligned16(q) || !mla::aligned16(k) || !mla::aligned16(v) || !mla::aligned16(out))
    return mla::fail(MLA_ERR_INVALID_ARGUMENT, "q, k, v and out must be 16-byte aligned");
  if (lse != nullptr && lse_stride < total_q)
    return mla::fail(MLA_ERR_INVALID_ARGUMENT, "lse_stride < total_q");
  mla::PrefillArgs a{q, k, v, cu_seqlens_q, cu_seqlens_k, batch, max_seqlen_q, total_q, total_k,
                     n_heads, descale_q, descale_k, descale_v, softmax_scale, causal, out, 0, lse,
                     lse_stride};
  a.max_seqlen_k = max_seqlen_k;
  return mla::prefill_launch(a, static_cast<hipStream_t>(stream));
}

#endif  // MLA_PREFILL_SMALL_GRID
