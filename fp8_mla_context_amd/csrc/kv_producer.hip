// Un-absorbed MLA K/V producer fused with the static per-head FP8 quantizer (gfx950).
//
// vLLM #60110, Purpose:
// prefill keeps the un-absorbed form, so keys and values are expanded from the latent
// cache per head; the page gives latent rank 512, 192-wide key heads of which 64 dims
// are the rope part, and 12 heads per rank. The quantizer is the static per-head one of
// "[ROCm][MLA] Add guarded gfx942 FP8 context prefill" (#51551), Summary.
//
// For token t and head h, with latent row c_t (512 bf16) and rope key p_t (64 bf16):
//   K[t, h] = [ RN_bf16(W_UK[h] c_t) | p_t ],  V[t, h] = RN_bf16(W_UV[h] c_t)
//   k8 = E4M3(K / dk[h]),  v8 = E4M3(V / dv[h])   (exact quotient, nearest even)
// W is [H * 256, 512] bf16: rows 256 h .. 256 h + 127 are W_UK[h], the next 128 W_UV[h].
//
// Design:
//  * One workgroup = 16 waves = 256 tokens x one head's 256 output features, one per CU.
//    Y^T = W_h C^T on v_mfma_f32_32x32x16_bf16 with weight rows as the A operand and
//    latent rows as the B operand, so a lane's accumulator holds one token and 4 x 4
//    consecutive features. Wave w owns tokens 64 (w & 3) .. + 63 and features
//    64 (w >> 2) .. + 63. Each XCD takes half of the heads over a quarter of the token
//    tiles, so that its L2 holds those heads' weights and serves each token tile's
//    latent rows to them.
//  * The 512-deep reduction runs in 8 chunks of 64; chunk c's weight rows (256 x 128 B)
//    and latent rows (256 x 128 B) are DMA'd (global_load_lds_dwordx4) into LDS buffer
//    c % 2, one chunk ahead of their use, the eight 16-byte pieces of a row XOR-swizzled
//    so that the operand reads of 16 consecutive rows hit distinct banks. Each wave runs
//    16 MFMAs between two barriers. (Measured against 16 chunks of 32 with two 8-wave
//    workgroups of 128 tokens per CU and three buffers: 140 against 156 us for 32K
//    tokens; the 64-byte chunks gave 8 MFMAs per barrier and a burst of loads after each.)
//  * Epilogue: fp32 -> bf16 (v_cvt_pk_bf16_f32, nearest even) -> E4M3 code, looked up in
//    per-head tables of the exact quantizer's codes, filled in LDS during the first
//    chunks of the reduction. The codes pass through LDS so that each thread stores
//    whole 16-byte pieces of k8 / v8 rows, with non-temporal stores: the 126 MB of codes
//    of a 32K-token call would otherwise push the weight and the shared latent rows out
//    of L2 (3x the HBM reads). The rope part is quantized with the head's key scale, 16
//    values per thread. The bf16 K and V can be written as well (for a BF16 attention
//    path).
#include "device_common.h"
#include "e4m3_quant.h"
#include "mla_internal.h"

namespace {

using namespace mla::dev;

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int kLatent = 512;
constexpr int kRope = 64;
constexpr int kNope = 128;
constexpr int kDv = 128;
constexpr int kFeat = kNope + kDv;  // 256 output features per head
constexpr int kWaves = 16;
constexpr int kThreads = 64 * kWaves;
constexpr int kTM = 256;            // tokens per workgroup
constexpr int kKC = 64;             // reduction chunk
constexpr int kNChunks = kLatent / kKC;
constexpr int kRowBytes = 128;      // one chunk of a row: eight 16-byte pieces, swizzled
constexpr int kWRegion = kFeat * kRowBytes;  // 32768
constexpr int kCRegion = kTM * kRowBytes;    // 32768
constexpr int kStage = kWRegion + kCRegion;  // 65536
// Two LDS buffers (128 KB) and the code tables: one workgroup per CU.
constexpr int kStages = 2;
constexpr int kWgPerCu = 1;
constexpr int kWInstr = kFeat * 8 / 64;  // 32 DMA instructions (8 pieces per row)
constexpr int kCInstr = kTM * 8 / 64;    // 32
constexpr int kInstr = kWInstr + kCInstr;
constexpr int kPerWave = (kInstr + kWaves - 1) / kWaves;  // 4
// piece p of row r sits at position p ^ ((r >> 1) & 7): the 16-byte operand reads of 16
// consecutive rows (same piece; 128-byte rows, two rows per 256 bytes of banks) then
// cover all 64 banks
__device__ __forceinline__ int piece_pos(int row, int piece) { return piece ^ ((row >> 1) & 7); }
constexpr int kCodeStride = kFeat + 16;  // LDS bytes per token row of the code tile
static_assert(kStages * kStage >= kTM * kCodeStride, "the code tile reuses the stage buffers");

constexpr int kLdsBytes = kStages * kStage + 2 * kTabBytes;  // stages, then the K and V tables

struct ProducerParams {
  const uint16_t* c_kv;
  const uint16_t* k_pe;
  const uint16_t* w;
  const float* dk;
  const float* dv;
  uint8_t* k8;
  uint8_t* v8;
  uint16_t* kb;  // optional bf16 K [T, H, 192]
  uint16_t* vb;  // optional bf16 V [T, H, 128]
  int64_t c_stride;   // elements between latent rows
  int64_t pe_stride;  // elements between rope rows
  int64_t n_tokens;
  int32_t n_heads;
  int32_t xcd_order;  // 2 or 1: XCD-aware work item orders (see the block mapping)
};

__device__ __forceinline__ v16f mfma_bf16(const v8bf& a, const v8bf& b, const v16f& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(kThreads, kWgPerCu) void kv_producer_kernel(ProducerParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = p.n_heads;
  // Work items (token tile, head); workgroup b is dealt to XCD b % 8. With xcd_order 2
  // (H even, tile count a multiple of 4) XCD x takes half of the heads (x & 1) over a
  // quarter of the token tiles (x >> 1), heads fastest: its L2 then holds the weights of
  // H/2 heads (1.5 MB at 12 heads, against 4 MB of L2) and serves a token tile's latent
  // rows to those heads, each latent row being read by two XCDs. (All H heads of a
  // contiguous range per XCD, xcd_order 1, left the 3 MB of weights competing with the
  // latent rows: 120 MB fetched from HBM on 32K tokens against 94 MB, and 3 % slower.)
  // Otherwise v = blockIdx is (tile, head), heads fastest.
  const int nb = gridDim.x;
  int h, tile;
  if (p.xcd_order == 2) {
    const int x = blockIdx.x & 7, s = blockIdx.x >> 3, hh = H >> 1;
    tile = (x >> 1) * (nb / (4 * H)) + s / hh;
    h = hh * (x & 1) + s % hh;
  } else {
    const int v = p.xcd_order ? (blockIdx.x & 7) * (nb >> 3) + (blockIdx.x >> 3) : blockIdx.x;
    h = v % H;
    tile = v / H;
  }
  const int64_t t0 = static_cast<int64_t>(tile) * kTM;
  const int n_tok = static_cast<int>(min<int64_t>(kTM, p.n_tokens - t0));  // >= 1

  // DMA slots: instruction i (i = wave + 16 j) writes 16-byte LDS slots 64 i + lane of the
  // stage; slots 0..2047 are weight rows (8 per row), then 2048 slots of latent rows (rows
  // past the last token repeat it). Slot position q of row r holds piece q ^ ((r >> 1) & 7).
  const uint8_t* w_base = reinterpret_cast<const uint8_t*>(p.w) +
                          static_cast<int64_t>(h) * kFeat * kLatent * 2;
  const uint8_t* c_base = reinterpret_cast<const uint8_t*>(p.c_kv) + t0 * p.c_stride * 2;
  uint32_t dma_off[kPerWave];
#pragma unroll
  for (int j = 0; j < kPerWave; ++j) {
    const int i = min(wave + kWaves * j, kInstr - 1);
    const int s = (i < kWInstr ? i * 64 : (i - kWInstr) * 64) + lane;
    const int row = s >> 3;
    const int piece = piece_pos(row, s & 7);  // the swizzle is its own inverse
    if (i < kWInstr)
      dma_off[j] = static_cast<uint32_t>(row * kLatent * 2 + 16 * piece);
    else
      dma_off[j] = static_cast<uint32_t>(min(row, n_tok - 1) * p.c_stride * 2 + 16 * piece);
  }
  auto issue = [&](int c) {
    uint8_t* stage = lds + (c % kStages) * kStage;
#pragma unroll
    for (int j = 0; j < kPerWave; ++j) {
      const int i = wave + kWaves * j;  // wave-uniform
      if (i < kInstr) {
        const uint8_t* base = uniform_ptr((i < kWInstr ? w_base : c_base) + c * kKC * 2);
        const uint32_t dst =
            lds_address(stage) + (i < kWInstr ? 1024u * i : kWRegion + 1024u * (i - kWInstr));
        dma_load16(base, dma_off[j], dst);
      }
    }
  };
  const int n_mine = (kInstr - wave + kWaves - 1) / kWaves;  // DMA instructions of this wave per chunk

  const int g = lane >> 5, col = lane & 31;
  const int tq = wave & 3, fq = wave >> 2;
  v16f acc[2][2];
#pragma unroll
  for (int fb = 0; fb < 2; ++fb)
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[fb][tb][r] = 0.f;

  // The rope part, K[t, h, 128 + i] = E4M3(p_t[i] / dk[h]): 16 values per thread, loaded
  // here (older than the first chunks' loads, so the waits below cover them) and
  // quantized in the epilogue.
  const int pe_tok = tid >> 2, pe_pc = tid & 3;
  uint4 pe_a = make_uint4(0, 0, 0, 0), pe_b = pe_a;
  if (pe_tok < n_tok) {
    const uint16_t* src = p.k_pe + (t0 + pe_tok) * p.pe_stride + 16 * pe_pc;
    pe_a = *reinterpret_cast<const uint4*>(src);
    pe_b = *reinterpret_cast<const uint4*>(src + 8);
  }
  // chunks [0, next) have been issued; before the barrier that ends iteration c, chunk
  // c + 1 must have landed, so the loads of chunks c + 2 .. next - 1 may stay in flight
  int next = 0;
  for (; next < kStages - 1; ++next) issue(next);
  // The code tables of this head (K then V, 2 kTabEntries entries) are filled during the
  // first chunks, entry tid + kThreads c in chunk c, in VALU time the loop leaves idle;
  // descales outside [2^-126, 2^126] skip them (every code then comes from quant16).
  const float dk = p.dk[h], dv = p.dv[h];
  const bool tab_ok = table_ok(dk) && table_ok(dv);
  uint8_t* tab_k = lds + kStages * kStage;
  uint8_t* tab_v = tab_k + kTabBytes;
  const float rk = 1.0f / dk, rv = 1.0f / dv;
  const int elo_k = table_elo(dk), elo_v = table_elo(dv);
  constexpr int kTabChunks = (2 * kTabEntries + kThreads - 1) / kThreads;
  static_assert(kTabChunks <= kNChunks, "the tables are filled within the loop");
  wait_vmcnt(n_mine * (next - 1));
  block_barrier();
  for (int c = 0; c < kNChunks; ++c) {
    if (next < kNChunks) issue(next++);
    const uint8_t* stage = lds + (c % kStages) * kStage;
#pragma unroll
    for (int ks = 0; ks < kKC / 16; ++ks) {
      v8bf a[2], b[2];
#pragma unroll
      for (int fb = 0; fb < 2; ++fb) {
        const int row = 64 * fq + 32 * fb + col;
        a[fb] = *reinterpret_cast<const v8bf*>(stage + row * kRowBytes +
                                                16 * piece_pos(row, 2 * ks + g));
      }
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int row = 64 * tq + 32 * tb + col;
        b[tb] = *reinterpret_cast<const v8bf*>(stage + kWRegion + row * kRowBytes +
                                                16 * piece_pos(row, 2 * ks + g));
      }
#pragma unroll
      for (int fb = 0; fb < 2; ++fb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) acc[fb][tb] = mfma_bf16(a[fb], b[tb], acc[fb][tb]);
    }
    if (tab_ok && c < kTabChunks) {
      const int i = tid + kThreads * c;
      if (i < kTabEntries)
        tab_k[i] = table_entry(i, dk, rk, elo_k);
      else if (i < 2 * kTabEntries)
        tab_v[i - kTabEntries] = table_entry(i - kTabEntries, dv, rv, elo_v);
    }
    wait_vmcnt(next > c + 2 ? n_mine * (next - c - 2) : 0);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the table stores too
    block_barrier();
  }

  // Epilogue. Lane (g, col) of block (fb, tb) holds token 64 tq + 32 tb + col and features
  // 64 fq + 32 fb + 8 q + 4 g + (0..3), q = 0..3. Their codes go to an LDS tile of 128
  // token rows (kCodeStride bytes apart: consecutive tokens start 4 banks apart), then
  // out in 16-byte pieces.
  const float d = fq < 2 ? dk : dv;  // features 0..127 are k_nope, 128..255 v
  const float rr = fq < 2 ? rk : rv;
  const uint8_t* tab = fq < 2 ? tab_k : tab_v;
  const int base = (fq < 2 ? elo_k : elo_v) << 7;
  const int64_t kst = static_cast<int64_t>(H) * 192, vst = static_cast<int64_t>(H) * kDv;
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int tok = 64 * tq + 32 * tb + col;
    const int64_t t = t0 + tok;
    const bool store_bf16 = tok < n_tok && (p.kb != nullptr || p.vb != nullptr);
#pragma unroll
    for (int fb = 0; fb < 2; ++fb) {
      uint32_t pr[8];  // the block's 16 values (q, i) as bf16 pairs, element 4 q + i
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // v_cvt_pk_bf16_f32: two fp32 values to bf16, nearest even
        pr[2 * q] = __builtin_bit_cast(
            uint32_t, __builtin_convertvector(v2f{acc[fb][tb][4 * q], acc[fb][tb][4 * q + 1]}, v2bf));
        pr[2 * q + 1] = __builtin_bit_cast(
            uint32_t,
            __builtin_convertvector(v2f{acc[fb][tb][4 * q + 2], acc[fb][tb][4 * q + 3]}, v2bf));
      }
      const uint4 cd = tab_ok ? quant16_tab(pr, tab, base, d, rr) : quant16(pr, d, rr);
      const uint32_t cw[4] = {cd.x, cd.y, cd.z, cd.w};  // word q: codes of (q, 0..3)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int f = 64 * fq + 32 * fb + 8 * q + 4 * g;
        *reinterpret_cast<uint32_t*>(lds + tok * kCodeStride + f) = cw[q];
        if (store_bf16) {
          const uint2 val = make_uint2(pr[2 * q], pr[2 * q + 1]);
          if (f < kNope) {
            if (p.kb != nullptr) *reinterpret_cast<uint2*>(p.kb + t * kst + h * 192 + f) = val;
          } else if (p.vb != nullptr) {
            *reinterpret_cast<uint2*>(p.vb + t * vst + h * kDv + (f - kNope)) = val;
          }
        }
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kTM * 16 / kThreads; ++j) {
    const int id = tid + kThreads * j;
    const int tok = id >> 4, pc = id & 15;
    if (tok < n_tok) {
      const uint4 v = *reinterpret_cast<const uint4*>(lds + tok * kCodeStride + 16 * pc);
      const int64_t t = t0 + tok;
      if (pc < 8)
        __builtin_nontemporal_store(__builtin_bit_cast(v4u, v),
                                    reinterpret_cast<v4u*>(p.k8 + t * kst + h * 192 + 16 * pc));
      else
        __builtin_nontemporal_store(__builtin_bit_cast(v4u, v),
                                    reinterpret_cast<v4u*>(p.v8 + t * vst + h * kDv + 16 * (pc - 8)));
    }
  }
  if (pe_tok < n_tok) {
    const uint32_t w[8] = {pe_a.x, pe_a.y, pe_a.z, pe_a.w, pe_b.x, pe_b.y, pe_b.z, pe_b.w};
    const int64_t o = (t0 + pe_tok) * kst + h * 192 + kNope + 16 * pe_pc;
    const uint4 cr = tab_ok ? quant16_tab(w, tab_k, elo_k << 7, dk, rk) : quant16(w, dk, rk);
    __builtin_nontemporal_store(__builtin_bit_cast(v4u, cr), reinterpret_cast<v4u*>(p.k8 + o));
    if (p.kb != nullptr) {
      *reinterpret_cast<uint4*>(p.kb + o) = pe_a;
      *reinterpret_cast<uint4*>(p.kb + o + 8) = pe_b;
    }
  }
}

}  // namespace

extern "C" int mla_fp8_kv_produce(const void* c_kv, int64_t c_kv_stride, const void* k_pe,
                                  int64_t k_pe_stride, const void* w_kv_b, int64_t n_tokens,
                                  int32_t n_heads, int32_t kv_lora_rank, int32_t rope_dim,
                                  const float* descale_k, const float* descale_v, void* k8,
                                  void* v8, void* k_bf16, void* v_bf16, void* stream) {
  if (kv_lora_rank != kLatent || rope_dim != kRope)
    return mla::fail(MLA_ERR_UNSUPPORTED, "latent rank %d / rope dim %d: only 512 / 64",
                     kv_lora_rank, rope_dim);
  if (n_heads < 1) return mla::fail(MLA_ERR_INVALID_ARGUMENT, "n_heads = %d < 1", n_heads);
  if (n_tokens < 0) return mla::fail(MLA_ERR_INVALID_ARGUMENT, "negative n_tokens");
  if (n_tokens == 0) return mla::ok();
  if (c_kv == nullptr || k_pe == nullptr || w_kv_b == nullptr || descale_k == nullptr ||
      descale_v == nullptr || k8 == nullptr || v8 == nullptr)
    return mla::fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (c_kv_stride < kLatent || k_pe_stride < kRope || c_kv_stride % 8 != 0 ||
      k_pe_stride % 8 != 0 || c_kv_stride >= (1 << 24) || k_pe_stride >= (1 << 24))
    return mla::fail(MLA_ERR_INVALID_ARGUMENT,
                     "row strides must be multiples of 8 elements, >= the row, < 2^24");
  if (!mla::aligned16(c_kv) || !mla::aligned16(k_pe) || !mla::aligned16(w_kv_b) ||
      !mla::aligned16(k8) || !mla::aligned16(v8) || !mla::aligned16(k_bf16) ||
      !mla::aligned16(v_bf16))
    return mla::fail(MLA_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
  const int64_t tiles = (n_tokens + kTM - 1) / kTM;
  if (tiles * n_heads >= (1ll << 31)) return mla::fail(MLA_ERR_UNSUPPORTED, "grid too large");
  ProducerParams prm{};
  prm.c_kv = static_cast<const uint16_t*>(c_kv);
  prm.k_pe = static_cast<const uint16_t*>(k_pe);
  prm.w = static_cast<const uint16_t*>(w_kv_b);
  prm.dk = descale_k;
  prm.dv = descale_v;
  prm.k8 = static_cast<uint8_t*>(k8);
  prm.v8 = static_cast<uint8_t*>(v8);
  prm.kb = static_cast<uint16_t*>(k_bf16);
  prm.vb = static_cast<uint16_t*>(v_bf16);
  prm.c_stride = c_kv_stride;
  prm.pe_stride = k_pe_stride;
  prm.n_tokens = n_tokens;
  prm.n_heads = n_heads;
  prm.xcd_order = (n_heads % 2 == 0 && tiles % 4 == 0) ? 2 : ((tiles * n_heads) % 8 == 0 ? 1 : 0);
  hipLaunchKernelGGL(kv_producer_kernel, dim3(static_cast<unsigned>(tiles * n_heads)),
                     dim3(kThreads), 0, static_cast<hipStream_t>(stream), prm);
  return mla::check_launch("kv_producer_kernel");
}
