// BF16 varlen context-prefill attention for MLA shapes (Q/K 192, V 128) on gfx950: the
// comparator of the FP8 path.
//
// "[ROCm][MLA] Add guarded gfx942 FP8 context prefill" (vLLM #51551): the close comment
// measures the FP8 kernel against the BF16 attention that already covers D192/V128 (faster
// on the non-causal 4K x 65K chunk, slower on both causal shapes). This kernel computes the
// same attention on bf16 Q/K/V with no scales, with the same blocking and schedule as the
// FP8 kernel so that the two differ only in the data type:
//  * One workgroup = 4 waves = 128 query rows of one (sequence, head), each wave 32 rows;
//    two workgroups per CU. Heaviest query tiles first; the XCD-aware order of the FP8
//    kernel for one sequence.
//  * 32-key K/V tiles (a bf16 key is twice the bytes of an FP8 one, so 32 keys keep three
//    buffers of two workgroups inside the CU's LDS) in three rotating LDS buffers filled by
//    global->LDS DMA. K rows are padded to 400 bytes; V rows are 256 bytes with XOR-swizzled
//    16-byte chunks (see v_swizzle). Iteration t issues the loads of K(t+3) and V(t+1) and
//    computes, interleaved, the PV MFMAs of tile t-1, the S MFMAs of tile t+1 and the
//    softmax of tile t. One barrier per tile.
//  * S^T = K * Q^T on v_mfma_f32_32x32x16_bf16 (12 per tile, K-dim 192 = 12 x 16): the Q
//    fragment (32 rows x 192) stays in registers as the B operand. In the accumulator every
//    lane holds one query row (lane % 32) and 16 of the tile's keys.
//  * Online softmax in base 2 as in the FP8 kernel (c = softmax_scale * log2 e), with a
//    lazy rescale slack of 8: P = 2^(c*s - m) <= 256 is rounded to bf16 (nearest even);
//    the row sum adds the rounded weights (v_dot2c_f32_bf16), so the normalised weights
//    sum to one.
//  * O^T = V^T * P^T on the same MFMA (8 per tile). The P^T operand is the S accumulator
//    repacked: MFMA k-index 8 * (lane / 32) + i of key chunk c stands for tile key
//    16 c + 8 (i / 4) + 4 (lane / 32) + i % 4, which is accumulator register 8 c + i of the
//    lane. The V^T operand uses the same key order, read with ds_read_b64_tr_b16: within a
//    16-lane group, output lane i component j is element i % 4 of the 8-byte window of
//    source lane 4 j + i / 4; with source lane 4 j + u at key j and dims d0 + 4u .. d0 + 4u
//    + 3, lane i receives dim d0 + i of four consecutive keys.
//  * Causal (bottom-right aligned) and ragged tiles are masked as in the FP8 kernel.
//  * Epilogue: out = O / l in bf16, lse = ln2 * (m + log2 l).
#include "mla_internal.h"
#include "device_common.h"

namespace {

using namespace mla::dev;

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v2f __attribute__((ext_vector_type(2)));

constexpr int kDqk = 192;
constexpr int kDv = 128;
#ifndef MLA_BF16_WAVES
#define MLA_BF16_WAVES 4
#endif
constexpr int kWaves = MLA_BF16_WAVES;  // waves per workgroup (4 or 8)
constexpr int kWgPerCu = 8 / kWaves;    // resident workgroups per CU (2 waves per SIMD)
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // query rows per workgroup
constexpr int kBN = 32;           // keys per tile
constexpr int kKStride = 400;     // LDS bytes per K row: 384 + 16 (16 consecutive rows hit distinct banks)
constexpr int kKSlots = kKStride / 16;                 // 25 16-byte slots per K row
constexpr int kKInstr = (kBN * kKSlots + 63) / 64;     // 13 DMA instructions per K tile
constexpr int kKRegion = kKInstr * 1024;               // the last instruction's spare lanes land past the tile
constexpr int kVStride = 256;                          // LDS bytes per V row, chunks swizzled
constexpr int kVInstr = kBN * (kVStride / 16) / 64;    // 8
constexpr int kVRegion = kVInstr * 1024;
constexpr int kStage = kKRegion + kVRegion;            // 21504 bytes
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleSlack = 8.0f;
#ifndef MLA_BF16_AHEAD
#define MLA_BF16_AHEAD 3
#endif
constexpr int kAhead = MLA_BF16_AHEAD;  // LDS operand prefetch distance, in MFMAs
static_assert(kAhead >= 1 && kAhead <= 4, "prefetch distance");
static_assert(kBN * kKSlots <= kKInstr * 64, "K tile slots");
static_assert(kWgPerCu * 3 * kStage <= 160 * 1024, "resident workgroups fit the LDS");

struct Bf16Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* cu_q;
  const int32_t* cu_k;
  uint16_t* out;
  float* lse;
  int64_t lse_stride;
  int64_t total_q;
  int64_t total_k;
  int32_t batch;
  int32_t n_heads;
  int32_t n_m_tiles;
  int32_t causal;
  int32_t xcd_order;  // 1: XCD-aware block order (one sequence, H % 4 == 0, even tile count)
  float scale_log2;
};

__device__ __forceinline__ v16f mfma_bf16(const v8bf& a, const v8bf& b, const v16f& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v4bf read_tr16(const uint8_t* lds_ptr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (__attribute__((address_space(3))) v4bf*)(lds_ptr));
}

// V rows hold sixteen 16-byte chunks (8 dims each); chunk c of key row k sits at position
// c ^ v_swizzle(k). For the transposed reads (four keys x 64 bytes per 16 lanes, two
// 16-lane groups on other keys) this puts every 16 lanes on distinct banks with 32
// four-byte banks and every 32 lanes with 64 banks.
__device__ __forceinline__ int v_swizzle(int key) { return ((key & 1) << 2) ^ (((key >> 1) & 1) * 10); }

__global__ __launch_bounds__(kThreads, kWgPerCu) void prefill_bf16_kernel(Bf16Params p) {
  // three K/V tile buffers: tile t is in buffer t % 3
  __shared__ __attribute__((aligned(16))) uint8_t lds[3 * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = p.n_heads;

  int h, b = 0, m_tile;
  if (p.xcd_order) {
    // one sequence: each XCD (block % 8) takes H/4 consecutive half-heads (even or odd
    // query tiles of a head), heaviest tile first, so that its L2 serves few heads' K/V
    const int hp = H >> 2;
    const int xcd = blockIdx.x & 7;
    const int slot = blockIdx.x >> 3;
    const int half = hp * xcd + slot % hp;
    const int rank = slot / hp;
    h = half >> 1;
    m_tile = p.n_m_tiles - 2 + (half & 1) - 2 * rank;
  } else {
    // heaviest query tiles first; (sequence, head) pairs rotated by 3 per tile index so
    // that each XCD (block % 8) sees every pair (the FP8 kernel's varlen order)
    const int pairs = H * p.batch;
    const int mi = blockIdx.x / pairs;
    const int pr = (blockIdx.x - mi * pairs + 3 * mi) % pairs;
    h = pr % H;
    b = pr / H;
    m_tile = p.n_m_tiles - 1 - mi;
  }

  int64_t q0 = p.cu_q[b], q1 = p.cu_q[b + 1], k0 = p.cu_k[b], k1 = p.cu_k[b + 1];
  q0 = min(max(q0, (int64_t)0), p.total_q);
  q1 = min(max(q1, q0), p.total_q);
  k0 = min(max(k0, (int64_t)0), p.total_k);
  k1 = min(max(k1, k0), p.total_k);
  const bool causal = p.causal != 0;
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
  int wave_kend = (wrow0 < Lq) ? kend : 0;
  if (causal && wrow0 < Lq) wave_kend = min(Lk, max(0, min(Lq, wrow0 + 32) + off));
  const int wave_tiles = (wave_kend + kBN - 1) / kBN;
  const int wave_iters = wave_tiles > 0 ? wave_tiles + 1 : 0;  // + the trailing PV

  // row strides in bytes
  const int64_t q_rs = static_cast<int64_t>(H) * kDqk * 2;
  const int64_t k_rs = static_cast<int64_t>(H) * kDqk * 2;
  const int64_t v_rs = static_cast<int64_t>(H) * kDv * 2;

  // Q fragment (B operand of S MFMA kb): row my_row, dims 16 kb + 8 g .. + 7
  v8bf qf[12];
  if (row_ok) {
    const uint8_t* qp = reinterpret_cast<const uint8_t*>(p.q) + (q0 + my_row) * q_rs +
                        h * (kDqk * 2) + 16 * g;
#pragma unroll
    for (int kb = 0; kb < 12; ++kb) qf[kb] = *reinterpret_cast<const v8bf*>(qp + 32 * kb);
  } else {
#pragma unroll
    for (int kb = 0; kb < 12; ++kb) qf[kb] = v8bf{};
  }

  const float c = p.scale_log2;
  float m_run = -INFINITY;
  float l_run = 0.f;  // this lane's part of the row sum (its 16 keys of every tile)
  v16f o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;

  const uint8_t* kbase =
      uniform_ptr(reinterpret_cast<const uint8_t*>(p.k) + k0 * k_rs + h * (kDqk * 2));
  const uint8_t* vbase =
      uniform_ptr(reinterpret_cast<const uint8_t*>(p.v) + k0 * v_rs + h * (kDv * 2));

  // Tile fill by global_load_lds_dwordx4 (lane l of an instruction writes 16-byte LDS slot
  // l). A K tile is 32 rows x 25 slots (24 data + 1 pad) in 13 instructions whose last 32
  // slots fall past the tile; a V tile is 32 rows x 16 slots in 8. The instructions of a
  // tile are dealt round-robin to the waves. Pad and spare slots load a duplicate chunk;
  // rows past the sequence load its last row (masked to -inf / weight 0 in the math).
  // Schedule and waits as in the FP8 kernel: iteration t reads K(t+1) and V(t-1) and
  // issues K(t+3) and V(t+1); the wait before the barrier leaves only this iteration's
  // loads in flight.
  constexpr int kPerK = (kKInstr + kWaves - 1) / kWaves;
  constexpr int kPerV = (kVInstr + kWaves - 1) / kWaves;
  const int n_k_instr = (kKInstr - wave + kWaves - 1) / kWaves;
  const int n_v_instr = (kVInstr - wave + kWaves - 1) / kWaves;
  auto dma_row = [&](int j, bool is_k) {
    const int slot = (wave + j * kWaves) * 64 + lane;
    if (is_k) {
      const int row = slot / kKSlots;
      const int chunk = min(slot - kKSlots * row, 23);  // pad slot -> last data chunk
      return make_int2(min(row, kBN - 1), 16 * chunk);  // spare slots past the tile
    }
    const int row = slot >> 4;
    return make_int2(row, 16 * ((slot & 15) ^ v_swizzle(row)));
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
  auto kbuf = [&](int t) { return lds + (t % 3) * kStage; };
  auto issue = [&](int t, bool is_k) {
    const int kt = t * kBN;
    const int64_t rs = is_k ? k_rs : v_rs;
    const uint32_t rs32 = is_k ? k_rs32 : v_rs32;
    const uint8_t* base = uniform_ptr((is_k ? kbase : vbase) + static_cast<int64_t>(kt) * rs);
    const uint32_t dst0 = lds_address(kbuf(t) + (is_k ? 0 : kKRegion));
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

  // transposed-read address of this lane (16-lane group G, source lane s): key
  // 4 (G / 2) + s / 4 (+ 16 c + 8 t), dims 32 db + 16 (G % 2) + 4 (s % 4) .. + 3. Keys
  // that differ by multiples of 4 share the swizzle, and block db flips address bits 6..7.
  const int grp = lane >> 4, sl = lane & 15;
  const int vt_key0 = 4 * (grp >> 1) + (sl >> 2);
  const int vt_chunk = 2 * (grp & 1) + ((sl & 3) >> 1);
  const int vt_off = vt_key0 * kVStride + 16 * (vt_chunk ^ v_swizzle(vt_key0)) + 8 * (sl & 1);
  auto vt_operand = [&](const uint8_t* vl, int db, int ck) {
    const uint8_t* vp = vl + (vt_off ^ (db << 6)) + 16 * ck * kVStride;
    const v4bf r0 = read_tr16(vp);
    const v4bf r1 = read_tr16(vp + 8 * kVStride);
    return v8bf{r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
  };
  // A operand of S MFMA kb: key row col, dims 16 kb + 8 g .. + 7
  auto k_operand = [&](const uint8_t* kl, int kb) {
    return *reinterpret_cast<const v8bf*>(kl + col * kKStride + 32 * kb + 16 * g);
  };

  // prologue: K(0), V(0), K(1) in LDS, K(2) in flight, S of tile 0 computed
  int in_flight = 0;
  if (n_tiles > 0) { issue(0, true); issue(0, false); }
  if (n_tiles > 1) issue(1, true);
  if (n_tiles > 2) { issue(2, true); in_flight += n_k_instr; }
  wait_vmcnt(in_flight);
#pragma unroll
  for (int kb = 0; kb < 12; ++kb) asm volatile("" ::"v"(qf[kb]));
  block_barrier();
  v16f s_cur;
  for (int r = 0; r < 16; ++r) s_cur[r] = 0.f;
  if (wave_tiles > 0) {
    const uint8_t* kl = kbuf(0);
#pragma unroll
    for (int kb = 0; kb < 12; ++kb) s_cur = mfma_bf16(k_operand(kl, kb), qf[kb], s_cur);
  }

  const v2bf ones2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  // P of accumulator registers 8 ck .. 8 ck + 7 as one bf16 B operand; the row sum adds
  // the rounded weights
  auto softmax_chunk = [&](const v16f& sc, float nbias, int ck) {
    v8bf pb;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const float e0 = __builtin_amdgcn_exp2f(fmaf(sc[8 * ck + i], c, nbias));
      const float e1 = __builtin_amdgcn_exp2f(fmaf(sc[8 * ck + i + 1], c, nbias));
      const v2bf pr = __builtin_convertvector(v2f{e0, e1}, v2bf);
      l_run = __builtin_amdgcn_fdot2_f32_bf16(pr, ones2, l_run, false);
      pb[i] = pr[0];
      pb[i + 1] = pr[1];
    }
    return pb;
  };

  // One software-pipelined iteration: PV of tile it-1 (8 MFMAs), S of tile it+1 (12) and
  // the softmax of tile it, interleaved. The last iteration of a wave is a fully masked
  // tile that only completes the PV of its last tile; on iteration 0 the previous P is
  // zero.
  auto step = [&](int it, v16f& s_c, v16f& s_n, const v8bf (&pb_prev)[2], v8bf (&pb_cur)[2]) {
    const bool active = it < wave_iters;
    const uint8_t* kl = kbuf(it + 1);
    const uint8_t* vl = kbuf(it > 0 ? it - 1 : 0) + kKRegion;
    // operands are read kAhead MFMAs of their kind ahead of use (a ring of kAhead
    // registers each): a bf16 MFMA is too short to cover an LDS read issued just before it
    v8bf va[kAhead], ka[kAhead];
    if (active) {
#pragma unroll
      for (int j = 0; j < kAhead; ++j) {
        va[j] = vt_operand(vl, j & 3, j >> 2);
        ka[j] = k_operand(kl, j);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    int issued = 0;
    if (it + 3 < n_tiles) { issue(it + 3, true); issued += n_k_instr; }
    if (it + 1 < n_tiles) { issue(it + 1, false); issued += n_v_instr; }

    if (active) {
      const int kt = it * kBN;
      const bool need_mask =
          it >= wave_tiles || (kt + kBN > Lk) || (causal && kt + kBN - 1 > wrow0 + off);
      if (need_mask) {
        asm volatile("" ::: "memory");  // keep the rare masking a real branch
        const bool all = it >= wave_tiles;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt + 8 * (r >> 2) + 4 * g + (r & 3);
          if (all || key >= Lk || (causal && key > my_row + off)) s_c[r] = -INFINITY;
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; r += 4)
        mx = vmax3(mx, vmax3(s_c[r], s_c[r + 1], s_c[r + 2]), s_c[r + 3]);
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
      const float nbias = (m_run == -INFINITY) ? 0.f : -m_run;

      for (int r = 0; r < 16; ++r) s_n[r] = 0.f;
      // 20 MFMA slots: PV (db, ck) alternate with S kb; the softmax of the two key chunks
      // sits after the fourth and the eighth PV MFMA
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int db = j & 3, ck = j >> 2;
        o[db] = mfma_bf16(va[j % kAhead], pb_prev[ck], o[db]);
        if (j + kAhead < 8) va[j % kAhead] = vt_operand(vl, (j + kAhead) & 3, (j + kAhead) >> 2);
        __builtin_amdgcn_sched_barrier(0);
        s_n = mfma_bf16(ka[j % kAhead], qf[j], s_n);
        ka[j % kAhead] = k_operand(kl, j + kAhead);
        if (j == 3) pb_cur[0] = softmax_chunk(s_c, nbias, 0);
        if (j == 7) pb_cur[1] = softmax_chunk(s_c, nbias, 1);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int kb = 8; kb < 12; ++kb) {
        s_n = mfma_bf16(ka[kb % kAhead], qf[kb], s_n);
        if (kb + kAhead < 12) ka[kb % kAhead] = k_operand(kl, kb + kAhead);
      }
      asm volatile("" ::"v"(pb_cur[0]), "v"(pb_cur[1]), "v"(l_run));

      if (rescale) {
        asm volatile("" : "+v"(alpha)::"memory");
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      }
    }
    wait_vmcnt(issued);
    block_barrier();
  };

  v16f s_alt;
  v8bf pb_a[2] = {v8bf{}, v8bf{}}, pb_b[2] = {v8bf{}, v8bf{}};
  for (int it = 0; it <= n_tiles; it += 2) {
    step(it, s_cur, s_alt, pb_a, pb_b);
    if (it + 1 <= n_tiles) step(it + 1, s_alt, s_cur, pb_b, pb_a);
  }

  // epilogue: this lane holds row my_row, dims 32 db + 8 (r / 4) + 4 g + r % 4
  float l_tot;
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run),
                                                     false, false);
    l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  if (row_ok) {
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    uint16_t* op = p.out + (q0 + my_row) * (static_cast<int64_t>(H) * kDv) + h * kDv;
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
    if (g == 0 && p.lse != nullptr)
      p.lse[static_cast<int64_t>(h) * p.lse_stride + q0 + my_row] =
          (l_tot > 0.f) ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

}  // namespace

extern "C" int mla_bf16_prefill_varlen(const void* q, const void* k, const void* v,
                                       const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                       int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                       int64_t total_q, int64_t total_k, int32_t n_heads,
                                       int32_t head_dim_qk, int32_t head_dim_v, float softmax_scale,
                                       int32_t causal, void* out, float* lse, int64_t lse_stride,
                                       void* stream) {
  int st = mla::prefill_check_common(n_heads, head_dim_qk, head_dim_v, softmax_scale, causal);
  if (st != MLA_OK) return st;
  if (batch < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || total_q < 0 || total_k < 0)
    return mla::fail(MLA_ERR_INVALID_ARGUMENT, "negative size");
  if (total_q >= (1ll << 31) || total_k >= (1ll << 31))
    return mla::fail(MLA_ERR_UNSUPPORTED, "total_q and total_k must be < 2^31");
  if (static_cast<int64_t>(n_heads) * kDqk * 2 * kBN >= (1ll << 31))
    return mla::fail(MLA_ERR_UNSUPPORTED, "n_heads too large");
  if (total_q == 0 || batch == 0 || max_seqlen_q == 0) return mla::ok();
  if (q == nullptr || out == nullptr || cu_seqlens_q == nullptr || cu_seqlens_k == nullptr)
    return mla::fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (total_k > 0 && (k == nullptr || v == nullptr))
    return mla::fail(MLA_ERR_INVALID_ARGUMENT, "k or v is NULL");
  if (!mla::aligned16(q) || !mla::aligned16(k) || !mla::aligned16(v) || !mla::aligned16(out))
    return mla::fail(MLA_ERR_INVALID_ARGUMENT, "q, k, v and out must be 16-byte aligned");
  if (lse != nullptr && lse_stride < total_q)
    return mla::fail(MLA_ERR_INVALID_ARGUMENT, "lse_stride < total_q");
  const int64_t n_m = (static_cast<int64_t>(max_seqlen_q) + kBM - 1) / kBM;
  const int64_t blocks = n_m * batch * n_heads;
  if (blocks >= (1ll << 31)) return mla::fail(MLA_ERR_UNSUPPORTED, "grid too large");
  Bf16Params prm{};
  prm.q = static_cast<const uint16_t*>(q);
  prm.k = static_cast<const uint16_t*>(k);
  prm.v = static_cast<const uint16_t*>(v);
  prm.cu_q = cu_seqlens_q;
  prm.cu_k = cu_seqlens_k;
  prm.out = static_cast<uint16_t*>(out);
  prm.lse = lse;
  prm.lse_stride = lse_stride;
  prm.total_q = total_q;
  prm.total_k = total_k;
  prm.batch = batch;
  prm.n_heads = n_heads;
  prm.n_m_tiles = static_cast<int32_t>(n_m);
  prm.causal = causal;
  prm.xcd_order = (batch == 1 && n_heads % 4 == 0 && n_m % 2 == 0) ? 1 : 0;
  prm.scale_log2 = softmax_scale * 1.44269504088896340736f;
  hipLaunchKernelGGL(prefill_bf16_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), prm);
  return mla::check_launch("prefill_bf16_kernel");
}
