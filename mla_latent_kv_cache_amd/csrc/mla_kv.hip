// Absorbed MLA decode over a quantized latent KV cache, for MI355X (gfx950).
//
// The operation (one layer, one new query token per sequence) is defined in
// include/mla_kv.h. Sources on the pages this follows:
//   * "Absorbed MLA Cache Optimization on DeepSeek-V2-Lite", section 2.1 (the
//     cache stores the 512-d latent plus the 64-d k_pe per token, quantizing
//     on store, and projects at compute time), section 3.2 / 4.2 tables
//     (per-channel INT8 in 32 blocks, k_pe INT8 in 8 blocks, asymmetric INT4
//     in 32 blocks).
//   * "DeepSeek的MLA技术", MLA mechanism step 2 (K_i = C W_i^upK,
//     V_i = C W_i^upV) and MLAttentionWithCache (per-head softmax(q K^T s) V
//     over every cached token). Absorbing W_UK into the query and applying
//     W_UV after the softmax-weighted latent sum is the same computation by
//     associativity; no token is expanded here.
//
// Kernels, in launch order:
//   append_kernel       quantize new bf16 rows into the cache planes
//   seqlen_kernel       advance seq_lens after an append
//   absorb_kernel       q_abs = scale*log2(e) * q_nope W_UK[h]  -> fp16 hi/lo
//                       records in the workspace
//   append_step_kernel  one new token per sequence (the decode step's append)
//   step_kernel         the fused step's first launch: absorb, turn and store
//   split16_kernel      split-KV partial attention: each workgroup takes an
//                       equal run of the batch's 32-token tiles for 16 heads
//                       (a head slice of the query); 16-byte loads of codes,
//                       in-register dequant to fp16, MFMA scores and value
//                       sums, online softmax in base 2
//   wide_kernel         the same for 32 heads per workgroup (BF16 and INT8
//                       latents at 32-128 heads)
//   combine_kernel      log-sum-exp merge of the splits for 16 sequences,
//                       then o_lat W_UV[h] on MFMA (grids of 1024+ blocks)
//   reduce_kernel       the same merge, W_UV on VALU, 4 sequences per block
//   reduce1_kernel      the same, one sequence per block (small grids)
//   get_kernel          dequantize a layer to fp32 (inspection aid)
//   rope_table_kernel   the fused step's fp32 angle tables
//   stream_read_kernel, mfma_rate_kernel   measurement aids (read ceiling,
//                       matrix-unit rate)

#include <hip/hip_runtime.h>

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "mla_kv.h"

namespace {

// ----------------------------------------------------------------- constants

constexpr int kLatent = 512;               // kv_lora_rank
constexpr int kRope = 64;                  // qk_rope_head_dim
constexpr int kRow = kLatent + kRope;      // 576 channels scored per token
constexpr int kNope = 128;                 // qk_nope_head_dim
constexpr int kVDim = 128;                 // v_head_dim
constexpr int kGroupL = 16;                // latent channels per quantization group
constexpr int kGroupR = 8;                 // k_pe channels per quantization group
constexpr int kNGroupL = kLatent / kGroupL;  // 32
constexpr int kNGroupR = kRope / kGroupR;    // 8
constexpr int kNScale = kNGroupL + kNGroupR; // 40 quantization groups per row

// What each format stores: the latent as one of BF16 / INT8 / INT4, the k_pe
// as bf16, INT8 or INT4 (symmetric), the fp16 scales per row, the row bytes.
enum { kKpeBf16 = 0, kKpeI8 = 1, kKpeI4 = 2 };
constexpr int lat_fmt(int f) {
  return f == MLA_FMT_INT8_KBF16 ? MLA_FMT_INT8 : f == MLA_FMT_INT4_KINT4 ? MLA_FMT_INT4 : f;
}
constexpr int kpe_fmt(int f) {
  return (f == MLA_FMT_BF16 || f == MLA_FMT_INT8_KBF16) ? kKpeBf16 : f == MLA_FMT_INT4_KINT4 ? kKpeI4 : kKpeI8;
}
constexpr int n_scales(int f) { return f == MLA_FMT_BF16 ? 0 : f == MLA_FMT_INT8_KBF16 ? kNGroupL : kNScale; }
constexpr int ckv_bytes(int f) {
  return lat_fmt(f) == MLA_FMT_BF16 ? kLatent * 2 : lat_fmt(f) == MLA_FMT_INT8 ? kLatent : kLatent / 2;
}
constexpr int kpe_bytes(int f) {
  return kpe_fmt(f) == kKpeBf16 ? kRope * 2 : kpe_fmt(f) == kKpeI8 ? kRope : kRope / 2;
}
constexpr bool has_zero(int f) { return lat_fmt(f) == MLA_FMT_INT4; }
constexpr int64_t kMaxSeqPlaneBytes = (int64_t)1 << 30;  // bytes of one sequence's rows in any plane
constexpr int64_t kMaxGrid = INT32_MAX;    // workgroups in one launch
constexpr int kWaves = 4;                  // waves per split workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kMaxSplits = 4096;
constexpr int kAutoMinTiles = 4;           // fewest 32-token tiles per range of the automatic plan (full sequences)
constexpr int kAutoShortRuns = 8;          // ranges per sequence the automatic plan allows a short cache
constexpr int kWgPerCu = 3;                // resident partial workgroups per CU
#ifndef MLA_COMBINE_MFMA
#define MLA_COMBINE_MFMA 1
#endif
constexpr bool kCombineMfma = MLA_COMBINE_MFMA;  // merge + W_UV projection on MFMA (combine_kernel)
constexpr float kLazy = 8.0f;              // log2 of the largest softmax weight before a rescale
constexpr float kLog2e = 1.4426950408889634f;

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

template <typename To, typename From>
__device__ __forceinline__ To bitcast(From v) {
  static_assert(sizeof(To) == sizeof(From), "size");
  return __builtin_bit_cast(To, v);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return (float)bitcast<_Float16>(b);
}

// ------------------------------------------------------- exact quantization
// One IEEE fp32 operation per step, no contraction, correctly rounded
// division (the compiler default for HIP), rintf = round half to even.

#pragma clang fp contract(off)

// fp32 -> fp16 bits, round to nearest even, saturating at +-65504.
__device__ __forceinline__ uint16_t f16_rne_sat(float v) {
  uint16_t b = bitcast<uint16_t>((_Float16)v);
  if ((b & 0x7FFFu) == 0x7C00u) b = (uint16_t)((b & 0x8000u) | 0x7BFFu);
  return b;
}

// fp32 -> fp16 bits, rounded toward -inf, saturating, zero stored as +0.
__device__ __forceinline__ uint16_t f16_rd_sat(float v) {
  uint16_t b = bitcast<uint16_t>((_Float16)v);
  if (b == 0x7C00u) b = 0x7BFFu;  // above the largest finite: round down to it
  if (f16_bits_to_f32(b) > v) {   // nearest was above v: step one toward -inf
    if ((b & 0x7FFFu) == 0) b = 0x8001u;
    else if (b & 0x8000u) b = (uint16_t)(b + 1);
    else b = (uint16_t)(b - 1);
  }
  if (b == 0xFC00u) b = 0xFBFFu;
  if (b == 0x8000u) b = 0x0000u;
  return b;
}

// Symmetric quantization of n values to codes in [-QMAX, QMAX] (127: INT8,
// 7: INT4): returns the fp16 scale bits, writes codes.
template <int N, int QMAX = 127>
__device__ __forceinline__ uint16_t quant_sym8(const float (&x)[N], int8_t (&q)[N]) {
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < N; ++i) a = fmaxf(a, fabsf(x[i]));
  uint16_t sb = f16_rne_sat(__fdiv_rn(a, (float)QMAX));
  float s = f16_bits_to_f32(sb);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    float c = 0.0f;
    if (s != 0.0f) c = fminf(fmaxf(rintf(__fdiv_rn(x[i], s)), -(float)QMAX), (float)QMAX);
    q[i] = (int8_t)(int)c;
  }
  return sb;
}

// Asymmetric INT4 of 16 values: writes scale and zero bits and codes 0..15.
__device__ __forceinline__ void quant_asym4(const float (&x)[kGroupL], uint8_t (&q)[kGroupL],
                                            uint16_t &sb, uint16_t &zb) {
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int i = 1; i < kGroupL; ++i) {
    mn = fminf(mn, x[i]);
    mx = fmaxf(mx, x[i]);
  }
  zb = f16_rd_sat(mn);
  float z = f16_bits_to_f32(zb);
  sb = f16_rne_sat(__fdiv_rn(__fsub_rn(mx, z), 15.0f));
  if ((sb & 0x7FFFu) == 0) sb = 0;  // zero scale stored as +0 (sign of max - z is not defined)
  float s = f16_bits_to_f32(sb);
#pragma unroll
  for (int i = 0; i < kGroupL; ++i) {
    float c = 0.0f;
    if (s != 0.0f) c = fminf(fmaxf(rintf(__fdiv_rn(__fsub_rn(x[i], z), s)), 0.0f), 15.0f);
    q[i] = (uint8_t)(int)c;
  }
}

#pragma clang fp contract(on)

// Wait until every LDS instruction this wave issued has completed, with no
// instruction moved across: a conservative fence, used at a few places off
// the per-tile path of the 16-head kernel.
__device__ __forceinline__ void lds_stores_done() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt left at their maxima
  __builtin_amdgcn_sched_barrier(0);
}

// ------------------------------------------------------------------ append

// Sequences are numbered across the layers a call covers: sequence j is
// batch entry j % batch of layer j / batch (counted from the call's first
// layer, whose planes the kernels receive). Contiguous planes keep the rows of
// sequence j at j * cap (the planes are [layer][batch][cap] rows).
// Paged planes: token p of sequence j is row p % size of page
// table[j % batch][p / size] of layer j / batch's pool (layer_rows rows
// apart); size = 0 means contiguous rows.
struct Paging {
  const int32_t *table;  // [batch][max_pages]
  int size, shift, max_pages, num_pages;  // size = 1 << shift (a power of two >= 32)
  int batch;             // sequences per layer
  int64_t layer_rows;    // rows of one layer's pool (num_pages * size)
};

// Page of token p of sequence j, or -1 when the table entry is outside the pool.
__device__ __forceinline__ int page_of(const Paging &pg, int j, int p) {
  const int page = pg.table[(int64_t)(j % pg.batch) * pg.max_pages + (p >> pg.shift)];
  return (page >= 0 && page < pg.num_pages) ? page : -1;
}

// Row within the planes of token p of sequence j, or -1 (no page).
__device__ __forceinline__ int64_t plane_row(const Paging &pg, int j, int cap, int p) {
  if (pg.size == 0) return (int64_t)j * cap + p;
  const int page = page_of(pg, j, p);
  return page < 0 ? -1
                  : (int64_t)(j / pg.batch) * pg.layer_rows + ((int64_t)page << pg.shift) + (p & (pg.size - 1));
}

// The latent plane keeps its rows in blocks of 16: within a block, the
// 16-byte chunk c of row i lies at byte (16 c + i) * 16, so chunk c of the
// block's 16 rows is 256 contiguous bytes, and a 64-lane load of chunks
// c..c+3 of a block (lane 16 g + i: chunk c + g of row i, the operand layout
// of the matrix instructions) reads 1 KB in one piece. Each sequence's rows
// start on a block: in the contiguous layout its latent rows are
// lat_stride(capacity) apart (capacity rounded up to 16); a page holds whole
// blocks. The other planes keep plain rows.
__host__ __device__ constexpr int lat_stride(int cap) { return (cap + 15) & ~15; }

// Byte offset of chunk c of row `row` (rows counted from a block start).
__device__ __forceinline__ int64_t lat_off(int64_t row, int c, int row_bytes) {
  return (row >> 4) * (int64_t)(16 * row_bytes) + (int64_t)(c * 16 + (int)(row & 15)) * 16;
}

// Latent row of a token whose row in the other planes is `row` (from plane_row).
__device__ __forceinline__ int64_t lat_row_of(const Paging &pg, int64_t row, int b, int cap, int p) {
  return pg.size ? row : (int64_t)b * lat_stride(cap) + p;
}

struct AppendArgs {
  void *ckv;            // layer base of the ckv plane
  void *kpe;
  uint16_t *scale;
  uint16_t *zero;
  int32_t *seq_lens;        // layer row of seq_lens
  const uint16_t *ckv_new;  // bf16 [B][T][512]
  const uint16_t *kpe_new;  // bf16 [B][T][64]
  const int32_t *n_new;     // optional [B]
  const float *rope_cos;    // optional fp32 [rows][32]: the k_pe of new tokens turns by its row
  const float *rope_sin;    // (fused decode step only; plain appends store k_pe as given)
  Paging pg;
  int B, T, cap;
};

// One RoPE turn of a channel pair by a table angle, in fp32 with every
// product and every sum rounded (no contraction into a fused multiply-add),
// so that the turned value is the same on any IEEE fp32 machine.
__device__ __forceinline__ void rope_pair_exact(float x0, float x1, float c, float s, float &y0, float &y1) {
#pragma clang fp contract(off)
  const float a = x0 * c, b = x1 * s, d = x0 * s, e = x1 * c;
  y0 = a - b;
  y1 = d + e;
}

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Quantize and store one group (grp < 32: latent group, else k_pe group) of
// new token t of sequence b at row `pos` of the cache.
template <int FMT>
__device__ __forceinline__ void append_group(const AppendArgs &a, int b, int t, int grp, int pos) {
  const int64_t row = plane_row(a.pg, b, a.cap, pos);
  if (row < 0) return;  // no page for this position: nothing is stored
  if (grp < kNGroupL) {
    const int64_t lrow = lat_row_of(a.pg, row, b, a.cap, pos);
    const uint16_t *src = a.ckv_new + ((int64_t)b * a.T + t) * kLatent + grp * kGroupL;
    const u32x4 v0 = *(const u32x4 *)src;
    const u32x4 v1 = *(const u32x4 *)(src + 8);
    if (lat_fmt(FMT) == MLA_FMT_BF16) {  // 16 channels: chunks 2 grp and 2 grp + 1
      *(u32x4 *)((uint8_t *)a.ckv + lat_off(lrow, 2 * grp, kLatent * 2)) = v0;
      *(u32x4 *)((uint8_t *)a.ckv + lat_off(lrow, 2 * grp + 1, kLatent * 2)) = v1;
      return;
    }
    float x[kGroupL];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_bits_to_f32(v0[i] & 0xFFFFu);
      x[2 * i + 1] = bf16_bits_to_f32(v0[i] >> 16);
      x[8 + 2 * i] = bf16_bits_to_f32(v1[i] & 0xFFFFu);
      x[8 + 2 * i + 1] = bf16_bits_to_f32(v1[i] >> 16);
    }
    if (lat_fmt(FMT) == MLA_FMT_INT8) {
      int8_t q[kGroupL];
      const uint16_t sb = quant_sym8<kGroupL>(x, q);
      u32x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = (uint32_t)(uint8_t)q[4 * i] | ((uint32_t)(uint8_t)q[4 * i + 1] << 8) |
               ((uint32_t)(uint8_t)q[4 * i + 2] << 16) | ((uint32_t)(uint8_t)q[4 * i + 3] << 24);
      *(u32x4 *)((uint8_t *)a.ckv + lat_off(lrow, grp, kLatent)) = w;  // chunk grp
      a.scale[row * n_scales(FMT) + grp] = sb;
    } else {
      uint8_t q[kGroupL];
      uint16_t sb, zb;
      quant_asym4(x, q, sb, zb);
      u32x2 w;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        uint32_t v = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) v |= (uint32_t)q[8 * i + j] << (4 * j);
        w[i] = v;
      }
      // the first or second half of chunk grp / 2
      *(u32x2 *)((uint8_t *)a.ckv + lat_off(lrow, grp >> 1, kLatent / 2) + (grp & 1) * 8) = w;
      a.scale[row * n_scales(FMT) + grp] = sb;
      a.zero[row * kNGroupL + grp] = zb;
    }
  } else {
    const int g = grp - kNGroupL;
    const uint16_t *src = a.kpe_new + ((int64_t)b * a.T + t) * kRope + g * kGroupR;
    u32x4 v = *(const u32x4 *)src;
    if (a.rope_cos) {
      // turn the group's 4 channel pairs by the row's angles, round to bf16
      const float *cr = a.rope_cos + (int64_t)pos * (kRope / 2) + g * (kGroupR / 2);
      const float *sr = a.rope_sin + (int64_t)pos * (kRope / 2) + g * (kGroupR / 2);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float y0, y1;
        rope_pair_exact(bf16_bits_to_f32(v[j] & 0xFFFFu), bf16_bits_to_f32(v[j] >> 16), cr[j], sr[j], y0, y1);
        v[j] = f32_to_bf16_rne(y0) | (f32_to_bf16_rne(y1) << 16);
      }
    }
    if (kpe_fmt(FMT) == kKpeBf16) {
      *(u32x4 *)((uint16_t *)a.kpe + row * kRope + g * kGroupR) = v;
      return;
    }
    float x[kGroupR];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_bits_to_f32(v[i] & 0xFFFFu);
      x[2 * i + 1] = bf16_bits_to_f32(v[i] >> 16);
    }
    int8_t q[kGroupR];
    if (kpe_fmt(FMT) == kKpeI8) {
      const uint16_t sb = quant_sym8<kGroupR>(x, q);
      u32x2 w;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        w[i] = (uint32_t)(uint8_t)q[4 * i] | ((uint32_t)(uint8_t)q[4 * i + 1] << 8) |
               ((uint32_t)(uint8_t)q[4 * i + 2] << 16) | ((uint32_t)(uint8_t)q[4 * i + 3] << 24);
      *(u32x2 *)((int8_t *)a.kpe + row * kRope + g * kGroupR) = w;
      a.scale[row * n_scales(FMT) + grp] = sb;
    } else {  // symmetric INT4: nibble code + 8, the even channel low
      const uint16_t sb = quant_sym8<kGroupR, 7>(x, q);
      uint32_t w = 0;
#pragma unroll
      for (int j = 0; j < kGroupR; ++j) w |= (uint32_t)(q[j] + 8) << (4 * j);
      *(uint32_t *)((uint8_t *)a.kpe + row * (kRope / 2) + g * (kGroupR / 2)) = w;
      a.scale[row * n_scales(FMT) + grp] = sb;
    }
  }
}

// Bulk append: one thread per quantization group of one new row; grid row y
// serves sequences y, y + gridDim.y, ..., whose n_new[b] rows take the first
// n_new[b] * 40 threads of the row (blocks past them skip the sequence at once,
// so the padding of a ragged batch costs nothing, and no index needs a
// division by a runtime count). seq_lens advances in seqlen_kernel, launched
// after it on the same stream, so every block reads the old length.
template <int FMT>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int t = (int)(idx / kNScale);
  const int grp = (int)(idx % kNScale);
  for (int b = blockIdx.y; b < a.B; b += gridDim.y) {
    const int n = a.n_new ? min(max(a.n_new[b], 0), a.T) : a.T;
    if (t >= n) continue;
    const int pos = a.seq_lens[b] + t;
    if (pos < 0 || pos >= a.cap) continue;
    append_group<FMT>(a, b, t, grp, pos);
  }
}

// Counts are clamped to [0, T] here as in append_kernel, so a length never
// moves past the rows that were stored.
__global__ void seqlen_kernel(int32_t *seq_lens, const int32_t *n_new, int B, int T, int cap) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int n = n_new ? min(max(n_new[b], 0), T) : T;
  const int64_t v = (int64_t)seq_lens[b] + n;
  seq_lens[b] = (int32_t)(v > cap ? cap : v);
}

// Small appends (a decode step): one block per sequence stores its T*40 groups,
// then advances its own length after a block barrier. One launch.
constexpr int kStepAppendMaxT = 8;

template <int FMT>
__global__ __launch_bounds__(128) void append_step_kernel(AppendArgs a) {
  const int b = blockIdx.x;
  const int n = a.n_new ? min(max(a.n_new[b], 0), a.T) : a.T;
  const int base = a.seq_lens[b];
  for (int i = threadIdx.x; i < a.T * kNScale; i += blockDim.x) {
    const int t = i / kNScale, grp = i % kNScale;
    const int pos = base + t;
    if (t < n && pos >= 0 && pos < a.cap) append_group<FMT>(a, b, t, grp, pos);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int64_t v = (int64_t)base + n;
    a.seq_lens[b] = (int32_t)(v > a.cap ? a.cap : v);
  }
}

// ------------------------------------------------------------------ absorb

constexpr int kAbsorbBT = 64;              // batch rows per absorb block (four MFMA column blocks)
constexpr int kAbsorbCB = 128;             // latent channels per absorb block, 32 per wave
constexpr int kAbsorbWRow = kAbsorbCB + 16;  // bf16 per LDS row of the staged W_UK tile (see below)
// fp16 per LDS row of the staged records: 128 hi, 128 lo, 8 + 8 group sums, and
// 8 of padding (rows 35 x 16 bytes apart, so the 16 rows of one store fall on
// different banks)
constexpr int kAbsorbORow = 2 * kAbsorbCB + 16 + 8;
static_assert(kAbsorbBT * kAbsorbORow <= kNope * kAbsorbWRow, "the record stage fits in the W_UK tile's LDS");
static_assert(kAbsorbCB == 128, "34 record pieces of 16 bytes per row (16 + 16 + 1 + 1), as the copy-out assumes");

// Per (sequence, head) record of absorbed queries, in fp16, each value v kept
// as hi = fp16(v) and lo = fp16(v - hi), so that hi + lo carries ~22 bits:
//   [0, 576)          hi of (q_abs | q_pe) * softmax_scale * log2(e)
//   [576, 1152)       lo of the same
//   [1152, 1184)      hi of the 32 latent-group sums of q_abs (INT4 zero-points)
//   [1184, 1216)      lo of those sums
constexpr int kQHi = 0, kQLo = kRow, kQSumHi = 2 * kRow, kQSumLo = 2 * kRow + kNGroupL;
constexpr int kQRec = 2 * kRow + 2 * kNGroupL;  // 1216 halves

// Transposed LDS read (ds_read_b64_tr_b16): the 16 lanes of a lane group
// each give the address of 4 consecutive 16-bit values, together a block of 4
// rows x 16 columns; lane i receives column i of those 4 rows.
__device__ __forceinline__ i16x4 lds_read_tr16_i16(const uint16_t *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(p));
}

// v as an fp16 pair: hi = fp16(v), lo = fp16(v - hi). v passes through an
// empty asm first, so that both uses of hi round this very fp32 value: the
// compiler may otherwise fold the product that made v into a mixed-precision
// fma that rounds to fp16 once (v_fma_mixlo_f16) for one use and keep the fp32
// product for the other, and in the rare cases where the two roundings differ
// lo then carries the wrong sign and hi + lo is off by one fp16 ulp of hi.
__device__ __forceinline__ void split_f16(float v, _Float16 &hi, _Float16 &lo) {
  asm volatile("" : "+v"(v));
  hi = (_Float16)v;
  lo = (_Float16)(v - (float)hi);
}

__device__ __forceinline__ void split_store(_Float16 *hi, _Float16 *lo, float v) {
  _Float16 h, l;
  split_f16(v, h, l);
  *hi = h;
  *lo = l;
}

// q_abs[b,h,c] = qs * sum_d q_nope[b,h,d] W_UK[h,d,c] for c < 512, and
// qs * q_pe[b,h,d] for the 64 RoPE channels; qs = softmax_scale * log2(e),
// so the attention kernels work in base 2.
// One block of the absorption: head h, channel block cb (128 channels), batch
// block bz (64 rows); 256 threads. The block stages its W_UK tile (128 d x
// 128 c, rows padded to 144 bf16 = 72 dwords, so the four rows of a
// transposed read start 8 banks apart) in LDS once. The block's channels form
// eight 16-channel column blocks (each one latent group) and its batch rows
// groups of 16; each wave takes one row group and some of the column blocks
// (the work split below), as [16 c x 32 d] x [32 d x 16 b] bf16 MFMAs with
// fp32 accumulation (bf16 products are exact in fp32). The W_UK operand comes
// from LDS through transposed reads, 8 consecutive d per lane; the query
// operand is those same 8 d of one batch row, one 16-byte load. With with_pe,
// the blocks of channel block 0 also write the scaled RoPE part.
__device__ __forceinline__ void absorb_block(const uint16_t *q_nope, const uint16_t *q_pe,
                                             const uint16_t *w_uk, int B, int H, float qs, _Float16 *qa,
                                             int h, int cb, int bz, bool with_pe) {
  __shared__ __attribute__((aligned(16))) uint16_t wt[kNope * kAbsorbWRow];
  const int b0 = bz * kAbsorbBT;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, g = lane >> 4, i = lane & 15;
  constexpr int kCPR = kAbsorbCB / 8;  // 16-byte chunks per W_UK tile row

  // W_UK[h][:, 128cb .. 128cb+127]: 128 rows of 256 bytes, 16 bytes per lane
  const uint16_t *wsrc = w_uk + (int64_t)h * kNope * kLatent + cb * kAbsorbCB;
  constexpr int kWLoads = kNope * kAbsorbCB / 8 / 256;
  u32x4 wl[kWLoads];
#pragma unroll
  for (int j = 0; j < kWLoads; ++j) {
    const int k = tid + 256 * j, row = k / kCPR, c8 = k % kCPR;
    wl[j] = *(const u32x4 *)(wsrc + (int64_t)row * kLatent + 8 * c8);
  }
  // Work split: the block's rows form nbb groups of 16; each group is served by
  // wpb waves (4 / nbb rounded up to a power of two), each of which takes
  // kCBk / wpb of the 16-channel column blocks. A full block (64 rows) gives
  // each wave one row group and all 128 channels, so every query row is loaded
  // once; a small batch keeps all four waves busy on its rows.
  constexpr int kCBk = kAbsorbCB / 16;
  const int nbb = (min(kAbsorbBT, B - b0) + 15) >> 4;  // 1 .. 4
  const int wpb = nbb == 1 ? 4 : nbb == 2 ? 2 : 1;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int bbw = wu / wpb;                           // this wave's row group
  const int c0 = (wu % wpb) * (kCBk / wpb), c1 = c0 + kCBk / wpb;  // its column blocks
  const bool rows_live = bbw < nbb;                   // uniform
  // the query operands of this wave's 16 batch rows (rows past the batch
  // repeat its last row and are not stored), in flight together with the tile
  u32x4 qv[kNope / 32];
  {
    const int b = min(b0 + 16 * bbw + i, B - 1);
    const uint16_t *qrow = q_nope + ((int64_t)b * H + h) * kNope + 8 * g;
#pragma unroll
    for (int kk = 0; kk < kNope / 32; ++kk) qv[kk] = *(const u32x4 *)(qrow + 32 * kk);
  }
  // blocks of channel block 0 also scale the RoPE part: 8 values per 16-byte
  // chunk, 64 rows of 8 chunks
  constexpr int kPLoads = kAbsorbBT * kRope / 8 / 256;
  u32x4 qpv[kPLoads];
  const bool pe = with_pe && cb == 0;
  if (pe) {
#pragma unroll
    for (int j = 0; j < kPLoads; ++j) {
      const int k = tid + 256 * j, b = min(b0 + (k >> 3), B - 1);
      qpv[j] = *(const u32x4 *)(q_pe + ((int64_t)b * H + h) * kRope + 8 * (k & 7));
    }
  }
#pragma unroll
  for (int j = 0; j < kWLoads; ++j) {
    const int k = tid + 256 * j, row = k / kCPR, c8 = k % kCPR;
    *(u32x4 *)(wt + row * kAbsorbWRow + 8 * c8) = wl[j];
  }
  __syncthreads();
  // The wave's column blocks, one 16-channel block (one latent group) at a
  // time: lane (i, g) of k-step kk takes column 16 cbk + i, rows 32kk + 8g ..
  // +7 of the tile (two transposed reads of four rows each), and ends with
  // channels 16 cbk + 4g .. +3 of row 16 bbw + i. The results wait in
  // registers until every wave has read the tile; its LDS then stages the
  // block's records (row r: the 128 hi, the 128 lo, the 8 group-sum hi, the 8
  // lo), so that they leave in whole 16-byte pieces of contiguous record bytes
  // instead of 8-byte pieces of 16 different records per store.
  f16x4 vh[kCBk], vl[kCBk];
  float gs[kCBk];
  if (rows_live) {
#pragma unroll
    for (int cbk = 0; cbk < kCBk; ++cbk) {
      if (cbk < c0 || cbk >= c1) continue;  // uniform
      f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < kNope / 32; ++kk) {
        const uint16_t *p = wt + (32 * kk + 8 * g + (i >> 2)) * kAbsorbWRow + 16 * cbk + 4 * (i & 3);
        const i16x4 r0 = lds_read_tr16_i16(p), r1 = lds_read_tr16_i16(p + 4 * kAbsorbWRow);
        const bf16x8 wa = bitcast<bf16x8>(i16x8{r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w});
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, bitcast<bf16x8>(qv[kk]), d, 0, 0, 0);
      }
      float gsum = 0.0f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = d[r] * qs;
        _Float16 h16, l16;
        split_f16(v, h16, l16);
        vh[cbk][r] = h16;
        vl[cbk][r] = l16;
        gsum += v;
      }
      // the column block's 16 channels are one latent group: add the four lane groups
      gsum += __shfl_xor(gsum, 16);
      gsum += __shfl_xor(gsum, 32);
      gs[cbk] = gsum;
    }
  }
  __syncthreads();  // every wave has read the W_UK tile
  _Float16 *srec = (_Float16 *)wt;
  if (rows_live) {
    _Float16 *srow = srec + (16 * bbw + i) * kAbsorbORow;
#pragma unroll
    for (int cbk = 0; cbk < kCBk; ++cbk) {
      if (cbk < c0 || cbk >= c1) continue;  // uniform
      *(f16x4 *)(srow + 16 * cbk + 4 * g) = vh[cbk];
      *(f16x4 *)(srow + kAbsorbCB + 16 * cbk + 4 * g) = vl[cbk];
      if (g == 0) split_store(srow + 2 * kAbsorbCB + cbk, srow + 2 * kAbsorbCB + 8 + cbk, gs[cbk]);
    }
  }
  __syncthreads();
  // 34 pieces of 16 bytes per row: 16 of hi, 16 of lo, the sums' hi and lo
  const int nrows = min(kAbsorbBT, B - b0);
  for (int k = tid; k < nrows * 34; k += 256) {
    const int row = k / 34, part = k - 34 * row;
    const u32x4 v = *(const u32x4 *)(srec + row * kAbsorbORow + 8 * part);
    _Float16 *rec = qa + ((int64_t)(b0 + row) * H + h) * kQRec;
    const int off = part < 16   ? kQHi + cb * kAbsorbCB + 8 * part
                    : part < 32 ? kQLo + cb * kAbsorbCB + 8 * (part - 16)
                    : part == 32 ? kQSumHi + cb * (kAbsorbCB / 16)
                                 : kQSumLo + cb * (kAbsorbCB / 16);
    *(u32x4 *)(rec + off) = v;
  }
  if (pe) {
#pragma unroll
    for (int j = 0; j < kPLoads; ++j) {
      const int k = tid + 256 * j, b = b0 + (k >> 3);
      if (b < B) {
        f16x8 vh, vl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t bits = (qpv[j][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
          _Float16 h16, l16;
          split_f16(bf16_bits_to_f32(bits) * qs, h16, l16);
          vh[e] = h16;
          vl[e] = l16;
        }
        _Float16 *rec = qa + ((int64_t)b * H + h) * kQRec + kLatent + 8 * (k & 7);
        *(f16x8 *)(rec + kQHi) = vh;
        *(f16x8 *)(rec + kQLo) = vl;
      }
    }
  }
}

// Grid (H, 512/128, layers x nbz): blockIdx.z = l * nbz + bz. Every argument is
// layer-stacked: layer l's queries, weights and records follow layer l-1's.
__global__ __launch_bounds__(256) void absorb_kernel(const uint16_t *q_nope, const uint16_t *q_pe,
                                                     const uint16_t *w_uk, int B, int H, float qs,
                                                     _Float16 *qa, int nbz) {
  const int l = blockIdx.z / nbz, bz = blockIdx.z % nbz;
  const int64_t rows = (int64_t)l * B * H;
  absorb_block(q_nope + rows * kNope, q_pe + rows * kRope, w_uk + (int64_t)l * H * kNope * kLatent, B, H, qs,
               qa + rows * kQRec, blockIdx.x, blockIdx.y, bz, true);
}

// ------------------------------------------------------------ fused step

// First launch of the fused decode step (append one token, then attend) of
// one or more layers. The grid holds, for each layer, n_absorb absorption
// blocks (head-major over (h, cb, bz)), and then one block per sequence j
// (layer-major over the layers' batches, see Paging), which
//   * reads its length pos (the new token's position), quantizes and stores
//     the new token at row pos with its k_pe turned by table row pos
//     (unless the sequence is full), and advances the length after a barrier;
//   * turns every head's q_pe by the same row (fp32), scales it and writes the
//     RoPE part of the query records, which the absorption blocks leave alone.
// No block reads a length another block writes.
struct StepArgs {
  AppendArgs ap;            // T = 1; B = sequences of every layer; rope tables optional
  const uint16_t *q_nope, *q_pe, *w_uk;  // layer-stacked
  _Float16 *qa;
  float qs;
  int H, n_absorb;          // absorption blocks per layer
  int batch, layers;        // sequences per layer, layers of the call
};

template <int FMT>
__global__ __launch_bounds__(256) void step_kernel(StepArgs s) {
  const int blk = blockIdx.x;
  if (blk < s.n_absorb * s.layers) {  // uniform
    const int l = blk / s.n_absorb, r = blk % s.n_absorb;
    const int h = r % s.H, cb = (r / s.H) % (kLatent / kAbsorbCB), bz = r / (s.H * (kLatent / kAbsorbCB));
    const int64_t rows = (int64_t)l * s.batch * s.H;
    absorb_block(s.q_nope + rows * kNope, s.q_pe, s.w_uk + (int64_t)l * s.H * kNope * kLatent, s.batch, s.H,
                 s.qs, s.qa + rows * kQRec, h, cb, bz, false);
    return;
  }
  const int b = blk - s.n_absorb * s.layers;
  const int tid = threadIdx.x;
  const int pos = s.ap.seq_lens[b];
  if (tid < kNScale && pos >= 0 && pos < s.ap.cap) append_group<FMT>(s.ap, b, 0, tid, pos);
  const int row = min(max(pos, 0), s.ap.cap);  // tables hold cap + 1 rows
  for (int e = tid; e < s.H * (kRope / 2); e += 256) {
    const int h = e / (kRope / 2), i = e % (kRope / 2);
    const uint32_t v = *(const uint32_t *)(s.q_pe + ((int64_t)b * s.H + h) * kRope + 2 * i);
    float x0 = bf16_bits_to_f32(v & 0xFFFFu), x1 = bf16_bits_to_f32(v >> 16);
    if (s.ap.rope_cos) {
      const float c = s.ap.rope_cos[(int64_t)row * (kRope / 2) + i];
      const float sn = s.ap.rope_sin[(int64_t)row * (kRope / 2) + i];
      const float y0 = x0 * c - x1 * sn, y1 = x0 * sn + x1 * c;
      x0 = y0;
      x1 = y1;
    }
    _Float16 *rec = s.qa + ((int64_t)b * s.H + h) * kQRec + kLatent + 2 * i;
    split_store(rec + kQHi, rec + kQLo, x0 * s.qs);
    split_store(rec + kQHi + 1, rec + kQLo + 1, x1 * s.qs);
  }
  __syncthreads();
  if (tid == 0 && pos >= 0) s.ap.seq_lens[b] = min(pos + 1, s.ap.cap);
}

// ------------------------------------------------------------- split-KV core

// Row bytes of a format's latent and k_pe planes.
template <int FMT> struct Fmt {
  static constexpr int kLatRowBytes = ckv_bytes(FMT);
  static constexpr int kKpeRowBytes = kpe_bytes(FMT);
};

struct SplitArgs {
  const void *ckv;
  const void *kpe;
  const uint16_t *scale;
  const uint16_t *zero;
  const int32_t *seq_lens;  // [B]: the call's layers' rows (layer-major)
  const _Float16 *qa;       // [B][H][kQRec]
  float *ws_m;              // [records][H], records <= W + B (the balanced plan)
  float *ws_l;              // [records][H]
  float *ws_acc;            // [records][H][512]
  int32_t *rec_tab;         // [B][2] first record and record count
  Paging pg;
  int B, H, cap;            // B: sequences of every layer of the call
  int W;  // ranges of the balanced plan
};

// Buffer descriptors over one split's rows of each plane. A buffer load past
// the descriptor's byte count returns zero without touching memory, so rows
// past the split or the sequence need no branch, and every load of a tile is
// issued unconditionally (which lets the compiler count outstanding loads
// exactly instead of draining the queue before each use).
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // gfx9 buffer resource dword 3
constexpr int kOffNone = 0x7FFFFFF0;        // an offset past any descriptor
constexpr int kLatLoadPolicy = 2;           // buffer-load cache policy operand: nt (non-temporal)
#ifndef MLA_SLICE_POLICY
#define MLA_SLICE_POLICY 0
#endif
// more than 16 heads: every head slice reads the latent, so the lines are
// worth keeping in the caches (the default policy)
constexpr int kSliceLoadPolicy = MLA_SLICE_POLICY;

struct SplitRsrc {
  __amdgpu_buffer_rsrc_t ckv, kpe, scale, zero;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, (int)kRsrcWord3);
}

// Descriptors over n plane rows starting at row0, latent row lrow0 (a block
// start; n = 0: empty, every load reads zeros). The latent descriptor covers
// whole 16-row blocks: rows past n in the last block are read too, and the
// kernels neutralize them (zero scales, or zeroed registers for bf16).
template <int FMT>
__device__ __forceinline__ SplitRsrc rows_rsrc(const SplitArgs &a, int64_t row0, int64_t lrow0, int64_t n) {
  SplitRsrc r;
  r.ckv = make_rsrc((const uint8_t *)a.ckv + lrow0 * Fmt<FMT>::kLatRowBytes,
                    ((n + 15) & ~(int64_t)15) * Fmt<FMT>::kLatRowBytes);
  r.kpe = make_rsrc((const uint8_t *)a.kpe + row0 * Fmt<FMT>::kKpeRowBytes, n * Fmt<FMT>::kKpeRowBytes);
  constexpr int NS = n_scales(FMT);
  r.scale = make_rsrc(NS == 0 ? a.kpe : (const void *)(a.scale + row0 * NS), n * NS * 2);
  r.zero = make_rsrc(has_zero(FMT) ? (const void *)(a.zero + row0 * kNGroupL) : a.kpe,
                     has_zero(FMT) ? n * kNGroupL * 2 : 0);
  return r;
}

// Rows [t_begin, t_end) of sequence b in the contiguous layout.
template <int FMT>
__device__ __forceinline__ SplitRsrc split_rsrc(const SplitArgs &a, int b, int t_begin, int t_end) {
  return rows_rsrc<FMT>(a, (int64_t)b * a.cap + t_begin, (int64_t)b * lat_stride(a.cap) + t_begin,
                        t_end - t_begin);
}

// Paged layout: rows [r0, t_end) of a sequence whose layer's pool starts at
// row `base`, cut at the end of r0's page (`page`, from page_of; -1 or
// r0 >= t_end: empty).
template <int FMT>
__device__ __forceinline__ SplitRsrc page_rsrc(const SplitArgs &a, int64_t base, int page, int r0, int t_end) {
  if (page < 0 || r0 >= t_end) return rows_rsrc<FMT>(a, 0, 0, 0);
  const int off = r0 & (a.pg.size - 1);
  const int end = min(t_end, r0 - off + a.pg.size);
  const int64_t row0 = base + ((int64_t)page << a.pg.shift) + off;
  return rows_rsrc<FMT>(a, row0, row0, end - r0);
}

// 4 signed bytes -> the 4 codes as exact fp16: one conversion per code, each
// sign-extending one byte of w (sub-dword operand select) and writing its
// fp16 to one half of a pair while keeping the other half. Four instructions
// for four codes; the splice of the biased bytes into 1024.0 and the
// subtraction it replaces took five (and a constant register), and the
// 16-head INT8 partial launch is 4-5% faster for it.
__device__ __forceinline__ void codes_i8x4(uint32_t w, f16x2 &lo, f16x2 &hi) {
  uint32_t a, c;
  asm("v_cvt_f16_i16_sdwa %0, sext(%2) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_0\n\t"
      "v_cvt_f16_i16_sdwa %0, sext(%2) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1\n\t"
      "v_cvt_f16_i16_sdwa %1, sext(%2) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_2\n\t"
      "v_cvt_f16_i16_sdwa %1, sext(%2) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_3"
      : "=&v"(a), "=&v"(c)
      : "v"(w));
  lo = bitcast<f16x2>(a);
  hi = bitcast<f16x2>(c);
}

// x = q*s as hi + lo in fp16: hi = fp16(q*s), lo = q*s - hi, which a fused
// multiply-add gives exactly (q has at most 8 significant bits, s 11).
__device__ __forceinline__ void scale_split(f16x2 q, f16x2 s, f16x2 &hi, f16x2 &lo) {
  hi = q * s;
  lo = __builtin_elementwise_fma(q, s, -hi);
}

__device__ __forceinline__ f16x2 bf16x2_to_f16x2(uint32_t w) {
  return f16x2{(_Float16)bf16_bits_to_f32(w & 0xFFFFu), (_Float16)bf16_bits_to_f32(w >> 16)};
}

__device__ __forceinline__ f16x2 splat_f16_bits(uint32_t bits16) {
  const _Float16 h = bitcast<_Float16>((uint16_t)bits16);
  return f16x2{h, h};
}

typedef __fp16 fp16x4_lds __attribute__((__vector_size__(4 * sizeof(__fp16))));

// LDS transpose read (gfx950 ds_read_b64_tr_b16): in each 16-lane group g,
// lane 4r+c points at row r, columns 4c..4c+3 of a 4x16 block of fp16, and
// lane i of the group receives column i, rows 0..3.
__device__ __forceinline__ f16x4 lds_read_tr16(const _Float16 *p) {
  const fp16x4_lds v = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
      (__attribute__((address_space(3))) fp16x4_lds *)(p));
  return bitcast<f16x4>(v);
}

// ------------------------------------------------------- split-KV core

// For one slice of 16 heads the four waves of a workgroup share each 32-token
// tile and divide the channels: wave w owns latent channels [128w, 128w+128)
// and k_pe channels [16w, 16w+16). Each wave loads its channels of the tile straight
// into the MFMA operand layout, dequantizes them in registers (as fp16 hi and
// exact residual lo), and
//   scores  adds its share of S^T[t][h] = sum_c C[t][c] Q[h][c] as
//           C_hi Q_hi + C_hi Q_lo + C_lo Q_hi (16x16x32 f16 MFMA, fp32
//           accumulation); the four partial score tiles meet in LDS and every
//           wave adds them in the same order, so all waves hold the same
//           scores and the same softmax state;
//   values  accumulates O^T[c][h] = sum_t C[t][c] P[t][h] for its own 128
//           channels: its C_hi (INT4: the exact codes) goes to a wave-private
//           LDS block and comes back transposed (ds_read_b64_tr_b16) as the A
//           operand; P is the B operand as the score MFMA left it in
//           registers (INT4: P times each group's scales, as an exact fp16
//           hi/lo pair).
// Lane l = 16g + i: in the score, row i of each 16-token half of the tile and
// the 32 channels of the wave's block that lane_chan gives lane group g (two
// quantization groups); in the accumulators, head i.
constexpr int kT16 = 32;             // tokens per tile
constexpr int kNpf16 = 1;            // tiles of loads in flight per wave
// A wave's value block: 32 rows (tokens) of 128 channels, then (INT4) the 8
// zero-points of the wave's groups in one 16-byte chunk and the wave's group
// scales, transposed, in the other; rows of 144 fp16 (72 dwords, 8 banks
// apart), so the four rows a transposed read spans start 8 banks apart and
// never share a bank. Writes go row per lane, 16 bytes at a time; there the
// 16-byte chunks of rows with bit 2 xor bit 3 of the row set are swapped in
// pairs (chunk c stored at c ^ 1), which puts rows r, r + 4 and r + 8 on
// different banks too.
constexpr int kVRow = 144;           // fp16 per row
constexpr int kWBlk = kT16 * kVRow;  // fp16 per wave block
__device__ __forceinline__ int vswz(int row) { return ((row >> 2) ^ (row >> 3)) & 1; }
constexpr int kPart16 = kWaves * 64 * 8;              // floats: 4 waves x 64 lanes x 8

// The small planes of a tile (latent scales, k_pe codes and scales, INT4
// zero-points) are few bytes per row, and loading each lane's few bytes
// straight from its row costs one memory request per row and instruction.
// Instead the workgroup loads a tile's rows of each small plane as whole
// 16-byte chunks (consecutive lanes, consecutive chunks), stages them in LDS,
// and every lane then reads its own bytes from there.
constexpr int kAuxRow = 80;      // staged row stride (bytes) of the scale, k_pe and zero blocks
constexpr int kAuxRowBf16 = 144; // staged k_pe row stride for bf16 (128-byte rows, padded)

// Staging area of each format (byte offsets of its blocks):
//   k_pe bf16 (BF16, INT8_KBF16): k_pe block of 32 rows x 144 B first;
//   latent scales (all quantized formats): 32 rows x 80 B;
//   k_pe codes (INT8, INT4, INT4_KINT4): 32 rows x 80 B (64 or 32 B used);
//   zero-points (INT4, INT4_KINT4): 32 rows x 80 B.
template <int FMT> struct Aux16 {
  static constexpr bool kKBf = kpe_fmt(FMT) == kKpeBf16;
  static constexpr int kKpeBytes = kKBf ? kT16 * kAuxRowBf16 : kT16 * kAuxRow;
  static constexpr int kScale = kKBf ? kKpeBytes : 0;
  static constexpr int kKpe = kKBf ? 0 : kT16 * kAuxRow;
  static constexpr int kZero = 2 * kT16 * kAuxRow;
  static constexpr int kBytes = FMT == MLA_FMT_BF16 ? kKpeBytes
                                : kKBf ? kKpeBytes + kT16 * kAuxRow
                                : has_zero(FMT) ? 3 * kT16 * kAuxRow : 2 * kT16 * kAuxRow;
};

template <int LF> struct RawLat16;
template <> struct RawLat16<MLA_FMT_INT8> {
  static constexpr int kLat = 2;  // 16-byte loads per half-tile row: 32 codes
  u32x4 lat[2][2];
  u32x4 sa, sb;                   // this lane's chunks of the small planes
};
template <> struct RawLat16<MLA_FMT_INT4> {
  static constexpr int kLat = 1;  // 32 nibbles
  u32x4 lat[2][1];
  u32x4 sa, sb;
};
template <> struct RawLat16<MLA_FMT_BF16> {
  static constexpr int kLat = 4;  // 32 bf16
  u32x4 lat[2][4];
  u32x4 sa, sb;
};
template <int FMT> using Raw16 = RawLat16<lat_fmt(FMT)>;

// What a lane reads back from the staged small planes for rows i and 16+i.
struct Meta16 {
  uint32_t sc[2], ks[2], zp[2];
  u32x2 kq[2];
};

// The latent channels that lane group g of wave w holds in k-step kk (8
// channels from the returned one on): each 16-byte load of a lane is one
// latent chunk, and the 64 lanes of a load read 4 consecutive chunks of the
// 16 rows of a block (1 KB in one piece). INT8: 16-channel chunks
// 8w + 4j + g (j = kk / 2); INT4: the 32-channel chunk 4w + g (nibble order
// within it); BF16: 8-channel chunks 16w + 4kk + g.
template <int FMT> __device__ __forceinline__ constexpr int lane_chan(int w, int g, int kk) {
  return lat_fmt(FMT) == MLA_FMT_INT8   ? 128 * w + 64 * (kk >> 1) + 16 * g + 8 * (kk & 1)
         : lat_fmt(FMT) == MLA_FMT_INT4 ? 128 * w + 32 * g + 8 * kk
                                        : 128 * w + 32 * kk + 8 * g;
}

// Byte offsets of this lane's data within a tile (the same for every tile).
//   latent: rows i and 16+i (blocks rb = 0, 1), the chunks of lane_chan
//   small planes: chunk plan of the staging loads, 16-byte chunks of the
//   tile's contiguous rows; wave w (uniform) loads
//     slot A: bf16 k_pe chunks 64w+l (256 = 32 rows x 128 B) where k_pe is
//             bf16, else scale chunks 64w+l (w < 3; 160 = 32 rows x 80 B);
//     slot B: INT8_KBF16: scale chunks 64w+l (w < 2; 128 = 32 rows x 64 B);
//             otherwise k_pe code chunks 64w+l (INT8 k_pe: w < 2, 128 =
//             32 rows x 64 B; INT4 k_pe: w = 0, 64 = 32 rows x 32 B), and
//             with zero-points, their chunks 64(w-2)+l (w >= 2; 128).
//   A chunk past its plane's tile reads nothing (kOffNone) and is not staged.
template <int FMT> struct Off16 {
  int lat[2][Raw16<FMT>::kLat];
  int ga, gb;    // byte offsets in the tile (or kOffNone)
  int la, lb;    // LDS byte offsets in the staging area (or -1: not staged)
  bool b_zero;   // slot B reads the zero-point plane (waves 2 and 3)
};

template <int FMT>
__device__ __forceinline__ Off16<FMT> offsets16(int w, int lane) {
  using AX = Aux16<FMT>;
  Off16<FMT> o;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
    for (int j = 0; j < Raw16<FMT>::kLat; ++j) {
      // chunk c of row i of block rb: rb * 16 * row_bytes + (16 c + i) * 16
      if (lat_fmt(FMT) == MLA_FMT_INT8) o.lat[rb][j] = rb * 16 * kLatent + (8 * w + 4 * j) * 256 + lane * 16;
      else if (lat_fmt(FMT) == MLA_FMT_INT4) o.lat[rb][j] = rb * 16 * (kLatent / 2) + 4 * w * 256 + lane * 16;
      else o.lat[rb][j] = rb * 16 * (kLatent * 2) + (16 * w + 4 * j) * 256 + lane * 16;
    }
  }
  o.ga = o.gb = kOffNone;
  o.la = o.lb = -1;
  o.b_zero = false;
  const int c = 64 * w + lane;
  if (AX::kKBf) {
    o.ga = 16 * c;  // < 256 chunks: every lane of every wave
    o.la = AX::kKpe + (c >> 3) * kAuxRowBf16 + 16 * (c & 7);
    if (FMT != MLA_FMT_BF16 && w < 2) {  // the 64-byte scale rows
      o.gb = 16 * c;
      o.lb = AX::kScale + (c >> 2) * kAuxRow + 16 * (c & 3);
    }
  } else {
    if (c < kT16 * n_scales(FMT) * 2 / 16) {  // the 80-byte scale rows: staged as they lie
      o.ga = 16 * c;
      o.la = AX::kScale + 16 * c;
    }
    constexpr int per_row = kpe_bytes(FMT) / 16;  // k_pe chunks per row: 4 or 2
    if (w < 2) {
      if (c < kT16 * per_row) {
        o.gb = 16 * c;
        o.lb = AX::kKpe + (c / per_row) * kAuxRow + 16 * (c % per_row);
      }
    } else if (has_zero(FMT)) {
      const int cz = 64 * (w - 2) + lane;  // zero-point chunk, 4 per 64-byte row
      o.gb = 16 * cz;
      o.lb = AX::kZero + (cz >> 2) * kAuxRow + 16 * (cz & 3);
      o.b_zero = true;
    }
  }
  return o;
}

// Descriptors over rows [r0, t_end) of the split (empty when r0 >= t_end):
// the tile's own base, so per-lane offsets stay constant across tiles and
// the range check still covers every byte read. All scalar arithmetic.
template <int FMT>
__device__ __forceinline__ SplitRsrc tile_rsrc(const SplitArgs &a, int b, int r0, int t_end) {
  const int r = min(r0, t_end);
  return split_rsrc<FMT>(a, b, r, t_end);
}

// Issue every load of one tile. `zero_b` is wave-uniform: it selects the
// descriptor of slot B. Rows past the descriptor read as zeros.
//
// Every latent byte is read once, by one load that takes whole 64-byte pieces
// of its lines, so the latent loads carry the non-temporal hint (the cache
// policy operand's nt bit): streamed lines are not kept in the caches, which
// measured some 7% faster than the default policy on the ragged INT8 decode.
//
// The latent descriptor covers whole 16-row blocks, so the rows of the last
// block past the split are read too. Quantized rows there dequantize to zero
// (their scales and zero-points, read through plain row descriptors, are
// zero); bf16 rows could hold anything, so from row `left` of the tile on
// (bf16 latents only) their loads are pointed past the descriptor.
template <int FMT, int POL>
__device__ __forceinline__ void load16_lat(Raw16<FMT> &r, const SplitRsrc &rs, const Off16<FMT> &o, int left,
                                           int i) {
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int j = 0; j < Raw16<FMT>::kLat; ++j) {
      const int off = lat_fmt(FMT) == MLA_FMT_BF16 && 16 * rb + i >= left ? kOffNone : o.lat[rb][j];
      r.lat[rb][j] = bitcast<u32x4>(__builtin_amdgcn_raw_buffer_load_b128(rs.ckv, off, 0, POL));
    }
}

// The latent loads of half-tile rb only (the 16-head kernel's early issue
// for INT8 latents). Kept apart from load16_lat: written as a loop over
// this function, load16_lat compiles to a schedule that spills in the
// 32-head bf16 kernel.
template <int FMT, int POL>
__device__ __forceinline__ void load16_lat_half(Raw16<FMT> &r, const SplitRsrc &rs, const Off16<FMT> &o, int left,
                                                int i, int rb) {
#pragma unroll
  for (int j = 0; j < Raw16<FMT>::kLat; ++j) {
    const int off = lat_fmt(FMT) == MLA_FMT_BF16 && 16 * rb + i >= left ? kOffNone : o.lat[rb][j];
    r.lat[rb][j] = bitcast<u32x4>(__builtin_amdgcn_raw_buffer_load_b128(rs.ckv, off, 0, POL));
  }
}

// The small planes' loads of a tile. They are issued a tile ahead of their
// use and before the same tile's latent loads: loads return in order, so the
// staging of the small planes never waits for latent bytes.
template <int FMT>
__device__ __forceinline__ void load16_small(Raw16<FMT> &r, const SplitRsrc &rs, const Off16<FMT> &o,
                                             bool zero_b) {
  constexpr bool kKBf = kpe_fmt(FMT) == kKpeBf16;
  r.sa = bitcast<u32x4>(__builtin_amdgcn_raw_buffer_load_b128(kKBf ? rs.kpe : rs.scale, o.ga, 0, 0));
  if (FMT != MLA_FMT_BF16)
    r.sb = bitcast<u32x4>(
        __builtin_amdgcn_raw_buffer_load_b128(zero_b ? rs.zero : kKBf ? rs.scale : rs.kpe, o.gb, 0, 0));
}

// This lane's chunks into the staging area.
template <int FMT>
__device__ __forceinline__ void stage16(const Raw16<FMT> &r, const Off16<FMT> &o, uint8_t *aux) {
  if (o.la >= 0) *(u32x4 *)(aux + o.la) = r.sa;
  if (FMT != MLA_FMT_BF16 && o.lb >= 0) *(u32x4 *)(aux + o.lb) = r.sb;
}

// This lane's small-plane values of rows i and 16+i from the staging area.
template <int FMT>
__device__ __forceinline__ Meta16 meta16(const uint8_t *aux, int w, int g, int i) {
  Meta16 m;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int row = 16 * rb + i;
    using AX = Aux16<FMT>;
    // k_pe channels 16w+4g .. +3 of the row
    if (kpe_fmt(FMT) == kKpeBf16) {
      m.kq[rb] = *(const u32x2 *)(aux + AX::kKpe + row * kAuxRowBf16 + 2 * (16 * w + 4 * g));
    } else if (kpe_fmt(FMT) == kKpeI8) {
      m.kq[rb] = u32x2{*(const uint32_t *)(aux + AX::kKpe + row * kAuxRow + 16 * w + 4 * g), 0u};
    } else {  // four nibbles
      m.kq[rb] = u32x2{*(const uint16_t *)(aux + AX::kKpe + row * kAuxRow + 8 * w + 2 * g), 0u};
    }
    m.sc[rb] = m.ks[rb] = m.zp[rb] = 0;
    if (FMT != MLA_FMT_BF16) {
      const uint8_t *srow = aux + AX::kScale + row * kAuxRow;
      if (lat_fmt(FMT) == MLA_FMT_INT8)  // the groups of chunks 8w + g and 8w + 4 + g
        m.sc[rb] = (uint32_t)*(const uint16_t *)(srow + 2 * (8 * w + g)) |
                   ((uint32_t)*(const uint16_t *)(srow + 2 * (8 * w + 4 + g)) << 16);
      else  // INT4: groups 8w + 2g and 8w + 2g + 1 (the chunk's 32 channels)
        m.sc[rb] = *(const uint32_t *)(srow + 2 * (8 * w + 2 * g));
      if (kpe_fmt(FMT) != kKpeBf16) m.ks[rb] = *(const uint16_t *)(srow + 2 * (kNGroupL + 2 * w + (g >> 1)));
    }
    if (has_zero(FMT))
      m.zp[rb] = *(const uint32_t *)(aux + AX::kZero + row * kAuxRow + 2 * (8 * w + 2 * g));
  }
  return m;
}

// Max and sum over the four 16-lane groups (lanes i, i+16, i+32, i+48) with the
// gfx950 lane-swap instructions: VALU only, no LDS round trip. A swap of x with
// itself leaves, in the two results, the lane's own value and its partner's.
__device__ __forceinline__ float max_across_groups(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t v = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float sum_across_groups(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t v = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ f16x8 cat8(f16x2 a, f16x2 b, f16x2 c, f16x2 d) {
  return f16x8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// Dequantize one half-tile row of this lane: hi/lo operands of the 4 latent
// k-steps (8 channels each) and of the k_pe k-step (4 channels), and in vdat
// the row's value-block data of the 4 k-steps (vstore16 stores it).
//
// INT4 operands keep the channel order in which the nibbles come out of a
// dword, (0,4,1,5,2,6,3,7) within each 8 channels, and the queries are
// permuted to match once per workgroup. The value block in LDS keeps that
// order too, so the value product's output channels come out in it and are
// re-paired once, when the unit's sums are stored. The MFMA operands and the
// LDS copy are then whole registers straight from the packed multiply-adds,
// as in the other formats.
template <int FMT>
__device__ __forceinline__ void dequant16(const Raw16<FMT> &r, const Meta16 &m, int rb, f16x8 (&hi)[4],
                                          f16x8 (&lo)[4], f16x8 (&vdat)[4], uint2 magic, f16x4 &khi,
                                          f16x4 &klo) {
  if (lat_fmt(FMT) == MLA_FMT_INT8) {
    const f16x2 s0 = splat_f16_bits(m.sc[rb] & 0xFFFFu), s1 = splat_f16_bits(m.sc[rb] >> 16);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const u32x4 v = r.lat[rb][kk >> 1];
      const f16x2 s2 = kk < 2 ? s0 : s1;
      f16x2 q0, q1, q2, q3, h0, h1, h2, h3, l0, l1, l2, l3;
      codes_i8x4(v[2 * (kk & 1)], q0, q1);
      codes_i8x4(v[2 * (kk & 1) + 1], q2, q3);
      scale_split(q0, s2, h0, l0);
      scale_split(q1, s2, h1, l1);
      scale_split(q2, s2, h2, l2);
      scale_split(q3, s2, h3, l3);
      hi[kk] = cat8(h0, h1, h2, h3);
      lo[kk] = cat8(l0, l1, l2, l3);
      vdat[kk] = hi[kk];
    }
  } else if (lat_fmt(FMT) == MLA_FMT_INT4) {
    const f16x2 s0 = splat_f16_bits(m.sc[rb] & 0xFFFFu), s1 = splat_f16_bits(m.sc[rb] >> 16);
    const f16x2 bias0 = {(_Float16)1024.0f, (_Float16)1024.0f};
    const f16x2 bias1 = {(_Float16)64.0f, (_Float16)64.0f};
    // A nibble q in bits 0..3 of a half-word under the exponent bits of 1024
    // reads as the fp16 1024 + q; in bits 4..7 under those of 64, as 64 + q
    // (the mantissa's unit there is 1/16). So both lower nibbles of each
    // half-word come out without a shift, and the upper two after one shift
    // by 8. (x & mask) | magic is one bit-field insert: the magics sit in
    // registers the compiler cannot see through, so the pattern stays one
    // instruction.
    const auto nib0 = [magic](uint32_t x) { return (x & 0x000F000Fu) | (magic.x & ~0x000F000Fu); };
    const auto nib1 = [magic](uint32_t x) { return (x & 0x00F000F0u) | (magic.y & ~0x00F000F0u); };
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const uint32_t w = r.lat[rb][0][kk], w8 = w >> 8;
      const f16x2 s2 = kk < 2 ? s0 : s1;
      const f16x2 q04 = bitcast<f16x2>(nib0(w)) - bias0;
      const f16x2 q15 = bitcast<f16x2>(nib1(w)) - bias1;
      const f16x2 q26 = bitcast<f16x2>(nib0(w8)) - bias0;
      const f16x2 q37 = bitcast<f16x2>(nib1(w8)) - bias1;
      f16x2 h04, l04, h15, l15, h26, l26, h37, l37;
      scale_split(q04, s2, h04, l04);
      scale_split(q15, s2, h15, l15);
      scale_split(q26, s2, h26, l26);
      scale_split(q37, s2, h37, l37);
      hi[kk] = cat8(h04, h15, h26, h37);  // channels 0,4,1,5,2,6,3,7
      lo[kk] = cat8(l04, l15, l26, l37);
      // the codes themselves (exact in fp16) go to the value block: the
      // values take the scale on the softmax side, as an exact hi/lo pair
      vdat[kk] = cat8(q04, q15, q26, q37);
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const u32x4 v = r.lat[rb][kk];
      hi[kk] = cat8(bf16x2_to_f16x2(v[0]), bf16x2_to_f16x2(v[1]), bf16x2_to_f16x2(v[2]),
                    bf16x2_to_f16x2(v[3]));
      lo[kk] = f16x8{};
      vdat[kk] = hi[kk];
    }
  }
  if (kpe_fmt(FMT) != kKpeBf16) {
    const f16x2 ks = splat_f16_bits(m.ks[rb]);
    f16x2 q0, q1, h0, h1, l0, l1;
    if (kpe_fmt(FMT) == kKpeI8) {
      codes_i8x4(m.kq[rb].x, q0, q1);
    } else {  // nibbles code + 8 of channels 0..3: spliced into 1024.0, minus 1032
      const uint32_t x = m.kq[rb].x;
      const f16x2 bias = {(_Float16)1032.0f, (_Float16)1032.0f};
      q0 = bitcast<f16x2>((x & 0xFu) | ((x & 0xF0u) << 12) | 0x64006400u) - bias;
      q1 = bitcast<f16x2>(((x >> 8) & 0xFu) | ((x & 0xF000u) << 4) | 0x64006400u) - bias;
    }
    scale_split(q0, ks, h0, l0);
    scale_split(q1, ks, h1, l1);
    khi = f16x4{h0.x, h0.y, h1.x, h1.y};
    klo = f16x4{l0.x, l0.y, l1.x, l1.y};
  } else {
    const f16x2 a = bf16x2_to_f16x2(m.kq[rb].x), b = bf16x2_to_f16x2(m.kq[rb].y);
    khi = f16x4{a.x, a.y, b.x, b.y};
    klo = f16x4{};
  }
}

// Store one half-tile row's value-block data (from dequant16) to this wave's
// value block `vblk`, row 16 rb + i:
//   INT8: columns lane_chan - 128 w = 16 g + 64 j + 8 h (k-step kk = 2 j + h);
//   INT4: columns 32 g + 8 kk, the codes in the nibble order; and the
//         zero-points of the wave's 8 groups in columns 128..135 (chunk 16),
//         the scales of groups 2g, 2g+1 of token 16 rb + i transposed into the
//         other chunk of columns 128..143: group n's 32 scales take rows
//         4n..4n+3, in the token order the value product's B operand holds
//         (lane group g': tokens 4g'..4g'+3, then 16+4g'..16+4g'+3);
//   BF16: columns 32 kk + 8 g.
// Chunk pairs of rows with vswz(row) set are swapped (see kVRow).
template <int FMT>
__device__ __forceinline__ void vstore16(_Float16 *vblk, int rb, int g, int i, const f16x8 (&vdat)[4],
                                         const Meta16 &m) {
  const int row = 16 * rb + i, swz = vswz(i);
  _Float16 *vrow = vblk + row * kVRow;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    if (lat_fmt(FMT) == MLA_FMT_INT8) *(f16x8 *)(vrow + 16 * g + 64 * (kk >> 1) + 8 * ((kk & 1) ^ swz)) = vdat[kk];
    else if (lat_fmt(FMT) == MLA_FMT_INT4) *(f16x8 *)(vrow + 32 * g + 8 * (kk ^ swz)) = vdat[kk];
    else *(f16x8 *)(vrow + 8 * (g ^ swz) + 32 * kk) = vdat[kk];
  }
  if (has_zero(FMT)) {
    *(uint32_t *)(vrow + 128 + 8 * swz + 2 * g) = m.zp[rb];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int trow = 4 * (2 * g + h2) + (i >> 2);
      *(uint16_t *)(vblk + trow * kVRow + 136 - 8 * vswz(trow) + 4 * rb + (i & 3)) = (uint16_t)(m.sc[rb] >> (16 * h2));
    }
  }
}

// Per tile, every wave:
//   1. stages its chunks of the tile's small planes, barrier (the staging
//      area and the partial-score slots of the previous tile are then free),
//      and issues the next tile's small-plane loads;
//   2. reads its scales, k_pe codes and zero-points back, dequantizes its
//      latent channels in registers, stores C_hi (INT4: the codes) to its
//      value block, and issues the MFMAs of its partial scores;
//   3. issues the next tile's latent loads (INT8 latents: each half-tile's
//      share in step 2, right after that half's dequantization);
//   4. stores its partial scores, barrier, and adds the four waves' partials
//      in a fixed order;
//   5. online softmax and the value MFMAs of its channels.

// ---- balanced plan of the 16-head partial kernel
//
// The batch's tiles (ceil(L_b / 32) per sequence, sequences in batch order)
// form one list of T tiles, and workgroup w of the W in the grid takes tiles
// [w q, min((w + 1) q, T)) with q = ceil(T / W): every workgroup gets the same
// number of tiles (within one), whatever the mix of lengths, and a range may
// cover the end of one sequence and the start of the next. Each (workgroup,
// sequence) pair it covers is one partial record, at index w + b: along the
// list, w and b never decrease and one of them grows at every new pair, so
// w + b is unique, below W + B. Workgroup 0 writes, for every sequence, its
// first record and record count, which the combine reads.
__device__ __forceinline__ int tiles_of(int L) { return (L + kT16 - 1) / kT16; }
__device__ __forceinline__ int clamp_len(int v, int cap) { return min(max(v, 0), cap); }

// Inclusive prefix sum of v over the workgroup's threads, and in `total` the
// sum over all of them. Every thread calls it; sh holds kWaves ints.
__device__ __forceinline__ int wg_scan(int v, int *sh, int &total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(v, off);
    if (lane >= off) v += u;
  }
  if (lane == 63) sh[w] = v;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) {
    const int t = sh[k];
    before += k < w ? t : 0;
    total += t;
  }
  __syncthreads();  // sh may be written again by the next call
  return v + before;
}

struct PlanStart {
  int b, S, L;  // first sequence of the range (B: none), its first global tile, its length
  int g0, g1;   // the workgroup's global tiles [g0, g1)
};

// Range wg of the W ranges. Every thread calls it (barriers inside); sh holds
// at least kWaves + 3 ints.
__device__ __forceinline__ PlanStart plan_start(const SplitArgs &a, int W, int wg, int *sh) {
  const int tid = threadIdx.x;
  int T = 0, n0 = 0, incl0 = 0, L0 = 0, tot0 = 0;
  for (int c0 = 0; c0 < a.B; c0 += kThreads) {  // total tiles
    const int b = c0 + tid;
    const int L = b < a.B ? clamp_len(a.seq_lens[b], a.cap) : 0;
    const int n = tiles_of(L);
    int tot;
    const int incl = wg_scan(n, sh, tot);
    if (c0 == 0) {
      n0 = n;
      incl0 = incl;
      L0 = L;
      tot0 = tot;
    }
    T += tot;
  }
  const int q = T > 0 ? (int)(((int64_t)T + W - 1) / W) : 1;
  const int g0 = (int)min((int64_t)wg * q, (int64_t)T);
  const int g1 = min(g0 + q, T);
  if (tid == 0) {
    sh[kWaves] = a.B;
    sh[kWaves + 1] = 0;
    sh[kWaves + 2] = 0;
  }
  __syncthreads();
  int carry = 0;
  for (int c0 = 0; c0 < a.B; c0 += kThreads) {  // locate g0; the record table
    const int b = c0 + tid;
    int n = n0, incl = incl0, L = L0, tot = tot0;
    if (c0 > 0) {
      L = b < a.B ? clamp_len(a.seq_lens[b], a.cap) : 0;
      n = tiles_of(L);
      incl = wg_scan(n, sh, tot);
    }
    const int S = carry + incl - n;
    if (b < a.B) {
      if (n > 0 && S <= g0 && g0 < S + n) {  // at most one thread of the grid's batch
        sh[kWaves] = b;
        sh[kWaves + 1] = S;
        sh[kWaves + 2] = L;
      }
      if (blockIdx.x == 0) {  // the first workgroup of the grid
        const int first = n > 0 ? S / q : 0;
        a.rec_tab[2 * b] = first + b;
        a.rec_tab[2 * b + 1] = n > 0 ? (S + n - 1) / q - first + 1 : 0;
      }
    }
    carry += tot;
  }
  __syncthreads();
  PlanStart p;
  p.b = __builtin_amdgcn_readfirstlane(sh[kWaves]);
  p.S = __builtin_amdgcn_readfirstlane(sh[kWaves + 1]);
  p.L = __builtin_amdgcn_readfirstlane(sh[kWaves + 2]);
  p.g0 = __builtin_amdgcn_readfirstlane(g0);
  p.g1 = __builtin_amdgcn_readfirstlane(g1);
  __syncthreads();  // sh is reused by the first tile
  return p;
}

// PAGED: the cache is paged (a compile-time choice: the per-tile descriptor code
// of the other layout is then absent from the tile loop). SLICED: more than 16
// heads, run as head slices that each read the latent.
template <int FMT, bool PAGED, bool SLICED>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(3, 3)))
void split16_kernel(SplitArgs a) {
  constexpr bool kLo = FMT != MLA_FMT_BF16;
  constexpr bool kZp = has_zero(FMT);  // INT4 latent: zero-points, and the nibble operand order
  constexpr bool kEarly = lat_fmt(FMT) == MLA_FMT_INT8;  // the next tile's latent loads per half-tile (step 3)
  // The softmax weights are p = 2^(s - m_run) for a reference m_run that
  // moves lazily (below). kSlack: log2 of the largest weight allowed before
  // the reference moves; kHead: how far above the tile maximum it is placed.
  // INT8 / BF16: weights up to 2^8 (exact in fp16 relative terms). INT4: the
  // weights multiply the group scales in fp16 (p s as an fp16 hi/lo pair), so
  // they stay at or below 1 and p s is finite for every fp16 scale; the
  // reference sits 2^4 above the maximum, so it still moves only when a
  // head's maximum rises by more than 4.
  constexpr float kSlack = kZp ? 0.0f : kLazy;
  constexpr float kHead = kZp ? 4.0f : 0.0f;
  __shared__ __attribute__((aligned(16))) _Float16 wblk[kWaves * kWBlk];
  // partial scores of a tile; before the first tile, the plan's scratch
  __shared__ __attribute__((aligned(16))) float part[kPart16];
  // read only between the two barriers of a tile (the next tile's staging
  // writes come after the second)
  __shared__ __attribute__((aligned(16))) uint8_t aux[Aux16<FMT>::kBytes];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g = lane >> 4, i = lane & 15;

  // More than 16 heads: the grid holds W ranges x (H / 16) head slices, the
  // slices of a range adjacent, so that they run together and read the
  // range's tiles while they are still in the caches; slice hs serves heads
  // 16 hs .. 16 hs + 15 (its queries and its rows of every record).
  // Workgroups are handed to the 8 XCDs (each with its own L2) round-robin
  // by index, so the slices of a range sit 8 indices apart: all on one XCD,
  // in one window of 8 * nslice indices. Indices past the W ranges (the grid
  // is rounded up to whole windows) get empty ranges.
  const int nslice = a.H / 16;
  const int win = blockIdx.x / (8 * nslice), in_win = blockIdx.x % (8 * nslice);
  const int hs = in_win / 8, rng = 8 * win + in_win % 8;
  const PlanStart plan = plan_start(a, a.W, rng, (int *)part);
  int b = plan.b, S = plan.S, L = plan.L;
  // one pass per sequence the range covers (all uniform across the workgroup)
  while (b < a.B) {
  // all wave-uniform; said so, so that the descriptors built from them stay
  // in scalar registers
  b = __builtin_amdgcn_readfirstlane(b);
  S = __builtin_amdgcn_readfirstlane(S);
  L = __builtin_amdgcn_readfirstlane(L);
  const int n = tiles_of(L);
  const int t_begin = __builtin_amdgcn_readfirstlane((max(plan.g0, S) - S) * kT16);
  const int t_end = __builtin_amdgcn_readfirstlane(min(L, (min(plan.g1, S + n) - S) * kT16));
  const int64_t ws_row = ((int64_t)rng + b) * a.H + 16 * hs;
  const int ntiles = (t_end - t_begin + kT16 - 1) / kT16;

  // queries of head i for this wave's channels, in the MFMA B layout
  f16x8 qh[4], ql[4];
  f16x8 kzh, kzl;  // k_pe channels 16w+4g..+3, then (INT4) the sums of groups 8w+2g, +1, then 0
  {
    const _Float16 *q = a.qa + ((int64_t)b * a.H + 16 * hs + i) * kQRec;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      qh[kk] = *(const f16x8 *)(q + kQHi + lane_chan<FMT>(w, g, kk));
      ql[kk] = *(const f16x8 *)(q + kQLo + lane_chan<FMT>(w, g, kk));
      if (kZp) {  // the INT4 operand order: channels 0,4,1,5,2,6,3,7
        qh[kk] = f16x8{qh[kk][0], qh[kk][4], qh[kk][1], qh[kk][5], qh[kk][2], qh[kk][6], qh[kk][3], qh[kk][7]};
        ql[kk] = f16x8{ql[kk][0], ql[kk][4], ql[kk][1], ql[kk][5], ql[kk][2], ql[kk][6], ql[kk][3], ql[kk][7]};
      }
    }
    const f16x4 kh = *(const f16x4 *)(q + kQHi + kLatent + 16 * w + 4 * g);
    const f16x4 kl = *(const f16x4 *)(q + kQLo + kLatent + 16 * w + 4 * g);
    const _Float16 z0 = (_Float16)0.0f;
    if (kZp) {
      const f16x2 sh = *(const f16x2 *)(q + kQSumHi + 8 * w + 2 * g);
      const f16x2 sl = *(const f16x2 *)(q + kQSumLo + 8 * w + 2 * g);
      kzh = f16x8{kh.x, kh.y, kh.z, kh.w, sh.x, sh.y, z0, z0};
      kzl = f16x8{kl.x, kl.y, kl.z, kl.w, sl.x, sl.y, z0, z0};
    } else {
      kzh = f16x8{kh.x, kh.y, kh.z, kh.w, z0, z0, z0, z0};
      kzl = f16x8{kl.x, kl.y, kl.z, kl.w, z0, z0, z0, z0};
    }
  }

  _Float16 *vblk = wblk + w * kWBlk;  // [32][kVRow] C_hi of this wave's channels
  // INT4: the fp16 exponent bits of 1024 and of 64 in both halves, in VGPRs
  // opaque to the optimizer (see dequant16)
  uint2 magic = {0u, 0u};
  if constexpr (kZp) {
    asm("v_mov_b32 %0, 0x64006400" : "=v"(magic.x));
    asm("v_mov_b32 %0, 0x54005400" : "=v"(magic.y));
  }

  f32x4 acc[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 accz = {0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;

  const Off16<FMT> off = offsets16<FMT>(w, lane);
  const bool zero_b = off.b_zero;  // uniform: depends on the wave only
  Raw16<FMT> raw[kNpf16];
  // Paged layout: each tile's descriptors come from its page. The page index
  // is read from the sequence's block-table row one tile ahead, with a buffer
  // (vector) load: a scalar load would share its wait counter with LDS
  // traffic, and every LDS wait of the tile would then wait for it too.
  constexpr bool paged = PAGED;
  constexpr int kPol = SLICED ? kSliceLoadPolicy : kLatLoadPolicy;  // latent loads' cache policy
  // the sequence's block-table row and its layer's pool (paged layout)
  const int pb = paged ? b % a.pg.batch : 0;
  const int64_t pool = paged ? (int64_t)(b / a.pg.batch) * a.pg.layer_rows : 0;
  const __amdgpu_buffer_rsrc_t trow =
      make_rsrc(paged ? (const void *)(a.pg.table + (int64_t)pb * a.pg.max_pages) : a.kpe,
                paged ? a.pg.max_pages * 4 : 0);
  auto page_entry = [&](int r) {  // raw table entry of token r (any lane; reads 0 past the row)
    return __builtin_amdgcn_raw_buffer_load_b32(trow, (r >> a.pg.shift) * 4, 0, 0);
  };
  auto checked = [&](uint32_t entry, int r) {  // the page of token r, or -1
    const int pg = (int)__builtin_amdgcn_readfirstlane(entry);
    return (r < t_end && pg >= 0 && pg < a.pg.num_pages) ? pg : -1;
  };
  auto rsrc_of = [&](int r0, int page) {
    if constexpr (PAGED) return page_rsrc<FMT>(a, pool, page, r0, t_end);
    else return tile_rsrc<FMT>(a, b, r0, t_end);
  };
#pragma unroll
  for (int p = 0; p < kNpf16; ++p) {
    const int r0 = t_begin + p * kT16;
    const SplitRsrc rs0 = rsrc_of(r0, paged ? checked(page_entry(r0), r0) : 0);
    load16_small<FMT>(raw[p], rs0, off, zero_b);
    load16_lat<FMT, kPol>(raw[p], rs0, off, t_end - r0, i);
  }
  uint32_t next_entry = paged ? page_entry(t_begin + kNpf16 * kT16) : 0u;

  for (int it0 = 0; it0 < ntiles; it0 += kNpf16) {
#pragma unroll
  for (int p = 0; p < kNpf16; ++p) {
    const int it = it0 + p;
    if (it >= ntiles) break;  // uniform across the workgroup
    // ---- 1. the tile's small planes into the shared staging area
    stage16<FMT>(raw[p], off, aux);
    __syncthreads();
    const Meta16 mt = meta16<FMT>(aux, w, g, i);
    // the small planes of the tile kNpf16 ahead (their registers were read by
    // the staging stores, which the barrier has waited for)
    const int r_next = t_begin + (it + kNpf16) * kT16;
    const SplitRsrc rs_next = rsrc_of(r_next, paged ? checked(next_entry, r_next) : 0);
    __builtin_amdgcn_sched_barrier(0);
    load16_small<FMT>(raw[p], rs_next, off, zero_b);
    __builtin_amdgcn_sched_barrier(0);

    // ---- 2. dequantize in registers; partial scores; C_hi to the value block
    f32x4 sc[2];
    // Wave priority: a wave issuing its dequantization and score MFMAs (and,
    // below, its value MFMAs) goes before the other waves of the SIMD, which
    // are then mostly waiting on loads or a barrier; the matrix and vector
    // pipes stay fed. About 3% on the INT8 and INT4 partial launches.
    __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      f16x8 hi[4], lo[4];
      f16x4 khi, klo;
      f16x8 vdat[4];
      dequant16<FMT>(raw[p], mt, rb, hi, lo, vdat, magic, khi, klo);
      if constexpr (kEarly) {
        // this half-tile's codes are consumed: its share of the next tile's
        // latent loads goes out now (the raw registers stay live, so the
        // score products below read other registers)
        __builtin_amdgcn_sched_barrier(0);
        load16_lat_half<FMT, kPol>(raw[p], rs_next, off, t_end - r_next, i, rb);
        __builtin_amdgcn_sched_barrier(0);
      }
      vstore16<FMT>(vblk, rb, g, i, vdat, mt);
      // Every score product is a 16x16x32 MFMA, so each accumulator is fed
      // by one MFMA shape only: on this GPU a 16x16x16 MFMA that takes as its
      // accumulator the result of a 16x16x32 MFMA issued just before it reads
      // a stale value (the matrix unit forwards a result only to an identical
      // instruction), and the compiler does not separate the two. The k_pe
      // channels and (INT4) the zero-points share one k-step: slots 0..3 of
      // each lane group hold k_pe, slots 4..5 the zero-points, 6..7 zeros.
      const _Float16 z0 = (_Float16)0.0f;
      f16x2 z = {z0, z0};
      if (kZp) z = bitcast<f16x2>(mt.zp[rb]);
      const f16x8 akh = {khi.x, khi.y, khi.z, khi.w, z.x, z.y, z0, z0};
      const f16x8 akl = {klo.x, klo.y, klo.z, klo.w, z0, z0, z0, z0};
      // one accumulator chain per half-tile (the two halves interleave)
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        s = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi[kk], qh[kk], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi[kk], ql[kk], s, 0, 0, 0);
        if (kLo) s = __builtin_amdgcn_mfma_f32_16x16x32_f16(lo[kk], qh[kk], s, 0, 0, 0);
      }
      s = __builtin_amdgcn_mfma_f32_16x16x32_f16(akh, kzh, s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_16x16x32_f16(akh, kzl, s, 0, 0, 0);
      if (kLo) s = __builtin_amdgcn_mfma_f32_16x16x32_f16(akl, kzh, s, 0, 0, 0);
      sc[rb] = s;
    }

    __builtin_amdgcn_s_setprio(0);
    // ---- 3. the next tile's latent loads (INT4 and BF16 latents), after
    // this tile's score products have been issued. INT8 latents issue each
    // half-tile's share earlier, right after that half's dequantization
    // (above), so their loads are in flight during the score products too
    // (1-4% on the INT8 launches); for the other formats the registers that
    // keeps live spill in the tile loop. Always issued, so the count of
    // outstanding loads is the same on every path.
    if constexpr (!kEarly) {
      __builtin_amdgcn_sched_barrier(0);
      load16_lat<FMT, kPol>(raw[p], rs_next, off, t_end - r_next, i);
    }
    if (paged) next_entry = page_entry(r_next + kT16);

    // ---- 4. partial scores of the four waves
    // [wave][half][lane][4]: consecutive lanes use consecutive 16 bytes
    *(f32x4 *)(part + ((2 * w) * 64 + lane) * 4) = sc[0];
    *(f32x4 *)(part + ((2 * w + 1) * 64 + lane) * 4) = sc[1];
    __syncthreads();  // every wave's partial scores of this tile are in LDS
    const float *pb_in = part + lane * 4;
    f32x4 t0 = *(const f32x4 *)pb_in, t1 = *(const f32x4 *)(pb_in + 64 * 4);
#pragma unroll
    for (int v = 1; v < kWaves; ++v) {
      t0 += *(const f32x4 *)(pb_in + (2 * v) * 64 * 4);
      t1 += *(const f32x4 *)(pb_in + (2 * v + 1) * 64 * 4);
    }

    // ---- 5. online softmax (base 2), identical in every wave; lane (g, i)
    // holds tokens 4g+r and 16+4g+r of head i
    float p8[8] = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
    const int left = t_end - (t_begin + it * kT16);  // uniform
    if (left < kT16) {  // only the last tile of a split is partial
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (4 * g + r >= left) p8[r] = -INFINITY;
        if (16 + 4 * g + r >= left) p8[4 + r] = -INFINITY;
      }
    }
    float tmax = fmaxf(fmaxf(fmaxf(p8[0], p8[1]), fmaxf(p8[2], p8[3])),
                       fmaxf(fmaxf(p8[4], p8[5]), fmaxf(p8[6], p8[7])));
    tmax = max_across_groups(tmax);
    // Lazy running max: the reference point moves only when some head's tile
    // maximum exceeds it by more than kSlack, so weights stay at or below
    // 2^kSlack and most tiles skip the rescale.
    // Every wave holds the same scores and takes the same decision.
    if (__builtin_amdgcn_ballot_w64(tmax > m_run + kSlack)) {
      const float m_new = fmaxf(m_run, tmax + kHead);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
#pragma unroll
      for (int n = 0; n < 8; ++n) acc[n] *= alpha;
      if (kZp) accz *= alpha;
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) p8[r] = __builtin_amdgcn_exp2f(p8[r] - m_run);
    f16x8 pb;
#pragma unroll
    for (int r = 0; r < 8; ++r) pb[r] = (_Float16)p8[r];
    // The normalizer sums the same fp16 weights the value products take (two
    // per dot instruction, fp32 accumulation), so the output is a weighted
    // mean of the value rows with exactly those weights.
    {
      const f16x2 one2 = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
      for (int r = 0; r < 4; ++r) l_run = __builtin_amdgcn_fdot2(f16x2{pb[2 * r], pb[2 * r + 1]}, one2, l_run, false);
    }

    __builtin_amdgcn_s_setprio(2);
    // values of this wave's 128 channels (its own block, no barrier needed)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // rows 4g..4g+3 (and 16 more) share bits 2 and 3, so one swap bit per lane group
    const int sg = vswz(4 * g);
    const int col = 8 * (((i >> 1) & 1) ^ sg) + 4 * (i & 1);  // this lane's 4 fp16 of 16
    const _Float16 *v0 = vblk + (4 * g + (i >> 2)) * kVRow + col;
    const _Float16 *v1 = v0 + 16 * kVRow;
    if (kZp) {
      // INT4: block n holds group n's codes; its scales s_t (transposed, rows
      // 4n..4n+3) go into the weights: p_t s_t = ph + pl exactly (fp16 hi/lo;
      // p <= 1 here, so the product is finite for every fp16 scale), and acc
      // gets sum_t p_t s_t q_t with no rounding of s q. The fp16 weights stay
      // normal down to p = 2^-14.
      const f16x8 pbs = pb;
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const f16x4 a0 = lds_read_tr16(v0 + 16 * n);
        const f16x4 a1 = lds_read_tr16(v1 + 16 * n);
        const f16x8 av = f16x8{a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        const int trow = 4 * n + g;
        const f16x8 st = *(const f16x8 *)(vblk + trow * kVRow + 136 - 8 * vswz(trow));
        const f16x8 ph = pbs * st;
        const f16x8 pl = __builtin_elementwise_fma(pbs, st, -ph);
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, ph, acc[n], 0, 0, 0);
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pl, acc[n], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const f16x4 a0 = lds_read_tr16(v0 + 16 * n);
        const f16x4 a1 = lds_read_tr16(v1 + 16 * n);
        const f16x8 av = f16x8{a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pb, acc[n], 0, 0, 0);
      }
    }
    if (kZp) {
      // columns 128..135 of the block are the 8 groups' zero-points; the
      // lanes that read the other chunk (the transposed scales) fill the
      // unused slots 8..15 of this product
      const _Float16 *z0 = vblk + (4 * g + (i >> 2)) * kVRow + 128 + col;
      const f16x4 a0 = lds_read_tr16(z0);
      const f16x4 a1 = lds_read_tr16(z0 + 16 * kVRow);
      const f16x8 az = f16x8{a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      accz = __builtin_amdgcn_mfma_f32_16x16x32_f16(az, pb, accz, 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
  }

  }
  // ---- write this unit's partial: m and l (same in every wave), this wave's channels
  l_run = sum_across_groups(l_run);
  if (kZp) {
    // accz lane (g, i) holds zero-point group 4g+r of this wave (slots 8..15 are
    // padding); channel block n of the wave is group n
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float *oz = (float *)vblk;  // [16 heads][16 slots], the value block is free now
#pragma unroll
    for (int r = 0; r < 4; ++r) oz[i * 16 + 4 * g + r] = accz[r];
    lds_stores_done();
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[n] += oz[i * 16 + n];
  }
  if (kZp) {
    // INT4 value blocks hold each 8 channels in the order 0,4,1,5,2,6,3,7, so
    // lane group g holds channels {0,4,1,5} (g even) or {2,6,3,7} (g odd) of
    // its 8: slots 0 and 2 are a channel pair, and so are slots 1 and 3
    float *dst = a.ws_acc + (ws_row + i) * kLatent + 128 * w + 8 * (g >> 1) + 2 * (g & 1);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      *(float2 *)(dst + 16 * n) = float2{acc[n][0], acc[n][2]};
      *(float2 *)(dst + 16 * n + 4) = float2{acc[n][1], acc[n][3]};
    }
  } else {
    float *dst = a.ws_acc + (ws_row + i) * kLatent + 128 * w + 4 * g;
#pragma unroll
    for (int n = 0; n < 8; ++n) *(f32x4 *)(dst + 16 * n) = acc[n];
  }
  if (w == 0 && g == 0) {
    a.ws_m[ws_row + i] = m_run;
    a.ws_l[ws_row + i] = l_run;
  }
  S += n;
  if (S >= plan.g1) break;
  do {  // the next sequence that holds tokens (one exists: the range is not done)
    ++b;
    L = b < a.B ? clamp_len(a.seq_lens[b], a.cap) : 0;
  } while (b < a.B && L == 0);
  }
}

// ---- 32 heads per workgroup (32, 64 and 128 heads; BF16 and INT8 latents)
//
// The 16-head kernel run once per 16-head slice dequantizes every tile once
// per slice; with many heads its vector work (the dequantization, the score
// sums and the softmax that each of the four waves repeats) bounds it. This
// kernel serves a slice of 32 heads per workgroup as two head groups of 16
// (hg), so each tile is dequantized once for 32 heads and each dequantized
// operand feeds the score products of both groups; and the softmax of the
// tile is computed once, not in every wave: wave w takes heads 8w .. 8w+7 of
// the slice (lane l: head 8w + l/8, tokens l%8 + 8k, k = 0..3), adds the four
// waves' partial scores, moves each head's lazy reference, and writes the
// weights (fp16, in the value product's operand order) and each head's
// rescale factor to LDS, from where every wave takes all 32 heads' weights
// for its value products. Per tile: dequantize and score (both groups),
// partial scores to LDS, barrier, softmax of its 8 heads, stage the next
// tile's small planes, barrier, values (both groups). Two workgroups per CU
// (the queries and sums of 32 heads take 256 registers per lane). INT4
// latents are not served here: their exact value product (codes times p s as
// an fp16 hi/lo pair, per head group) needs more registers than two waves per
// SIMD allow, and at one wave per SIMD the kernel was slower than the 16-head
// kernel per slice.
__device__ __forceinline__ float dpp_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
}
__device__ __forceinline__ float dpp_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
}
__device__ __forceinline__ float dpp_mirror8(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));  // row_half_mirror
}
// max and sum over each group of 8 lanes (8k .. 8k+7)
__device__ __forceinline__ float max8(float x) {
  x = fmaxf(x, dpp_xor1(x));
  x = fmaxf(x, dpp_xor2(x));
  return fmaxf(x, dpp_mirror8(x));
}
__device__ __forceinline__ float sum8(float x) {
  x += dpp_xor1(x);
  x += dpp_xor2(x);
  return x + dpp_mirror8(x);
}

constexpr int kWideHeads = 32;
constexpr int kWideWgPerCu = 2;
constexpr int kPartWide = kWaves * 2 * 2 * 64 * 4;  // floats: [wave][hg][half][lane][4]

// (one workgroup of four waves per SIMD slot: kWideWgPerCu waves per SIMD)
template <int FMT, bool PAGED>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(kWideWgPerCu, kWideWgPerCu)))
void wide_kernel(SplitArgs a) {
  static_assert(!has_zero(FMT), "INT4 latents take the 16-head kernel per slice");
  constexpr bool kLo = FMT != MLA_FMT_BF16;
  constexpr int kPol = kSliceLoadPolicy;  // slices of a range read its latent from the caches
  __shared__ __attribute__((aligned(16))) _Float16 wblk[kWaves * kWBlk];
  __shared__ __attribute__((aligned(16))) float part[kPartWide];
  __shared__ __attribute__((aligned(16))) uint8_t aux[Aux16<FMT>::kBytes];
  __shared__ __attribute__((aligned(16))) _Float16 pw[kWideHeads * kT16];
  __shared__ float alpha_s[kWideHeads];
  __shared__ int resc_s[kWaves];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g = lane >> 4, i = lane & 15;
  // slices of 32 heads, the slices of a range 8 workgroup indices apart (one XCD)
  const int nslice = a.H / kWideHeads;
  const int win = blockIdx.x / (8 * nslice), in_win = blockIdx.x % (8 * nslice);
  const int hs = in_win / 8, rng = 8 * win + in_win % 8;
  const PlanStart plan = plan_start(a, a.W, rng, (int *)part);
  int b = plan.b, S = plan.S, L = plan.L;
  // the softmax lanes: head hh of the slice, tokens j + 8k
  const int hh = 8 * w + (lane >> 3), j = lane & 7;
  _Float16 *vblk = wblk + w * kWBlk;
  const Off16<FMT> off = offsets16<FMT>(w, lane);
  const bool zero_b = off.b_zero;

  while (b < a.B) {
  b = __builtin_amdgcn_readfirstlane(b);
  S = __builtin_amdgcn_readfirstlane(S);
  L = __builtin_amdgcn_readfirstlane(L);
  const int n = tiles_of(L);
  const int t_begin = __builtin_amdgcn_readfirstlane((max(plan.g0, S) - S) * kT16);
  const int t_end = __builtin_amdgcn_readfirstlane(min(L, (min(plan.g1, S + n) - S) * kT16));
  const int64_t ws_row = ((int64_t)rng + b) * a.H + kWideHeads * hs;
  const int ntiles = (t_end - t_begin + kT16 - 1) / kT16;

  // queries of head 16 hg + i of the slice for this wave's channels
  f16x8 qh[2][4], ql[2][4], kzh[2], kzl[2];
#pragma unroll
  for (int hg = 0; hg < 2; ++hg) {
    const _Float16 *q = a.qa + ((int64_t)b * a.H + kWideHeads * hs + 16 * hg + i) * kQRec;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      qh[hg][kk] = *(const f16x8 *)(q + kQHi + lane_chan<FMT>(w, g, kk));
      ql[hg][kk] = *(const f16x8 *)(q + kQLo + lane_chan<FMT>(w, g, kk));
    }
    const f16x4 kh = *(const f16x4 *)(q + kQHi + kLatent + 16 * w + 4 * g);
    const f16x4 kl = *(const f16x4 *)(q + kQLo + kLatent + 16 * w + 4 * g);
    const _Float16 z0 = (_Float16)0.0f;
    kzh[hg] = f16x8{kh.x, kh.y, kh.z, kh.w, z0, z0, z0, z0};
    kzl[hg] = f16x8{kl.x, kl.y, kl.z, kl.w, z0, z0, z0, z0};
  }

  f32x4 acc[2][8];
#pragma unroll
  for (int hg = 0; hg < 2; ++hg)
#pragma unroll
    for (int nn = 0; nn < 8; ++nn) acc[hg][nn] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_part = 0.0f;  // head hh (same in its 8 lanes); this lane's share of l

  Raw16<FMT> raw;
  constexpr bool paged = PAGED;
  const int pb_row = paged ? b % a.pg.batch : 0;
  const int64_t pool = paged ? (int64_t)(b / a.pg.batch) * a.pg.layer_rows : 0;
  const __amdgpu_buffer_rsrc_t trow =
      make_rsrc(paged ? (const void *)(a.pg.table + (int64_t)pb_row * a.pg.max_pages) : a.kpe,
                paged ? a.pg.max_pages * 4 : 0);
  auto page_entry = [&](int r) { return __builtin_amdgcn_raw_buffer_load_b32(trow, (r >> a.pg.shift) * 4, 0, 0); };
  auto checked = [&](uint32_t entry, int r) {
    const int pg = (int)__builtin_amdgcn_readfirstlane(entry);
    return (r < t_end && pg >= 0 && pg < a.pg.num_pages) ? pg : -1;
  };
  auto rsrc_of = [&](int r0, int page) {
    if constexpr (PAGED) return page_rsrc<FMT>(a, pool, page, r0, t_end);
    else return tile_rsrc<FMT>(a, b, r0, t_end);
  };
  {
    const SplitRsrc rs0 = rsrc_of(t_begin, paged ? checked(page_entry(t_begin), t_begin) : 0);
    load16_small<FMT>(raw, rs0, off, zero_b);
    load16_lat<FMT, kPol>(raw, rs0, off, t_end - t_begin, i);
  }
  uint32_t next_entry = paged ? page_entry(t_begin + kT16) : 0u;
  stage16<FMT>(raw, off, aux);
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    // ---- dequantize once, scores of both head groups
    const Meta16 mt = meta16<FMT>(aux, w, g, i);
    const int r_next = t_begin + (it + 1) * kT16;
    const SplitRsrc rs_next = rsrc_of(r_next, paged ? checked(next_entry, r_next) : 0);
    __builtin_amdgcn_sched_barrier(0);
    load16_small<FMT>(raw, rs_next, off, zero_b);
    __builtin_amdgcn_sched_barrier(0);
    f32x4 sc[2][2];
    __builtin_amdgcn_s_setprio(2);  // as in split16_kernel
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      f16x8 hi[4], lo[4], vdat[4];
      f16x4 khi, klo;
      dequant16<FMT>(raw, mt, rb, hi, lo, vdat, uint2{0u, 0u}, khi, klo);
      vstore16<FMT>(vblk, rb, g, i, vdat, mt);
      const _Float16 z0 = (_Float16)0.0f;
      const f16x8 akh = {khi.x, khi.y, khi.z, khi.w, z0, z0, z0, z0};
      const f16x8 akl = {klo.x, klo.y, klo.z, klo.w, z0, z0, z0, z0};
#pragma unroll
      for (int hg = 0; hg < 2; ++hg) {
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          s = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi[kk], qh[hg][kk], s, 0, 0, 0);
          s = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi[kk], ql[hg][kk], s, 0, 0, 0);
          if (kLo) s = __builtin_amdgcn_mfma_f32_16x16x32_f16(lo[kk], qh[hg][kk], s, 0, 0, 0);
        }
        s = __builtin_amdgcn_mfma_f32_16x16x32_f16(akh, kzh[hg], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_16x16x32_f16(akh, kzl[hg], s, 0, 0, 0);
        if (kLo) s = __builtin_amdgcn_mfma_f32_16x16x32_f16(akl, kzh[hg], s, 0, 0, 0);
        sc[hg][rb] = s;
      }
    }
    __builtin_amdgcn_s_setprio(0);
    // partial scores [wave][hg][half][lane][4]; then the next tile's latent
    // loads (after the score results were read back: see split16_kernel)
#pragma unroll
    for (int hg = 0; hg < 2; ++hg)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) *(f32x4 *)(part + (((w * 2 + hg) * 2 + rb) * 64 + lane) * 4) = sc[hg][rb];
    __builtin_amdgcn_sched_barrier(0);
    load16_lat<FMT, kPol>(raw, rs_next, off, t_end - r_next, i);
    if (paged) next_entry = page_entry(r_next + kT16);
    __syncthreads();

    // ---- softmax (base 2) of head hh: tokens j + 8k. The partial score of
    // (token 16 h + 4 g' + r, head 16 hg + c) sits at lane 16 g' + c, slot r
    // of block (hg, h) of each wave.
    {
      const int hg = hh >> 4, c = hh & 15;
      const int left = t_end - (t_begin + it * kT16);  // uniform
      float sv[4];
      float tmax = -INFINITY;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int t = j + 8 * k, h = t >> 4, tt = t & 15;
        const float *pp = part + ((hg * 2 + h) * 64 + 16 * (tt >> 2) + c) * 4 + (tt & 3);
        float x = pp[0];
#pragma unroll
        for (int v = 1; v < kWaves; ++v) x += pp[v * 2 * 2 * 64 * 4];
        sv[k] = t < left ? x : -INFINITY;
        tmax = fmaxf(tmax, sv[k]);
      }
      tmax = max8(tmax);
      float alpha = 1.0f;
      const bool mv = tmax > m_run + kLazy;  // the lazy reference of split16_kernel
      if (mv) {
        const float m_new = fmaxf(m_run, tmax);
        alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
      }
      float ps = 0.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int t = j + 8 * k;
        const float p = __builtin_amdgcn_exp2f(sv[k] - m_run);
        ps += p;
        // the value product's B order: head c, lane group g' holds tokens
        // 4g'..4g'+3 then 16+4g'..16+4g'+3
        pw[hh * kT16 + 8 * ((t & 15) >> 2) + 4 * (t >> 4) + (t & 3)] = (_Float16)p;
      }
      l_part = l_part * alpha + ps;
      if (j == 0) alpha_s[hh] = alpha;
      const bool any = __builtin_amdgcn_ballot_w64(mv) != 0;
      if (lane == 0) resc_s[w] = any;
    }
    stage16<FMT>(raw, off, aux);  // the next tile's small planes
    __syncthreads();

    // ---- values of this wave's 128 channels, both head groups
    if (resc_s[0] | resc_s[1] | resc_s[2] | resc_s[3]) {  // uniform
#pragma unroll
      for (int hg = 0; hg < 2; ++hg) {
        const float al = alpha_s[16 * hg + i];
#pragma unroll
        for (int nn = 0; nn < 8; ++nn) acc[hg][nn] *= al;
      }
    }
    __builtin_amdgcn_s_setprio(2);
    f16x8 pb[2];
#pragma unroll
    for (int hg = 0; hg < 2; ++hg) pb[hg] = *(const f16x8 *)(pw + (16 * hg + i) * kT16 + 8 * g);
    const int sg = vswz(4 * g);
    const int col = 8 * (((i >> 1) & 1) ^ sg) + 4 * (i & 1);
    const _Float16 *v0 = vblk + (4 * g + (i >> 2)) * kVRow + col;
    const _Float16 *v1 = v0 + 16 * kVRow;
#pragma unroll
    for (int nn = 0; nn < 8; ++nn) {
      const f16x4 a0 = lds_read_tr16(v0 + 16 * nn);
      const f16x4 a1 = lds_read_tr16(v1 + 16 * nn);
      const f16x8 av = f16x8{a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
      for (int hg = 0; hg < 2; ++hg)
        acc[hg][nn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pb[hg], acc[hg][nn], 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
    // the value block is rewritten by the next tile's dequantization: its
    // transposed reads above come first (in-order LDS queue; the fence keeps
    // the compiler from moving the stores above them)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- this unit's partial record
  const float l_run = sum8(l_part);
#pragma unroll
  for (int hg = 0; hg < 2; ++hg) {
    float *dst = a.ws_acc + (ws_row + 16 * hg + i) * kLatent + 128 * w + 4 * g;
#pragma unroll
    for (int nn = 0; nn < 8; ++nn) *(f32x4 *)(dst + 16 * nn) = acc[hg][nn];
  }
  if (j == 0) {
    a.ws_m[ws_row + hh] = m_run;
    a.ws_l[ws_row + hh] = l_run;
  }
  S += n;
  if (S >= plan.g1) break;
  do {
    ++b;
    L = b < a.B ? clamp_len(a.seq_lens[b], a.cap) : 0;
  } while (b < a.B && L == 0);
  __syncthreads();  // the staging area and the softmax state in LDS are reused by the next pass
  }
}

// ------------------------------------------------------------------ reduce

constexpr int kReduceBT = 4;  // batch rows per combine block

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

constexpr int kMergeChunk = 16;  // splits merged per round of loads

// Per (head h, 4 batch rows), two waves per row (each half of the 512 latent
// channels): merge the sequence's partial records (the splits: first record
// and count from the partial kernel's table) with log-sum-exp weights and
// normalize, then all
// eight waves form out[b,h,:] = o_lat W_UV[h]. The merge takes the splits 16 at
// a time: lane s loads m and l of split s while every lane loads its 4 latent
// channels of all 16 splits, in one round of loads. The chunk's maximum updates
// a running maximum (what was merged before is rescaled by 2^(M_old - M_new)),
// and each split's weight 2^(m_s - M) is taken from its lane as a scalar. A
// split with l = 0 holds no tokens and its sums were never written: it gets
// weight zero and its sums are skipped, not multiplied. Grid (H, ceil(B/4),
// layers), 512 threads: layer l's sequences are l * B .. l * B + B - 1 of the
// record table and of out, and its W_UV follows layer l-1's.
constexpr int kReduceThreads = 512;
constexpr int kReduceCS = kReduceThreads / 16;  // latent row chunks of the projection (16 rows each)
static_assert(kReduceBT * kVDim == kReduceThreads && kReduceCS * 16 == kLatent && 2 * kReduceBT * 64 == kReduceThreads,
              "two waves per row, one output per thread");
__global__ __launch_bounds__(kReduceThreads) void reduce_kernel(const float *ws_m, const float *ws_l,
                                                                const float *ws_acc, const int32_t *rec_tab,
                                                                const uint16_t *w_uv, int B, int H, float *out) {
  __shared__ float olat[kReduceBT][kLatent];
  __shared__ float red[kReduceCS][kReduceBT][kVDim];
  const int h = blockIdx.x;
  const int b0 = blockIdx.y * kReduceBT;
  const int64_t layer_seq = (int64_t)blockIdx.z * B;  // the layer's first sequence
  rec_tab += 2 * layer_seq;
  out += layer_seq * H * kVDim;
  w_uv += (int64_t)blockIdx.z * H * kLatent * kVDim;
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int bt = wv >> 1, half = wv & 1;
  const int b = b0 + bt;  // uniform across the wave
  f32x4 o0 = {0.f, 0.f, 0.f, 0.f};
  if (b < B) {
    // the sequence's records, as the partial kernel's table lists them
    const int first = __builtin_amdgcn_readfirstlane(rec_tab[2 * b]);
    const int count = __builtin_amdgcn_readfirstlane(rec_tab[2 * b + 1]);
    const int64_t base = (int64_t)first * H + h;
    const float *acc = ws_acc + base * kLatent + (kLatent / 2) * half + 4 * lane;
    float M = -INFINITY, Ls = 0.0f;
    for (int c0 = 0; c0 < count; c0 += kMergeChunk) {
      const int cn = min(kMergeChunk, count - c0);  // uniform
      float ml = -INFINITY, ll = 0.0f;
      if (lane < cn) {
        ll = ws_l[base + (int64_t)(c0 + lane) * H];
        ml = ws_m[base + (int64_t)(c0 + lane) * H];
      }
      f32x4 a0[kMergeChunk];
#pragma unroll
      for (int j = 0; j < kMergeChunk; ++j)
        if (j < cn) a0[j] = *(const f32x4 *)(acc + (int64_t)(c0 + j) * H * kLatent);
      const float mc = wave_max(ll > 0.0f ? ml : -INFINITY);
      if (mc == -INFINITY) continue;  // no split of the chunk holds tokens
      const float mn = fmaxf(M, mc);
      const float alpha = __builtin_amdgcn_exp2f(M - mn);  // 0 while nothing is merged
      o0 *= alpha;
      Ls *= alpha;
      M = mn;
      const float wl = ll > 0.0f ? __builtin_amdgcn_exp2f(ml - M) : 0.0f;
      Ls += wave_sum(wl * ll);
#pragma unroll
      for (int j = 0; j < kMergeChunk; ++j) {
        if (j < cn) {
          const float wgt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), j));
          if (wgt != 0.0f) {  // uniform
#pragma unroll
            for (int k = 0; k < 4; ++k) o0[k] = fmaf(wgt, a0[j][k], o0[k]);
          }
        }
      }
    }
    const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
    o0 *= inv;
  }
  // this thread's W_UV rows for the projection (8 output columns of 16 latent
  // rows), in flight while the merged rows go through LDS
  const int eg = tid & 15, cs = tid >> 4;
  const uint16_t *w = w_uv + ((int64_t)h * kLatent + cs * 16) * kVDim + 8 * eg;
  u32x4 wr[16];
#pragma unroll
  for (int cc = 0; cc < 16; ++cc) wr[cc] = *(const u32x4 *)(w + cc * kVDim);
  *(f32x4 *)&olat[bt][(kLatent / 2) * half + 4 * lane] = o0;
  __syncthreads();
  float acc[kReduceBT][8];
#pragma unroll
  for (int r = 0; r < kReduceBT; ++r)
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[r][k] = 0.0f;
#pragma unroll
  for (int c4 = 0; c4 < 4; ++c4) {
    f32x4 ov[kReduceBT];
#pragma unroll
    for (int r = 0; r < kReduceBT; ++r) ov[r] = *(const f32x4 *)&olat[r][cs * 16 + 4 * c4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 wq = wr[4 * c4 + q];
      float wf[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        wf[2 * k] = bf16_bits_to_f32(wq[k] & 0xFFFFu);
        wf[2 * k + 1] = bf16_bits_to_f32(wq[k] >> 16);
      }
#pragma unroll
      for (int r = 0; r < kReduceBT; ++r)
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[r][k] += ov[r][q] * wf[k];
    }
  }
#pragma unroll
  for (int r = 0; r < kReduceBT; ++r)
#pragma unroll
    for (int k = 0; k < 8; ++k) red[cs][r][8 * eg + k] = acc[r][k];
  lds_stores_done();
  __syncthreads();
  // one output per thread: kReduceBT * kVDim = 512
  const int r = tid / kVDim, e = tid % kVDim;
  const int bo = b0 + r;
  float v = 0.0f;
#pragma unroll
  for (int q = 0; q < kReduceCS; ++q) v += red[q][r][e];
  if (bo < B) out[((int64_t)bo * H + h) * kVDim + e] = v;
}

// The same merge and projection for small grids, one sequence per block
// (grid (H, B, layers), 512 threads): every one of the eight waves takes
// records w, w + 8, ... (kReduce1Recs of them per round of loads, so a
// sequence of up to 48 records is read in one round), all 512 channels of
// each (8 per lane), and merges them with its own running maximum; the waves'
// merges then meet in LDS under the block's maximum. The block's W_UV rows
// are requested first, so they arrive during the merge. Used where the grid
// has at most one block per CU: there the latency of the rounds of loads is
// the launch's time, and one sequence per block spreads the records over
// more CUs (each block reads its head's W_UV, from L2 after the first).
constexpr int kReduce1Recs = 6;
constexpr int kReduce1MaxBlocks = 256;

__global__ __launch_bounds__(kReduceThreads) void reduce1_kernel(const float *ws_m, const float *ws_l,
                                                                 const float *ws_acc, const int32_t *rec_tab,
                                                                 const uint16_t *w_uv, int B, int H, float *out) {
  __shared__ __attribute__((aligned(16))) float olat[kReduceThreads / 64][kLatent];
  __shared__ float orow[kLatent];
  __shared__ float red[kReduceCS][kVDim];
  __shared__ float wm[kReduceThreads / 64], wls[kReduceThreads / 64];
  constexpr int NW = kReduceThreads / 64;
  const int h = blockIdx.x, b = blockIdx.y;
  const int64_t layer_seq = (int64_t)blockIdx.z * B;
  rec_tab += 2 * layer_seq;
  out += layer_seq * H * kVDim;
  w_uv += ((int64_t)blockIdx.z * H + h) * kLatent * kVDim;
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  // this thread's W_UV rows (8 output columns of 16 latent rows)
  const int eg = tid & 15, cs = tid >> 4;
  const uint16_t *w = w_uv + ((int64_t)cs * 16) * kVDim + 8 * eg;
  u32x4 wr[16];
#pragma unroll
  for (int cc = 0; cc < 16; ++cc) wr[cc] = *(const u32x4 *)(w + cc * kVDim);

  const int first = __builtin_amdgcn_readfirstlane(rec_tab[2 * b]);
  const int count = __builtin_amdgcn_readfirstlane(rec_tab[2 * b + 1]);
  const int64_t base = (int64_t)first * H + h;
  float M = -INFINITY, Ls = 0.0f;
  f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
  for (int r0 = 0; r0 < count; r0 += NW * kReduce1Recs) {
    f32x4 a[kReduce1Recs][2];
    float ms[kReduce1Recs], ls[kReduce1Recs];
#pragma unroll
    for (int k = 0; k < kReduce1Recs; ++k) {
      const int sidx = r0 + wv + NW * k;  // uniform across the wave
      const int64_t rec = base + (int64_t)min(sidx, count - 1) * H;
      ls[k] = sidx < count ? ws_l[rec] : 0.0f;
      ms[k] = ws_m[rec];
      if (ls[k] > 0.0f) {
        const f32x4 *src = (const f32x4 *)(ws_acc + rec * kLatent + 8 * lane);
        a[k][0] = src[0];
        a[k][1] = src[1];
      }
    }
    float mb = -INFINITY;
#pragma unroll
    for (int k = 0; k < kReduce1Recs; ++k)
      if (ls[k] > 0.0f) mb = fmaxf(mb, ms[k]);
    if (mb == -INFINITY) continue;  // no record of the round holds tokens (uniform)
    const float mn = fmaxf(M, mb);
    const float alpha = __builtin_amdgcn_exp2f(M - mn);  // 0 while nothing is merged
    Ls *= alpha;
    o0 *= alpha;
    o1 *= alpha;
    M = mn;
#pragma unroll
    for (int k = 0; k < kReduce1Recs; ++k) {
      if (ls[k] > 0.0f) {
        const float wgt = __builtin_amdgcn_exp2f(ms[k] - M);
        Ls += wgt * ls[k];
        o0 += wgt * a[k][0];
        o1 += wgt * a[k][1];
      }
    }
  }
  if (lane == 0) {
    wm[wv] = M;
    wls[wv] = Ls;
  }
  __syncthreads();
  float Mall = -INFINITY;
#pragma unroll
  for (int v = 0; v < NW; ++v) Mall = fmaxf(Mall, wm[v]);
  const float sc = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(M - Mall);
  *(f32x4 *)&olat[wv][8 * lane] = o0 * sc;
  *(f32x4 *)&olat[wv][8 * lane + 4] = o1 * sc;
  __syncthreads();
  float Lall = 0.0f;
#pragma unroll
  for (int v = 0; v < NW; ++v)
    if (wm[v] != -INFINITY) Lall += wls[v] * __builtin_amdgcn_exp2f(wm[v] - Mall);
  const float inv = Lall > 0.0f ? 1.0f / Lall : 0.0f;
  {
    float x = 0.0f;
#pragma unroll
    for (int v = 0; v < NW; ++v) x += olat[v][tid];
    orow[tid] = x * inv;
  }
  __syncthreads();
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.0f;
#pragma unroll
  for (int cc = 0; cc < 16; ++cc) {
    const float ov = orow[cs * 16 + cc];
    const u32x4 wq = wr[cc];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc[2 * k] += ov * bf16_bits_to_f32(wq[k] & 0xFFFFu);
      acc[2 * k + 1] += ov * bf16_bits_to_f32(wq[k] >> 16);
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) red[cs][8 * eg + k] = acc[k];
  __syncthreads();
  if (tid < kVDim) {
    float v = 0.0f;
#pragma unroll
    for (int q = 0; q < kReduceCS; ++q) v += red[q][tid];
    out[((int64_t)b * H + h) * kVDim + tid] = v;
  }
}
static_assert(kReduceThreads == kLatent && 64 * 8 == kLatent,
              "one latent channel per thread in the sum over the waves, 8 per lane in the merge");

// ------------------------------------------------------------------ combine

// Merge of the partial records and projection through W_UV. Grid
// (H, ceil(B / R), layers), 256 threads: the block serves head h and R
// sequences of one layer (layer l's sequences are l * B .. l * B + B - 1 of
// the record table and of out, and its W_UV follows layer l-1's). Launched
// with R = 16 where the grid is large (a layer-range call: few blocks share
// each W_UV[h], so it is read from the caches fewer times); smaller grids take
// reduce_kernel, whose two waves per sequence keep more record loads in
// flight (measured: 5-9 µs against 6-13 µs for one layer of 1 to 64
// sequences, 49 against 62 µs at 128 heads; 36 µs for both forms over 27
// layers of 64 sequences, where reduce_kernel alone took 89 µs), and grids of
// at most 256 (head, sequence) pairs reduce1_kernel.
//   1. Merge. TPR = 256 / R threads per sequence, each with CPT = 512 / TPR
//      of the latent channels. The row's records (first record and count from
//      the partial kernel's table) are weighted by
//      2^(m_s - M) / sum_s 2^(m_s - M) l_s with M the largest m_s of a record
//      holding tokens (l_s > 0); records with no tokens get weight zero and
//      their sums are not read. One pass, NB records at a time with all their
//      loads issued together, and a running maximum. o_lat goes to LDS as a
//      bf16 hi/lo pair (hi = bf16(o),
//      lo = bf16(o - hi)): the pair carries ~16 bits, and W_UV is bf16, so
//      the products are exact in fp32. An empty sequence gives o_lat = 0.
//   2. Projection on 16x16x32 bf16 MFMA (rows past R are zero), 64 latent
//      channels of W_UV[h] at a time staged in LDS and read transposed
//      (ds_read_b64_tr_b16): wave w computes output columns 32w .. 32w + 31 as
//      o_hi W + o_lo W. The first two chunks are requested before the merge,
//      each later one two chunks ahead. With 64-row chunks the block takes
//      52 KB of LDS and 128 VGPRs, so three blocks share a CU (47.5 -> 40.3 us
//      for 27 layers of 64 sequences with cold caches, against 128-row chunks
//      at two blocks per CU).
constexpr int kCombChunk = 64;            // latent channels of W_UV staged at a time
constexpr int kCombARow = kLatent + 8;    // bf16 per LDS row of o_lat (hi or lo): 16 B of padding
constexpr int kCombWRow = kVDim + 16;     // bf16 per LDS row of the staged W_UV chunk (see absorb_block)
constexpr int kCombBigGrid = 1024;        // blocks of 16 rows from which the 16-row form is used
template <int R>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3)))
void combine_kernel(const float *ws_m, const float *ws_l, const float *ws_acc, const int32_t *rec_tab,
                    const uint16_t *w_uv, int B, int H, float *out) {
  constexpr int TPR = 256 / R;           // merge threads per sequence
  constexpr int CPT = kLatent / TPR;     // channels per merge thread
  constexpr int NV = CPT / 4;            // 16-byte loads per record and thread
  constexpr int NB = NV < 8 ? 16 / NV : 1;  // records whose loads are in flight together
  __shared__ __attribute__((aligned(16))) uint16_t ahi[R * kCombARow];
  __shared__ __attribute__((aligned(16))) uint16_t alo[R * kCombARow];
  __shared__ __attribute__((aligned(16))) uint16_t wt[kCombChunk * kCombWRow];
  const int h = blockIdx.x;
  const int b0 = blockIdx.y * R;
  const int64_t layer_seq = (int64_t)blockIdx.z * B;  // the layer's first sequence
  rec_tab += 2 * layer_seq;
  out += layer_seq * H * kVDim;
  w_uv += ((int64_t)blockIdx.z * H + h) * kLatent * kVDim;
  const int tid = threadIdx.x;
  const int wv = tid >> 6, lane = tid & 63, g = lane >> 4, i = lane & 15;
  // W_UV rows ch0 .. ch0 + 63 of a chunk (256 bytes each): 4 x 16 bytes per
  // thread and chunk, two chunks in flight
  constexpr int kWL = kCombChunk * kVDim / 8 / 256;
  constexpr int kNChunk = kLatent / kCombChunk;
  constexpr int kAhead = 2;
  u32x4 wl[kAhead][kWL];
  auto load_chunk = [&](int ck, int slot) {
#pragma unroll
    for (int jj = 0; jj < kWL; ++jj) {
      const int k = tid + 256 * jj, row = k >> 4, c8 = k & 15;
      wl[slot][jj] = *(const u32x4 *)(w_uv + (int64_t)(kCombChunk * ck + row) * kVDim + 8 * c8);
    }
  };
#pragma unroll
  for (int ck = 0; ck < kAhead; ++ck) load_chunk(ck, ck);

  // ---- 1. merge
  {
    const int r = tid / TPR, c = tid % TPR;
    const int b = b0 + r;
    f32x4 o[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) o[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int first = b < B ? rec_tab[2 * b] : 0, count = b < B ? rec_tab[2 * b + 1] : 0;
    // one pass over the records, NB at a time: their m, l and sums are loaded
    // together; the running maximum M moves with each batch's maximum and what
    // was merged before is rescaled by 2^(M_old - M_new)
    float M = -INFINITY, Ls = 0.0f;
    for (int s0 = 0; s0 < count; s0 += NB) {
      f32x4 v[NB][NV];
      float ms[NB], ls[NB];
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const int s = s0 + k;
        const int64_t rec = (int64_t)(first + min(s, count - 1)) * H + h;
        ls[k] = s < count ? ws_l[rec] : 0.0f;
        ms[k] = ws_m[rec];
        if (ls[k] > 0.0f) {
          const f32x4 *src = (const f32x4 *)(ws_acc + rec * kLatent + CPT * c);
#pragma unroll
          for (int q = 0; q < NV; ++q) v[k][q] = src[q];
        }
      }
      float mb = -INFINITY;
#pragma unroll
      for (int k = 0; k < NB; ++k)
        if (ls[k] > 0.0f) mb = fmaxf(mb, ms[k]);
      if (mb == -INFINITY) continue;  // no record of the batch holds tokens (uniform per row)
      const float mn = fmaxf(M, mb);
      const float alpha = __builtin_amdgcn_exp2f(M - mn);  // 0 while nothing is merged
      Ls *= alpha;
#pragma unroll
      for (int q = 0; q < NV; ++q) o[q] *= alpha;
      M = mn;
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        if (ls[k] > 0.0f) {
          const float wgt = __builtin_amdgcn_exp2f(ms[k] - M);
          Ls += wgt * ls[k];
#pragma unroll
          for (int q = 0; q < NV; ++q) o[q] += wgt * v[k][q];
        }
      }
    }
    const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
#pragma unroll
    for (int q = 0; q < NV; ++q) o[q] *= inv;
    // bf16 hi / lo of the thread's channels, 8 at a time
#pragma unroll
    for (int k2 = 0; k2 < NV / 2; ++k2) {
      u32x4 hv, lv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = o[2 * k2 + e / 2][2 * (e & 1)], x1 = o[2 * k2 + e / 2][2 * (e & 1) + 1];
        const uint32_t h0 = f32_to_bf16_rne(x0), h1 = f32_to_bf16_rne(x1);
        const uint32_t l0 = f32_to_bf16_rne(x0 - bf16_bits_to_f32(h0)), l1 = f32_to_bf16_rne(x1 - bf16_bits_to_f32(h1));
        hv[e] = h0 | (h1 << 16);
        lv[e] = l0 | (l1 << 16);
      }
      *(u32x4 *)(ahi + r * kCombARow + CPT * c + 8 * k2) = hv;
      *(u32x4 *)(alo + r * kCombARow + CPT * c + 8 * k2) = lv;
    }
  }

  // ---- 2. projection
  f32x4 d[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int ck = 0; ck < kNChunk; ++ck) {
    const int ch0 = kCombChunk * ck;
    __syncthreads();  // the previous chunk's reads of wt (and, the first time, the merge's stores) are done
#pragma unroll
    for (int jj = 0; jj < kWL; ++jj) {
      const int k = tid + 256 * jj, row = k >> 4, c8 = k & 15;
      *(u32x4 *)(wt + row * kCombWRow + 8 * c8) = wl[ck % kAhead][jj];
    }
    lds_stores_done();
    if (ck + kAhead < kNChunk) load_chunk(ck + kAhead, ck % kAhead);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kCombChunk / 32; ++kk) {
      // A: row i, channels ch0 + 32 kk + 8 g .. +7 (zero past the block's R rows)
      bf16x8 a_hi = {}, a_lo = {};
      if (i < R) {
        a_hi = *(const bf16x8 *)(ahi + i * kCombARow + ch0 + 32 * kk + 8 * g);
        a_lo = *(const bf16x8 *)(alo + i * kCombARow + ch0 + 32 * kk + 8 * g);
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        // B: output column 32 wv + 16 nt + i, channels 32 kk + 8 g .. +7 of the chunk
        const uint16_t *p = wt + (32 * kk + 8 * g + (i >> 2)) * kCombWRow + 32 * wv + 16 * nt + 4 * (i & 3);
        const i16x4 r0 = lds_read_tr16_i16(p), r1 = lds_read_tr16_i16(p + 4 * kCombWRow);
        const bf16x8 bw = bitcast<bf16x8>(i16x8{r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w});
        d[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_hi, bw, d[nt], 0, 0, 0);
        d[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_lo, bw, d[nt], 0, 0, 0);
      }
    }
  }
  // lane (g, i) holds rows 4g .. 4g + 3 of column 32 wv + 16 nt + i
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int b = b0 + 4 * g + r;
      if (4 * g + r < R && b < B) out[((int64_t)b * H + h) * kVDim + 32 * wv + 16 * nt + i] = d[nt][r];
    }
}

// -------------------------------------------------------- stream-read probe

// Reads n16 16-byte words with the access pattern of a plain streaming read
// (grid-stride, consecutive lanes on consecutive words, four loads in flight
// per thread) and folds them into one word per workgroup, so that no load is
// dead. NT: non-temporal loads (the lines are not kept in the caches);
// otherwise the default policy, so the lines are allocated in the caches
// like any read's. A measurement aid for the achievable HBM read rate.
template <bool NT>
__device__ __forceinline__ u32x4 stream_ld(const u32x4 *p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *buf, int64_t n16, uint32_t *sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t x = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = stream_ld<NT>(buf + i), b = stream_ld<NT>(buf + i + stride);
    const u32x4 c = stream_ld<NT>(buf + i + 2 * stride);
    const u32x4 d = stream_ld<NT>(buf + i + 3 * stride);
    x ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const u32x4 a = buf[i];
    x ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  __shared__ uint32_t red[4];
  for (int off = 32; off >= 1; off >>= 1) x ^= __shfl_xor(x, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

// ---------------------------------------------------------------- rope tables

// theta_i = base^(-2i/64) of the 32 channel pairs, computed on the host.
struct RopeTheta {
  double t[kRope / 2];
};

// cos / sin of p * theta_i in fp64, rounded to fp32 (nearest even), for
// table row p and pair i: one thread per entry.
__global__ __launch_bounds__(256) void rope_table_kernel(float *cos_out, float *sin_out, int rows, RopeTheta th) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)rows * (kRope / 2)) return;
  const int i = (int)(idx % (kRope / 2));
  const double a = (double)(idx / (kRope / 2)) * th.t[i];
  cos_out[idx] = (float)cos(a);
  sin_out[idx] = (float)sin(a);
}

// --------------------------------------------------------------------- get

template <int FMT>
__global__ __launch_bounds__(256) void get_kernel(const void *ckv, const void *kpe,
                                                  const uint16_t *scale, const uint16_t *zero,
                                                  const int32_t *seq_lens, Paging pg, int B, int cap,
                                                  float *ckv_out, float *kpe_out) {
  const int64_t total = (int64_t)B * cap * kRow;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(idx % kRow);
    const int64_t orow = idx / kRow;  // output row [B][cap]
    const int b = (int)(orow / cap), t = (int)(orow % cap);
    float v = 0.0f;
    const int64_t row = t < seq_lens[b] ? plane_row(pg, b, cap, t) : -1;  // plane row
    if (row >= 0) {
      constexpr int NS = n_scales(FMT);
      if (c < kLatent) {
        const int64_t lrow = lat_row_of(pg, row, b, cap, t);
        const uint8_t *lat = (const uint8_t *)ckv;
        if (lat_fmt(FMT) == MLA_FMT_BF16) {
          v = bf16_bits_to_f32(*(const uint16_t *)(lat + lat_off(lrow, c / 8, kLatent * 2) + (c % 8) * 2));
        } else if (lat_fmt(FMT) == MLA_FMT_INT8) {
          v = (float)*(const int8_t *)(lat + lat_off(lrow, c / 16, kLatent) + c % 16) *
              f16_bits_to_f32(scale[row * NS + c / kGroupL]);
        } else {
          const uint8_t byte = lat[lat_off(lrow, c / 32, kLatent / 2) + (c % 32) / 2];
          const float q = (float)((c & 1) ? (byte >> 4) : (byte & 15));
          v = fmaf(q, f16_bits_to_f32(scale[row * NS + c / kGroupL]),
                   f16_bits_to_f32(zero[row * kNGroupL + c / kGroupL]));
        }
      } else {
        const int d = c - kLatent;
        if (kpe_fmt(FMT) == kKpeBf16) {
          v = bf16_bits_to_f32(((const uint16_t *)kpe)[row * kRope + d]);
        } else if (kpe_fmt(FMT) == kKpeI8) {
          v = (float)((const int8_t *)kpe)[row * kRope + d] *
              f16_bits_to_f32(scale[row * NS + kNGroupL + d / kGroupR]);
        } else {
          const uint8_t byte = ((const uint8_t *)kpe)[row * (kRope / 2) + d / 2];
          const float q = (float)((int)((d & 1) ? (byte >> 4) : (byte & 15)) - 8);
          v = q * f16_bits_to_f32(scale[row * NS + kNGroupL + d / kGroupR]);
        }
      }
    }
    if (c < kLatent) {
      if (ckv_out) ckv_out[orow * kLatent + c] = v;
    } else if (kpe_out) {
      kpe_out[orow * kRope + (c - kLatent)] = v;
    }
  }
}

// -------------------------------------------------------------- host side

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int check_cache(const mla_cache *c) {
  if (!c) return MLA_ERR_INVALID_ARG;
  if (c->format < MLA_FMT_BF16 || c->format > MLA_FMT_INT4_KINT4) return MLA_ERR_INVALID_ARG;
  if (c->num_layers < 1 || c->batch < 1 || c->capacity < 1) return MLA_ERR_INVALID_ARG;
  if (c->kv_lora_rank != kLatent || c->rope_dim != kRope || c->group_latent != kGroupL ||
      c->group_rope != kGroupR)
    return MLA_ERR_UNSUPPORTED;
  // The kernels address one sequence's rows of a plane through a buffer
  // descriptor whose byte count is a 32-bit number, with kOffNone as an offset
  // past every descriptor: a sequence's plane must stay below 2^30 bytes.
  if ((int64_t)lat_stride(c->capacity) * ckv_bytes(c->format) > kMaxSeqPlaneBytes ||
      (int64_t)c->capacity * (kpe_bytes(c->format) > 2 * kNScale ? kpe_bytes(c->format) : 2 * kNScale) >
          kMaxSeqPlaneBytes)
    return MLA_ERR_UNSUPPORTED;
  if (!c->ckv || !c->kpe || !c->seq_lens) return MLA_ERR_INVALID_ARG;
  if (!aligned16(c->ckv) || !aligned16(c->kpe) || ((uintptr_t)c->seq_lens & 3u)) return MLA_ERR_INVALID_ARG;
  const bool quant = c->format != MLA_FMT_BF16;
  if (quant != (c->scale != nullptr)) return MLA_ERR_INVALID_ARG;
  if (has_zero(c->format) != (c->zero != nullptr)) return MLA_ERR_INVALID_ARG;
  if (c->scale && !aligned16(c->scale)) return MLA_ERR_INVALID_ARG;
  if (c->zero && !aligned16(c->zero)) return MLA_ERR_INVALID_ARG;
  if (c->page_size < 0) return MLA_ERR_INVALID_ARG;
  if (c->page_size == 0) return c->block_table ? MLA_ERR_INVALID_ARG : MLA_OK;
  // paged: pages are a power of two of at least 32 tokens (whole 32-token
  // tiles) and tile the capacity
  if (c->page_size < 32 || (c->page_size & (c->page_size - 1)) || c->capacity % c->page_size)
    return MLA_ERR_INVALID_ARG;
  if (c->num_pages < 1 || !c->block_table || ((uintptr_t)c->block_table & 3u)) return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

Paging paging_of(const mla_cache *c) {
  Paging p;
  p.table = c->page_size ? c->block_table : nullptr;
  p.size = c->page_size;
  p.shift = 0;
  while (c->page_size && (1 << p.shift) < c->page_size) ++p.shift;
  p.max_pages = c->page_size ? c->capacity / c->page_size : 0;
  p.num_pages = c->page_size ? c->num_pages : 0;
  p.batch = c->batch;
  p.layer_rows = (int64_t)p.num_pages * c->page_size;
  return p;
}

int64_t ckv_row_bytes(int fmt) { return ckv_bytes(fmt); }
int64_t kpe_row_bytes(int fmt) { return kpe_bytes(fmt); }

struct LayerPlanes {
  void *ckv, *kpe;
  uint16_t *scale, *zero;
  int32_t *seq_lens;
};

LayerPlanes layer_planes(const mla_cache *c, int layer) {
  // rows of one layer: batch * capacity contiguous, or its pool of pages; the
  // latent plane's sequences are lat_stride(capacity) rows apart
  const int64_t rows = (int64_t)layer * (c->page_size ? (int64_t)c->num_pages * c->page_size
                                                      : (int64_t)c->batch * c->capacity);
  const int64_t lrows = (int64_t)layer * (c->page_size ? (int64_t)c->num_pages * c->page_size
                                                       : (int64_t)c->batch * lat_stride(c->capacity));
  LayerPlanes p;
  p.ckv = (uint8_t *)c->ckv + lrows * ckv_row_bytes(c->format);
  p.kpe = (uint8_t *)c->kpe + rows * kpe_row_bytes(c->format);
  p.scale = c->scale ? c->scale + rows * n_scales(c->format) : nullptr;
  p.zero = c->zero ? c->zero + rows * kNGroupL : nullptr;
  p.seq_lens = c->seq_lens + (int64_t)layer * c->batch;
  return p;
}

bool heads_ok(int heads) { return heads == 16 || heads == 32 || heads == 64 || heads == 128; }

// Calls f(std::integral_constant<int, FMT>) for the cache's (validated) format.
template <typename F> void with_format(int fmt, F &&f) {
  switch (fmt) {
    case MLA_FMT_INT8: f(std::integral_constant<int, MLA_FMT_INT8>{}); break;
    case MLA_FMT_INT4: f(std::integral_constant<int, MLA_FMT_INT4>{}); break;
    case MLA_FMT_INT8_KBF16: f(std::integral_constant<int, MLA_FMT_INT8_KBF16>{}); break;
    case MLA_FMT_INT4_KINT4: f(std::integral_constant<int, MLA_FMT_INT4_KINT4>{}); break;
    default: f(std::integral_constant<int, MLA_FMT_BF16>{}); break;
  }
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct WsLayout {
  size_t qa, m, l, acc, tab, total;
};

// The workspace of a decode over `layers` layers of a batch (S = batch x
// layers sequences): the absorbed queries of every sequence; the partial
// records, one per (range, sequence) pair of the balanced plan, at most W + S
// with W = nsplit * batch ranges, each with rows for all H heads; then the
// per-sequence record table.
WsLayout ws_layout(int batch, int layers, int H, int nsplit) {
  const size_t S = (size_t)batch * layers;
  const size_t recs = (size_t)batch * nsplit + S;
  WsLayout w;
  size_t off = 0;
  w.qa = off;
  off = align256(off + S * H * kQRec * 2);
  w.m = off;
  off = align256(off + recs * H * 4);
  w.l = off;
  off = align256(off + recs * H * 4);
  w.acc = off;
  off = align256(off + recs * H * kLatent * 4);
  w.tab = off;
  off = align256(off + S * 2 * 4);
  w.total = off;
  return w;
}

// More than 16 heads: the 32-head kernel for the formats without zero-points;
// INT4 latents run the 16-head kernel per slice (the 32-head kernel's INT4
// value product needs registers for only one wave per SIMD, and was slower).
bool use_wide(int fmt, int heads) { return heads > 16 && !has_zero(fmt); }

int auto_splits(const mla_cache *c, int heads, int layers, int *out) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return MLA_ERR_HIP;
  if (cus < 1) cus = 1;
  // Balanced plan: nsplit * batch ranges of equal work (times heads / 32 head
  // slices for more than 16 heads), as many workgroups as are resident at
  // once (three per CU for 16 heads, two for the 32-head workgroups), and at
  // least kAutoMinTiles tiles per range when every sequence is full.
  int64_t ns = use_wide(c->format, heads) ? (int64_t)kWideWgPerCu * cus / ((int64_t)c->batch * (heads / kWideHeads))
                               : (int64_t)kWgPerCu * cus / ((int64_t)c->batch * (heads / 16));
  // Short caches (under kAutoShortRuns * kAutoMinTiles tiles) may still take
  // kAutoShortRuns runs of a tile or more: there the launch is latency-bound
  // and the few records merge at once.
  const int64_t cap_tiles = ((int64_t)c->capacity * layers + kT16 - 1) / kT16;
  int64_t by_len = (cap_tiles + kAutoMinTiles - 1) / kAutoMinTiles;
  if (by_len < kAutoShortRuns) by_len = cap_tiles < kAutoShortRuns ? cap_tiles : kAutoShortRuns;
  if (ns > by_len) ns = by_len;
  if (ns < 1) ns = 1;
  if (ns > kMaxSplits) ns = kMaxSplits;
  *out = (int)ns;
  return MLA_OK;
}


// Head slices of the partial kernel: 16 heads per workgroup (split16_kernel),
// or 32 for more than 16 heads when the 32-head kernel is built in.
int head_slices(int fmt, int heads) { return use_wide(fmt, heads) ? heads / kWideHeads : heads / 16; }

template <int FMT>
hipError_t launch_split_fmt(const SplitArgs &a, dim3 grid, hipStream_t st) {
  const bool paged = a.pg.size != 0;
  if constexpr (!has_zero(FMT)) {
    if (use_wide(FMT, a.H)) {
      if (paged) hipLaunchKernelGGL((wide_kernel<FMT, true>), grid, dim3(kThreads), 0, st, a);
      else hipLaunchKernelGGL((wide_kernel<FMT, false>), grid, dim3(kThreads), 0, st, a);
      return hipGetLastError();
    }
  }
  if (a.H > 16) {
    if (paged) hipLaunchKernelGGL((split16_kernel<FMT, true, true>), grid, dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL((split16_kernel<FMT, false, true>), grid, dim3(kThreads), 0, st, a);
  } else {
    if (paged) hipLaunchKernelGGL((split16_kernel<FMT, true, false>), grid, dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL((split16_kernel<FMT, false, false>), grid, dim3(kThreads), 0, st, a);
  }
  return hipGetLastError();
}

struct DecodePlan {
  int ns;      // ranges per batch entry (W = ns * batch)
  int layers;  // layers of the call
  WsLayout wl;
};

bool layers_ok(const mla_cache *c, int layer0, int layers) {
  return layer0 >= 0 && layers >= 1 && (int64_t)layer0 + layers <= c->num_layers;
}

// Validation shared by the decode entry points: cache, layers, heads, split
// count and workspace. Fills the plan (split count, workspace layout) on success.
int plan_decode(const mla_cache *cache, int layers, int heads, int num_splits, const void *workspace,
                size_t workspace_bytes, DecodePlan *plan) {
  int st = check_cache(cache);
  if (st != MLA_OK) return st;
  if (layers < 1 || layers > cache->num_layers) return MLA_ERR_INVALID_ARG;
  if (!heads_ok(heads)) return MLA_ERR_UNSUPPORTED;
  if (num_splits < 0 || num_splits > kMaxSplits) return MLA_ERR_INVALID_ARG;
  int ns = num_splits;
  if (ns == 0) {
    st = auto_splits(cache, heads, layers, &ns);
    if (st != MLA_OK) return st;
  }
  // ranges x head slices, rounded up to whole windows of 8 ranges; the plan
  // counts the tiles of all the call's sequences in 32-bit integers
  const int64_t seqs = (int64_t)cache->batch * layers;
  if (((int64_t)ns * cache->batch + 7) / 8 * 8 * head_slices(cache->format, heads) > kMaxGrid)
    return MLA_ERR_UNSUPPORTED;
  if (seqs * ((cache->capacity + kT16 - 1) / kT16) > kMaxGrid) return MLA_ERR_UNSUPPORTED;
  plan->ns = ns;
  plan->layers = layers;
  plan->wl = ws_layout(cache->batch, layers, heads, ns);
  if (!workspace || workspace_bytes < plan->wl.total || ((uintptr_t)workspace & 255u))
    return MLA_ERR_WORKSPACE;
  return MLA_OK;
}

int check_absorb_args(const void *q_nope, const void *q_pe, const void *w_uk, float softmax_scale) {
  if (!q_nope || !q_pe || !w_uk) return MLA_ERR_INVALID_ARG;
  if (!aligned16(q_nope) || !aligned16(q_pe) || !aligned16(w_uk)) return MLA_ERR_INVALID_ARG;
  if (!(softmax_scale == softmax_scale) || isinf(softmax_scale)) return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

int check_combine_args(const void *w_uv, const float *out) {
  if (!w_uv || !out || !aligned16(w_uv) || !aligned16(out)) return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

int run_absorb(const mla_cache *cache, const DecodePlan &pl, const void *q_nope, const void *q_pe,
               const void *w_uk, int heads, float softmax_scale, void *workspace, hipStream_t s) {
  const int B = cache->batch;
  const int nbz = (B + kAbsorbBT - 1) / kAbsorbBT;
  _Float16 *qa = (_Float16 *)((uint8_t *)workspace + pl.wl.qa);
  hipLaunchKernelGGL(absorb_kernel, dim3(heads, kLatent / kAbsorbCB, nbz * pl.layers), dim3(256), 0, s,
                     (const uint16_t *)q_nope, (const uint16_t *)q_pe, (const uint16_t *)w_uk, B, heads,
                     softmax_scale * kLog2e, qa, nbz);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int run_partial(const mla_cache *cache, const DecodePlan &pl, int layer0, int heads, void *workspace,
                hipStream_t s) {
  const LayerPlanes p = layer_planes(cache, layer0);
  uint8_t *ws = (uint8_t *)workspace;
  SplitArgs a;
  a.ckv = p.ckv;
  a.kpe = p.kpe;
  a.scale = p.scale;
  a.zero = p.zero;
  a.seq_lens = p.seq_lens;
  a.qa = (const _Float16 *)(ws + pl.wl.qa);
  a.ws_m = (float *)(ws + pl.wl.m);
  a.ws_l = (float *)(ws + pl.wl.l);
  a.ws_acc = (float *)(ws + pl.wl.acc);
  a.B = cache->batch * pl.layers;  // the sequences of every layer, layer after layer
  a.H = heads;
  a.cap = cache->capacity;
  a.pg = paging_of(cache);
  a.rec_tab = (int32_t *)(ws + pl.wl.tab);
  // the balanced plan's nsplit * batch ranges, each as head_slices workgroups,
  // rounded up to whole windows of 8 ranges (see split16_kernel)
  a.W = pl.ns * cache->batch;
  const dim3 grid((unsigned)(((int64_t)a.W + 7) / 8 * 8 * head_slices(cache->format, heads)));
  hipError_t e = hipSuccess;
  with_format(cache->format, [&](auto f) { e = launch_split_fmt<decltype(f)::value>(a, grid, s); });
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int run_combine(const mla_cache *cache, const DecodePlan &pl, const void *w_uv, int heads,
                void *workspace, float *out, hipStream_t s) {
  const int B = cache->batch;
  uint8_t *ws = (uint8_t *)workspace;
  const int64_t big = (int64_t)heads * ((B + 15) / 16) * pl.layers;
  if (kCombineMfma && big >= kCombBigGrid)
    hipLaunchKernelGGL(combine_kernel<16>, dim3(heads, (B + 15) / 16, pl.layers), dim3(256), 0, s,
                       (const float *)(ws + pl.wl.m), (const float *)(ws + pl.wl.l), (const float *)(ws + pl.wl.acc),
                       (const int32_t *)(ws + pl.wl.tab), (const uint16_t *)w_uv, B, heads, out);
  else if ((int64_t)heads * B * pl.layers <= kReduce1MaxBlocks)
    hipLaunchKernelGGL(reduce1_kernel, dim3(heads, B, pl.layers), dim3(kReduceThreads), 0, s,
                       (const float *)(ws + pl.wl.m), (const float *)(ws + pl.wl.l), (const float *)(ws + pl.wl.acc),
                       (const int32_t *)(ws + pl.wl.tab), (const uint16_t *)w_uv, B, heads, out);
  else
    hipLaunchKernelGGL(reduce_kernel, dim3(heads, (B + kReduceBT - 1) / kReduceBT, pl.layers),
                       dim3(kReduceThreads), 0, s, (const float *)(ws + pl.wl.m), (const float *)(ws + pl.wl.l),
                       (const float *)(ws + pl.wl.acc), (const int32_t *)(ws + pl.wl.tab),
                       (const uint16_t *)w_uv, B, heads, out);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

// Decode of layers [layer0, layer0 + layers): three launches.
int decode_layers(const mla_cache *cache, int32_t layer0, int32_t layers, const void *q_nope, const void *q_pe,
                  const void *w_uk, const void *w_uv, int32_t heads, float softmax_scale, int32_t num_splits,
                  void *workspace, size_t workspace_bytes, float *out, hipStream_t s) {
  int st = check_cache(cache);
  if (st != MLA_OK) return st;
  if (!layers_ok(cache, layer0, layers)) return MLA_ERR_INVALID_ARG;
  if (!heads_ok(heads)) return MLA_ERR_UNSUPPORTED;
  if ((st = check_absorb_args(q_nope, q_pe, w_uk, softmax_scale)) != MLA_OK) return st;
  if ((st = check_combine_args(w_uv, out)) != MLA_OK) return st;
  DecodePlan pl;
  if ((st = plan_decode(cache, layers, heads, num_splits, workspace, workspace_bytes, &pl)) != MLA_OK) return st;
  if ((st = run_absorb(cache, pl, q_nope, q_pe, w_uk, heads, softmax_scale, workspace, s)) != MLA_OK) return st;
  if ((st = run_partial(cache, pl, layer0, heads, workspace, s)) != MLA_OK) return st;
  return run_combine(cache, pl, w_uv, heads, workspace, out, s);
}

// Validation and first launch of the fused decode step of layers
// [layer0, layer0 + layers) (store the new tokens, turn and absorb the
// queries). Fills the plan on success.
int step_begin(const mla_cache *cache, int32_t layer0, int32_t layers, const void *ckv_new, const void *kpe_new,
               const void *q_nope, const void *q_pe, const float *rope_cos, const float *rope_sin,
               int32_t rope_rows, const void *w_uk, int32_t heads, float softmax_scale, int32_t num_splits,
               void *workspace, size_t workspace_bytes, hipStream_t s, DecodePlan *pl) {
  int st = check_cache(cache);
  if (st != MLA_OK) return st;
  if (!layers_ok(cache, layer0, layers)) return MLA_ERR_INVALID_ARG;
  if (!ckv_new || !kpe_new || !aligned16(ckv_new) || !aligned16(kpe_new)) return MLA_ERR_INVALID_ARG;
  if ((rope_cos == nullptr) != (rope_sin == nullptr)) return MLA_ERR_INVALID_ARG;
  if (rope_cos && (((uintptr_t)rope_cos & 3u) || ((uintptr_t)rope_sin & 3u) ||
                   (int64_t)rope_rows < (int64_t)cache->capacity + 1))
    return MLA_ERR_INVALID_ARG;
  if (!heads_ok(heads)) return MLA_ERR_UNSUPPORTED;
  if ((st = check_absorb_args(q_nope, q_pe, w_uk, softmax_scale)) != MLA_OK) return st;
  if ((st = plan_decode(cache, layers, heads, num_splits, workspace, workspace_bytes, pl)) != MLA_OK) return st;
  const int64_t n_absorb =
      (int64_t)heads * (kLatent / kAbsorbCB) * ((cache->batch + kAbsorbBT - 1) / kAbsorbBT);
  if ((n_absorb + cache->batch) * layers > kMaxGrid) return MLA_ERR_UNSUPPORTED;
  const LayerPlanes p = layer_planes(cache, layer0);
  StepArgs sa;
  sa.ap.ckv = p.ckv;
  sa.ap.kpe = p.kpe;
  sa.ap.scale = p.scale;
  sa.ap.zero = p.zero;
  sa.ap.seq_lens = p.seq_lens;
  sa.ap.ckv_new = (const uint16_t *)ckv_new;
  sa.ap.kpe_new = (const uint16_t *)kpe_new;
  sa.ap.n_new = nullptr;
  sa.ap.rope_cos = rope_cos;
  sa.ap.rope_sin = rope_sin;
  sa.ap.pg = paging_of(cache);
  sa.ap.B = cache->batch * layers;
  sa.ap.T = 1;
  sa.ap.cap = cache->capacity;
  sa.q_nope = (const uint16_t *)q_nope;
  sa.q_pe = (const uint16_t *)q_pe;
  sa.w_uk = (const uint16_t *)w_uk;
  sa.qa = (_Float16 *)((uint8_t *)workspace + pl->wl.qa);
  sa.qs = softmax_scale * kLog2e;
  sa.H = heads;
  sa.n_absorb = (int)n_absorb;
  sa.batch = cache->batch;
  sa.layers = layers;
  const dim3 g((unsigned)((n_absorb + cache->batch) * layers)), bl(256);
  with_format(cache->format, [&](auto f) { hipLaunchKernelGGL(step_kernel<decltype(f)::value>, g, bl, 0, s, sa); });
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int step_layers(const mla_cache *cache, int32_t layer0, int32_t layers, const void *ckv_new, const void *kpe_new,
                const void *q_nope, const void *q_pe, const float *rope_cos, const float *rope_sin,
                int32_t rope_rows, const void *w_uk, const void *w_uv, int32_t heads, float softmax_scale,
                int32_t num_splits, void *workspace, size_t workspace_bytes, float *out, hipStream_t s) {
  // everything the later launches need is validated before the first one
  if (check_combine_args(w_uv, out) != MLA_OK) return MLA_ERR_INVALID_ARG;
  DecodePlan pl;
  int st = step_begin(cache, layer0, layers, ckv_new, kpe_new, q_nope, q_pe, rope_cos, rope_sin, rope_rows, w_uk,
                      heads, softmax_scale, num_splits, workspace, workspace_bytes, s, &pl);
  if (st != MLA_OK) return st;
  if ((st = run_partial(cache, pl, layer0, heads, workspace, s)) != MLA_OK) return st;
  return run_combine(cache, pl, w_uv, heads, workspace, out, s);
}

// ------------------------------------------------ the no-allocation variant

// The workspace of mla_decode_attn_static: a file-scope device array, one
// copy per GPU the library runs on, kept until the process ends. Host code
// never passes the array's name to a kernel (in host code it is a stand-in,
// not a device address): it passes the address hipGetSymbolAddress returns
// for the current device, looked up once per device.
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
static_assert(kStaticScratchBytes == (size_t)MLA_STATIC_SCRATCH_BYTES, "header and library agree");
__device__ __attribute__((aligned(256))) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (null on a HIP error).
void *static_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

// ================================================================== C ABI

extern "C" int mla_decode_attn_static(const mla_cache *cache, int32_t layer, const void *q_nope, const void *q_pe,
                                      const void *w_uk, const void *w_uv, int32_t heads, float softmax_scale,
                                      int32_t num_splits, float *out, void *hip_stream) {
  // every argument first, the size limit before any HIP call
  int st = check_cache(cache);
  if (st != MLA_OK) return st;
  if (layer < 0 || layer >= cache->num_layers) return MLA_ERR_INVALID_ARG;
  if (!heads_ok(heads)) return MLA_ERR_UNSUPPORTED;
  if ((st = check_absorb_args(q_nope, q_pe, w_uk, softmax_scale)) != MLA_OK) return st;
  if ((st = check_combine_args(w_uv, out)) != MLA_OK) return st;
  if (num_splits < 0 || num_splits > kMaxSplits) return MLA_ERR_INVALID_ARG;
  int ns = num_splits;
  if (ns == 0 && (st = auto_splits(cache, heads, 1, &ns)) != MLA_OK) return st;
  if (ws_layout(cache->batch, 1, heads, ns).total > kStaticScratchBytes) return MLA_ERR_WORKSPACE;
  void *ws = static_scratch();
  if (!ws) return MLA_ERR_HIP;
  return decode_layers(cache, layer, 1, q_nope, q_pe, w_uk, w_uv, heads, softmax_scale, ns, ws,
                       kStaticScratchBytes, out, (hipStream_t)hip_stream);
}

extern "C" const char *mla_status_str(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported dimension or head count";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small";
    case MLA_ERR_CAPACITY: return "append exceeds cache capacity";
    case MLA_ERR_HIP: return "HIP runtime or launch error";
    default: return "unknown status";
  }
}

extern "C" int mla_cache_append(const mla_cache *cache, int32_t layer, const void *ckv_new,
                                const void *kpe_new, int32_t t_new, const int32_t *n_new,
                                void *hip_stream) {
  int st = check_cache(cache);
  if (st != MLA_OK) return st;
  if (layer < 0 || layer >= cache->num_layers || t_new < 0) return MLA_ERR_INVALID_ARG;
  if (t_new == 0) return MLA_OK;
  if (!ckv_new || !kpe_new || !aligned16(ckv_new) || !aligned16(kpe_new)) return MLA_ERR_INVALID_ARG;
  if (n_new && ((uintptr_t)n_new & 3u)) return MLA_ERR_INVALID_ARG;
  const LayerPlanes p = layer_planes(cache, layer);
  AppendArgs a;
  a.ckv = p.ckv;
  a.kpe = p.kpe;
  a.scale = p.scale;
  a.zero = p.zero;
  a.seq_lens = p.seq_lens;
  a.ckv_new = (const uint16_t *)ckv_new;
  a.kpe_new = (const uint16_t *)kpe_new;
  a.n_new = n_new;
  a.rope_cos = a.rope_sin = nullptr;
  a.pg = paging_of(cache);
  a.B = cache->batch;
  a.T = t_new;
  a.cap = cache->capacity;
  hipStream_t s = (hipStream_t)hip_stream;
  if (t_new <= kStepAppendMaxT) {  // a decode step: one launch, lengths advanced in-kernel
    const dim3 g((unsigned)a.B), bl(128);
    with_format(cache->format, [&](auto f) {
      hipLaunchKernelGGL(append_step_kernel<decltype(f)::value>, g, bl, 0, s, a);
    });
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
  }
  const int64_t blocks = ((int64_t)a.T * kNScale + 255) / 256;
  const unsigned rows = (unsigned)(a.B < 65535 ? a.B : 65535);  // grid rows (sequences strided over them)
  with_format(cache->format, [&](auto f) {
    hipLaunchKernelGGL(append_kernel<decltype(f)::value>, dim3((unsigned)blocks, rows), dim3(256), 0, s, a);
  });
  if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP;
  hipLaunchKernelGGL(seqlen_kernel, dim3((a.B + 255) / 256), dim3(256), 0, s, p.seq_lens, n_new, a.B,
                     a.T, a.cap);
  if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}

extern "C" int mla_decode_auto_splits(const mla_cache *cache, int32_t heads, int32_t *num_splits) {
  return mla_decode_auto_splits_layers(cache, 1, heads, num_splits);
}

extern "C" int mla_decode_auto_splits_layers(const mla_cache *cache, int32_t layer_count, int32_t heads,
                                             int32_t *num_splits) {
  int st = check_cache(cache);
  if (st != MLA_OK) return st;
  if (!num_splits || layer_count < 1 || layer_count > cache->num_layers) return MLA_ERR_INVALID_ARG;
  if (!heads_ok(heads)) return MLA_ERR_UNSUPPORTED;
  return auto_splits(cache, heads, layer_count, num_splits);
}

extern "C" int mla_decode_workspace_bytes(const mla_cache *cache, int32_t heads, int32_t num_splits,
                                          size_t *bytes) {
  return mla_decode_workspace_bytes_layers(cache, 1, heads, num_splits, bytes);
}

extern "C" int mla_decode_workspace_bytes_layers(const mla_cache *cache, int32_t layer_count, int32_t heads,
                                                 int32_t num_splits, size_t *bytes) {
  int st = check_cache(cache);
  if (st != MLA_OK) return st;
  if (!bytes || layer_count < 1 || layer_count > cache->num_layers) return MLA_ERR_INVALID_ARG;
  if (!heads_ok(heads)) return MLA_ERR_UNSUPPORTED;
  if (num_splits < 0 || num_splits > kMaxSplits) return MLA_ERR_INVALID_ARG;
  int ns = num_splits;
  if (ns == 0) {
    st = auto_splits(cache, heads, layer_count, &ns);
    if (st != MLA_OK) return st;
  }
  *bytes = ws_layout(cache->batch, layer_count, heads, ns).total;
  return MLA_OK;
}

extern "C" int mla_decode_attn(const mla_cache *cache, int32_t layer, const void *q_nope,
                               const void *q_pe, const void *w_uk, const void *w_uv, int32_t heads,
                               float softmax_scale, int32_t num_splits, void *workspace,
                               size_t workspace_bytes, float *out, void *hip_stream) {
  return decode_layers(cache, layer, 1, q_nope, q_pe, w_uk, w_uv, heads, softmax_scale, num_splits, workspace,
                       workspace_bytes, out, (hipStream_t)hip_stream);
}

extern "C" int mla_decode_attn_layers(const mla_cache *cache, int32_t layer0, int32_t layer_count,
                                      const void *q_nope, const void *q_pe, const void *w_uk, const void *w_uv,
                                      int32_t heads, float softmax_scale, int32_t num_splits, void *workspace,
                                      size_t workspace_bytes, float *out, void *hip_stream) {
  return decode_layers(cache, layer0, layer_count, q_nope, q_pe, w_uk, w_uv, heads, softmax_scale, num_splits,
                       workspace, workspace_bytes, out, (hipStream_t)hip_stream);
}

extern "C" int mla_decode_step(const mla_cache *cache, int32_t layer, const void *ckv_new,
                               const void *kpe_new, const void *q_nope, const void *q_pe,
                               const float *rope_cos, const float *rope_sin, int32_t rope_rows,
                               const void *w_uk, const void *w_uv, int32_t heads, float softmax_scale,
                               int32_t num_splits, void *workspace, size_t workspace_bytes, float *out,
                               void *hip_stream) {
  return step_layers(cache, layer, 1, ckv_new, kpe_new, q_nope, q_pe, rope_cos, rope_sin, rope_rows, w_uk, w_uv,
                     heads, softmax_scale, num_splits, workspace, workspace_bytes, out, (hipStream_t)hip_stream);
}

extern "C" int mla_decode_step_layers(const mla_cache *cache, int32_t layer0, int32_t layer_count,
                                      const void *ckv_new, const void *kpe_new, const void *q_nope,
                                      const void *q_pe, const float *rope_cos, const float *rope_sin,
                                      int32_t rope_rows, const void *w_uk, const void *w_uv, int32_t heads,
                                      float softmax_scale, int32_t num_splits, void *workspace,
                                      size_t workspace_bytes, float *out, void *hip_stream) {
  return step_layers(cache, layer0, layer_count, ckv_new, kpe_new, q_nope, q_pe, rope_cos, rope_sin, rope_rows,
                     w_uk, w_uv, heads, softmax_scale, num_splits, workspace, workspace_bytes, out,
                     (hipStream_t)hip_stream);
}

extern "C" int mla_decode_step_begin_layers(const mla_cache *cache, int32_t layer0, int32_t layer_count,
                                            const void *ckv_new, const void *kpe_new, const void *q_nope,
                                            const void *q_pe, const float *rope_cos, const float *rope_sin,
                                            int32_t rope_rows, const void *w_uk, int32_t heads,
                                            float softmax_scale, int32_t num_splits, void *workspace,
                                            size_t workspace_bytes, void *hip_stream) {
  DecodePlan pl;
  return step_begin(cache, layer0, layer_count, ckv_new, kpe_new, q_nope, q_pe, rope_cos, rope_sin, rope_rows,
                    w_uk, heads, softmax_scale, num_splits, workspace, workspace_bytes, (hipStream_t)hip_stream,
                    &pl);
}

extern "C" int mla_decode_absorb_layers(const mla_cache *cache, int32_t layer_count, const void *q_nope,
                                        const void *q_pe, const void *w_uk, int32_t heads, float softmax_scale,
                                        int32_t num_splits, void *workspace, size_t workspace_bytes,
                                        void *hip_stream) {
  int st = check_cache(cache);
  if (st != MLA_OK) return st;
  if (!heads_ok(heads)) return MLA_ERR_UNSUPPORTED;
  if ((st = check_absorb_args(q_nope, q_pe, w_uk, softmax_scale)) != MLA_OK) return st;
  DecodePlan pl;
  if ((st = plan_decode(cache, layer_count, heads, num_splits, workspace, workspace_bytes, &pl)) != MLA_OK)
    return st;
  return run_absorb(cache, pl, q_nope, q_pe, w_uk, heads, softmax_scale, workspace, (hipStream_t)hip_stream);
}

extern "C" int mla_decode_partial_layers(const mla_cache *cache, int32_t layer0, int32_t layer_count,
                                         int32_t heads, int32_t num_splits, void *workspace,
                                         size_t workspace_bytes, void *hip_stream) {
  int st = check_cache(cache);
  if (st != MLA_OK) return st;
  if (!layers_ok(cache, layer0, layer_count)) return MLA_ERR_INVALID_ARG;
  DecodePlan pl;
  if ((st = plan_decode(cache, layer_count, heads, num_splits, workspace, workspace_bytes, &pl)) != MLA_OK)
    return st;
  return run_partial(cache, pl, layer0, heads, workspace, (hipStream_t)hip_stream);
}

extern "C" int mla_decode_combine_layers(const mla_cache *cache, int32_t layer_count, const void *w_uv,
                                         int32_t heads, int32_t num_splits, void *workspace,
                                         size_t workspace_bytes, float *out, void *hip_stream) {
  int st = check_cache(cache);
  if (st != MLA_OK) return st;
  if (!heads_ok(heads)) return MLA_ERR_UNSUPPORTED;
  if ((st = check_combine_args(w_uv, out)) != MLA_OK) return st;
  DecodePlan pl;
  if ((st = plan_decode(cache, layer_count, heads, num_splits, workspace, workspace_bytes, &pl)) != MLA_OK)
    return st;
  return run_combine(cache, pl, w_uv, heads, workspace, out, (hipStream_t)hip_stream);
}

extern "C" int mla_decode_step_begin(const mla_cache *cache, int32_t layer, const void *ckv_new,
                                     const void *kpe_new, const void *q_nope, const void *q_pe,
                                     const float *rope_cos, const float *rope_sin, int32_t rope_rows,
                                     const void *w_uk, int32_t heads, float softmax_scale,
                                     int32_t num_splits, void *workspace, size_t workspace_bytes,
                                     void *hip_stream) {
  DecodePlan pl;
  return step_begin(cache, layer, 1, ckv_new, kpe_new, q_nope, q_pe, rope_cos, rope_sin, rope_rows, w_uk, heads,
                    softmax_scale, num_splits, workspace, workspace_bytes, (hipStream_t)hip_stream, &pl);
}

extern "C" int mla_decode_absorb(const mla_cache *cache, const void *q_nope, const void *q_pe,
                                 const void *w_uk, int32_t heads, float softmax_scale,
                                 int32_t num_splits, void *workspace, size_t workspace_bytes,
                                 void *hip_stream) {
  int st = check_cache(cache);
  if (st != MLA_OK) return st;
  if (!heads_ok(heads)) return MLA_ERR_UNSUPPORTED;
  if ((st = check_absorb_args(q_nope, q_pe, w_uk, softmax_scale)) != MLA_OK) return st;
  DecodePlan pl;
  if ((st = plan_decode(cache, 1, heads, num_splits, workspace, workspace_bytes, &pl)) != MLA_OK) return st;
  return run_absorb(cache, pl, q_nope, q_pe, w_uk, heads, softmax_scale, workspace, (hipStream_t)hip_stream);
}

extern "C" int mla_decode_partial(const mla_cache *cache, int32_t layer, int32_t heads,
                                  int32_t num_splits, void *workspace, size_t workspace_bytes,
                                  void *hip_stream) {
  int st = check_cache(cache);
  if (st != MLA_OK) return st;
  if (layer < 0 || layer >= cache->num_layers) return MLA_ERR_INVALID_ARG;
  DecodePlan pl;
  if ((st = plan_decode(cache, 1, heads, num_splits, workspace, workspace_bytes, &pl)) != MLA_OK) return st;
  return run_partial(cache, pl, layer, heads, workspace, (hipStream_t)hip_stream);
}

extern "C" int mla_decode_combine(const mla_cache *cache, const void *w_uv, int32_t heads,
                                  int32_t num_splits, void *workspace, size_t workspace_bytes,
                                  float *out, void *hip_stream) {
  int st = check_cache(cache);
  if (st != MLA_OK) return st;
  if (!heads_ok(heads)) return MLA_ERR_UNSUPPORTED;
  if ((st = check_combine_args(w_uv, out)) != MLA_OK) return st;
  DecodePlan pl;
  if ((st = plan_decode(cache, 1, heads, num_splits, workspace, workspace_bytes, &pl)) != MLA_OK) return st;
  return run_combine(cache, pl, w_uv, heads, workspace, out, (hipStream_t)hip_stream);
}

// Issues 16x16x32 f16 MFMAs in 8 independent accumulator chains per wave, iters
// rounds, and writes each lane's sum of its accumulators to sink, so that no
// product is dead. A measurement aid for the matrix units' achievable rate.
__global__ __launch_bounds__(256) void mfma_rate_kernel(float *sink, int iters, float seed) {
  f32x4 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  const _Float16 u = (_Float16)(seed * (float)threadIdx.x), v = u + (_Float16)1.0f;
  const f16x8 a = {u, u, u, u, u, u, u, u}, b = {v, v, v, v, v, v, v, v};
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[c], 0, 0, 0);
  float t = 0.0f;
#pragma unroll
  for (int c = 0; c < 8; ++c) t += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = t;
}

extern "C" int mla_mfma_rate(float *sink, int32_t workgroups, int32_t iters, void *hip_stream) {
  if (!sink || ((uintptr_t)sink & 3u) || workgroups < 1 || iters < 0) return MLA_ERR_INVALID_ARG;
  hipLaunchKernelGGL(mfma_rate_kernel, dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)hip_stream, sink,
                     (int)iters, 1e-3f);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

extern "C" int mla_stream_read(const void *buf, size_t bytes, uint32_t *sink, int32_t sink_words,
                               int32_t nontemporal, void *hip_stream) {
  if (!buf || !sink || !aligned16(buf) || (bytes & 15u) || ((uintptr_t)sink & 3u) || sink_words < 1)
    return MLA_ERR_INVALID_ARG;
  if (bytes == 0) return MLA_OK;
  if (nontemporal)
    hipLaunchKernelGGL(stream_read_kernel<true>, dim3((unsigned)sink_words), dim3(256), 0, (hipStream_t)hip_stream,
                       (const u32x4 *)buf, (int64_t)(bytes / 16), sink);
  else
    hipLaunchKernelGGL(stream_read_kernel<false>, dim3((unsigned)sink_words), dim3(256), 0, (hipStream_t)hip_stream,
                       (const u32x4 *)buf, (int64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

extern "C" int mla_rope_tables(float *cos_out, float *sin_out, int32_t rows, double base, void *hip_stream) {
  if (!cos_out || !sin_out || ((uintptr_t)cos_out & 3u) || ((uintptr_t)sin_out & 3u)) return MLA_ERR_INVALID_ARG;
  if (rows < 0 || !(base > 0.0) || isinf(base)) return MLA_ERR_INVALID_ARG;
  if (rows == 0) return MLA_OK;
  RopeTheta th;
  for (int i = 0; i < kRope / 2; ++i) th.t[i] = pow(base, (-2.0 * i) / kRope);
  const int64_t blocks = ((int64_t)rows * (kRope / 2) + 255) / 256;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)hip_stream, cos_out,
                     sin_out, rows, th);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

extern "C" int mla_cache_get(const mla_cache *cache, int32_t layer, float *ckv_out, float *kpe_out,
                             void *hip_stream) {
  int st = check_cache(cache);
  if (st != MLA_OK) return st;
  if (layer < 0 || layer >= cache->num_layers) return MLA_ERR_INVALID_ARG;
  if (!ckv_out && !kpe_out) return MLA_OK;
  const LayerPlanes p = layer_planes(cache, layer);
  hipStream_t s = (hipStream_t)hip_stream;
  const int64_t total = (int64_t)cache->batch * cache->capacity * kRow;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  const dim3 g((unsigned)blocks), bl(256);
  with_format(cache->format, [&](auto f) {
    hipLaunchKernelGGL(get_kernel<decltype(f)::value>, g, bl, 0, s, p.ckv, p.kpe, p.scale, p.zero, p.seq_lens,
                       paging_of(cache), cache->batch, cache->capacity, ckv_out, kpe_out);
  });
  if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}
