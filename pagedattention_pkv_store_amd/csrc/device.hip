// Device half of libpkv: the KV scatter into the page pools and paged
// attention (decode and prefill/append) for gfx950 (CDNA4, wave64).
//
// What is computed (see include/pkv.h for the exact contracts):
//  * store_kv: each new token's K and V vectors go to the pools at their slot
//    (TileInfer.jl docs "KV cache", "Pages and block tables": store_kv!).
//  * attention: a query at position p attends to positions 0..p of its own
//    sequence, read in place through the block table ("KV Cache Management
//    and PagedAttention", "Compute attention over scattered KV", Figure 4).
//
// Kernel design (MI355X-first, not a translation of any page's design):
//  * One workgroup (4 waves) owns one (sequence, KV head, query tile, KV
//    split).  Its query rows are (query, head-in-group) pairs of one GQA
//    group, so every K/V byte a workgroup reads serves the whole group.
//  * K/V are staged 64 positions at a time in LDS, gathered page by page
//    through the block table with 16-byte coalesced loads; the next tile's
//    loads are in flight while the current tile is computed.
//  * Scores are computed transposed, S^T = K Q^T, on MFMA (bf16:
//    v_mfma_f32_16x16x32_bf16; fp32: v_mfma_f32_16x16x4_f32).  In that layout
//    each lane holds one query row and four key positions, so the running
//    max / sum of the online softmax need only in-lane work plus two
//    wavefront shuffles, and the probabilities are already in the MFMA
//    operand layout of O^T = V^T P^T (bf16: v_mfma_f32_16x16x16_bf16).  V is
//    read transposed out of LDS.
//  * Waves either split the query tile (long prefill tiles) or split the
//    staged keys (decode, few rows); partial softmax states of waves are
//    combined in LDS.  Long contexts are split across workgroups at fixed
//    logical positions and merged with log-sum-exp by a second kernel, so
//    the result depends only on the logical sequence, never on which
//    physical pages hold it.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <string>
#include <type_traits>

#include "../../include/pkv.h"
#include "status.h"

using pkv::fail;

namespace {

constexpr int kWave = 64;
constexpr int kThreads = 256;   // 4 waves
constexpr int kTileKeys = 64;   // positions staged in LDS per iteration
constexpr int kTargetWorkgroups = 2048;
constexpr int kDecodeTargetWorkgroups = 8192;
constexpr int kMinSplitKeys = 256;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));   // 16-byte load unit

__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;  // NaN stays NaN
  u += 0x7fffu + ((u >> 16) & 1u);                      // round to nearest even
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Four fp32 -> bf16 (round to nearest even, gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ i16x4 pack_bf16x4(f32x4 x) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const bf16x4 v = {static_cast<__bf16>(x[0]), static_cast<__bf16>(x[1]), static_cast<__bf16>(x[2]),
                    static_cast<__bf16>(x[3])};
  return __builtin_bit_cast(i16x4, v);
}

// Element storage: float for fp32, uint16_t bit patterns for bf16.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kQkPerMfma = 1;  // k-elements per lane per QK MFMA
};
template <> struct Elem<uint16_t> {
  static constexpr int kQkPerMfma = 8;
};

// MFMA operand fragments of the QK product, held in their operand type (no
// type-punned local arrays, which the compiler would keep in scratch).
// A lane's share of a row is kDl contiguous elements: bf16 -> kDl/8 packs of
// 8 (16x16x32 bf16 MFMA), fp32 -> kDl floats (16x16x4 f32 MFMA).
template <typename T, int kDl> struct QkFrag;
template <int kDl> struct QkFrag<uint16_t, kDl> {
  static constexpr int kN = kDl / 8;
  bf16x8 v[kN];
  __device__ __forceinline__ void load16(int c, u32x4 x) { v[c] = __builtin_bit_cast(bf16x8, x); }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < kN; ++i) v[i] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  }
};
template <int kDl> struct QkFrag<float, kDl> {
  static constexpr int kN = kDl;
  float v[kN];
  __device__ __forceinline__ void load16(int c, u32x4 x) {
    v[4 * c + 0] = __uint_as_float(x[0]);
    v[4 * c + 1] = __uint_as_float(x[1]);
    v[4 * c + 2] = __uint_as_float(x[2]);
    v[4 * c + 3] = __uint_as_float(x[3]);
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < kN; ++i) v[i] = 0.f;
  }
};

__device__ __forceinline__ f32x4 mfma_qk(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_qk(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

struct AttnArgs {
  const void* q;
  void* out;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* cu_q;  // nullptr: decode, sequence b owns query row b
  float* ws_o;          // split partials [tok][Hq][n_splits][D], or nullptr
  float* ws_ml;         // [tok][Hq][n_splits][2] = (running max, sum)
  int32_t bt_stride;
  int32_t n_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t num_pages;
  int32_t page_size;
  int32_t ps_shift;     // log2(page_size), or -1
  int32_t total_q;
  int32_t ws_tokens;    // rows of the split workspace: n_seqs * max_q_per_seq
  int32_t split_len;    // positions per KV split (multiple of kTileKeys)
  int32_t epi_rows;     // decode kernel: query rows per 16-row block (<= 16)
  int32_t n_splits;
  int32_t max_q;        // queries computed per sequence (later ones are not)
  float scale_log2;     // softmax scale * log2(e)
};

// Elements per LDS row of a staged K/V tile: a 16-byte pad staggers rows
// across banks; 512-byte rows go unpadded so two tiles fit in 64 KiB.
template <typename T, int D>
constexpr int row_stride() {
  return D + (D * static_cast<int>(sizeof(T)) >= 512 ? 0 : 16 / static_cast<int>(sizeof(T)));
}

// LDS bytes: two staged tiles (K, V), reused by the epilogue.
template <typename T, int D>
constexpr int lds_bytes() {
  constexpr int rs = row_stride<T, D>() * static_cast<int>(sizeof(T));
  constexpr int tiles = 2 * kTileKeys * rs;
  constexpr int epi = 64 * (D + 4) * 4 + 2 * 64 * 4;
  return tiles > epi ? tiles : epi;
}

// Combine the partial softmax states of NW producers per row, staged in LDS
// (eo [NW][n_rows][D + 4] un-normalised outputs, em / el [NW][n_rows] running
// max and sum, log2 domain), and write rows row0 .. row0 + n_rows - 1 of the
// (sequence, KV head) tile: normalised to `out` when the launch has one KV
// split, else as this split's partial to the workspace.
template <typename T, int D, int NW>
__device__ __forceinline__ void combine_rows(const AttnArgs& args, const float* eo, const float* em,
                                             const float* el, int n_rows, int row0, int rows_total,
                                             int q0, int g, bool final_write, int split) {
  const int kRows = n_rows;
  constexpr int kEpiStride = D + 4;
  constexpr int kQuads = D / 4;
  const int group = args.group;
  const bool split_mode = !final_write;
  for (int idx = threadIdx.x; idx < kRows * kQuads; idx += kThreads) {
    const int tr = idx / kQuads;
    const int d4 = (idx - tr * kQuads) * 4;
    const int r = row0 + tr;
    if (r >= rows_total) continue;
    const int qi = r / group;
    const int tok = q0 + qi;
    if (tok >= args.total_q) continue;
    const int h = g * group + (r - qi * group);
    float mmax = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mmax = fmaxf(mmax, em[w * kRows + tr]);
    const float mref = mmax == -INFINITY ? 0.f : mmax;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    float lsum = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float wt = fast_exp2(em[w * kRows + tr] - mref);
      lsum += wt * el[w * kRows + tr];
      acc += wt * *reinterpret_cast<const f32x4*>(eo + (w * kRows + tr) * kEpiStride + d4);
    }
    const int64_t orow = static_cast<int64_t>(tok) * args.num_q_heads + h;
    if (split_mode) {
      if (tok >= args.ws_tokens) continue;
      const int64_t slot = orow * args.n_splits + split;
      *reinterpret_cast<f32x4*>(args.ws_o + slot * D + d4) = acc;
      if (d4 == 0) {
        args.ws_ml[slot * 2] = mmax;
        args.ws_ml[slot * 2 + 1] = lsum;
      }
    } else {
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
      acc *= inv;
      if constexpr (sizeof(T) == 2) {
        uint16_t* o = static_cast<uint16_t*>(args.out) + orow * D + d4;
        uint2 packed;
        packed.x = float_to_bf16_bits(acc[0]) | (static_cast<uint32_t>(float_to_bf16_bits(acc[1])) << 16);
        packed.y = float_to_bf16_bits(acc[2]) | (static_cast<uint32_t>(float_to_bf16_bits(acc[3])) << 16);
        *reinterpret_cast<uint2*>(o) = packed;
      } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(args.out) + orow * D + d4) = acc;
      }
    }
  }
}

// RB: 16-row query blocks per workgroup; KG: waves sharing one row block,
// each taking kTileKeys / KG of the staged positions.  RB * KG == 4.
template <typename T, int D, int RB, int KG>
__global__ __launch_bounds__(kThreads) void paged_attention_kernel(AttnArgs args) {
  static_assert(RB * KG == kThreads / kWave, "4 waves");
  constexpr int kEs = sizeof(T);
  constexpr int kRowStride = row_stride<T, D>();
  constexpr int kChunksPerRow = D * kEs / 16;        // 16-byte chunks per K/V row
  constexpr int kChunks = kTileKeys * kChunksPerRow / kThreads;  // per thread per pool
  constexpr int kDl = D / 4;                         // dims per lane in the QK operands
  constexpr int kQkMfmas = kDl / Elem<T>::kQkPerMfma;
  constexpr int kKeysPerWave = kTileKeys / KG;
  constexpr int kBlocks = kKeysPerWave / 16;         // 16-position MFMA blocks per wave
  constexpr int kDimBlocks = D / 16;
  constexpr int kTileRows = 16 * RB;
  static_assert(kChunks * kThreads == kTileKeys * kChunksPerRow, "even split of the tile");

  extern __shared__ __align__(16) char smem[];
  T* ks = reinterpret_cast<T*>(smem);
  T* vs = ks + kTileKeys * kRowStride;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int rb = wave / KG;
  const int kg = wave % KG;
  const int lrow = lane & 15;   // MFMA column: query row within the 16-row block
  const int lgrp = lane >> 4;   // MFMA k/row group 0..3

  const int hkv = args.num_kv_heads;
  const int b = blockIdx.z / hkv;
  const int g = blockIdx.z % hkv;
  const int group = args.group;

  int q0, n_b;
  if (args.cu_q) {
    q0 = args.cu_q[b];
    n_b = args.cu_q[b + 1] - q0;
  } else {
    q0 = b;
    n_b = 1;
  }
  const int rows_total = n_b * group;
  const int row0 = blockIdx.y * kTileRows;
  if (row0 >= rows_total) return;
  const int seq_len = args.seq_lens[b];
  const int start = seq_len - n_b;                    // position of new query 0
  const int row_last = min(row0 + kTileRows, rows_total) - 1;
  const int kv_end = start + row_last / group + 1;    // positions this tile can see
  const int k_lo = blockIdx.x * args.split_len;
  if (k_lo >= kv_end) return;
  const int k_hi = min(k_lo + args.split_len, kv_end);

  const int ps = args.page_size;
  const int ps_shift = args.ps_shift;
  const int32_t* bt_row = args.block_tables + static_cast<int64_t>(b) * args.bt_stride;
  const T* kpool = static_cast<const T*>(args.k_pool);
  const T* vpool = static_cast<const T*>(args.v_pool);

  // ---- this lane's query row (B operand of S^T = K Q^T) ----
  const int my_row = row0 + rb * 16 + lrow;           // row within (sequence, KV head)
  const bool row_ok = my_row < rows_total;
  const int my_qpos = start + (row_ok ? my_row / group : rows_total / group);
  T qv[kDl];
  {
    const int qi = my_row / group;
    const int hh = my_row - qi * group;
    const int tok = q0 + qi;
    if (row_ok && tok < args.total_q) {
      const T* src = static_cast<const T*>(args.q) +
                     (static_cast<int64_t>(tok) * args.num_q_heads + g * group + hh) * D +
                     lgrp * kDl;
#pragma unroll
      for (int c = 0; c < kDl * kEs / 16; ++c)
        *reinterpret_cast<uint4*>(&qv[c * 16 / kEs]) = reinterpret_cast<const uint4*>(src)[c];
    } else {
#pragma unroll
      for (int c = 0; c < kDl; ++c) qv[c] = T(0);
    }
  }

  // ---- global -> register staging of one tile of K and V ----
  uint4 kreg[kChunks], vreg[kChunks];
  auto load_tile = [&](int base) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int chunk = c * kThreads + tid;
      const int row = chunk / kChunksPerRow;
      const int part = chunk - row * kChunksPerRow;
      const int pos = base + row;
      uint4 kx = make_uint4(0, 0, 0, 0), vx = make_uint4(0, 0, 0, 0);
      if (pos < k_hi) {
        const int blk = ps_shift >= 0 ? (pos >> ps_shift) : pos / ps;
        const int off = pos - blk * ps;
        if (blk < args.bt_stride) {
          const int page = bt_row[blk];
          if (static_cast<unsigned>(page) < static_cast<unsigned>(args.num_pages)) {
            const int64_t e = ((static_cast<int64_t>(page) * hkv + g) * ps + off) * D +
                              part * (16 / kEs);
            kx = *reinterpret_cast<const uint4*>(kpool + e);
            vx = *reinterpret_cast<const uint4*>(vpool + e);
          }
        }
      }
      kreg[c] = kx;
      vreg[c] = vx;
    }
  };
  auto store_tile = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int chunk = c * kThreads + tid;
      const int row = chunk / kChunksPerRow;
      const int part = chunk - row * kChunksPerRow;
      *reinterpret_cast<uint4*>(ks + row * kRowStride + part * (16 / kEs)) = kreg[c];
      *reinterpret_cast<uint4*>(vs + row * kRowStride + part * (16 / kEs)) = vreg[c];
    }
  };

  // ---- online softmax state (log2 domain) ----
  float m_run = -INFINITY;
  float l_part = 0.f;                 // this lane's share of the row sum
  f32x4 o_acc[kDimBlocks];            // O^T: lane holds row lrow, dims 4*lgrp+i of each block
#pragma unroll
  for (int d = 0; d < kDimBlocks; ++d) o_acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_tile(k_lo);
  for (int base = k_lo; base < k_hi; base += kTileKeys) {
    __syncthreads();                  // previous tile fully consumed
    store_tile();
    __syncthreads();
    if (base + kTileKeys < k_hi) load_tile(base + kTileKeys);

    const int wbase = base + kg * kKeysPerWave;
    if (wbase >= k_hi) continue;      // nothing valid for this wave in this tile

    // S^T blocks: rows = 16 key positions, columns = 16 query rows.
    f32x4 s[kBlocks];
#pragma unroll
    for (int nb = 0; nb < kBlocks; ++nb) {
      s[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
      const T* krow = ks + (kg * kKeysPerWave + nb * 16 + lrow) * kRowStride + lgrp * kDl;
#pragma unroll
      for (int kk = 0; kk < kQkMfmas; ++kk) {
        if constexpr (sizeof(T) == 2) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + kk * 8);
          const bf16x8 bq = *reinterpret_cast<const bf16x8*>(&qv[kk * 8]);
          s[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bq, s[nb], 0, 0, 0);
        } else {
          s[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(krow[kk], qv[kk], s[nb], 0, 0, 0);
        }
      }
    }

    // Mask, then the running max over this wave's positions.
    float mx = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < kBlocks; ++nb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pos = wbase + nb * 16 + lgrp * 4 + i;
        const float x = s[nb][i] * args.scale_log2;
        s[nb][i] = (pos < k_hi && pos <= my_qpos) ? x : -INFINITY;
        mx = fmaxf(mx, s[nb][i]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int nb = 0; nb < kBlocks; ++nb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[nb][i] = fast_exp2(s[nb][i] - m_use);
        psum += s[nb][i];
      }
    }
    l_part = l_part * alpha + psum;
#pragma unroll
    for (int d = 0; d < kDimBlocks; ++d) o_acc[d] *= alpha;

    // O^T += V^T P^T, 16 positions per step.
#pragma unroll
    for (int nb = 0; nb < kBlocks; ++nb) {
      const T* vblk = vs + (kg * kKeysPerWave + nb * 16 + lgrp * 4) * kRowStride + lrow;
      if constexpr (sizeof(T) == 2) {
        i16x4 pb;
#pragma unroll
        for (int i = 0; i < 4; ++i) pb[i] = static_cast<short>(float_to_bf16_bits(s[nb][i]));
#pragma unroll
        for (int d = 0; d < kDimBlocks; ++d) {
          i16x4 a;
#pragma unroll
          for (int i = 0; i < 4; ++i) a[i] = static_cast<short>(vblk[i * kRowStride + d * 16]);
          o_acc[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb, o_acc[d], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int d = 0; d < kDimBlocks; ++d)
            o_acc[d] = __builtin_amdgcn_mfma_f32_16x16x4f32(vblk[i * kRowStride + d * 16],
                                                            s[nb][i], o_acc[d], 0, 0, 0);
        }
      }
    }
  }

  // ---- epilogue: combine the KG waves of each row block in LDS ----
  float l_row = l_part;
  l_row += __shfl_xor(l_row, 16);
  l_row += __shfl_xor(l_row, 32);
  __syncthreads();                    // tiles no longer needed
  constexpr int kEpiStride = D + 4;
  float* eo = reinterpret_cast<float*>(smem);               // [KG][kTileRows][kEpiStride]
  float* em = eo + 64 * kEpiStride;                         // [KG][kTileRows]
  float* el = em + 64;
  {
    const int erow = kg * kTileRows + rb * 16 + lrow;
#pragma unroll
    for (int d = 0; d < kDimBlocks; ++d)
      *reinterpret_cast<f32x4*>(eo + erow * kEpiStride + d * 16 + lgrp * 4) = o_acc[d];
    if (lgrp == 0) {
      em[erow] = m_run;
      el[erow] = l_row;
    }
  }
  __syncthreads();

  combine_rows<T, D, KG>(args, eo, em, el, kTileRows, row0, rows_total, q0, g, args.n_splits == 1,
                         blockIdx.x);
}

// ---------------------------------------------------------------------------
// Paged decode and short appends (at most 16 * RBW query rows per sequence and
// KV head): a schedule kernel, a persistent attention kernel and a merge.
//
// Work is cut into equal items of `chunk` positions of one sequence and one KV
// head.  decode_schedule_kernel lists every (sequence, chunk) in a dense
// array and resets the work-queue counter; paged_decode_kernel runs as many
// workgroups as the chip holds at once, and each workgroup repeatedly takes
// the next item from the queue (one atomic per item), so long and short
// sequences balance across all CUs.  Inside an item, 16-position block j goes
// to wave j % 4:
//  * its K and V rows are loaded with fully coalesced 16-byte loads (each
//    instruction reads 1 KB of whole rows) and written into a 16-row slice of
//    LDS private to the wave.  The 16-byte chunks of row r are stored XOR-
//    swizzled by r, so the MFMA operand reads that follow hit distinct banks;
//  * the next block's loads are issued before the current block is computed;
//    every load is unconditional (a position past the item re-reads the
//    item's first row and is masked), so no branch forces a full wait on
//    outstanding loads;
//  * S^T = K Q^T and O^T = V^T P^T run on MFMA, the softmax max/sum on
//    wavefront shuffles.
// At the end of an item the four waves' softmax states are combined in LDS and
// written: normalised to `out` when the item spans its whole sequence, else
// as a partial that merge_chunks_kernel folds in with log-sum-exp.
// ---------------------------------------------------------------------------

// Positions of sequence b's KV range for its (single) row tile and the number
// of chunks covering it.  Shared by the schedule and merge kernels.
template <int RBW>
__device__ __forceinline__ int decode_kv_end(const AttnArgs& a, int b, int* q0_out, int* n_b_out) {
  int q0, n_b;
  if (a.cu_q) {
    q0 = a.cu_q[b];
    n_b = a.cu_q[b + 1] - q0;
  } else {
    q0 = b;
    n_b = 1;
  }
  *q0_out = q0;
  *n_b_out = n_b;
  const int rows = min(n_b * a.group, 16 * RBW);
  if (rows <= 0) return 0;
  return a.seq_lens[b] - n_b + (rows - 1) / a.group + 1;
}

struct DecodeQueue {
  int32_t n_chunks;    // items listed by the schedule kernel
  int32_t pad[63];
};

// One work item: positions [k_lo, k_hi) of sequence b (for every KV head),
// with the scalars the attention kernel needs precomputed.
struct DecodeItem {
  int32_t b, k_lo, k_hi, n_chunks;      // n_chunks of the sequence (1: final write)
  int32_t q0, start, rows_total, pad;   // first query row, position of query 0, rows
};

template <int RBW>
__global__ __launch_bounds__(kThreads) void decode_schedule_kernel(AttnArgs a, DecodeQueue* q,
                                                                   DecodeItem* items) {
  __shared__ int s_scan[kThreads];
  __shared__ int s_carry;
  const int tid = threadIdx.x;
  if (tid == 0) s_carry = 0;
  __syncthreads();
  for (int base = 0; base < a.n_seqs; base += kThreads) {
    const int b = base + tid;
    int nc = 0, kv_end = 0, q0 = 0, n_b = 0;
    if (b < a.n_seqs) {
      kv_end = decode_kv_end<RBW>(a, b, &q0, &n_b);
      if (kv_end > 0) nc = min((kv_end + a.split_len - 1) / a.split_len, a.n_splits);
    }
    s_scan[tid] = nc;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
      const int v = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += v;
      __syncthreads();
    }
    const int first = s_carry + s_scan[tid] - nc;
    const int rows = min(n_b * a.group, 16 * RBW);
    const int start = b < a.n_seqs ? a.seq_lens[b] - n_b : 0;
    for (int c = 0; c < nc; ++c) {
      DecodeItem it;
      it.b = b;
      it.k_lo = c * a.split_len;
      it.k_hi = min((c + 1) * a.split_len, kv_end);
      it.n_chunks = nc;
      it.q0 = q0;
      it.start = start;
      it.rows_total = rows;
      it.pad = 0;
      items[first + c] = it;
    }
    __syncthreads();
    if (tid == kThreads - 1) s_carry += s_scan[tid];
    __syncthreads();
  }
  if (tid == 0) q->n_chunks = s_carry;
}

// kPageMode 0: page_size a power of two >= 16 (a 16-position block lies in
// one page); 1: a power of two < 16; 2: any other page size.
#ifndef PKV_DECODE_WAVES_PER_SIMD
#define PKV_DECODE_WAVES_PER_SIMD 2
#endif
template <typename T, int D, int RBW, int kPageMode>
__global__ __launch_bounds__(kThreads, RBW == 1 ? PKV_DECODE_WAVES_PER_SIMD : 1) void paged_decode_kernel(
    AttnArgs args, const DecodeQueue* queue, const DecodeItem* __restrict__ items) {
  constexpr int kEs = sizeof(T);
  constexpr int kRowBytes = D * kEs;
  constexpr int kCpr = kRowBytes / 16;                  // 16-byte chunks per row
  constexpr int kLoads = 16 * kRowBytes / (16 * kWave); // 16-byte loads per lane per pool per block
  constexpr int kDl = D / 4;                            // dims per lane in the QK operands
  constexpr int kFragChunks = kDl * kEs / 16;           // 16-byte chunks of one lane's K fragment
  constexpr int kQkMfmas = kDl / Elem<T>::kQkPerMfma;
  constexpr int kDimBlocks = D / 16;
  constexpr int kWaves = kThreads / kWave;
  constexpr int kEpiStride = D + 4;
  // LDS rows are padded by 16 bytes: the 16-lane phases of the K operand
  // reads, the transposed V reads and the staging writes then all hit
  // distinct banks, and every address is a per-lane base plus an immediate.
  // (512-byte rows stay unpadded so four waves' slices fit in 64 KiB.)
  constexpr int kLdsRow = kRowBytes + (kRowBytes >= 512 ? 0 : 16);
  constexpr int kStageBytes = 2 * 16 * kLdsRow;         // K + V slice of one wave

  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lrow = lane & 15;
  const int lgrp = lane >> 4;
  char* kst = smem + wave * kStageBytes;
  char* vst = kst + 16 * kLdsRow;

  const int hkv = args.num_kv_heads;
  const int group = args.group;
  const int ps = args.page_size;
  const int ps_shift = args.ps_shift;
  const T* kpool = static_cast<const T*>(args.k_pool);
  const T* vpool = static_cast<const T*>(args.v_pool);
  const int n_work = queue->n_chunks * hkv;
  const int grid = gridDim.x;

  auto slot = [](int r, int c) __attribute__((always_inline)) { return r * kLdsRow + c * 16; };

  // ---- per-item scalars (wave-uniform) ----
  struct ItemS {
    int valid, b, g, k_lo, k_hi, nb, whole, q0, start, rows_total, blk_lo;
  };
  auto fetch = [&](int wi) __attribute__((always_inline)) {
    ItemS s;
    s.valid = wi < n_work;
    const int idx = s.valid ? wi / hkv : 0;
    const DecodeItem rec = items[idx];
    s.b = __builtin_amdgcn_readfirstlane(rec.b);
    s.g = s.valid ? wi % hkv : 0;
    s.k_lo = __builtin_amdgcn_readfirstlane(rec.k_lo);
    s.k_hi = __builtin_amdgcn_readfirstlane(rec.k_hi);
    s.whole = __builtin_amdgcn_readfirstlane(rec.n_chunks) == 1;
    s.q0 = __builtin_amdgcn_readfirstlane(rec.q0);
    s.start = __builtin_amdgcn_readfirstlane(rec.start);
    s.rows_total = __builtin_amdgcn_readfirstlane(rec.rows_total);
    s.nb = s.valid ? (s.k_hi - s.k_lo + 15) >> 4 : 0;
    s.blk_lo = kPageMode != 2 ? (s.k_lo >> ps_shift) : s.k_lo / ps;
    return s;
  };
  // The item's block-table slice lives in lane registers (lane i holds the
  // page of logical block blk_lo + i, -1 if out of range); items span at most
  // 64 pages.  Reading it needs no memory access once loaded.
  // Branch-free: the load always goes to an in-range entry of the table
  // (a record of an invalid item is item 0's, a real sequence).
  auto load_bt = [&](const ItemS& it) __attribute__((always_inline)) {
    const int blk = it.blk_lo + lane;
    const int last = kPageMode != 2 ? ((it.k_hi - 1) >> ps_shift) : (it.k_hi - 1) / ps;
    const int blk_c = max(0, min(blk, min(last, args.bt_stride - 1)));
    const int p = args.block_tables[static_cast<int64_t>(it.b) * args.bt_stride + blk_c];
    const bool ok = it.valid && blk <= last && blk < args.bt_stride &&
                    static_cast<unsigned>(p) < static_cast<unsigned>(args.num_pages);
    return ok ? p : -1;
  };
  // Query rows (B operand of S^T = K Q^T): row r = (query r / group, head
  // g * group + r % group); this lane holds row rb * 16 + lrow, dims
  // lgrp * kDl .. + kDl.
  auto load_q = [&](const ItemS& it, QkFrag<T, kDl> (&qv)[RBW], int (&qpos)[RBW]) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      const int r = rb * 16 + lrow;
      const int qi = r / group;
      const int tok = it.q0 + qi;
      const bool ok = it.valid && r < it.rows_total && tok < args.total_q;
      qpos[rb] = it.start + (r < it.rows_total ? qi : it.rows_total / group);
      // branch-free: rows without a query read row 0 and are zeroed
      const int tok_c = ok ? tok : 0;
      const T* src = static_cast<const T*>(args.q) +
                     (static_cast<int64_t>(tok_c) * args.num_q_heads + it.g * group + (r - qi * group)) * D +
                     lgrp * kDl;
      const unsigned keep = ok ? ~0u : 0u;
#pragma unroll
      for (int c = 0; c < kFragChunks; ++c) qv[rb].load16(c, reinterpret_cast<const u32x4*>(src)[c] & keep);
    }
  };

  // Issue the loads of block j of item `it` (clamped into the item; an
  // invalid item reads page 0 and flags everything for zeroing).  Load c of
  // a lane covers 16-byte chunk q % kCpr of row q / kCpr (q = c * 64 +
  // lane): consecutive lanes read consecutive bytes of whole rows.
  auto load_block = [&](const ItemS& it, int bt, int j, u32x4 (&kr)[kLoads], u32x4 (&vr)[kLoads],
                        uint32_t& okm) __attribute__((always_inline)) {
    j = max(0, min(j, it.nb - 1));
    const int pos0 = it.k_lo + 16 * j;
    okm = 0;
    if constexpr (kPageMode == 0) {
      const int blk = pos0 >> ps_shift;
      int page = __builtin_amdgcn_readlane(bt, blk - it.blk_lo);
      const bool page_ok = it.valid && page >= 0;
      page = page_ok ? page : 0;
      const int64_t base = ((static_cast<int64_t>(page) * hkv + it.g) * ps + (pos0 & (ps - 1))) * D;
      const T* kb = kpool + base;     // wave-uniform row-0 pointers: scalar base +
      const T* vb = vpool + base;     // a 32-bit per-lane offset per load
#pragma unroll
      for (int c = 0; c < kLoads; ++c) {
        const int q = c * kWave + lane;
        const int r = q / kCpr;
        const int chunk = q % kCpr;
        okm |= (page_ok && pos0 + r < it.k_hi) ? (1u << c) : 0u;
        const int off = r * D + chunk * (16 / kEs);
        kr[c] = *reinterpret_cast<const u32x4*>(kb + off);
        vr[c] = *reinterpret_cast<const u32x4*>(vb + off);
      }
    } else {
#pragma unroll
      for (int c = 0; c < kLoads; ++c) {
        const int q = c * kWave + lane;
        const int r = q / kCpr;
        const int chunk = q % kCpr;
        const int pos_raw = pos0 + r;
        const int pos = max(0, min(pos_raw, it.k_hi - 1));
        const int blk = kPageMode == 1 ? (pos >> ps_shift) : pos / ps;
        const int page = __shfl(bt, max(0, min(blk - it.blk_lo, kWave - 1)));
        const bool ok = it.valid && pos_raw < it.k_hi && page >= 0;
        okm |= ok ? (1u << c) : 0u;
        const int64_t e = ((static_cast<int64_t>(ok ? page : 0) * hkv + it.g) * ps + (ok ? pos - blk * ps : 0)) * D +
                          chunk * (16 / kEs);
        kr[c] = *reinterpret_cast<const u32x4*>(kpool + e);
        vr[c] = *reinterpret_cast<const u32x4*>(vpool + e);
      }
    }
  };

  // Write a block's loaded rows into the wave's LDS slice.  V rows past the
  // item or on an invalid page are zeroed (their probability is 0, but stale
  // slots may hold anything, NaN included); K rows need no zeroing, their
  // scores are masked.  Only a partial block needs the mask.
  auto stage_block = [&](const u32x4 (&kr)[kLoads], const u32x4 (&vr)[kLoads], uint32_t okm) __attribute__((always_inline)) {
    constexpr uint32_t kFull = (1u << kLoads) - 1u;
    if (__all(okm == kFull)) {
#pragma unroll
      for (int c = 0; c < kLoads; ++c) {
        const int q = c * kWave + lane;
        const int off = slot(q / kCpr, q % kCpr);
        *reinterpret_cast<u32x4*>(kst + off) = kr[c];
        *reinterpret_cast<u32x4*>(vst + off) = vr[c];
      }
    } else {
#pragma unroll
      for (int c = 0; c < kLoads; ++c) {
        const int q = c * kWave + lane;
        const int off = slot(q / kCpr, q % kCpr);
        const unsigned keep = 0u - ((okm >> c) & 1u);   // all ones or zero
        *reinterpret_cast<u32x4*>(kst + off) = kr[c];
        *reinterpret_cast<u32x4*>(vst + off) = vr[c] & keep;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // ---- online softmax state of the current item (log2 domain) ----
  float m_run[RBW], l_part[RBW];
  f32x4 o_acc[RBW][kDimBlocks];

  auto compute_block = [&](const ItemS& it, const QkFrag<T, kDl> (&qv)[RBW], const int (&qpos)[RBW],
                           int j) __attribute__((always_inline)) {
    const int pos0 = it.k_lo + 16 * j;
    // K fragment: position lrow, dims lgrp * kDl .. + kDl
    QkFrag<T, kDl> kf;
#pragma unroll
    for (int c = 0; c < kFragChunks; ++c)
      kf.load16(c, *reinterpret_cast<const u32x4*>(kst + slot(lrow, lgrp * kFragChunks + c)));
    f32x4 s[RBW];
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      s[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < kQkMfmas; ++kk) s[rb] = mfma_qk(kf.v[kk], qv[rb].v[kk], s[rb]);
    }
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pos = pos0 + lgrp * 4 + i;
        const float x = s[rb][i] * args.scale_log2;
        s[rb][i] = (pos < it.k_hi && pos <= qpos[rb]) ? x : -INFINITY;
        mx = fmaxf(mx, s[rb][i]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[rb], mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[rb] - m_use);
      m_run[rb] = m_new;
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[rb][i] = fast_exp2(s[rb][i] - m_use);
        psum += s[rb][i];
      }
      l_part[rb] = l_part[rb] * alpha + psum;
      if (__any(alpha != 1.f)) {       // the running max moved for some row
#pragma unroll
        for (int d = 0; d < kDimBlocks; ++d) o_acc[rb][d] *= alpha;
      }
    }
    // O^T += V^T P^T: the A operand is V transposed, read element-wise
    if constexpr (sizeof(T) == 2) {
      i16x4 pb[RBW];
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) pb[rb] = pack_bf16x4(s[rb]);
#pragma unroll
      for (int d = 0; d < kDimBlocks; ++d) {
        const int dim = d * 16 + lrow;
        i16x4 a;
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const short*>(vst + slot(lgrp * 4 + i, 0) + dim * 2);
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb)
          o_acc[rb][d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb[rb], o_acc[rb][d], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int d = 0; d < kDimBlocks; ++d) {
          const int dim = d * 16 + lrow;
          const float a = *reinterpret_cast<const float*>(vst + slot(lgrp * 4 + i, 0) + dim * 4);
#pragma unroll
          for (int rb = 0; rb < RBW; ++rb)
            o_acc[rb][d] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, s[rb][i], o_acc[rb][d], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // ---- the item stream of this workgroup: items w, w + grid, w + 2 grid ... ----
  int w = blockIdx.x;
  ItemS cur = fetch(w);
  if (!cur.valid) return;
  int bt_cur = load_bt(cur);
  QkFrag<T, kDl> q_cur[RBW];
  int qpos_cur[RBW];
  load_q(cur, q_cur, qpos_cur);
  ItemS nxt = fetch(w + grid);

  // Two register buffers, two blocks in flight per wave.  A block is staged
  // to LDS, the loads two steps ahead go out into the registers it freed,
  // then the staged block is computed.  An item's last step issues the next
  // item's first two blocks instead, so loads stay in flight through the
  // epilogue and the next item's start.  Loads are never skipped (an index
  // past the item is clamped and the rows masked), so every path carries the
  // same outstanding loads and each staging waits for the older buffer only.
  u32x4 ka[kLoads], va[kLoads], kb[kLoads], vb[kLoads];
  uint32_t oka, okb;
  load_block(cur, bt_cur, wave, ka, va, oka);
  load_block(cur, bt_cur, wave + kWaves, kb, vb, okb);

  for (;;) {
    const int bt_nxt = load_bt(nxt);
    QkFrag<T, kDl> q_nxt[RBW];
    int qpos_nxt[RBW];
    load_q(nxt, q_nxt, qpos_nxt);
    const ItemS nxt2 = fetch(w + 2 * grid);

#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      m_run[rb] = -INFINITY;
      l_part[rb] = 0.f;
#pragma unroll
      for (int d = 0; d < kDimBlocks; ++d) o_acc[rb][d] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    for (int j = wave;; j += 2 * kWaves) {
      const bool last = j + 2 * kWaves >= cur.nb;   // the item's final step for this wave
      // where the loads issued in this step go: two steps ahead in this item,
      // or the next item's first two steps (a dummy re-read when none)
      const bool to_next = last && nxt.valid;
      const ItemS tgt = to_next ? nxt : cur;
      const int tgt_bt = to_next ? bt_nxt : bt_cur;
      const int ja = last ? (to_next ? wave : cur.nb - 1) : j + 2 * kWaves;
      const int jb = last ? (to_next ? wave + kWaves : cur.nb - 1) : j + 3 * kWaves;
      stage_block(ka, va, oka);
      load_block(tgt, tgt_bt, ja, ka, va, oka);
      if (j < cur.nb) compute_block(cur, q_cur, qpos_cur, j);
      stage_block(kb, vb, okb);
      load_block(tgt, tgt_bt, jb, kb, vb, okb);
      if (j + kWaves < cur.nb) compute_block(cur, q_cur, qpos_cur, j + kWaves);
      if (last) break;
    }

    // ---- combine the four waves, one 16-row block at a time ----
    const int er = args.epi_rows;
    float* eo = reinterpret_cast<float*>(smem);
    float* em = eo + kWaves * er * kEpiStride;
    float* el = em + kWaves * er;
    const int chunk_idx = cur.k_lo / args.split_len;
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      float l_row = l_part[rb];
      l_row += __shfl_xor(l_row, 16);
      l_row += __shfl_xor(l_row, 32);
      __syncthreads();
      if (lrow < er) {
        const int erow = wave * er + lrow;
#pragma unroll
        for (int d = 0; d < kDimBlocks; ++d)
          *reinterpret_cast<f32x4*>(eo + erow * kEpiStride + d * 16 + lgrp * 4) = o_acc[rb][d];
        if (lgrp == 0) {
          em[erow] = m_run[rb];
          el[erow] = l_row;
        }
      }
      __syncthreads();
      combine_rows<T, D, kWaves>(args, eo, em, el, er, rb * 16, cur.rows_total, cur.q0, cur.g, cur.whole,
                                 chunk_idx);
    }
    __syncthreads();   // the epilogue's LDS reads finish before the next staging

    if (!nxt.valid) break;
    w += grid;
    cur = nxt;
    bt_cur = bt_nxt;
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      q_cur[rb] = q_nxt[rb];
      qpos_cur[rb] = qpos_nxt[rb];
    }
    nxt = nxt2;
  }
}

// ---------------------------------------------------------------------------
// Paged prefill/append in bf16 for more than 48 query rows per sequence and
// KV head.
//  * A workgroup owns 128 query rows of one (sequence, KV head) unit; rows are
//    (query, head-in-group) pairs, so every K/V byte it stages serves the
//    whole GQA group.  Wave w owns rows 32w..32w+31 as two 16-row MFMA
//    blocks and keeps its own softmax state: no cross-wave combine.
//  * K/V tiles of 64 positions are gathered through the block table with
//    16-byte loads into registers one tile ahead and written to one of two
//    LDS buffers; rows are padded by 16 bytes so every operand read below is
//    free of bank conflicts.  One barrier per tile.  Block-table entries are
//    fetched a further tile ahead.
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 with Q held in registers.  A
//    lane then holds one query row and 4 positions of each 16-key block: the
//    row max is in-lane work plus two shuffles.  The reference max of a row
//    is raised only when a tile's max exceeds it by more than 8 (log2
//    units), so most tiles skip the rescale and probabilities stay <= 256.
//  * O^T += V^T P^T on the same MFMA.  P^T is already in B-operand layout
//    once the MFMA's k index is permuted the same way on both operands
//    (k-slots 8g..8g+3 <-> keys 4g..4g+3 of the first 16-key block, 8g+4..
//    8g+7 <-> the same of the second), and V^T comes straight out of LDS with
//    ds_read_b64_tr_b16.  Row sums run on the MFMA as well (a ones operand
//    times P^T), from the same bf16 P the numerator uses.
//  * Workgroups are dealt to the 8 XCDs round robin, so workgroup i serves
//    unit i % 8 of a block of 8 units: all q-tiles of a unit run on one XCD
//    and re-read its K/V from that XCD's L2.  Within a block the tiles with
//    the most keys go first.  A one-workgroup schedule kernel lists the
//    blocks' tile counts; the grid is a host-side upper bound and surplus
//    workgroups exit at once.
// ---------------------------------------------------------------------------
constexpr int kPfRows = 128;   // query rows per workgroup
constexpr int kPfKeys = 64;    // positions per staged tile

template <int D>
constexpr int pf_row_bytes() { return D * 2 + 16; }
template <int D>
constexpr int pf_lds_bytes() { return 2 * 2 * kPfKeys * pf_row_bytes<D>(); }

// row_off[k] = sum over blocks < k of (q-tiles of the block) * n_splits,
// where a block's q-tiles are the most any of its 8 units needs.
__global__ __launch_bounds__(kThreads) void prefill_schedule_kernel(AttnArgs a, int32_t* row_off,
                                                                    int n_blocks) {
  __shared__ int s_scan[kThreads];
  __shared__ int s_carry;
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_carry = 0;
    row_off[0] = 0;
  }
  __syncthreads();
  const int units = a.n_seqs * a.num_kv_heads;
  for (int base = 0; base < n_blocks; base += kThreads) {
    const int blk = base + tid;
    int tiles = 0;
    if (blk < n_blocks) {
      int prev = -1;
      for (int u = blk * 8; u < min(units, blk * 8 + 8); ++u) {
        const int b = u / a.num_kv_heads;
        if (b == prev) continue;
        prev = b;
        const int n_b = min(a.cu_q[b + 1] - a.cu_q[b], a.max_q);
        tiles = max(tiles, (n_b * a.group + kPfRows - 1) / kPfRows);
      }
    }
    const int v = tiles * a.n_splits;
    s_scan[tid] = v;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
      const int w = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += w;
      __syncthreads();
    }
    if (blk < n_blocks) row_off[blk + 1] = s_carry + s_scan[tid];
    __syncthreads();
    if (tid == kThreads - 1) s_carry += s_scan[tid];
    __syncthreads();
  }
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Four bf16 of one column of a 4 x 16 block, transposed across a 16-lane
// group (gfx950 ds_read_b64_tr_b16): lane i of the group receives column i
// of rows 0..3 when lane k of the group addresses row k / 4, columns
// 4 (k % 4) .. 4 (k % 4) + 3.
__device__ __forceinline__ bf16x4 lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

// kPow2: page_size is a power of two (block index by shift).
template <int D, bool kPow2>
__global__ __launch_bounds__(kThreads, 2) void paged_prefill_kernel(AttnArgs a,
                                                                   const int32_t* __restrict__ row_off,
                                                                   int n_blocks) {
  constexpr int kRowB = pf_row_bytes<D>();              // LDS row stride, bytes
  constexpr int kCpr = D * 2 / 16;                      // 16-byte chunks per K/V row
  constexpr int kChunks = kPfKeys * kCpr / kThreads;    // per thread per pool
  constexpr int kRowsPerPass = kThreads / kCpr;         // rows staged per chunk index
  constexpr int kQk = D / 32;                           // MFMAs per 16x16 score block
  constexpr int kDb = D / 16;                           // 16-dim blocks of O^T
  constexpr int kTileB = kPfKeys * kRowB;               // bytes of one staged K or V tile
  static_assert(kChunks * kRowsPerPass == kPfKeys, "tile split");
  extern __shared__ __align__(16) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int lrow = lane & 15;
  const int lgrp = lane >> 4;

  // ---- work item ----
  const int r = blockIdx.x >> 3;
  if (r >= row_off[n_blocks]) return;
  int lo = 0, hi = n_blocks;   // row_off[lo] <= r < row_off[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (row_off[mid] <= r) lo = mid;
    else hi = mid;
  }
  const int n_sp = a.n_splits;
  const int local = r - row_off[lo];
  const int tiles_blk = (row_off[lo + 1] - row_off[lo]) / n_sp;
  const int qt = tiles_blk - 1 - local / n_sp;
  const int split = local - (local / n_sp) * n_sp;
  const int hkv = a.num_kv_heads;
  const int u = lo * 8 + (blockIdx.x & 7);
  if (u >= a.n_seqs * hkv) return;
  const int b = u / hkv;
  const int g = u - b * hkv;
  const int group = a.group;
  const int q0 = a.cu_q[b];
  const int n_b = a.cu_q[b + 1] - q0;
  const int rows_total = min(n_b, a.max_q) * group;   // queries past max_q are not computed
  const int row0 = qt * kPfRows;
  if (row0 >= rows_total) return;
  const int start = a.seq_lens[b] - n_b;                 // position of new query 0
  const int kv_end = start + (min(row0 + kPfRows, rows_total) - 1) / group + 1;
  const int k_lo = split * a.split_len;
  if (k_lo >= kv_end) return;
  const int k_hi = min(k_lo + a.split_len, kv_end);
  const int n_tiles = (k_hi - k_lo + kPfKeys - 1) / kPfKeys;

  // ---- staging: this thread's rows srow0 + c * kRowsPerPass, chunk spart ----
  const int ps = a.page_size;
  const int ps_shift = a.ps_shift;
  const int32_t* bt_row = a.block_tables + static_cast<int64_t>(b) * a.bt_stride;
  const int srow0 = tid / kCpr;
  const int spart = tid - srow0 * kCpr;
  const uint32_t head_bytes = static_cast<uint32_t>(ps) * D * 2;   // one (page, head) block
  const char* kbytes = static_cast<const char*>(a.k_pool);
  const char* vbytes = static_cast<const char*>(a.v_pool);

  int pg_next[kChunks], pg_next2[kChunks];
  u32x4 kr[kChunks], vr[kChunks];
  // position of staged row c of tile t (past the split's end: its last position)
  auto pos_of = [&](int t, int c) __attribute__((always_inline)) {
    return min(k_lo + t * kPfKeys + srow0 + c * kRowsPerPass, k_hi - 1);
  };
  auto blk_of = [&](int pos) __attribute__((always_inline)) {
    if constexpr (kPow2) return pos >> ps_shift;
    else return pos / ps;
  };
  auto fetch_pages = [&](int t) __attribute__((always_inline)) {
    const int tl = min(t, n_tiles - 1);
#pragma unroll
    for (int c = 0; c < kChunks; ++c) pg_next2[c] = bt_row[blk_of(pos_of(tl, c))];
  };
  auto load_kv = [&](int t) __attribute__((always_inline)) {
    const int tl = min(t, n_tiles - 1);
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int pos = pos_of(tl, c);
      const int off = pos - blk_of(pos) * ps;
      const uint32_t page = static_cast<uint32_t>(min(max(pg_next[c], 0), a.num_pages - 1));
      const uint64_t boff = static_cast<uint64_t>(page * hkv + g) * head_bytes +
                            static_cast<uint32_t>(off * (D * 2) + spart * 16);
      kr[c] = *reinterpret_cast<const u32x4*>(kbytes + boff);
      vr[c] = *reinterpret_cast<const u32x4*>(vbytes + boff);
    }
  };
  auto stage = [&](int buf) __attribute__((always_inline)) {
    char* kb = smem + buf * 2 * kTileB;
    char* vb = kb + kTileB;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int row = srow0 + c * kRowsPerPass;
      *reinterpret_cast<u32x4*>(kb + row * kRowB + spart * 16) = kr[c];
      *reinterpret_cast<u32x4*>(vb + row * kRowB + spart * 16) = vr[c];
    }
  };

  // ---- this lane's two query rows (B operand of S^T = K Q^T) ----
  // Lane group lgrp holds dims [lgrp * D/4, (lgrp + 1) * D/4); MFMA kk takes
  // the kk-th 8 of them (the same permutation is applied to K).
  const int wr0 = row0 + 32 * wave;
  bf16x8 qf[2][kQk];
  int qpos[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int rr = wr0 + 16 * rb + lrow;
    const int qi = rr / group;
    const bool ok = rr < rows_total && q0 + qi < a.total_q;
    qpos[rb] = ok ? start + qi : -1;
    const uint16_t* src = static_cast<const uint16_t*>(a.q) +
                          (static_cast<int64_t>(q0 + qi) * a.num_q_heads + g * group + (rr - qi * group)) * D +
                          lgrp * (D / 4);
#pragma unroll
    for (int kk = 0; kk < kQk; ++kk) {
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (ok) v = *reinterpret_cast<const u32x4*>(src + kk * 8);
      qf[rb][kk] = __builtin_bit_cast(bf16x8, v);
    }
  }

  const bool w_active = wr0 < rows_total;
  const int w_qmin = start + wr0 / group;
  const int w_qmax = start + (min(wr0 + 31, rows_total - 1)) / group;
  const float c2 = a.scale_log2;

  f32x4 o[kDb][2];
  f32x4 lsum[2];
  float mc[2] = {-INFINITY, -INFINITY};   // reference max per row, log2 units
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    lsum[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int d = 0; d < kDb; ++d) o[d][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});

  // lane parts of the LDS operand addresses
  const int k_lane = lrow * kRowB + lgrp * (D / 4) * 2;
  const int v_lane = (4 * lgrp + (lrow >> 2)) * kRowB + ((lrow & 3) >> 1) * 16 + (lrow & 1) * 8;

  auto compute = [&](const char* kt, const char* vt, int tb, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool kMask = decltype(mask_tag)::value;
    f32x4 s[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      bf16x8 kf[kQk];
#pragma unroll
      for (int kk = 0; kk < kQk; ++kk)
        kf[kk] = *reinterpret_cast<const bf16x8*>(kt + k_lane + kb * 16 * kRowB + kk * 16);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < kQk; ++kk) acc = mfma_qk(kf[kk], qf[rb][kk], acc);
        s[kb][rb] = acc;
      }
    }
    bf16x8 pk[2][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      if constexpr (kMask) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            s[kb][rb][i] = (tb + kb * 16 + 4 * lgrp + i <= qpos[rb]) ? s[kb][rb][i] : -INFINITY;
      }
      float mx = s[0][rb][0];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[kb][rb][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mxc = mx * c2;
      const bool up = mxc > mc[rb] + 8.f;
      const float mnew = up ? mxc : mc[rb];
      const float alpha = up ? fast_exp2(mc[rb] - mnew) : 1.f;
      mc[rb] = mnew;
      if (__any(up)) {
        lsum[rb] *= alpha;
#pragma unroll
        for (int d = 0; d < kDb; ++d) o[d][rb] *= alpha;
      }
      const float muse = mnew == -INFINITY ? 0.f : mnew;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 p;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[i] = static_cast<__bf16>(fast_exp2(fmaf(s[2 * ks][rb][i], c2, -muse)));
          p[4 + i] = static_cast<__bf16>(fast_exp2(fmaf(s[2 * ks + 1][rb][i], c2, -muse)));
        }
        pk[rb][ks] = p;
        lsum[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, p, lsum[rb], 0, 0, 0);
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int d = 0; d < kDb; ++d) {
        const char* vp = vt + v_lane + 32 * ks * kRowB + d * 32;
        const bf16x4 v0 = lds_read_tr(vp);
        const bf16x4 v1 = lds_read_tr(vp + 16 * kRowB);
        const bf16x8 vf = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          o[d][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pk[rb][ks], o[d][rb], 0, 0, 0);
      }
    }
  };

  // ---- main loop over the split's tiles ----
  fetch_pages(0);
#pragma unroll
  for (int c = 0; c < kChunks; ++c) pg_next[c] = pg_next2[c];
  load_kv(0);
  fetch_pages(1);
  stage(0);
#pragma unroll
  for (int c = 0; c < kChunks; ++c) pg_next[c] = pg_next2[c];
  __syncthreads();
  for (int t = 0; t < n_tiles; ++t) {
    load_kv(t + 1);            // clamped: the last tile reloads itself
    fetch_pages(t + 2);
    const int tb = k_lo + t * kPfKeys;
    if (w_active && tb <= w_qmax) {
      const char* kt = smem + (t & 1) * 2 * kTileB;
      if (tb + kPfKeys - 1 <= w_qmin)
        compute(kt, kt + kTileB, tb, std::integral_constant<bool, false>());
      else
        compute(kt, kt + kTileB, tb, std::integral_constant<bool, true>());
    }
    stage((t + 1) & 1);
#pragma unroll
    for (int c = 0; c < kChunks; ++c) pg_next[c] = pg_next2[c];
    __syncthreads();
  }

  // ---- epilogue: rows of this wave ----
  if (!w_active) return;
  const bool final_write = n_sp == 1;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int rr = wr0 + 16 * rb + lrow;
    if (qpos[rb] < 0) continue;
    const int qi = rr / group;
    const int tok = q0 + qi;
    const int64_t orow = static_cast<int64_t>(tok) * a.num_q_heads + g * group + (rr - qi * group);
    const float l = lsum[rb][0];
    if (final_write) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      uint16_t* dst = static_cast<uint16_t*>(a.out) + orow * D + 4 * lgrp;
#pragma unroll
      for (int d = 0; d < kDb; ++d)
        *reinterpret_cast<i16x4*>(dst + 16 * d) = pack_bf16x4(o[d][rb] * inv);
    } else {
      if (tok >= a.ws_tokens) continue;
      const int64_t slot = orow * n_sp + split;
      float* dst = a.ws_o + slot * D + 4 * lgrp;
#pragma unroll
      for (int d = 0; d < kDb; ++d) *reinterpret_cast<f32x4*>(dst + 16 * d) = o[d][rb];
      if (lgrp == 0) {
        a.ws_ml[slot * 2] = mc[rb];
        a.ws_ml[slot * 2 + 1] = l;
      }
    }
  }
}

// Log-sum-exp merge of the KV-split partials of one (query, head) row.  Grid:
// (num_q_heads, max_q_per_seq, n_seqs), one wave per row.  RBW > 0: the
// decode path, where rows whose sequence fits one chunk were written final
// by the attention kernel; RBW = 0: the tile kernel, every split partial.
template <typename T, int D, int RBW>
__global__ __launch_bounds__(kWave) void merge_chunks_kernel(AttnArgs args) {
  const int h = blockIdx.x;
  const int qi = blockIdx.y;
  const int b = blockIdx.z;
  int q0, n_b;
  int n_chunks = args.n_splits;
  if constexpr (RBW > 0) {
    const int kv_end = decode_kv_end<RBW>(args, b, &q0, &n_b);
    n_chunks = kv_end > 0 ? min((kv_end + args.split_len - 1) / args.split_len, args.n_splits) : 0;
    if (n_chunks <= 1) return;
  } else {
    if (args.cu_q) {
      q0 = args.cu_q[b];
      n_b = args.cu_q[b + 1] - q0;
    } else {
      q0 = b;
      n_b = 1;
    }
  }
  if (qi >= n_b) return;
  const int tok = q0 + qi;
  if (tok >= args.total_q || tok >= args.ws_tokens) return;
  const int qpos = args.seq_lens[b] - n_b + qi;
  const int ns = qpos < 0 ? 0 : min(n_chunks, qpos / args.split_len + 1);
  const int lane = threadIdx.x;
  const int64_t orow = static_cast<int64_t>(tok) * args.num_q_heads + h;
  const int64_t base = orow * args.n_splits;
  constexpr int kPer = D / kWave;
  // pass 1: global max; each lane holds the states of chunks lane, lane + 64, ...
  float mmax = -INFINITY;
  for (int s = lane; s < ns; s += kWave) mmax = fmaxf(mmax, args.ws_ml[(base + s) * 2]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mmax = fmaxf(mmax, __shfl_xor(mmax, off));
  const float mref = mmax == -INFINITY ? 0.f : mmax;
  float acc[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) acc[j] = 0.f;
  float lsum = 0.f;
  for (int s0 = 0; s0 < ns; s0 += kWave) {
    const int sl = s0 + lane;
    float wt = 0.f;
    if (sl < ns) {
      wt = fast_exp2(args.ws_ml[(base + sl) * 2] - mref);
      lsum += wt * args.ws_ml[(base + sl) * 2 + 1];
    }
    const int cnt = min(kWave, ns - s0);
    // eight partial rows in flight at a time (indices clamped, weights zero)
    for (int k0 = 0; k0 < cnt; k0 += 8) {
      float part[8][kPer];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int k = min(k0 + u, cnt - 1);
        const float* o = args.ws_o + (base + s0 + k) * D + lane * kPer;
#pragma unroll
        for (int j = 0; j < kPer; ++j) part[u][j] = o[j];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wk = __shfl(wt, min(k0 + u, kWave - 1));
        const float w_use = (k0 + u < cnt) ? wk : 0.f;
#pragma unroll
        for (int j = 0; j < kPer; ++j) acc[j] += w_use * part[u][j];
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) lsum += __shfl_xor(lsum, off);
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const float v = acc[j] * inv;
    const int64_t e = orow * D + lane * kPer + j;
    if constexpr (sizeof(T) == 2)
      static_cast<uint16_t*>(args.out)[e] = float_to_bf16_bits(v);
    else
      static_cast<float*>(args.out)[e] = v;
  }
}

// KV scatter: one thread per 16-byte chunk of a (token, KV head) row, K and
// V handled by the two halves of the grid.
template <int kEs>
__global__ __launch_bounds__(kThreads) void store_kv_kernel(
    char* __restrict__ k_pool, char* __restrict__ v_pool, const char* __restrict__ k_new,
    const char* __restrict__ v_new, const int64_t* __restrict__ slots, int32_t n_tokens,
    int32_t hkv, int32_t head_dim, int32_t page_size, int32_t ps_shift, int64_t pool_slots) {
  const int chunks_per_row = head_dim * kEs / 16;
  const int64_t per_pool = static_cast<int64_t>(n_tokens) * hkv * chunks_per_row;
  int64_t idx = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (idx >= 2 * per_pool) return;
  const bool is_v = idx >= per_pool;
  if (is_v) idx -= per_pool;
  const int part = static_cast<int>(idx % chunks_per_row);
  const int64_t row = idx / chunks_per_row;         // token * hkv + g
  const int64_t t = row / hkv;
  const int g = static_cast<int>(row - t * hkv);
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= pool_slots) return;
  const int64_t page = ps_shift >= 0 ? (slot >> ps_shift) : slot / page_size;
  const int64_t off = slot - page * page_size;
  const int64_t row_bytes = static_cast<int64_t>(head_dim) * kEs;
  const int64_t dst = ((page * hkv + g) * page_size + off) * row_bytes + part * 16;
  const int64_t src = row * row_bytes + part * 16;
  const uint4 val = *reinterpret_cast<const uint4*>((is_v ? v_new : k_new) + src);
  *reinterpret_cast<uint4*>((is_v ? v_pool : k_pool) + dst) = val;
}

// ---------------------------------------------------------------------------
// host-side launch planning
// ---------------------------------------------------------------------------
int log2_exact(int x) {
  if (x <= 0 || (x & (x - 1))) return -1;
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_desc(const pkv_pool_desc* d, const char* fn) {
  if (!d) return fail(PKV_ERR_INVALID_ARG, std::string(fn) + ": NULL desc");
  if (d->dtype != PKV_F32 && d->dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, std::string(fn) + ": dtype must be PKV_F32 or PKV_BF16");
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, std::string(fn) + ": head_dim must be 64 or 128");
  if (d->page_size < 1 || d->page_size > 256)
    return fail(PKV_ERR_UNSUPPORTED, std::string(fn) + ": page_size must be in 1..256");
  if (d->num_kv_heads < 1 || d->num_pages < 1)
    return fail(PKV_ERR_INVALID_ARG, std::string(fn) + ": num_kv_heads and num_pages must be >= 1");
  if (static_cast<int64_t>(d->num_pages) * d->num_kv_heads * d->page_size * d->head_dim >
      (int64_t{1} << 40))
    return fail(PKV_ERR_UNSUPPORTED, std::string(fn) + ": pool larger than 2^40 elements");
  if (static_cast<int64_t>(d->num_pages) * d->num_kv_heads > INT32_MAX)
    return fail(PKV_ERR_UNSUPPORTED, std::string(fn) + ": num_pages * num_kv_heads above 2^31 - 1");
  return PKV_OK;
}

struct Plan {
  int max_q = 0;
  bool decode = false;  // decode path (few rows) vs a tile kernel
  bool prefill = false; // bf16 tiles: paged_prefill_kernel, else paged_attention_kernel
  int n_blocks = 0;     // prefill: blocks of 8 (sequence, KV head) units
  int rbw = 1;          // decode: 16-row blocks each wave holds
  int epi_rows = 16;    // decode: rows of a block that carry queries
  int rb = 4, kg = 1;   // tile kernel: row blocks x key groups of the 4 waves
  int tile_rows = 64;
  int q_tiles = 0;
  int split_len = 0;    // tile kernel: positions per split; decode: positions per item
  int n_splits = 1;     // most splits / items of one sequence
  int grid = 0;         // decode: persistent workgroups
  size_t items_off = 0, partial_off = 0, ws_bytes = 0;
};

// Decode-path tunables (overridable at build time for sweeps).
#ifndef PKV_DECODE_WORKGROUPS
#define PKV_DECODE_WORKGROUPS 512    // persistent decode workgroups (2 per CU)
#endif
#ifndef PKV_DECODE_MIN_CHUNK
#define PKV_DECODE_MIN_CHUNK 256     // smallest work item, in positions
#endif
constexpr int kDecodeWorkgroups = PKV_DECODE_WORKGROUPS;

// The launch shape is a pure function of host scalars, so the workspace size
// and the split positions are reproducible from the same arguments.
int make_plan(const pkv_pool_desc* d, int n_seqs, int hq, int max_q, int max_seq_len, Plan* p,
              const char* fn) {
  int rc = check_desc(d, fn);
  if (rc != PKV_OK) return rc;
  if (n_seqs < 0 || max_q < 0 || max_seq_len < 0)
    return fail(PKV_ERR_INVALID_ARG, std::string(fn) + ": negative size");
  if (hq < 1 || hq % d->num_kv_heads != 0)
    return fail(PKV_ERR_UNSUPPORTED, std::string(fn) + ": num_q_heads must be a multiple of num_kv_heads");
  const int group = hq / d->num_kv_heads;
  p->max_q = max_q;
  if (group > 16) return fail(PKV_ERR_UNSUPPORTED, std::string(fn) + ": GQA group above 16");
  const int64_t rows = static_cast<int64_t>(max_q) * group;
  const int ps = d->page_size;
  if (n_seqs == 0 || max_q == 0) return PKV_OK;  // nothing to launch, no workspace
  if (rows <= 48) {
    // decode path: items of `chunk` positions.  Larger items for more rows
    // keep the partials small next to the K/V they summarise; smaller ones
    // keep enough items to balance the persistent workgroups.  An item spans
    // at most 64 pages (its block-table slice sits in one register per lane).
    p->decode = true;
    p->rbw = static_cast<int>(std::max<int64_t>(1, (rows + 15) / 16));
    p->epi_rows = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(16, rows)));
    p->tile_rows = 16 * p->rbw;
    p->q_tiles = 1;
    int64_t chunk = std::max<int64_t>(PKV_DECODE_MIN_CHUNK, 64 * rows);
    chunk = std::min<int64_t>(chunk, 4096);
    const int64_t est_len = std::max<int64_t>(1, max_seq_len);
    while (chunk > PKV_DECODE_MIN_CHUNK &&
           static_cast<int64_t>(n_seqs) * d->num_kv_heads * ((est_len + chunk - 1) / chunk) < 4 * kDecodeWorkgroups)
      chunk /= 2;
    chunk = std::min<int64_t>(chunk, static_cast<int64_t>(63) * ps);
    chunk = std::max<int64_t>(16, chunk & ~int64_t{15});
    p->split_len = static_cast<int>(chunk);
    p->n_splits = static_cast<int>(std::max<int64_t>(1, (est_len + chunk - 1) / chunk));
    if (static_cast<int64_t>(n_seqs) * p->n_splits > (int64_t{1} << 30))
      return fail(PKV_ERR_UNSUPPORTED, std::string(fn) + ": too many work items");
    const int64_t items = static_cast<int64_t>(n_seqs) * p->n_splits * d->num_kv_heads;
    p->grid = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(items, kDecodeWorkgroups)));
    p->items_off = 256;
    p->partial_off = p->items_off + static_cast<size_t>(n_seqs) * p->n_splits * 32;
    p->ws_bytes = p->partial_off;
    if (p->n_splits > 1)
      p->ws_bytes += static_cast<size_t>(n_seqs) * max_q * hq * p->n_splits * (d->head_dim + 2) * sizeof(float);
    return PKV_OK;
  }
  if (d->dtype == PKV_BF16) {
    // paged_prefill_kernel: 128-row tiles; KV splits only when the units'
    // tiles alone cannot fill the chip.
    p->prefill = true;
    p->tile_rows = kPfRows;
    if (rows > (int64_t{1} << 28)) return fail(PKV_ERR_UNSUPPORTED, std::string(fn) + ": too many queries per sequence");
    const int64_t q_tiles = (rows + kPfRows - 1) / kPfRows;
    p->q_tiles = static_cast<int>(q_tiles);
    const int64_t units = static_cast<int64_t>(n_seqs) * d->num_kv_heads;
    p->n_blocks = static_cast<int>((units + 7) / 8);
    const int64_t max_tiles = (static_cast<int64_t>(max_seq_len) + kPfKeys - 1) / kPfKeys;
    int64_t want = (kTargetWorkgroups + units * q_tiles - 1) / (units * q_tiles);
    want = std::max<int64_t>(1, std::min<int64_t>(want, (max_seq_len + kMinSplitKeys - 1) / kMinSplitKeys));
    const int64_t tiles_per_split = std::max<int64_t>(1, (max_tiles + want - 1) / want);
    p->split_len = static_cast<int>(tiles_per_split * kPfKeys);
    p->n_splits = static_cast<int>(std::max<int64_t>(1, (max_tiles + tiles_per_split - 1) / tiles_per_split));
    const int64_t sched_rows = static_cast<int64_t>(p->n_blocks) * q_tiles * p->n_splits;
    if (sched_rows > (int64_t{1} << 27)) return fail(PKV_ERR_UNSUPPORTED, std::string(fn) + ": too many work items");
    p->items_off = 0;
    p->partial_off = (static_cast<size_t>(p->n_blocks + 1) * sizeof(int32_t) + 255) & ~size_t{255};
    p->ws_bytes = p->partial_off;
    if (p->n_splits > 1)
      p->ws_bytes += static_cast<size_t>(n_seqs) * max_q * hq * p->n_splits * (d->head_dim + 2) * sizeof(float);
    return PKV_OK;
  }
  p->rb = 4;
  p->kg = 1;
  p->tile_rows = 16 * p->rb;
  const int64_t q_tiles = (rows + p->tile_rows - 1) / p->tile_rows;
  if (q_tiles > 65535) return fail(PKV_ERR_UNSUPPORTED, std::string(fn) + ": too many queries per sequence");
  p->q_tiles = static_cast<int>(q_tiles);
  const int64_t units = static_cast<int64_t>(n_seqs) * d->num_kv_heads * q_tiles;
  const int64_t max_tiles = (static_cast<int64_t>(max_seq_len) + kTileKeys - 1) / kTileKeys;
  int64_t want = units > 0 ? (kTargetWorkgroups + units - 1) / units : 1;
  const int64_t max_by_len = (max_seq_len + kMinSplitKeys - 1) / kMinSplitKeys;
  want = std::max<int64_t>(1, std::min<int64_t>(want, std::max<int64_t>(1, max_by_len)));
  int64_t tiles_per_split = (max_tiles + want - 1) / want;
  if (tiles_per_split < 1) tiles_per_split = 1;
  p->split_len = static_cast<int>(tiles_per_split * kTileKeys);
  p->n_splits = static_cast<int>(std::max<int64_t>(1, (max_tiles + tiles_per_split - 1) / tiles_per_split));
  if (p->n_splits > 65535) return fail(PKV_ERR_UNSUPPORTED, std::string(fn) + ": too many splits");
  p->partial_off = 0;
  p->ws_bytes = 0;
  if (p->n_splits > 1) {
    const int64_t rows_out = static_cast<int64_t>(n_seqs) * max_q * hq * p->n_splits;
    p->ws_bytes = static_cast<size_t>(rows_out) * (d->head_dim + 2) * sizeof(float);
  }
  return PKV_OK;
}

template <typename T, int D, int RB, int KG>
void launch_attention_t(const AttnArgs& a, const Plan& p, int n_seqs, int hkv, hipStream_t st) {
  dim3 grid(p.n_splits, p.q_tiles, n_seqs * hkv);
  constexpr int kLds = lds_bytes<T, D>();
  paged_attention_kernel<T, D, RB, KG><<<grid, dim3(kThreads), kLds, st>>>(a);
}

template <typename T, int D, int RBW>
void launch_decode_t(const AttnArgs& a, const Plan& p, int n_seqs, char* ws, hipStream_t st) {
  DecodeQueue* queue = reinterpret_cast<DecodeQueue*>(ws);
  DecodeItem* items = reinterpret_cast<DecodeItem*>(ws + p.items_off);
  decode_schedule_kernel<RBW><<<1, kThreads, 0, st>>>(a, queue, items);
  constexpr int kRowB = D * static_cast<int>(sizeof(T));
  constexpr int kStage = 4 * 2 * 16 * (kRowB + (kRowB >= 512 ? 0 : 16));
  const int epi = (4 * p.epi_rows * (D + 4) + 2 * 4 * p.epi_rows) * static_cast<int>(sizeof(float));
  const int lds = std::max(kStage, epi);
  if (a.ps_shift >= 4)
    paged_decode_kernel<T, D, RBW, 0><<<p.grid, dim3(kThreads), lds, st>>>(a, queue, items);
  else if (a.ps_shift >= 0)
    paged_decode_kernel<T, D, RBW, 1><<<p.grid, dim3(kThreads), lds, st>>>(a, queue, items);
  else
    paged_decode_kernel<T, D, RBW, 2><<<p.grid, dim3(kThreads), lds, st>>>(a, queue, items);
  if (p.n_splits > 1) {
    dim3 grid(a.num_q_heads, p.max_q, n_seqs);
    merge_chunks_kernel<T, D, RBW><<<grid, dim3(kWave), 0, st>>>(a);
  }
}

// Upper bound on the prefill tile-rows the schedule kernel can list, from
// host scalars: a block's q-tiles are at most its units' sequences' q-tiles
// summed, and a sequence's units fall in at most hkv / 8 + 2 blocks.
int64_t prefill_grid(const Plan& p, int n_seqs, int hkv, int group, int total_q) {
  const int64_t tiles_all = (static_cast<int64_t>(total_q) * group + kPfRows - 1) / kPfRows + n_seqs;
  const int64_t per_seq_blocks = hkv % 8 == 0 ? hkv / 8 : hkv / 8 + 2;
  const int64_t rows = std::min<int64_t>(static_cast<int64_t>(p.n_blocks) * p.q_tiles, per_seq_blocks * tiles_all);
  return 8 * rows * p.n_splits;
}

template <int D, bool kPow2>
int launch_prefill_t(const AttnArgs& a, const Plan& p, char* ws, hipStream_t st) {
  constexpr int kLds = pf_lds_bytes<D>();
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&paged_prefill_kernel<D, kPow2>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
  if (attr != hipSuccess) return fail(PKV_ERR_DEVICE, std::string("prefill: LDS attribute: ") + hipGetErrorString(attr));
  int32_t* row_off = reinterpret_cast<int32_t*>(ws + p.items_off);
  prefill_schedule_kernel<<<1, kThreads, 0, st>>>(a, row_off, p.n_blocks);
  const int64_t grid = prefill_grid(p, a.n_seqs, a.num_kv_heads, a.group, a.total_q);
  if (grid > INT32_MAX) return fail(PKV_ERR_UNSUPPORTED, "prefill: grid too large");
  if (grid > 0) paged_prefill_kernel<D, kPow2><<<static_cast<int>(grid), dim3(kThreads), kLds, st>>>(a, row_off, p.n_blocks);
  if (p.n_splits > 1) {
    dim3 mg(a.num_q_heads, p.max_q, a.n_seqs);
    merge_chunks_kernel<uint16_t, D, 0><<<mg, dim3(kWave), 0, st>>>(a);
  }
  return PKV_OK;
}

template <typename T, int D>
void launch_attention_d(const AttnArgs& a, const Plan& p, int n_seqs, int hkv, char* ws, hipStream_t st) {
  if (p.decode) {
    switch (p.rbw) {
      case 1: launch_decode_t<T, D, 1>(a, p, n_seqs, ws, st); break;
      case 2: launch_decode_t<T, D, 2>(a, p, n_seqs, ws, st); break;
      default: launch_decode_t<T, D, 3>(a, p, n_seqs, ws, st); break;
    }
    return;
  }
  launch_attention_t<T, D, 4, 1>(a, p, n_seqs, hkv, st);
  if (p.n_splits > 1) {
    dim3 grid(a.num_q_heads, p.max_q, n_seqs);
    merge_chunks_kernel<T, D, 0><<<grid, dim3(kWave), 0, st>>>(a);
  }
}

int run_attention(const char* fn, const pkv_pool_desc* desc, const void* k_pool,
                  const void* v_pool, const void* q, int32_t total_q, const int32_t* cu_q,
                  int32_t n_seqs, int32_t hq, const int32_t* block_tables, int32_t bt_stride,
                  const int32_t* seq_lens, int32_t max_q, int32_t max_seq_len, float scale,
                  void* out, void* workspace, size_t ws_bytes, void* stream) {
  Plan p;
  int rc = make_plan(desc, n_seqs, hq, max_q, max_seq_len, &p, fn);
  if (rc != PKV_OK) return rc;
  if (n_seqs == 0 || total_q == 0 || max_q == 0) return PKV_OK;
  if (total_q < 0 || bt_stride < 0) return fail(PKV_ERR_INVALID_ARG, std::string(fn) + ": negative size");
  if (!k_pool || !v_pool || !q || !out || !block_tables || !seq_lens)
    return fail(PKV_ERR_INVALID_ARG, std::string(fn) + ": NULL device pointer");
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(q) || !aligned16(out))
    return fail(PKV_ERR_INVALID_ARG, std::string(fn) + ": pools, q and out must be 16-byte aligned");
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(PKV_ERR_INVALID_ARG, std::string(fn) + ": scale must be positive and finite");
  if (p.ws_bytes > 0) {
    if (!workspace || ws_bytes < p.ws_bytes)
      return fail(PKV_ERR_BUFFER_TOO_SMALL, std::string(fn) + ": workspace needs " +
                                                std::to_string(p.ws_bytes) + " bytes");
    if (!aligned16(workspace))
      return fail(PKV_ERR_INVALID_ARG, std::string(fn) + ": workspace must be 16-byte aligned");
  }
  AttnArgs a{};
  a.q = q;
  a.out = out;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.cu_q = cu_q;
  a.bt_stride = bt_stride;
  a.n_seqs = n_seqs;
  a.num_q_heads = hq;
  a.num_kv_heads = desc->num_kv_heads;
  a.group = hq / desc->num_kv_heads;
  a.num_pages = desc->num_pages;
  a.page_size = desc->page_size;
  a.ps_shift = log2_exact(desc->page_size);
  a.total_q = total_q;
  a.ws_tokens = static_cast<int32_t>(std::min<int64_t>(INT32_MAX, static_cast<int64_t>(n_seqs) * max_q));
  a.split_len = p.split_len;
  a.epi_rows = p.epi_rows;
  a.n_splits = p.n_splits;
  a.max_q = max_q;
  a.scale_log2 = scale * 1.4426950408889634f;
  if (p.n_splits > 1) {
    const size_t rows_out = static_cast<size_t>(n_seqs) * max_q * hq * p.n_splits;
    a.ws_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.partial_off);
    a.ws_ml = a.ws_o + rows_out * desc->head_dim;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int hkv = desc->num_kv_heads;
  char* ws = static_cast<char*>(workspace);
  (void)hipGetLastError();
  if (p.prefill) {
    const bool pow2 = a.ps_shift >= 0;
    if (desc->head_dim == 128)
      rc = pow2 ? launch_prefill_t<128, true>(a, p, ws, st) : launch_prefill_t<128, false>(a, p, ws, st);
    else
      rc = pow2 ? launch_prefill_t<64, true>(a, p, ws, st) : launch_prefill_t<64, false>(a, p, ws, st);
    if (rc != PKV_OK) return rc;
  } else if (desc->dtype == PKV_BF16) {
    if (desc->head_dim == 128)
      launch_attention_d<uint16_t, 128>(a, p, n_seqs, hkv, ws, st);
    else
      launch_attention_d<uint16_t, 64>(a, p, n_seqs, hkv, ws, st);
  } else {
    if (desc->head_dim == 128)
      launch_attention_d<float, 128>(a, p, n_seqs, hkv, ws, st);
    else
      launch_attention_d<float, 64>(a, p, n_seqs, hkv, ws, st);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess)
    return fail(PKV_ERR_DEVICE, std::string(fn) + ": launch failed: " + hipGetErrorString(err));
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_store_kv(const pkv_pool_desc* desc, void* k_pool, void* v_pool, const void* k_new,
                 const void* v_new, const int64_t* slots, int32_t n_tokens, void* stream) {
  int rc = check_desc(desc, "pkv_store_kv");
  if (rc != PKV_OK) return rc;
  if (n_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "pkv_store_kv: n_tokens < 0");
  if (n_tokens == 0) return PKV_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !slots)
    return fail(PKV_ERR_INVALID_ARG, "pkv_store_kv: NULL device pointer");
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(k_new) || !aligned16(v_new) ||
      (reinterpret_cast<uintptr_t>(slots) & 7u))
    return fail(PKV_ERR_INVALID_ARG, "pkv_store_kv: misaligned device pointer");
  const int es = desc->dtype == PKV_BF16 ? 2 : 4;
  const int64_t chunks = 2 * static_cast<int64_t>(n_tokens) * desc->num_kv_heads *
                         (desc->head_dim * es / 16);
  const int64_t blocks = (chunks + kThreads - 1) / kThreads;
  if (blocks > INT32_MAX) return fail(PKV_ERR_UNSUPPORTED, "pkv_store_kv: too many tokens");
  const int64_t pool_slots = static_cast<int64_t>(desc->num_pages) * desc->page_size;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (es == 2)
    store_kv_kernel<2><<<dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, st>>>(
                       static_cast<char*>(k_pool), static_cast<char*>(v_pool),
                       static_cast<const char*>(k_new), static_cast<const char*>(v_new), slots,
                       n_tokens, desc->num_kv_heads, desc->head_dim, desc->page_size,
                       log2_exact(desc->page_size), pool_slots);
  else
    store_kv_kernel<4><<<dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, st>>>(
                       static_cast<char*>(k_pool), static_cast<char*>(v_pool),
                       static_cast<const char*>(k_new), static_cast<const char*>(v_new), slots,
                       n_tokens, desc->num_kv_heads, desc->head_dim, desc->page_size,
                       log2_exact(desc->page_size), pool_slots);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess)
    return fail(PKV_ERR_DEVICE, std::string("pkv_store_kv: launch failed: ") + hipGetErrorString(err));
  return PKV_OK;
}

size_t pkv_workspace_bytes(const pkv_pool_desc* desc, int32_t n_seqs, int32_t num_q_heads,
                           int32_t max_q_per_seq, int32_t max_seq_len) {
  Plan p;
  if (make_plan(desc, n_seqs, num_q_heads, max_q_per_seq, max_seq_len, &p, "pkv_workspace_bytes") != PKV_OK)
    return 0;
  return p.ws_bytes;
}

int pkv_decode(const pkv_pool_desc* desc, const void* k_pool, const void* v_pool, const void* q,
               int32_t n_seqs, int32_t num_q_heads, const int32_t* block_tables,
               int32_t bt_stride, const int32_t* seq_lens, int32_t max_seq_len, float scale,
               void* out, void* workspace, size_t ws_bytes, void* stream) {
  return run_attention("pkv_decode", desc, k_pool, v_pool, q, n_seqs, nullptr, n_seqs,
                       num_q_heads, block_tables, bt_stride, seq_lens, 1, max_seq_len, scale,
                       out, workspace, ws_bytes, stream);
}

int pkv_prefill_append(const pkv_pool_desc* desc, const void* k_pool, const void* v_pool,
                       const void* q, int32_t total_q, const int32_t* cu_q, int32_t n_seqs,
                       int32_t num_q_heads, const int32_t* block_tables, int32_t bt_stride,
                       const int32_t* seq_lens, int32_t max_q_per_seq, int32_t max_seq_len,
                       float scale, void* out, void* workspace, size_t ws_bytes, void* stream) {
  if (!cu_q && n_seqs > 0) return fail(PKV_ERR_INVALID_ARG, "pkv_prefill_append: NULL cu_q");
  return run_attention("pkv_prefill_append", desc, k_pool, v_pool, q, total_q, cu_q, n_seqs,
                       num_q_heads, block_tables, bt_stride, seq_lens, max_q_per_seq,
                       max_seq_len, scale, out, workspace, ws_bytes, stream);
}

}  // extern "C"
