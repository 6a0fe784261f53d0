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
// Kernels (MI355X-first, not a translation of any page's design):
//  * store_kv_kernel / store_kv_i8_kernel: one 16-byte chunk of a (token,
//    KV head) row per thread, coalesced; INT8 pages quantize on the way.
//  * paged_decode_kernel (decode and appends of at most 48 rows per unit):
//    one-wave workgroups split the list of 16-position blocks of all
//    (sequence, KV head) units into equal contiguous ranges ("stream-K").
//    A wave keeps two blocks in flight in registers (non-temporal loads),
//    takes K straight from its registers as the MFMA operand (bf16 pages),
//    stages V in LDS and runs S^T = K Q^T and O^T += V^T P^T on bf16 MFMA,
//    with each lane holding one query row.  A row's reference max is raised
//    only when a score exceeds it by more than 8 (log2 units), which each lane decides
//    from its own scores, so the shuffles of a row reduction run only then.
//    merge_segments_kernel folds the partial states of units that a range
//    boundary split, by log-sum-exp.
//  * paged_prefill_kernel (bf16 and INT8 pages, longer appends): a
//    workgroup owns 32 query rows per wave of one (sequence, KV head) unit
//    (8 waves, 128-position K/V tiles), stages K/V tiles in two LDS buffers
//    through the block table, and runs both products on
//    v_mfma_f32_16x16x32_bf16 with V^T read by ds_read_b64_tr_b16.  INT8
//    codes are staged as exact bf16 integers: the key scale multiplies the
//    scores and the value scale the probabilities.
//  * paged_prefill_stream_kernel (the same, when no context exceeds 2048
//    positions): persistent 8-wave workgroups with 64-position tiles that
//    run through their work items without draining between them; with bf16
//    pages, D = 128 and scalar page lookups the K/V tiles go straight from
//    memory into a ring of three LDS buffers, two tiles ahead.
//  * paged_attention_kernel: the fp32 prefill (4 waves, 64-position tiles,
//    v_mfma_f32_16x16x4_f32), kept for the fp32 parity cases.
//  * copy_pages_kernel, codec_encode_kernel / codec_decode_kernel,
//    stream_read_kernel: page copies, the group-wise codec and a read probe.
// Long contexts are split at fixed logical positions and merged with
// log-sum-exp, so every result depends only on the logical sequence, never
// on which physical pages hold it.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>
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

// Pairwise reductions across lanes l and l ^ 16 (l ^ 32) without LDS:
// v_permlane16_swap (v_permlane32_swap) with both operands x leaves, in
// every lane, its own value in one result and its partner's in the other.
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

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
  int32_t waves;        // decode: one-wave workgroups of the launch
  int32_t head_bytes;   // bytes of one (page, KV head) block of a pool
  int32_t kv_cap;       // min(bt_stride * page_size, max_seq_len): positions at
                        // or past it are never read, so a seq_lens entry past
                        // its block-table row (or the planned length) cannot
                        // index beyond the row
  float scale_log2;     // softmax scale * log2(e)
};

// INT8 pages: a (page, KV head) block holds page_size rows of head_dim codes,
// then page_size fp32 scales, padded to a multiple of 16 bytes.
__host__ __device__ constexpr int64_t i8_block_bytes(int64_t ps, int64_t d) { return ps * d + ((4 * ps + 15) & ~int64_t{15}); }

// Eight int8 codes -> eight bf16 in code order (exact: |code| <= 127 fits
// bf16's 8-bit significand).
__device__ __forceinline__ u32x4 i8x8_to_bf16(uint2 x) {
  u32x4 o;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const uint32_t v = w ? x.y : x.x;
    const f32x4 f = {static_cast<float>(static_cast<int8_t>(v)), static_cast<float>(static_cast<int8_t>(v >> 8)),
                     static_cast<float>(static_cast<int8_t>(v >> 16)), static_cast<float>(static_cast<int8_t>(v >> 24))};
    const auto p = __builtin_bit_cast(uint2, pack_bf16x4(f));
    o[2 * w] = p.x;
    o[2 * w + 1] = p.y;
  }
  return o;
}

// Non-temporal load (16 or 8 bytes): the line is not kept for reuse.  For
// reads that touch each byte once (the decode's K/V, page copies, the read
// probe) this lifts HBM throughput by a tenth or more over plain loads
// (decode: 120.8 -> 107.1 us for the 64-sequence batch).  Kernels that
// re-read lines from L2 (the prefill's q-tiles) or read one line in two
// halves (the codec) were slower with it and keep plain loads.
__device__ __forceinline__ u32x4 ld_stream(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ uint2 ld_stream(const uint2* p) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return uint2{v[0], v[1]};
}

// Unit of the K/V loads: 16 bytes of bf16 / fp32 rows, or 8 INT8 codes (which
// widen to 16 bytes of bf16, so staged rows are written in the same pattern).
template <bool kI8>
using KvLoad = std::conditional_t<kI8, uint2, u32x4>;

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
  const int kv_end = min(start + row_last / group + 1, args.kv_cap);   // positions this tile can see
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
// KV head), split evenly over waves ("stream-K").
//
// The work is the list of 16-position blocks of every (sequence, KV head)
// unit, sequence-major, then KV head, then position.  paged_decode_kernel runs
// a fixed number of one-wave workgroups; each wave scans the sequences' block
// counts (a wavefront prefix sum per 64 sequences) and takes the contiguous
// range of `per` blocks starting at w * per.  Every wave moves the same bytes
// and no wave ever waits on another: the kernel has no barrier.  A wave walks
// its range with two blocks in flight, across unit boundaries:
//  * a block's V rows are loaded with fully coalesced 16-byte loads (each
//    instruction reads 1 KB of whole rows) into registers, two blocks ahead,
//    then written to the wave's LDS slice (rows padded as dec_v_row_bytes
//    states, so the transposed reads below are free of bank conflicts).  On
//    bf16 pages each lane loads its K operand of the QK product straight
//    from the pool (16 bytes of each of 16 rows per instruction, the 4 KiB
//    run read once over 4 instructions), so K never passes through LDS;
//    fp32 and INT8 pages stage K like V.  Pool loads are non-temporal;
//  * S^T = K Q^T runs on MFMA with the unit's queries held in registers
//    (loaded when the wave enters the unit); a lane then holds one query row
//    and 4 positions.  The reference max of a row is raised only when a
//    score exceeds it by more than 8 (log2 units), so probabilities stay
//    <= 256; each lane checks its own 4 scores, and the two-shuffle row
//    reduction and the rescale run only when some lane finds one.
//    O^T += V^T P^T takes V^T straight out of LDS with ds_read_b64_tr_b16
//    (bf16);
//  * loads are never skipped: past the range's end the last block is read
//    again, past a unit's end rows are masked, so no branch forces a full
//    wait on outstanding loads.
// Where a wave's range covers a whole unit it writes the normalised output;
// otherwise it writes the unit's partial state (un-normalised O, max, sum) to
// slot unit + wave, and merge_segments_kernel folds a unit's slots with
// log-sum-exp.  Segment boundaries are fixed positions of the logical
// sequence, so results never depend on which physical pages hold it.
// ---------------------------------------------------------------------------

#ifndef PKV_DECODE_WAVES
#define PKV_DECODE_WAVES 1024          // one-wave workgroups (4 per CU)
#endif
#ifndef PKV_COPY_CHUNKS
#define PKV_COPY_CHUNKS 1              // 16-byte chunks per thread of the page copy
#endif
#ifndef PKV_DECODE_MIN_BLOCKS
#define PKV_DECODE_MIN_BLOCKS 4        // smallest range of a wave, in blocks
#endif
#ifndef PKV_DECODE_WAVES_PER_SIMD
#define PKV_DECODE_WAVES_PER_SIMD 2
#endif
#ifndef PKV_DECODE_DEPTH
#define PKV_DECODE_DEPTH 2             // blocks in flight per wave
#endif
constexpr int kDecodeWaves = PKV_DECODE_WAVES;
constexpr int kDecodeDepth = PKV_DECODE_DEPTH;

// Queries of sequence b seen by the decode path (at most 16 * RBW rows) and
// the positions they see: [0, kv_end).
template <int RBW>
__device__ __forceinline__ int decode_kv_end(const AttnArgs& a, int b, int* q0_out, int* n_b_out,
                                             int* rows_out) {
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
  const int rows = max(0, min(min(n_b, a.max_q) * a.group, 16 * RBW));
  *rows_out = rows;
  if (rows <= 0) return 0;
  return min(a.seq_lens[b] - n_b + (rows - 1) / a.group + 1, a.kv_cap);
}

// Blocks per wave: the same in the attention and merge kernels.
__device__ __forceinline__ int decode_per(int total, int waves, int min_blocks) {
  return max(min_blocks, (total + waves - 1) / waves);
}

typedef __bf16 dec_bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) dec_bf16x4 lds_dec_bf16x4;

// INT8 pages: a block is half the bytes, so a wave spends relatively longer
// waiting; twice the waves keep the same bytes in flight.
#ifndef PKV_DECODE_DEPTH_I8
#define PKV_DECODE_DEPTH_I8 2
#endif
#ifndef PKV_DECODE_WAVES_I8
#define PKV_DECODE_WAVES_I8 2048
#endif
#ifndef PKV_DECODE_WAVES_PER_SIMD_I8
#define PKV_DECODE_WAVES_PER_SIMD_I8 2
#endif

// LDS rows of the decode kernel's staged block.  bf16 (and INT8, staged as
// bf16): K and V rows padded by 32 bytes; the K operand read of MFMA step c
// takes dims 32 c + 8 g .. + 7 in lane group g, so it covers 64 contiguous
// bytes of each of 16 rows, and with this padding neither it nor the
// transposed V read has bank conflicts (gfx950's LDS has 128 banks).  fp32:
// K rows padded by 16 bytes, V rows by 32; 512-byte rows stay unpadded.
template <typename T, int D>
constexpr int dec_k_row_bytes() {
  return D * static_cast<int>(sizeof(T)) + (D * static_cast<int>(sizeof(T)) >= 512 ? 0 : (sizeof(T) == 2 ? 32 : 16));
}
template <typename T, int D>
constexpr int dec_v_row_bytes() {
  return D * static_cast<int>(sizeof(T)) + (D * static_cast<int>(sizeof(T)) >= 512 ? 0 : 32);
}
// bf16 pages stage V only: each lane loads its K operand straight from the pool.
template <typename T, int D, bool kI8>
constexpr int dec_lds_bytes() {
  return 16 * ((kI8 || sizeof(T) != 2 ? dec_k_row_bytes<T, D>() : 0) + dec_v_row_bytes<T, D>());
}

// kPageMode 0: page_size a power of two >= 16 (a 16-position block lies in
// one page); 1: a power of two < 16; 2: any other page size.  kI8: INT8
// pages (T is then the bf16 type of the queries and outputs).
template <typename T, int D, int RBW, int kPageMode, bool kI8>
__global__ __launch_bounds__(kWave, RBW == 1 ? (kI8 ? PKV_DECODE_WAVES_PER_SIMD_I8 : PKV_DECODE_WAVES_PER_SIMD)
                                             : 1) void paged_decode_kernel(
    AttnArgs args, int32_t* __restrict__ seq_blk, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ block_tables) {
  static_assert(!kI8 || sizeof(T) == 2, "INT8 pages take bf16 queries");
  constexpr int kEs = sizeof(T);
  using Ld = KvLoad<kI8>;
  constexpr int kLdB = sizeof(Ld);
  constexpr int kRowBytes = D * kEs;                    // bytes of a staged (LDS) row
  constexpr int kGRowBytes = kI8 ? D : kRowBytes;       // bytes of a pool row
  constexpr int kCpr = kGRowBytes / kLdB;               // load units per pool row
  constexpr int kLoads = 16 * kGRowBytes / (kLdB * kWave); // loads per lane per pool per block
  // fp32 rows of 128 elements: one block in flight (two would spill)
  constexpr int kDepth = kI8 ? PKV_DECODE_DEPTH_I8 : (kGRowBytes >= 512 ? 1 : kDecodeDepth);
  constexpr int kDl = D / 4;                            // dims per lane in the QK operands
  constexpr int kFragChunks = kDl * kEs / 16;           // 16-byte chunks of one lane's K fragment
  constexpr int kQkMfmas = kDl / Elem<T>::kQkPerMfma;
  constexpr int kDimBlocks = D / 16;
  constexpr int kRowsCap = 16 * RBW;
  constexpr int kKRow = dec_k_row_bytes<T, D>();
  constexpr int kVRow = dec_v_row_bytes<T, D>();
  static_assert(kLoads * kWave * kLdB == 16 * kGRowBytes, "block split");
  // bf16 pages: each lane loads its K fragment straight from the pool in the
  // MFMA operand layout (row lrow, dims 32 c + 8 lgrp .. + 7), so K skips LDS.
  constexpr bool kDirectK = !kI8 && kEs == 2;
  static_assert(!kDirectK || kLoads == kFragChunks, "direct K fragment");

  extern __shared__ __align__(16) char smem[];
  char* kst = smem;
  char* vst = smem + (kDirectK ? 0 : 16 * kKRow);
  const int lane = threadIdx.x;
  const int lrow = lane & 15;
  const int lgrp = lane >> 4;

  const int hkv = args.num_kv_heads;
  const int group = args.group;
  const int ps = args.page_size;
  const int ps_shift = args.ps_shift;
  const int n_seqs = args.n_seqs;
  const char* kbytes = static_cast<const char*>(args.k_pool);
  const char* vbytes = static_cast<const char*>(args.v_pool);

  // ---- the block list: each wave scans the sequences' block counts ----
  // nb(b) = 16-position blocks of sequence b per KV head.  Lane l of chunk c
  // handles sequence 64 c + l; wave 0 also writes the prefix seq_blk[] that
  // the merge kernel reads.
  // Queries of sequence b seen here (at most 16 * RBW rows) and the positions
  // they see, [0, kv_end) (the same rule as decode_kv_end, read through the
  // read-only kernel arguments so uniform indices use scalar loads).
  struct Unit {
    int q0, start, rows, kv_end;
  };
  auto unit_of = [&](int b) __attribute__((always_inline)) {
    Unit u;
    int n_b;
    if (cu_q) {
      u.q0 = cu_q[b];
      n_b = cu_q[b + 1] - u.q0;
    } else {
      u.q0 = b;
      n_b = 1;
    }
    u.rows = max(0, min(min(n_b, args.max_q) * group, 16 * RBW));
    u.start = seq_lens[b] - n_b;
    u.kv_end = u.rows > 0 ? min(u.start + (u.rows - 1) / group + 1, args.kv_cap) : 0;
    return u;
  };
  auto nb_of = [&](int b) __attribute__((always_inline)) {
    const int kv_end = unit_of(b).kv_end;
    return kv_end > 0 ? (kv_end + 15) >> 4 : 0;
  };
  int total_seq = 0;                       // blocks per KV head of all sequences
  for (int c0 = 0; c0 < n_seqs; c0 += kWave) {
    const int b = c0 + lane;
    const int nb = b < n_seqs ? nb_of(b) : 0;
    int incl = nb;                         // inclusive prefix within the chunk
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    if (blockIdx.x == 0 && b < n_seqs) seq_blk[b] = total_seq + incl - nb;
    total_seq += __builtin_amdgcn_readfirstlane(__shfl(incl, kWave - 1));
  }
  if (blockIdx.x == 0 && lane == 0) seq_blk[n_seqs] = total_seq;

  // ---- this wave's block range ----
  const int total = total_seq * hkv;
  const int per = decode_per(total, gridDim.x, args.split_len);
  const int i0 = blockIdx.x * per;
  if (i0 >= total) return;
  const int i1 = min(total, i0 + per);

  // A position in the block list: sequence b, KV head g, block j of nb.
  struct Cur {
    int b, g, j, nb;
  };
  auto locate = [&](int i) __attribute__((always_inline)) {
    // the sequence whose blocks hold i: first b with (prefix through b) * hkv > i
    int base = 0;
    Cur c;
    c.b = 0;
    c.nb = 0;
    for (int c0 = 0; c0 < n_seqs; c0 += kWave) {
      const int b = c0 + lane;
      const int nb = b < n_seqs ? nb_of(b) : 0;
      int incl = nb;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int v = __shfl_up(incl, off);
        if (lane >= off) incl += v;
      }
      const unsigned long long hit = __ballot((base + incl) * hkv > i);
      if (hit) {
        const int l = __builtin_ctzll(hit);
        c.b = __builtin_amdgcn_readfirstlane(c0 + l);
        c.nb = __builtin_amdgcn_readfirstlane(__shfl(nb, l));
        base += __builtin_amdgcn_readfirstlane(__shfl(incl, l)) - c.nb;
        break;
      }
      base += __builtin_amdgcn_readfirstlane(__shfl(incl, kWave - 1));
    }
    const int r = i - base * hkv;
    c.g = r / c.nb;
    c.j = r - c.g * c.nb;
    return c;
  };
  auto advance = [&](Cur& c) __attribute__((always_inline)) {
    if (++c.j < c.nb) return;
    c.j = 0;
    if (++c.g < hkv) return;
    c.g = 0;
    do {
      c.b = __builtin_amdgcn_readfirstlane(c.b + 1);
      c.nb = __builtin_amdgcn_readfirstlane(nb_of(c.b));
    } while (c.nb == 0 && c.b + 1 < n_seqs);
  };


  // Query rows (B operand of S^T = K Q^T): row r = (query r / group, head
  // g * group + r % group); this lane holds row rb * 16 + lrow, for MFMA
  // step c dims 32 c + 8 lgrp .. + 7 (bf16; fp32: dims lgrp * kDl .. + kDl,
  // the same assignment as K).  Branch-free: a row without a query reads the
  // batch's first query (finite values; its result is never written), and
  // the loaded values are not touched until the unit is computed, so the
  // loads stay in flight behind the K/V loads.
  auto load_q = [&](int b, int g, const Unit& u, QkFrag<T, kDl> (&qv)[RBW], int (&qpos)[RBW]) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      const int r = rb * 16 + lrow;
      const int qi = r / group;
      const int tok = u.q0 + qi;
      const bool ok = r < u.rows && tok < args.total_q;
      qpos[rb] = u.start + (r < u.rows ? qi : -1);
      const int tok_c = ok ? tok : 0;
      const int hh = ok ? g * group + (r - qi * group) : 0;
      const T* src = static_cast<const T*>(args.q) + (static_cast<int64_t>(tok_c) * args.num_q_heads + hh) * D +
                     (kEs == 2 ? lgrp * 8 : lgrp * kDl);
#pragma unroll
      for (int c = 0; c < kFragChunks; ++c)
        qv[rb].load16(c, *reinterpret_cast<const u32x4*>(src + (kEs == 2 ? c * 32 : c * 4)));
    }
  };

  // Issue the loads of the block at cursor c (kv_end: its unit's).  Load ci
  // of a lane covers load unit q % kCpr of row q / kCpr (q = ci * 64 +
  // lane): consecutive lanes read consecutive bytes of whole rows.  okm marks
  // the rows inside the unit.  INT8 pages: the lane also loads the key and
  // value scales of positions 4 lgrp .. 4 lgrp + 3 of the block, the rows
  // its score and probability registers hold; they are issued first, so the
  // wait for the block's rows covers them.
  const uint32_t head_bytes = static_cast<uint32_t>(args.head_bytes);
  const uint32_t scale_off = static_cast<uint32_t>(ps) * D;   // INT8: scales follow the codes
  auto load_block = [&](const Cur& c, int kv_end, int page_hint, Ld (&kr)[kLoads], Ld (&vr)[kLoads],
                        uint32_t& okm, f32x4& ks, f32x4& vs) __attribute__((always_inline)) {
    const int pos0 = 16 * c.j;
    const int32_t* bt_row = block_tables + static_cast<int64_t>(c.b) * args.bt_stride;
    okm = 0;
    if constexpr (kPageMode == 0) {
      const uint32_t page = static_cast<uint32_t>(min(max(page_hint, 0), args.num_pages - 1));
      const uint64_t head = static_cast<uint64_t>(page * hkv + c.g) * head_bytes;
      const uint32_t row0 = pos0 & (ps - 1);
      if constexpr (kI8) {
        const uint32_t so = scale_off + 4 * (row0 + 4 * lgrp);
        ks = *reinterpret_cast<const f32x4*>(kbytes + head + so);
        vs = *reinterpret_cast<const f32x4*>(vbytes + head + so);
      }
      const uint64_t base = head + row0 * kGRowBytes;
#pragma unroll
      for (int ci = 0; ci < kLoads; ++ci) {
        const int q = ci * kWave + lane;
        const int r = q / kCpr;
        okm |= (pos0 + r < kv_end) ? (1u << ci) : 0u;
        const uint32_t off = r * kGRowBytes + (q % kCpr) * kLdB;
        const uint32_t koff = kDirectK ? lrow * kGRowBytes + (ci * 4 + lgrp) * 16 : off;
        kr[ci] = ld_stream(reinterpret_cast<const Ld*>(kbytes + base + koff));
        vr[ci] = ld_stream(reinterpret_cast<const Ld*>(vbytes + base + off));
      }
    } else {
      if constexpr (kI8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int pos = min(pos0 + 4 * lgrp + i, kv_end - 1);
          const int blk = kPageMode == 1 ? (pos >> ps_shift) : pos / ps;
          const int page = min(max(bt_row[blk], 0), args.num_pages - 1);
          const uint64_t e = static_cast<uint64_t>(page * hkv + c.g) * head_bytes + scale_off + 4 * (pos - blk * ps);
          ks[i] = *reinterpret_cast<const float*>(kbytes + e);
          vs[i] = *reinterpret_cast<const float*>(vbytes + e);
        }
      }
#pragma unroll
      for (int ci = 0; ci < kLoads; ++ci) {
        const int q = ci * kWave + lane;
        const int r = q / kCpr;
        const int pos_raw = pos0 + r;
        const int pos = min(pos_raw, kv_end - 1);
        const int blk = kPageMode == 1 ? (pos >> ps_shift) : pos / ps;
        const int page = min(max(bt_row[blk], 0), args.num_pages - 1);
        okm |= (pos_raw < kv_end) ? (1u << ci) : 0u;
        const uint64_t e = static_cast<uint64_t>(page * hkv + c.g) * head_bytes + (pos - blk * ps) * kGRowBytes +
                           (q % kCpr) * kLdB;
        vr[ci] = ld_stream(reinterpret_cast<const Ld*>(vbytes + e));
        if constexpr (kDirectK) {
          const int kpos = min(pos0 + lrow, kv_end - 1);
          const int kblk = kPageMode == 1 ? (kpos >> ps_shift) : kpos / ps;
          const int kpage = min(max(bt_row[kblk], 0), args.num_pages - 1);
          const uint64_t ke = static_cast<uint64_t>(kpage * hkv + c.g) * head_bytes + (kpos - kblk * ps) * kGRowBytes +
                              (ci * 4 + lgrp) * 16;
          kr[ci] = ld_stream(reinterpret_cast<const Ld*>(kbytes + ke));
        } else {
          kr[ci] = ld_stream(reinterpret_cast<const Ld*>(kbytes + e));
        }
      }
    }
  };
  // page of the block at cursor c (page mode 0: one page per block)
  auto page_of = [&](const Cur& c) __attribute__((always_inline)) {
    const int b = __builtin_amdgcn_readfirstlane(c.b);
    const int blk = __builtin_amdgcn_readfirstlane((16 * c.j) >> max(ps_shift, 0));
    return block_tables[static_cast<int64_t>(b) * args.bt_stride + blk];
  };

  // Write a block's rows into the wave's LDS slices.  V rows past the unit
  // are zeroed (their probability is 0, but stale slots may hold anything,
  // NaN included); K rows need no zeroing, their scores are masked.  INT8
  // codes are widened to bf16 here (every code is finite; a row past the
  // unit gets value scale 0 instead).
  auto stage_block = [&](const Ld (&kr)[kLoads], const Ld (&vr)[kLoads], uint32_t okm) __attribute__((always_inline)) {
#pragma unroll
    for (int ci = 0; ci < kLoads; ++ci) {
      const int q = ci * kWave + lane;
      const int r = q / kCpr;
      const int cc = q % kCpr;
      if constexpr (kI8) {
        *reinterpret_cast<u32x4*>(kst + r * kKRow + cc * 16) = i8x8_to_bf16(kr[ci]);
        *reinterpret_cast<u32x4*>(vst + r * kVRow + cc * 16) = i8x8_to_bf16(vr[ci]);
      } else {
        const unsigned keep = 0u - ((okm >> ci) & 1u);   // all ones or zero
        if constexpr (!kDirectK) *reinterpret_cast<u32x4*>(kst + r * kKRow + cc * 16) = kr[ci];
        *reinterpret_cast<u32x4*>(vst + r * kVRow + cc * 16) = vr[ci] & keep;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // ---- online softmax state of the current segment (log2 domain) ----
  float m_run[RBW], m_use[RBW], l_part[RBW];   // m_use: m_run, or 0 while it is -inf
  f32x4 o_acc[RBW][kDimBlocks];
  auto reset_state = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      m_run[rb] = -INFINITY;
      m_use[rb] = 0.f;
      l_part[rb] = 0.f;
#pragma unroll
      for (int d = 0; d < kDimBlocks; ++d) o_acc[rb][d] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };

  // ks, vs (INT8 pages): key and value scales of this lane's positions
  // pos0 + 4 lgrp + i.  The key scale multiplies the scores, the value scale
  // the probabilities entering O^T (not the row sums).
  auto compute_block = [&](int pos0, int kv_end, const QkFrag<T, kDl> (&qv)[RBW], const int (&qpos)[RBW],
                           f32x4 ks, f32x4 vs, const Ld (&kreg)[kLoads]) __attribute__((always_inline)) {
    // K fragment: position lrow, the dims this lane's query fragment holds
    // (bf16 pages: the loaded registers themselves)
    QkFrag<T, kDl> kf;
#pragma unroll
    for (int c = 0; c < kFragChunks; ++c) {
      if constexpr (kDirectK)
        kf.load16(c, kreg[c]);
      else
        kf.load16(c, *reinterpret_cast<const u32x4*>(kst + lrow * kKRow + (kEs == 2 ? c * 4 + lgrp : lgrp * kFragChunks + c) * 16));
    }
    f32x4 s[RBW];
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      s[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < kQkMfmas; ++kk) s[rb] = mfma_qk(kf.v[kk], qv[rb].v[kk], s[rb]);
    }
    f32x4 sc;                          // score scale of each of the lane's positions
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = kI8 ? ks[i] * args.scale_log2 : args.scale_log2;
    // The reference max of a row is raised only when a score exceeds it by
    // more than 8 (log2 units), so probabilities stay <= 256.  A row needs
    // that exactly when one of its lanes' 4 scores does: the cross-lane
    // reduction and the rescale sit in one rarely taken branch.
    float lmx[RBW];
    bool up_lane = false;
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pos = pos0 + lgrp * 4 + i;
        const float x = s[rb][i] * sc[i];
        s[rb][i] = (pos < kv_end && pos <= qpos[rb]) ? x : -INFINITY;
        mx = fmaxf(mx, s[rb][i]);
      }
      lmx[rb] = mx;
      up_lane = up_lane || mx > m_run[rb] + 8.f;
    }
    if (__any(up_lane)) {
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) {
        const float mx = max_xor32(max_xor16(lmx[rb]));
        const bool up = mx > m_run[rb] + 8.f;
        const float m_new = up ? mx : m_run[rb];
        const float alpha = up ? fast_exp2(m_run[rb] - m_new) : 1.f;
        m_run[rb] = m_new;
        m_use[rb] = m_new == -INFINITY ? 0.f : m_new;
        l_part[rb] *= alpha;
#pragma unroll
        for (int d = 0; d < kDimBlocks; ++d) o_acc[rb][d] *= alpha;
      }
    }
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[rb][i] = fast_exp2(s[rb][i] - m_use[rb]);
        psum += s[rb][i];
      }
      l_part[rb] += psum;
    }
    // O^T += V^T P^T
    if constexpr (sizeof(T) == 2) {
      i16x4 pb[RBW];
      if constexpr (kI8) {
        f32x4 vsm;                     // rows past the unit: scale 0 (stale scales may be NaN)
#pragma unroll
        for (int i = 0; i < 4; ++i) vsm[i] = pos0 + lgrp * 4 + i < kv_end ? vs[i] : 0.f;
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) pb[rb] = pack_bf16x4(s[rb] * vsm);
      } else {
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) pb[rb] = pack_bf16x4(s[rb]);
      }
      // lane k of a 16-lane group addresses row 4 lgrp + k / 4, dims 4 (k % 4)..;
      // it receives dim lrow of rows 4 lgrp .. 4 lgrp + 3
      const char* vl = vst + (4 * lgrp + (lrow >> 2)) * kVRow + (lrow & 3) * 8;
#pragma unroll
      for (int d = 0; d < kDimBlocks; ++d) {
        const dec_bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_dec_bf16x4*)(vl + d * 32));
        const i16x4 a = __builtin_bit_cast(i16x4, v);
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
          const float a = *reinterpret_cast<const float*>(vst + (lgrp * 4 + i) * kVRow + dim * 4);
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

  // End of a segment of unit (b, g): normalised output when it covers the
  // unit, else the partial state in slot unit + wave.
  auto write_segment = [&](int b, int g, const Unit& u, bool whole) __attribute__((always_inline)) {
    const int slot = b * hkv + g + static_cast<int>(blockIdx.x);
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      const float l_row = sum_xor32(sum_xor16(l_part[rb]));
      const int r = rb * 16 + lrow;
      if (r >= u.rows) continue;
      const int qi = r / group;
      const int tok = u.q0 + qi;
      if (tok >= args.total_q) continue;
      const int64_t orow = static_cast<int64_t>(tok) * args.num_q_heads + g * group + (r - qi * group);
      if (whole) {
        const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
#pragma unroll
        for (int d = 0; d < kDimBlocks; ++d) {
          const f32x4 v = o_acc[rb][d] * inv;
          if constexpr (sizeof(T) == 2)
            *reinterpret_cast<i16x4*>(static_cast<uint16_t*>(args.out) + orow * D + d * 16 + lgrp * 4) = pack_bf16x4(v);
          else
            *reinterpret_cast<f32x4*>(static_cast<float*>(args.out) + orow * D + d * 16 + lgrp * 4) = v;
        }
      } else {
        const int64_t row = static_cast<int64_t>(slot) * kRowsCap + r;
#pragma unroll
        for (int d = 0; d < kDimBlocks; ++d)
          *reinterpret_cast<f32x4*>(args.ws_o + row * D + d * 16 + lgrp * 4) = o_acc[rb][d];
        if (lgrp == 0) {
          args.ws_ml[row * 2] = m_run[rb];
          args.ws_ml[row * 2 + 1] = l_row;
        }
      }
    }
  };

  // ---- the walk ----
  Cur cc = locate(i0);              // block being computed
  Cur lc = cc;                      // block whose loads are issued next
  Ld kbuf[kDepth][kLoads], vbuf[kDepth][kLoads];
  f32x4 ksb[kDepth] = {}, vsb[kDepth] = {};   // INT8 scales
  uint32_t okm[kDepth];
  Unit ul = unit_of(lc.b);          // unit of the load cursor
  int page_l = kPageMode == 0 ? page_of(lc) : 0;
  auto issue = [&](int li, Ld (&kr)[kLoads], Ld (&vr)[kLoads], uint32_t& okm, f32x4& ks, f32x4& vs)
      __attribute__((always_inline)) {
    load_block(lc, ul.kv_end, page_l, kr, vr, okm, ks, vs);
    if (li + 1 < i1) {              // move the load cursor on (it stays on the last block)
      const int b_old = lc.b;
      advance(lc);
      if (lc.b != b_old) ul = unit_of(lc.b);
      if constexpr (kPageMode == 0) page_l = page_of(lc);
    }
  };
#pragma unroll
  for (int d = 0; d < kDepth; ++d) issue(i0 + d, kbuf[d], vbuf[d], okm[d], ksb[d], vsb[d]);

  Unit uc = unit_of(cc.b);
  // The unit's queries load at its start (a wave's range meets few units);
  // they are first used by the next block's MFMAs, so the wait for them
  // leaves that block's K/V loads in flight.
  QkFrag<T, kDl> qv[RBW];
  int qpos[RBW];
  load_q(cc.b, cc.g, uc, qv, qpos);
  int seg_first = cc.j;             // block at which the current segment started
  reset_state();

  // One step: stage block ii from its registers, issue block ii + depth into
  // them, compute block ii, and close the segment at a unit's or the range's
  // end.
  auto step = [&](int ii, Ld (&kr)[kLoads], Ld (&vr)[kLoads], uint32_t& om, f32x4& ks, f32x4& vs)
      __attribute__((always_inline)) {
    stage_block(kr, vr, om);
    const f32x4 ks_c = ks, vs_c = vs;   // the buffer is refilled below
    Ld kc[kLoads];
#pragma unroll
    for (int ci = 0; ci < kLoads; ++ci) kc[ci] = kr[ci];
    issue(ii + kDepth, kr, vr, om, ks, vs);
    compute_block(16 * cc.j, uc.kv_end, qv, qpos, ks_c, vs_c, kc);
    const bool unit_end = cc.j == cc.nb - 1;
    if (unit_end || ii + 1 == i1) {
      write_segment(cc.b, cc.g, uc, seg_first == 0 && unit_end);
      if (ii + 1 < i1) {            // on to the next unit
        advance(cc);
        uc = unit_of(cc.b);
        load_q(cc.b, cc.g, uc, qv, qpos);
        seg_first = 0;
        reset_state();
      }
    } else {
      advance(cc);
    }
  };
  // Whole groups of `depth` steps, then the last few: every path back to the
  // top of the loop has issued all buffers' loads, so each staging waits for
  // the oldest buffer only.
  int i = i0;
  for (; i + kDepth <= i1; i += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) step(i + d, kbuf[d], vbuf[d], okm[d], ksb[d], vsb[d]);
  }
#pragma unroll
  for (int d = 0; d < kDepth - 1; ++d)
    if (i + d < i1) step(i + d, kbuf[d], vbuf[d], okm[d], ksb[d], vsb[d]);
}

// ---------------------------------------------------------------------------
// Paged prefill/append in bf16 for more than 48 query rows per sequence and
// KV head.
//  * A workgroup of 8 waves owns 256 query rows of one (sequence, KV head)
//    unit, with 128-position tiles, one workgroup per CU (when no context
//    exceeds kPfStreamCtx positions the persistent kernel further below takes
//    the launch instead).  Rows are (query,
//    head-in-group) pairs, so every K/V byte it stages serves the whole GQA
//    group.  Wave w owns rows 32w..32w+31 as two 16-row MFMA blocks and keeps
//    its own softmax state: no cross-wave combine.
//  * K/V tiles are gathered through the block table with
//    16-byte loads into registers one tile ahead and written to one of two
//    LDS buffers.  K and V rows are padded to D*2 + 32 bytes.  MFMA step kk
//    of S^T = K Q^T takes dims 32 kk + 8 g .. 32 kk + 8 g + 7 in lane group
//    g, so one K read covers 64 contiguous bytes of each of 16 rows; with
//    that padding neither it nor the transposed V read has bank conflicts
//    (the counters read 0.9% of busy cycles, against 10.4% with K rows of
//    D*2 + 16 and dims 32 g + 8 kk ..).
//    One barrier per tile; block-table entries are fetched a tile earlier
//    still.  When a power-of-two page holds all rows a wave stages in one
//    pass, the page lookup is scalar and each lane adds a 32-bit offset.
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 with Q held in registers.  A
//    lane then holds one query row and 4 positions of each 16-key block.
//    The reference max of a row is raised only when a tile's max exceeds it
//    by more than 8 (log2 units), so probabilities stay <= 256.  That holds
//    for the row exactly when it holds for one of its lanes' 16 scores, so
//    the two-shuffle row reduction and the rescale sit in one branch that
//    most tiles skip.
//  * O^T += V^T P^T on the same MFMA.  P^T is already in B-operand layout
//    once the MFMA's k index is permuted the same way on both operands
//    (k-slots 8g..8g+3 <-> keys 4g..4g+3 of the first 16-key block, 8g+4..
//    8g+7 <-> the same of the second), and V^T comes straight out of LDS with
//    ds_read_b64_tr_b16.  Row sums run on the MFMA as well (a ones operand
//    times P^T), from the same bf16 P the numerator uses.  The exponentials,
//    the row sums and the PV products of a tile form one basic block, so the
//    scheduler can overlap VALU and MFMA work.
//  * Workgroups are dealt to the 8 XCDs round robin, so workgroup i serves
//    unit i % 8 of a block of 8 units: all q-tiles of a unit run on one XCD
//    and re-read its K/V from that XCD's L2.  Within a block the tiles with
//    the most keys go first.  A one-workgroup schedule kernel lists the
//    blocks' tile counts; the grid is a host-side upper bound and surplus
//    workgroups exit at once.
// ---------------------------------------------------------------------------
#ifndef PKV_PREFILL_ROW_BLOCKS
#define PKV_PREFILL_ROW_BLOCKS 2
#endif
#ifndef PKV_PREFILL_WAVES
#define PKV_PREFILL_WAVES 8
#endif
constexpr int kPfRb = PKV_PREFILL_ROW_BLOCKS;   // 16-row MFMA blocks per wave
constexpr int kPfWaves = PKV_PREFILL_WAVES;
#ifndef PKV_PREFILL_KEYS
#define PKV_PREFILL_KEYS 128
#endif
constexpr int kPfKeys = PKV_PREFILL_KEYS;   // positions per staged tile (computed 64 at a time)
constexpr int kPfMaxRows = 16 * kPfRb * kPfWaves;   // rows per workgroup of the tiled kernel
// Contexts up to kPfStreamCtx positions take the persistent stream kernel
// (paged_prefill_stream_kernel): kPfStreamWaves waves, kPfStreamKeys-position
// tiles.
#ifndef PKV_PREFILL_STREAM_CTX
#define PKV_PREFILL_STREAM_CTX 2048
#endif
#ifndef PKV_PREFILL_STREAM_WAVES
#define PKV_PREFILL_STREAM_WAVES 8
#endif
#ifndef PKV_PREFILL_STREAM_KEYS
#define PKV_PREFILL_STREAM_KEYS 64
#endif
constexpr int kPfStreamCtx = PKV_PREFILL_STREAM_CTX;
constexpr int kPfStreamWaves = PKV_PREFILL_STREAM_WAVES;
constexpr int kPfStreamKeys = PKV_PREFILL_STREAM_KEYS;

template <int D>
constexpr int pf_k_row_bytes() { return D * 2 + 32; }
template <int D>
constexpr int pf_v_row_bytes() { return D * 2 + 32; }
// LDS of one staged K + V buffer, two buffers per workgroup.  INT8 codes are
// staged as bf16 in the same layout, followed by the tile's key scales and
// value scales (fp32, kKeys of each).
template <int D, int kKeys, bool kI8>
constexpr int pf_buf_bytes() { return kKeys * (pf_k_row_bytes<D>() + pf_v_row_bytes<D>()) + (kI8 ? 8 * kKeys : 0); }
template <int D, int kKeys, bool kI8>
constexpr int pf_lds_bytes() { return 2 * pf_buf_bytes<D, kKeys, kI8>(); }
// Rows one wave stages per pass (a pass = one 16-byte chunk per thread).
template <int D, bool kI8>
constexpr int pf_wave_rows() { return kWave / (D * (kI8 ? 1 : 2) / static_cast<int>(sizeof(KvLoad<kI8>))); }

// row_off[k] = sum over blocks < k of (q-tiles of the block) * n_splits,
// where a block's q-tiles are the most any of its 8 units needs.  With `rec`
// (the persistent short-append launch) it also writes one record per work
// item id = 8 * row + slot: int32 {b, g, q0, n_b, start, row0, kv_end, split},
// b = -1 for an item with no work.  One workgroup of kSchedThreads threads,
// one block per thread per pass: a block's 8 units read their sequence
// bounds with independent loads before any record is stored, so a pass
// waits on memory once.  The prefix over a pass's blocks is taken within
// each wave (lane shuffles) and then over the 16 wave totals: two barriers
// per pass.  With several workgroups (the persistent launch) each one takes
// the whole prefix and stores the records of every gridDim.x-th block, so
// the record stores (16-byte pieces 256 bytes apart across lanes) are
// issued from that many CUs; workgroup 0 writes row_off.
constexpr int kSchedThreads = 1024;
constexpr int kSchedRecGroups = 16;
__global__ __launch_bounds__(kSchedThreads) void prefill_schedule_kernel(AttnArgs a, int32_t* row_off,
                                                                         int n_blocks, int tile_rows,
                                                                         int32_t* __restrict__ rec) {
  __shared__ int s_wsum[kSchedThreads / kWave];
  __shared__ int s_carry;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const bool off_writer = blockIdx.x == 0;
  if (tid == 0) {
    s_carry = 0;
    if (off_writer) row_off[0] = 0;
  }
  __syncthreads();
  const int units = a.n_seqs * a.num_kv_heads;
  for (int base = 0; base < n_blocks; base += kSchedThreads) {
    const int blk = base + tid;
    int sb[8], sq0[8], snb[8], sstart[8];
    int tiles = 0;
#pragma unroll
    for (int slot = 0; slot < 8; ++slot) {
      const int u = blk * 8 + slot;
      const bool ok = blk < n_blocks && u < units;
      const int b = ok ? u / a.num_kv_heads : 0;
      const int q0 = a.cu_q[b];
      const int q1 = a.cu_q[b + 1];
      const int len = a.seq_lens[b];
      sb[slot] = ok ? b : -1;
      sq0[slot] = q0;
      snb[slot] = q1 - q0;
      sstart[slot] = len - (q1 - q0);
      if (ok) tiles = max(tiles, (min(q1 - q0, a.max_q) * a.group + tile_rows - 1) / tile_rows);
    }
    const int v = tiles * a.n_splits;
    // inclusive scan of v: within each wave, then over the waves' totals
    int incl = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int w = __shfl_up(incl, off);
      if (lane >= off) incl += w;
    }
    if (lane == kWave - 1) s_wsum[wave] = incl;
    __syncthreads();
    if (wave == 0) {
      int t = lane < kSchedThreads / kWave ? s_wsum[lane] : 0;
#pragma unroll
      for (int off = 1; off < kSchedThreads / kWave; off <<= 1) {
        const int w = __shfl_up(t, off);
        if (lane >= off) t += w;
      }
      if (lane < kSchedThreads / kWave) s_wsum[lane] = t;
    }
    __syncthreads();
    const int scan = (wave > 0 ? s_wsum[wave - 1] : 0) + incl;
    if (off_writer && blk < n_blocks) row_off[blk + 1] = s_carry + scan;
    if (rec && blk < n_blocks && blk % static_cast<int>(gridDim.x) == static_cast<int>(blockIdx.x)) {
      const int r0 = s_carry + scan - v;
#pragma unroll
      for (int slot = 0; slot < 8; ++slot) {
        const int b = sb[slot];
        const int n_b = snb[slot];
        const int rows_total = b >= 0 ? min(n_b, a.max_q) * a.group : 0;
        const int u = blk * 8 + slot;
        for (int local = 0; local < v; ++local) {
          const int qt = tiles - 1 - local / a.n_splits;
          const int split = local - (local / a.n_splits) * a.n_splits;
          const int row0 = qt * tile_rows;
          int kv_end = 0;
          bool ok = b >= 0 && row0 < rows_total;
          if (ok) {
            kv_end = min(sstart[slot] + (min(row0 + tile_rows, rows_total) - 1) / a.group + 1, a.kv_cap);
            ok = split * a.split_len < kv_end;
          }
          int32_t* o = rec + 8 * (static_cast<int64_t>(r0 + local) * 8 + slot);
          *reinterpret_cast<int4*>(o) =
              ok ? make_int4(b, u - b * a.num_kv_heads, sq0[slot], n_b) : make_int4(-1, 0, 0, 0);
          *reinterpret_cast<int4*>(o + 4) = make_int4(sstart[slot], row0, kv_end, split);
        }
      }
    }
    __syncthreads();
    if (tid == 0) s_carry += s_wsum[kSchedThreads / kWave - 1];
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

// One 64-key sub-tile of the attention core both prefill kernels share, for
// the wave's kPfRb 16-row blocks: S^T = K Q^T, the online softmax (the
// reference max of a row is raised only when a tile's max exceeds it by more
// than 8, log2 units; one rarely taken rescale branch for all row blocks) and
// O^T += V^T P^T, with the row sums from the same bf16 P.  kt, vt: the
// sub-tile's staged K and V rows; sk (INT8): its key scales, value scales at
// sk + kKeys; tb: the position of its first key; k_lane, v_lane: this lane's
// parts of the LDS operand addresses; mc, mu: each row's reference max (log2
// units) and the same with -inf replaced by 0, the value the exponents
// subtract.  kMask 0: no key is past any row's position; 1: causal mask;
// 2: causal mask, and every key of the upper 32 is past every row's
// position, so only the lower 32 are computed (the skipped keys would add
// exact zeros: the result is the same bit for bit).  kSwz: rows of D * 2
// bytes whose 16-byte chunks are XOR-permuted by the row's low 4 bits (the
// ring layout of the persistent kernel); koff, voff then hold the lane's
// K and V^T read offsets per MFMA step and per 16-dim block.
template <int D, int kKeys, bool kI8, int kMask, bool kSwz = false>
__device__ __forceinline__ void pf_sub_tile(const char* kt, const char* vt, const float* sk, int tb, int lgrp,
                                            int k_lane, int v_lane, float c2, const bf16x8& ones,
                                            const bf16x8 (&qf)[kPfRb][D / 32], const int (&qpos)[kPfRb],
                                            f32x4 (&o)[D / 16][kPfRb], f32x4 (&lsum)[kPfRb],
                                            float (&mc)[kPfRb], float (&mu)[kPfRb], float (&mt)[kPfRb],
                                            const int* koff = nullptr, const int* voff = nullptr) {
  constexpr int kKRowB = kSwz ? D * 2 : pf_k_row_bytes<D>();
  constexpr int kVRowB = kSwz ? D * 2 : pf_v_row_bytes<D>();
  constexpr int kQk = D / 32;
  constexpr int kDb = D / 16;
  constexpr int kKb = kMask == 2 ? 2 : 4;   // 16-key blocks computed
  f32x4 s[4][kPfRb];
#pragma unroll
  for (int kb = 0; kb < kKb; ++kb) {
    bf16x8 kf[kQk];
#pragma unroll
    for (int kk = 0; kk < kQk; ++kk)
      kf[kk] = *reinterpret_cast<const bf16x8*>(kt + kb * 16 * kKRowB + (kSwz ? koff[kk] : k_lane + kk * 64));
#pragma unroll
    for (int rb = 0; rb < kPfRb; ++rb) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < kQk; ++kk) acc = mfma_qk(kf[kk], qf[rb][kk], acc);
      s[kb][rb] = acc;
    }
  }
  if constexpr (kI8) {
    // INT8: each score becomes its exponent argument at once, score times
    // (key scale * c2) minus the row's reference, one fused multiply-add
    // (lane keys kb * 16 + 4 lgrp + i); the maxima below are taken over
    // these arguments
#pragma unroll
    for (int kb = 0; kb < kKb; ++kb) {
      const f32x4 kc = *reinterpret_cast<const f32x4*>(sk + kb * 16 + 4 * lgrp) * c2;
#pragma unroll
      for (int rb = 0; rb < kPfRb; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[kb][rb][i] = __builtin_fmaf(s[kb][rb][i], kc[i], -mu[rb]);
    }
  }
  // Lane-local maxima decide.  A row's maximum exceeds its reference by more
  // than 8 exactly when one of its lanes' local maxima does (rounding the
  // product with c2 > 0 is monotone), so the cross-lane reduction, the new
  // reference and the rescale all sit in one rarely taken branch.
  float lmx[kPfRb];
  bool up_lane = false;
#pragma unroll
  for (int rb = 0; rb < kPfRb; ++rb) {
    if constexpr (kMask != 0) {
#pragma unroll
      for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          s[kb][rb][i] = (tb + kb * 16 + 4 * lgrp + i <= qpos[rb]) ? s[kb][rb][i] : -INFINITY;
    }
    // a linear chain folds into three-input maxima (v_max3_f32)
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 4 * kKb; e += 2) mx = fmaxf(fmaxf(mx, s[e >> 2][rb][e & 3]), s[e >> 2][rb][(e & 3) + 1]);
    lmx[rb] = mx;
    if constexpr (kI8)
      up_lane = up_lane || mx > mt[rb] - mu[rb];
    else
      up_lane = up_lane || mx * c2 > mt[rb];
  }
  if (__any(up_lane)) {
#pragma unroll
    for (int rb = 0; rb < kPfRb; ++rb) {
      const float mxr = max_xor32(max_xor16(lmx[rb]));
      const float mxc = kI8 ? mxr + mu[rb] : mxr * c2;
      const bool up = mxc > mt[rb];
      const float mnew = up ? mxc : mc[rb];
      const float alpha = up ? fast_exp2(mc[rb] - mnew) : 1.f;
      const float mu_new = mnew == -INFINITY ? 0.f : mnew;
      if constexpr (kI8) {
        // the arguments move with the reference
        const float shift = mu[rb] - mu_new;
#pragma unroll
        for (int kb = 0; kb < kKb; ++kb) s[kb][rb] += shift;
      }
      mc[rb] = mnew;
      mu[rb] = mu_new;
      mt[rb] = mnew + 8.f;
      lsum[rb] *= alpha;
#pragma unroll
      for (int d = 0; d < kDb; ++d) o[d][rb] *= alpha;
    }
  }
#pragma unroll
  for (int ks = 0; ks < kKb / 2; ++ks) {
    bf16x8 pk[kPfRb];   // probabilities: row sums (and PV for bf16 pages)
    bf16x8 pv[kPfRb];   // INT8: probabilities times the value scales, for PV
    f32x4 vs0, vs1;     // INT8: value scales of this lane's keys
    if constexpr (kI8) {
      vs0 = *reinterpret_cast<const f32x4*>(sk + kKeys + 32 * ks + 4 * lgrp);
      vs1 = *reinterpret_cast<const f32x4*>(sk + kKeys + 32 * ks + 16 + 4 * lgrp);
    }
#pragma unroll
    for (int rb = 0; rb < kPfRb; ++rb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e0 = fast_exp2(kI8 ? s[2 * ks][rb][i] : fmaf(s[2 * ks][rb][i], c2, -mu[rb]));
        const float e1 = fast_exp2(kI8 ? s[2 * ks + 1][rb][i] : fmaf(s[2 * ks + 1][rb][i], c2, -mu[rb]));
        pk[rb][i] = static_cast<__bf16>(e0);
        pk[rb][4 + i] = static_cast<__bf16>(e1);
        if constexpr (kI8) {
          pv[rb][i] = static_cast<__bf16>(e0 * vs0[i]);
          pv[rb][4 + i] = static_cast<__bf16>(e1 * vs1[i]);
        }
      }
      lsum[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pk[rb], lsum[rb], 0, 0, 0);
    }
#pragma unroll
    for (int d = 0; d < kDb; ++d) {
      const char* vp = vt + 32 * ks * kVRowB + (kSwz ? voff[d] : v_lane + d * 32);
      const bf16x4 v0 = lds_read_tr(vp);
      const bf16x4 v1 = lds_read_tr(vp + 16 * kVRowB);
      const bf16x8 vf = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int rb = 0; rb < kPfRb; ++rb)
        o[d][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, kI8 ? pv[rb] : pk[rb], o[d][rb], 0, 0, 0);
    }
  }
}

// kPageMode 0: page_size a power of two >= the rows a wave stages per pass
// (those rows then share one page: scalar lookup); 1: other powers of two;
// 2: any page size.  kI8: INT8 pages (TileInfer.jl docs, "KV cache", "INT8
// cache"): the codes are staged as bf16 (exact, |code| <= 127), each score
// is multiplied by its key's scale before the softmax, and each probability
// by its value's scale before it enters O^T; the row sums take the unscaled
// probabilities.
template <int D, int kPageMode, int kPfThreads, int kPfKeys, bool kI8>
__global__ __launch_bounds__(kPfThreads, kPfRb >= 3 ? 1 : 2) void paged_prefill_kernel(AttnArgs a,
                                                                   const int32_t* __restrict__ row_off,
                                                                   int n_blocks) {
  constexpr int kPfRows = 16 * kPfRb * (kPfThreads / kWave);   // query rows per workgroup
  constexpr int kKRowB = pf_k_row_bytes<D>();            // LDS row strides, bytes
  constexpr int kVRowB = pf_v_row_bytes<D>();
  using Ld = KvLoad<kI8>;
  constexpr int kLdB = sizeof(Ld);
  constexpr int kGRowB = D * (kI8 ? 1 : 2);             // bytes of a pool row
  constexpr int kCpr = kGRowB / kLdB;                   // load units per pool row
  constexpr int kChunks = kPfKeys * kCpr / kPfThreads;  // per thread per pool
  constexpr int kRowsPerPass = kPfThreads / kCpr;       // rows staged per chunk index
  constexpr int kQk = D / 32;                           // MFMAs per 16x16 score block
  constexpr int kDb = D / 16;                           // 16-dim blocks of O^T
  constexpr int kKTileB = kPfKeys * kKRowB;             // bytes of one staged K tile
  constexpr int kBufB = pf_buf_bytes<D, kPfKeys, kI8>();  // one K + V buffer
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
  const int kv_end = min(start + (min(row0 + kPfRows, rows_total) - 1) / group + 1, a.kv_cap);
  const int k_lo = split * a.split_len;
  if (k_lo >= kv_end) return;
  const int k_hi = min(k_lo + a.split_len, kv_end);
  const int n_tiles = (k_hi - k_lo + kPfKeys - 1) / kPfKeys;

  // ---- staging: this thread's rows srow0 + c * kRowsPerPass, load unit spart ----
  const int ps = a.page_size;
  const int ps_shift = a.ps_shift;
  const int32_t* bt_row = a.block_tables + static_cast<int64_t>(b) * a.bt_stride;
  const uint32_t head_bytes = static_cast<uint32_t>(a.head_bytes);   // one (page, head) block
  const uint32_t scale_off = static_cast<uint32_t>(ps) * D;           // INT8: scales follow the codes
  const char* kbytes = static_cast<const char*>(a.k_pool);
  const char* vbytes = static_cast<const char*>(a.v_pool);
  const int srow0 = tid / kCpr;
  const int spart = tid - srow0 * kCpr;
  // first row this wave stages in a pass (wave-uniform)
  const int wrow0 = __builtin_amdgcn_readfirstlane(srow0);

  int pg_next[kChunks], pg_next2[kChunks];
  Ld kr[kChunks], vr[kChunks];
  float ksr[kChunks], vsr[kChunks];   // INT8: the staged rows' scales
  // position of staged row `row` of tile t (past the split's end: its last position)
  auto pos_of = [&](int t, int row) __attribute__((always_inline)) {
    return min(k_lo + t * kPfKeys + row, k_hi - 1);
  };
  auto blk_of = [&](int pos) __attribute__((always_inline)) {
    if constexpr (kPageMode <= 1) return pos >> ps_shift;
    else return pos / ps;
  };
  auto fetch_pages = [&](int t) __attribute__((always_inline)) {
    const int tl = min(t, n_tiles - 1);
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      if constexpr (kPageMode == 0)
        pg_next2[c] = bt_row[blk_of(pos_of(tl, wrow0 + c * kRowsPerPass))];
      else
        pg_next2[c] = bt_row[blk_of(pos_of(tl, srow0 + c * kRowsPerPass))];
    }
  };
  auto load_kv = [&](int t) __attribute__((always_inline)) {
    const int tl = min(t, n_tiles - 1);
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int pos = pos_of(tl, srow0 + c * kRowsPerPass);
      const uint32_t page = static_cast<uint32_t>(min(max(pg_next[c], 0), a.num_pages - 1));
      const uint32_t off = kPageMode <= 1 ? (pos & (ps - 1)) : (pos - blk_of(pos) * ps);
      const uint32_t voff = off * kGRowB + spart * kLdB;
      const uint64_t base = static_cast<uint64_t>(page * hkv + g) * head_bytes;
      if constexpr (kI8) {
        ksr[c] = *reinterpret_cast<const float*>(kbytes + base + scale_off + 4 * off);
        vsr[c] = *reinterpret_cast<const float*>(vbytes + base + scale_off + 4 * off);
      }
      kr[c] = *reinterpret_cast<const Ld*>(kbytes + base + voff);
      vr[c] = *reinterpret_cast<const Ld*>(vbytes + base + voff);
    }
  };
  auto stage = [&](int buf) __attribute__((always_inline)) {
    char* kb = smem + buf * kBufB;
    char* vb = kb + kKTileB;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int row = srow0 + c * kRowsPerPass;
      if constexpr (kI8) {
        // codes as exact bf16; part 0 of each row writes the row's scales
        *reinterpret_cast<u32x4*>(kb + row * kKRowB + spart * 16) = i8x8_to_bf16(kr[c]);
        *reinterpret_cast<u32x4*>(vb + row * kVRowB + spart * 16) = i8x8_to_bf16(vr[c]);
        if (spart == 0) {
          float* sc = reinterpret_cast<float*>(vb + kPfKeys * kVRowB);
          sc[row] = ksr[c];
          sc[kPfKeys + row] = vsr[c];
        }
      } else {
        *reinterpret_cast<u32x4*>(kb + row * kKRowB + spart * 16) = kr[c];
        *reinterpret_cast<u32x4*>(vb + row * kVRowB + spart * 16) = vr[c];
      }
    }
  };

  // ---- this lane's two query rows (B operand of S^T = K Q^T) ----
  // For MFMA step kk, lane group lgrp holds dims 32 kk + 8 lgrp .. + 7 (the
  // same assignment is applied to K).
  constexpr int kWr = 16 * kPfRb;                       // rows per wave
  const int wr0 = row0 + kWr * wave;
  bf16x8 qf[kPfRb][kQk];
  int qpos[kPfRb];
#pragma unroll
  for (int rb = 0; rb < kPfRb; ++rb) {
    const int rr = wr0 + 16 * rb + lrow;
    const int qi = rr / group;
    const bool ok = rr < rows_total && q0 + qi < a.total_q;
    qpos[rb] = ok ? min(start + qi, kv_end - 1) : -1;   // keys past kv_end are clamped copies: masked
    const uint16_t* src = static_cast<const uint16_t*>(a.q) +
                          (static_cast<int64_t>(q0 + qi) * a.num_q_heads + g * group + (rr - qi * group)) * D +
                          lgrp * 8;
#pragma unroll
    for (int kk = 0; kk < kQk; ++kk) {
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (ok) v = *reinterpret_cast<const u32x4*>(src + kk * 32);
      qf[rb][kk] = __builtin_bit_cast(bf16x8, v);
    }
  }

  const bool w_active = wr0 < rows_total;
  const int w_qmin = min(start + wr0 / group, kv_end - 1);
  const int w_qmax = min(start + (min(wr0 + kWr - 1, rows_total - 1)) / group, kv_end - 1);
  const float c2 = a.scale_log2;

  f32x4 o[kDb][kPfRb];
  f32x4 lsum[kPfRb];
  float mc[kPfRb];                        // reference max per row, log2 units
  float mu[kPfRb];                        // the same, 0 while it is -inf
  float mt[kPfRb];                        // the same plus 8: the rescale threshold
#pragma unroll
  for (int rb = 0; rb < kPfRb; ++rb) {
    lsum[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
    mc[rb] = -INFINITY;
    mu[rb] = 0.f;
    mt[rb] = -INFINITY;
#pragma unroll
    for (int d = 0; d < kDb; ++d) o[d][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});

  // lane parts of the LDS operand addresses
  const int k_lane = lrow * kKRowB + lgrp * 16;
  const int v_lane = (4 * lgrp + (lrow >> 2)) * kVRowB + ((lrow & 3) >> 1) * 16 + (lrow & 1) * 8;
  // kt, vt: the sub-tile's staged K and V rows; sk (INT8): its key scales.
  auto compute = [&](const char* kt, const char* vt, const float* sk, int tb, auto mask_tag)
      __attribute__((always_inline)) {
    pf_sub_tile<D, kPfKeys, kI8, decltype(mask_tag)::value>(kt, vt, sk, tb, lgrp, k_lane, v_lane, c2, ones, qf,
                                                            qpos, o, lsum, mc, mu, mt);
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
#pragma unroll
    for (int sub = 0; sub < kPfKeys / 64; ++sub) {
      const int tb = k_lo + t * kPfKeys + 64 * sub;
      if (w_active && tb <= w_qmax) {
        const char* kt = smem + (t & 1) * kBufB + sub * 64 * kKRowB;
        const char* vt = smem + (t & 1) * kBufB + kKTileB + sub * 64 * kVRowB;
        const float* sk = reinterpret_cast<const float*>(smem + (t & 1) * kBufB + kKTileB + kPfKeys * kVRowB) + sub * 64;
        if (tb + 63 <= w_qmin)
          compute(kt, vt, sk, tb, std::integral_constant<int, 0>());
        else
          compute(kt, vt, sk, tb, std::integral_constant<int, 1>());
      }
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
  for (int rb = 0; rb < kPfRb; ++rb) {
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

// ---------------------------------------------------------------------------
// Short appends, persistent ("stream"): paged_prefill_stream_kernel runs the
// same tiles, staging, scores and products as paged_prefill_kernel, but a
// workgroup takes the work items id = blockIdx.x + k * gridDim.x in turn
// (gridDim.x a multiple of 8, so every item of a unit slot stays on one XCD)
// and never drains between them: the K/V loads run one tile ahead and the
// block-table lookups two tiles ahead across item boundaries, and the next
// item's queries load during the current item's last tile.  Items come from
// records the schedule kernel writes (one scalar load per item, two items
// ahead).  With few tiles per item (a 50-token question over a 300-token
// document is 6 tiles of 64 positions) the per-item start and drain
// latency, not the tiles, had bounded the one-item-per-workgroup launch.
// The next item's queries go straight from memory to an LDS buffer
// (global_load_lds_dwordx4, issued before the last tile's K/V loads, so the
// wait that stages that tile also covers them) and into registers at the
// switch: holding them in registers during the last tile would spill.
// With bf16 pages, D = 128 and scalar page lookups (page sizes that are
// powers of two of at least 4) the K/V tiles skip the registers as well:
// they go straight into a ring of three LDS buffers two tiles ahead (the
// query buffer and the ring fill the CU's 160 KB), one wait and one barrier
// per tile, and no staging pass.
// ---------------------------------------------------------------------------
// 8-wave workgroups (one per CU) take the next item's queries through an
// LDS buffer; 4-wave workgroups (two per CU, which hide each other's waits)
// load them into registers at the switch.
template <int kThreads_>
constexpr bool pf_stream_q_lds() { return kThreads_ >= 512; }
// bf16 pages, D = 128, 64-position tiles, 8 waves, page mode 0 (scalar page
// lookups): the K/V tiles go straight from memory into a ring of three LDS
// buffers (rows unpadded, their 16-byte chunks XOR-permuted by the row's low
// 4 bits), loaded two tiles ahead.  Per-lane (vector) page lookups would be
// waited on together with the tile loads in flight, so the other page modes
// keep the register-staged double buffer.
template <int D, int kKeys, int kThreads_, bool kI8, int kPageMode>
constexpr bool pf_stream_ring() { return !kI8 && D == 128 && kKeys == 64 && kThreads_ == 512 && kPageMode == 0; }
template <int D, int kKeys>
constexpr int pf_ring_buf_bytes() { return 2 * kKeys * D * 2; }
template <int D, int kKeys, int kThreads_, bool kI8, int kPageMode>
constexpr int pf_stream_lds_bytes() {
  return (pf_stream_ring<D, kKeys, kThreads_, kI8, kPageMode>() ? 3 * pf_ring_buf_bytes<D, kKeys>()
                                                                : pf_lds_bytes<D, kKeys, kI8>()) +
         (pf_stream_q_lds<kThreads_>() ? 16 * kPfRb * (kThreads_ / kWave) * D * 2 : 0);
}

template <int D, int kPageMode, int kPfThreads, int kPfKeys, bool kI8>
__global__ __launch_bounds__(kPfThreads, kPfThreads >= 512 ? 1 : 2) void paged_prefill_stream_kernel(
    AttnArgs a, const int32_t* __restrict__ row_off, int n_blocks, const int32_t* __restrict__ rec) {
  constexpr int kPfRows = 16 * kPfRb * (kPfThreads / kWave);   // query rows per item
  constexpr int kKRowB = pf_k_row_bytes<D>();
  constexpr int kVRowB = pf_v_row_bytes<D>();
  using Ld = KvLoad<kI8>;
  constexpr int kLdB = sizeof(Ld);
  constexpr int kGRowB = D * (kI8 ? 1 : 2);
  constexpr int kCpr = kGRowB / kLdB;
  constexpr int kChunks = kPfKeys * kCpr / kPfThreads;
  constexpr int kRowsPerPass = kPfThreads / kCpr;
  constexpr int kQk = D / 32;
  constexpr int kDb = D / 16;
  constexpr int kKTileB = kPfKeys * kKRowB;
  constexpr int kBufB = pf_buf_bytes<D, kPfKeys, kI8>();
  static_assert(kChunks * kRowsPerPass == kPfKeys, "tile split");
  extern __shared__ __align__(16) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int lrow = lane & 15;
  const int lgrp = lane >> 4;
  const int hkv = a.num_kv_heads;
  const int group = a.group;
  const int n_sp = a.n_splits;
  const int G = gridDim.x;
  const int n_ids = row_off[n_blocks] * 8;   // records written by the schedule kernel

  // ---- work items ----
  struct Item {
    int valid, b, g, q0, n_b, start, row0, kv_end, split, k_lo, k_hi, n_tiles, rows_total;
  };
  auto make_item = [&](int4 x, int4 y) __attribute__((always_inline)) {
    Item it;
    it.valid = x.x >= 0;
    it.b = max(x.x, 0);
    it.g = x.y;
    it.q0 = x.z;
    it.n_b = x.w;
    it.start = y.x;
    it.row0 = y.y;
    it.kv_end = y.z;
    it.split = y.w;
    it.rows_total = min(it.n_b, a.max_q) * group;
    it.k_lo = it.split * a.split_len;
    it.k_hi = min(it.k_lo + a.split_len, it.kv_end);
    it.n_tiles = it.valid ? (it.k_hi - it.k_lo + kPfKeys - 1) / kPfKeys : 0;
    return it;
  };
  // The records of the next ids are loaded one item before they are used;
  // ids without work are skipped (a wait on a record only then).
  int next_id = blockIdx.x;
  int4 pend_x = make_int4(-1, 0, 0, 0), pend_y = make_int4(0, 0, 0, 0);
  // Records and (page mode 0) block-table entries are wave-uniform: read
  // through the constant address space they are scalar loads, waited on with
  // lgkmcnt, and never hold back the vmcnt waits of the K/V tiles.
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  typedef const __attribute__((address_space(4))) int32_t* cptr;
  typedef const __attribute__((address_space(4))) i32x4* cptr4;
  auto load_rec = [&](int id, int4& x, int4& y) __attribute__((always_inline)) {
    if (id < n_ids) {
      cptr4 p4 = (cptr4)((cptr)(rec) + 8 * static_cast<int64_t>(id));
      const i32x4 vx = p4[0], vy = p4[1];
      x = make_int4(vx.x, vx.y, vx.z, vx.w);
      y = make_int4(vy.x, vy.y, vy.z, vy.w);
    } else {
      x = make_int4(-1, 0, 0, 0);
      y = make_int4(0, 0, 0, 0);
    }
  };
  // the next item with work: the pending record, else records further on
  auto take_item = [&]() __attribute__((always_inline)) {
    int4 x = pend_x, y = pend_y;
    while (x.x < 0 && next_id < n_ids) {
      load_rec(next_id, x, y);
      next_id += G;
    }
    load_rec(next_id, pend_x, pend_y);   // the item after it, used at the next switch
    next_id += G;
    return make_item(x, y);
  };
  load_rec(next_id, pend_x, pend_y);
  next_id += G;
  Item W0 = take_item();
  if (!W0.valid) return;
  Item W1 = take_item();
  Item W2 = take_item();

  // ---- staging (as paged_prefill_kernel; the item is an argument) ----
  const int ps = a.page_size;
  const int ps_shift = a.ps_shift;
  const uint32_t head_bytes = static_cast<uint32_t>(a.head_bytes);
  const uint32_t scale_off = static_cast<uint32_t>(ps) * D;
  const char* kbytes = static_cast<const char*>(a.k_pool);
  const char* vbytes = static_cast<const char*>(a.v_pool);
  const int srow0 = tid / kCpr;
  const int spart = tid - srow0 * kCpr;
  const int wrow0 = __builtin_amdgcn_readfirstlane(srow0);

  int pg_next[kChunks], pg_next2[kChunks];
  Ld kr[kChunks], vr[kChunks];
  float ksr[kChunks], vsr[kChunks];
  auto pos_of = [&](const Item& it, int t, int row) __attribute__((always_inline)) {
    return min(it.k_lo + t * kPfKeys + row, it.k_hi - 1);
  };
  auto blk_of = [&](int pos) __attribute__((always_inline)) {
    if constexpr (kPageMode <= 1) return pos >> ps_shift;
    else return pos / ps;
  };
  auto fetch_pages = [&](const Item& it, int t) __attribute__((always_inline)) {
    const int64_t row = static_cast<int64_t>(it.b) * a.bt_stride;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      if constexpr (kPageMode == 0)
        pg_next2[c] = ((cptr)(a.block_tables))[row + blk_of(pos_of(it, t, wrow0 + c * kRowsPerPass))];
      else
        pg_next2[c] = a.block_tables[row + blk_of(pos_of(it, t, srow0 + c * kRowsPerPass))];
    }
  };
  auto load_kv = [&](const Item& it, int t) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int pos = pos_of(it, t, srow0 + c * kRowsPerPass);
      const uint32_t page = static_cast<uint32_t>(min(max(pg_next[c], 0), a.num_pages - 1));
      const uint32_t off = kPageMode <= 1 ? (pos & (ps - 1)) : (pos - blk_of(pos) * ps);
      const uint32_t voff = off * kGRowB + spart * kLdB;
      const uint64_t base = static_cast<uint64_t>(page * hkv + it.g) * head_bytes;
      if constexpr (kI8) {
        ksr[c] = *reinterpret_cast<const float*>(kbytes + base + scale_off + 4 * off);
        vsr[c] = *reinterpret_cast<const float*>(vbytes + base + scale_off + 4 * off);
      }
      kr[c] = *reinterpret_cast<const Ld*>(kbytes + base + voff);
      vr[c] = *reinterpret_cast<const Ld*>(vbytes + base + voff);
    }
  };
  auto stage = [&](int buf) __attribute__((always_inline)) {
    char* kb = smem + buf * kBufB;
    char* vb = kb + kKTileB;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int row = srow0 + c * kRowsPerPass;
      if constexpr (kI8) {
        // codes as exact bf16; part 0 of each row writes the row's scales
        *reinterpret_cast<u32x4*>(kb + row * kKRowB + spart * 16) = i8x8_to_bf16(kr[c]);
        *reinterpret_cast<u32x4*>(vb + row * kVRowB + spart * 16) = i8x8_to_bf16(vr[c]);
        if (spart == 0) {
          float* sc = reinterpret_cast<float*>(vb + kPfKeys * kVRowB);
          sc[row] = ksr[c];
          sc[kPfKeys + row] = vsr[c];
        }
      } else {
        *reinterpret_cast<u32x4*>(kb + row * kKRowB + spart * 16) = kr[c];
        *reinterpret_cast<u32x4*>(vb + row * kVRowB + spart * 16) = vr[c];
      }
    }
  };
  // The tile k steps after tile tc of W0 (k = 1, 2): (item 0..2, tile).  Past
  // the last item with work it names the last tile of the stream (reloaded,
  // never computed).
  auto after = [&](int tc, int k, int& which, int& t) __attribute__((always_inline)) {
    const int r0 = W0.n_tiles - 1 - tc;
    if (k <= r0) { which = 0; t = tc + k; return; }
    int kk = k - r0 - 1;                              // tile index into W1, W2, ...
    if (W1.valid && kk < W1.n_tiles) { which = 1; t = kk; return; }
    if (!W1.valid) { which = 0; t = W0.n_tiles - 1; return; }
    kk -= W1.n_tiles;
    if (W2.valid && kk < W2.n_tiles) { which = 2; t = kk; return; }
    if (!W2.valid) { which = 1; t = W1.n_tiles - 1; return; }
    which = 2;
    t = W2.n_tiles - 1;
  };
  auto item_ref = [&](int which) __attribute__((always_inline)) -> const Item& {
    return which == 0 ? W0 : which == 1 ? W1 : W2;
  };

  // ---- query rows of an item (B operand of S^T = K Q^T) ----
  constexpr int kWr = 16 * kPfRb;
  bf16x8 qf[kPfRb][kQk];
  // The next item's query tile, memory -> LDS: chunk q = c * kPfThreads + tid
  // of the tile (row q / kQcpr, 16-byte part q % kQcpr) lands at byte 16 q of
  // the buffer (each wave instruction writes 1 KB at its M0).  Rows without a
  // query read the item's first query row (finite; never written out).
  constexpr int kQcpr = D * 2 / 16;
  constexpr int kQChunks = kPfRows * kQcpr / kPfThreads;
  static_assert(kQChunks * kPfThreads == kPfRows * kQcpr, "query tile split");
  constexpr bool kRing = pf_stream_ring<D, kPfKeys, kPfThreads, kI8, kPageMode>();
  constexpr int kRBufB = pf_ring_buf_bytes<D, kPfKeys>();
  char* qbuf = smem + (kRing ? 3 * kRBufB : 2 * kBufB);
  auto dma_q = [&](const Item& it) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < kQChunks; ++c) {
      const int qc = c * kPfThreads + tid;
      const int row = qc / kQcpr;
      const int part = qc - row * kQcpr;
      const int rr = it.row0 + row;
      const int qi = rr / group;
      const bool ok = rr < it.rows_total && it.q0 + qi < a.total_q;
      const uint16_t* src = static_cast<const uint16_t*>(a.q) +
                            (static_cast<int64_t>(it.q0 + (ok ? qi : 0)) * a.num_q_heads + it.g * group +
                             (ok ? rr - qi * group : 0)) * D + part * 8;
      // Inline asm: the compiler neither counts these loads in its vmcnt
      // waits (so its waits stay sufficient, only stronger) nor makes LDS
      // reads wait for them; the staging wait of the tile loads issued
      // right after covers them (loads retire in order).
      const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
          (__attribute__((address_space(3))) char*)(qbuf + (c * kPfThreads + wave * kWave) * 16)));
      asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0) : "memory");
    }
  };
  auto read_q_lds = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < kPfRb; ++rb) {
      const char* src = qbuf + (kWr * wave + 16 * rb + lrow) * (D * 2) + lgrp * 16;
#pragma unroll
      for (int kk = 0; kk < kQk; ++kk) qf[rb][kk] = *reinterpret_cast<const bf16x8*>(src + kk * 64);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): read before the buffer is refilled
  };
  auto load_q = [&](const Item& it, bf16x8 (&dst)[kPfRb][kQk]) __attribute__((always_inline)) {
    const int wr0 = it.row0 + kWr * wave;
#pragma unroll
    for (int rb = 0; rb < kPfRb; ++rb) {
      const int rr = wr0 + 16 * rb + lrow;
      const int qi = rr / group;
      const bool ok = rr < it.rows_total && it.q0 + qi < a.total_q;
      const uint16_t* src = static_cast<const uint16_t*>(a.q) +
                            (static_cast<int64_t>(it.q0 + (ok ? qi : 0)) * a.num_q_heads + it.g * group +
                             (ok ? rr - qi * group : 0)) * D + lgrp * 8;
#pragma unroll
      for (int kk = 0; kk < kQk; ++kk) {
        u32x4 v = *reinterpret_cast<const u32x4*>(src + kk * 32);
        if (!ok) v = u32x4{0u, 0u, 0u, 0u};
        dst[rb][kk] = __builtin_bit_cast(bf16x8, v);
      }
    }
  };

  // per-item, per-wave row bookkeeping
  int qpos[kPfRb];
  bool w_active;
  int w_qmin, w_qmax, wr0;
  auto enter_item = [&](const Item& it) __attribute__((always_inline)) {
    wr0 = it.row0 + kWr * wave;
#pragma unroll
    for (int rb = 0; rb < kPfRb; ++rb) {
      const int rr = wr0 + 16 * rb + lrow;
      const int qi = rr / group;
      const bool ok = rr < it.rows_total && it.q0 + qi < a.total_q;
      qpos[rb] = ok ? min(it.start + qi, it.kv_end - 1) : -1;
    }
    w_active = wr0 < it.rows_total;
    w_qmin = min(it.start + wr0 / group, it.kv_end - 1);
    w_qmax = min(it.start + (min(wr0 + kWr - 1, it.rows_total - 1)) / group, it.kv_end - 1);
  };
  const float c2 = a.scale_log2;
  f32x4 o[kDb][kPfRb];
  f32x4 lsum[kPfRb];
  float mc[kPfRb];
  float mu[kPfRb];
  float mt[kPfRb];
  auto reset_state = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < kPfRb; ++rb) {
      lsum[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
      mc[rb] = -INFINITY;
      mu[rb] = 0.f;
      mt[rb] = -INFINITY;
#pragma unroll
      for (int d = 0; d < kDb; ++d) o[d][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
  const int k_lane = lrow * kKRowB + lgrp * 16;
  const int v_lane = (4 * lgrp + (lrow >> 2)) * kVRowB + ((lrow & 3) >> 1) * 16 + (lrow & 1) * 8;
  // kt, vt: the sub-tile's staged K and V rows; sk (INT8): its key scales.
  auto compute = [&](const char* kt, const char* vt, const float* sk, int tb, auto mask_tag)
      __attribute__((always_inline)) {
    pf_sub_tile<D, kPfKeys, kI8, decltype(mask_tag)::value>(kt, vt, sk, tb, lgrp, k_lane, v_lane, c2, ones, qf,
                                                            qpos, o, lsum, mc, mu, mt);
  };

  auto epilogue = [&](const Item& it) __attribute__((always_inline)) {
    if (!w_active) return;
    const bool final_write = n_sp == 1;
#pragma unroll
    for (int rb = 0; rb < kPfRb; ++rb) {
      const int rr = wr0 + 16 * rb + lrow;
      if (qpos[rb] < 0) continue;
      const int qi = rr / group;
      const int tok = it.q0 + qi;
      const int64_t orow = static_cast<int64_t>(tok) * a.num_q_heads + it.g * group + (rr - qi * group);
      const float l = lsum[rb][0];
      if (final_write) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        uint16_t* dst = static_cast<uint16_t*>(a.out) + orow * D + 4 * lgrp;
#pragma unroll
        for (int d = 0; d < kDb; ++d)
          *reinterpret_cast<i16x4*>(dst + 16 * d) = pack_bf16x4(o[d][rb] * inv);
      } else {
        if (tok >= a.ws_tokens) continue;
        const int64_t slot = orow * n_sp + it.split;
        float* dst = a.ws_o + slot * D + 4 * lgrp;
#pragma unroll
        for (int d = 0; d < kDb; ++d) *reinterpret_cast<f32x4*>(dst + 16 * d) = o[d][rb];
        if (lgrp == 0) {
          a.ws_ml[slot * 2] = mc[rb];
          a.ws_ml[slot * 2 + 1] = l;
        }
      }
    }
  };

  if constexpr (kRing) {
    // ---- ring: tile t in buffer t % 3, loaded at the top of tile t - 2 ----
    // Chunk p of staged row r holds the row's chunk p ^ (r & 15): lane
    // (lrow, lgrp) reads K rows kb * 16 + lrow, chunk (4 kk + lgrp) ^ lrow,
    // and V^T rows 4 lgrp + (lrow >> 2) (+ 16 / 32 multiples), chunk pair
    // d ^ (row >> 1 & 7); each group of lanes an LDS read serves then covers
    // distinct banks.
    constexpr int kRowB = D * 2;
    int tc_ring = 0;   // tile of W0 being computed
    int koff[kQk], voff[kDb];
#pragma unroll
    for (int kk = 0; kk < kQk; ++kk) koff[kk] = lrow * kRowB + 16 * ((4 * kk + lgrp) ^ lrow);
    {
      const int vr = 4 * lgrp + (lrow >> 2);
      const int h = (lrow & 3) >> 1;
#pragma unroll
      for (int d = 0; d < kDb; ++d) voff[d] = vr * kRowB + 16 * ((2 * d + h) ^ vr) + 8 * (lrow & 1);
    }
    // A tile by the fields its loads need (item fields picked by value, so
    // they stay in scalar registers).
    struct TileRef {
      int b, g, k_lo, k_hi, t;
    };
    auto tile_ref = [&](int k) __attribute__((always_inline)) {
      int wh, t;
      after(tc_ring, k, wh, t);
      TileRef r;
      r.b = wh == 0 ? W0.b : (wh == 1 ? W1.b : W2.b);
      r.g = wh == 0 ? W0.g : (wh == 1 ? W1.g : W2.g);
      r.k_lo = wh == 0 ? W0.k_lo : (wh == 1 ? W1.k_lo : W2.k_lo);
      r.k_hi = wh == 0 ? W0.k_hi : (wh == 1 ? W1.k_hi : W2.k_hi);
      r.t = t;
      return r;
    };
    auto rpos = [&](const TileRef& r, int row) __attribute__((always_inline)) {
      return min(r.k_lo + r.t * kPfKeys + row, r.k_hi - 1);
    };
    auto rfetch = [&](const TileRef& r) __attribute__((always_inline)) {
      const int64_t brow = static_cast<int64_t>(r.b) * a.bt_stride;
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {
        if constexpr (kPageMode == 0)
          pg_next2[c] = ((cptr)(a.block_tables))[brow + blk_of(rpos(r, wrow0 + c * kRowsPerPass))];
        else
          pg_next2[c] = a.block_tables[brow + blk_of(rpos(r, srow0 + c * kRowsPerPass))];
      }
    };
    // One wave instruction fills 1 KB of LDS at its M0 (lane l at 16 l):
    // rows wrow0 + c * kRowsPerPass .. + 3, each lane one chunk of its row.
    auto dma_kv = [&](const TileRef& it, int rb) __attribute__((always_inline)) {
      char* kb = smem + rb * kRBufB;
      char* vb = kb + kPfKeys * kRowB;
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {
        const int row = srow0 + c * kRowsPerPass;
        const int pos = rpos(it, row);
        const uint32_t page = static_cast<uint32_t>(min(max(pg_next[c], 0), a.num_pages - 1));
        const uint32_t off = kPageMode <= 1 ? (pos & (ps - 1)) : (pos - blk_of(pos) * ps);
        const uint32_t voff_g = off * kGRowB + 16 * (spart ^ (row & 15));
        const uint64_t base = static_cast<uint64_t>(page * hkv + it.g) * head_bytes;
        const char* ksrc = kbytes + base + voff_g;
        const char* vsrc = vbytes + base + voff_g;
        const int mrow = wrow0 + c * kRowsPerPass;
        const uint32_t mk = static_cast<uint32_t>(
            reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)(kb + mrow * kRowB)));
        const uint32_t mv = static_cast<uint32_t>(
            reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)(vb + mrow * kRowB)));
        asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(ksrc), "{m0}"(mk) : "memory");
        asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(vsrc), "{m0}"(mv) : "memory");
      }
    };
    // vmcnt(n), other counters untouched
    constexpr int kTileDma = 2 * kChunks;   // DMA instructions per wave per tile
    static_assert(kTileDma < 16, "wait count");
    auto wait_tile = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt(0x0F70 | kTileDma);   // vmcnt(kTileDma): only the next tile's may be in flight
    };
    auto rcompute = [&](const char* kt, const char* vt, int tb, auto mask_tag) __attribute__((always_inline)) {
      pf_sub_tile<D, kPfKeys, kI8, decltype(mask_tag)::value, true>(kt, vt, nullptr, tb, lgrp, 0, 0, c2, ones, qf, qpos,
                                                                   o, lsum, mc, mu, mt, koff, voff);
    };

    // prologue: the first item's queries; tiles 0 and 1 in flight
    load_q(W0, qf);
    enter_item(W0);
    reset_state();
    {
      const TileRef r0 = tile_ref(0);
      rfetch(r0);
#pragma unroll
      for (int c = 0; c < kChunks; ++c) pg_next[c] = pg_next2[c];
      dma_kv(r0, 0);
      const TileRef r1 = tile_ref(1);
      rfetch(r1);
#pragma unroll
      for (int c = 0; c < kChunks; ++c) pg_next[c] = pg_next2[c];
      dma_kv(r1, 1);
    }
    int rbuf = 0;
    int& tc = tc_ring;
    while (true) {
      const bool last = tc == W0.n_tiles - 1;
      const TileRef r2 = tile_ref(2);
      rfetch(r2);        // waited on at the barrier
      wait_tile();
      __syncthreads();   // tile tc is in LDS for every wave; tile tc - 1 is no longer read
      // the next item's queries, into the query buffer read at the switch
      if (W1.valid && tc == max(W0.n_tiles - 2, 0)) dma_q(W1);
#pragma unroll
      for (int c = 0; c < kChunks; ++c) pg_next[c] = pg_next2[c];
      dma_kv(r2, rbuf == 0 ? 2 : rbuf - 1);
      {
        const int tb = W0.k_lo + tc * kPfKeys;
        if (w_active && tb <= w_qmax) {
          const char* kt = smem + rbuf * kRBufB;
          const char* vt = kt + kPfKeys * kRowB;
          if (tb + 63 <= w_qmin)
            rcompute(kt, vt, tb, std::integral_constant<int, 0>());
          else if (tb + 32 > w_qmax)
            rcompute(kt, vt, tb, std::integral_constant<int, 2>());
          else
            rcompute(kt, vt, tb, std::integral_constant<int, 1>());
        }
      }
      rbuf = rbuf == 2 ? 0 : rbuf + 1;
      if (!last) {
        ++tc;
        continue;
      }
      if (W0.n_tiles == 1 && W1.valid) {
        // the queries were requested this iteration, before the tile DMAs
        wait_tile();
        __syncthreads();
      }
      epilogue(W0);
      if (!W1.valid) break;
      W0 = W1;
      W1 = W2;
      W2 = take_item();
      read_q_lds();
      enter_item(W0);
      reset_state();
      tc = 0;
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): no DMA outlives the wave
    return;
  }

  // ---- prologue: the first item's queries, pages and first tile ----
  load_q(W0, qf);
  enter_item(W0);
  reset_state();
  fetch_pages(W0, 0);
#pragma unroll
  for (int c = 0; c < kChunks; ++c) pg_next[c] = pg_next2[c];
  load_kv(W0, 0);
  {
    int wh, t;
    after(0, 1, wh, t);
    fetch_pages(item_ref(wh), t);
  }
  stage(0);
#pragma unroll
  for (int c = 0; c < kChunks; ++c) pg_next[c] = pg_next2[c];
  __syncthreads();

  // ---- the stream of tiles ----
  int buf = 0;
  int tc = 0;
  while (true) {
    const bool last = tc == W0.n_tiles - 1;
    if constexpr (pf_stream_q_lds<kPfThreads>())
      if (last && W1.valid) dma_q(W1);
    {
      int wh, t;
      after(tc, 1, wh, t);
      load_kv(item_ref(wh), t);
      after(tc, 2, wh, t);
      fetch_pages(item_ref(wh), t);
    }
#pragma unroll
    for (int sub = 0; sub < kPfKeys / 64; ++sub) {
      const int tb = W0.k_lo + tc * kPfKeys + 64 * sub;
      if (w_active && tb <= w_qmax) {
        const char* kt = smem + buf * kBufB + sub * 64 * kKRowB;
        const char* vt = smem + buf * kBufB + kKTileB + sub * 64 * kVRowB;
        const float* sk = reinterpret_cast<const float*>(smem + buf * kBufB + kKTileB + kPfKeys * kVRowB) + sub * 64;
        if (tb + 63 <= w_qmin)
          compute(kt, vt, sk, tb, std::integral_constant<int, 0>());
        else if (tb + 32 > w_qmax)
          compute(kt, vt, sk, tb, std::integral_constant<int, 2>());
        else
          compute(kt, vt, sk, tb, std::integral_constant<int, 1>());
      }
    }
    stage(buf ^ 1);
#pragma unroll
    for (int c = 0; c < kChunks; ++c) pg_next[c] = pg_next2[c];
    __syncthreads();
    buf ^= 1;
    if (!last) {
      ++tc;
      continue;
    }
    epilogue(W0);
    if (!W1.valid) break;
    W0 = W1;
    W1 = W2;
    W2 = take_item();
    if constexpr (pf_stream_q_lds<kPfThreads>()) {
      read_q_lds();
      // Every wave's query DMA writes rows that other waves read here.  An
      // item of one tile issues the next item's DMA in its first iteration,
      // so all reads must finish first; with more tiles a tile barrier lies
      // between.
      if (W0.n_tiles == 1 && W1.valid) __syncthreads();
    } else {
      load_q(W0, qf);
    }
    enter_item(W0);
    reset_state();
    tc = 0;
  }
}

// Fold ns partial states of one output row: state k has its un-normalised
// output at o[k * stride * D ..] and (max, sum) at ml[k * stride * 2 ..]
// (log2 domain), and the result goes to row orow of out.  One wave; each lane
// owns D / 64 dims; partial rows are read eight at a time.
template <typename T, int D>
__device__ __forceinline__ void merge_rows(const AttnArgs& args, const float* o, const float* ml, int stride,
                                           int ns, int64_t orow) {
  const int lane = threadIdx.x & (kWave - 1);
  constexpr int kPer = D / kWave;
  float mmax = -INFINITY;
  for (int s = lane; s < ns; s += kWave) mmax = fmaxf(mmax, ml[static_cast<int64_t>(s) * stride * 2]);
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
      const float* m = ml + static_cast<int64_t>(sl) * stride * 2;
      wt = fast_exp2(m[0] - mref);
      lsum += wt * m[1];
    }
    const int cnt = min(kWave, ns - s0);
    for (int k0 = 0; k0 < cnt; k0 += 8) {
      float part[8][kPer];
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const int k = min(k0 + v, cnt - 1);
        const float* src = o + static_cast<int64_t>(s0 + k) * stride * D + lane * kPer;
#pragma unroll
        for (int j = 0; j < kPer; ++j) part[v][j] = src[j];
      }
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const float wk = __shfl(wt, min(k0 + v, kWave - 1));
        const float w_use = (k0 + v < cnt) ? wk : 0.f;
#pragma unroll
        for (int j = 0; j < kPer; ++j) acc[j] += w_use * part[v][j];
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

// Log-sum-exp merge of the KV-split partials of one (query, head) row of the
// tile kernels.  Grid: (num_q_heads, max_q_per_seq, n_seqs), one wave per row.
template <typename T, int D>
__global__ __launch_bounds__(kWave) void merge_chunks_kernel(AttnArgs args) {
  const int h = blockIdx.x;
  const int qi = blockIdx.y;
  const int b = blockIdx.z;
  const int q0 = args.cu_q[b];
  const int n_b = args.cu_q[b + 1] - q0;
  if (qi >= n_b) return;
  const int tok = q0 + qi;
  if (tok >= args.total_q || tok >= args.ws_tokens) return;
  const int qpos = min(args.seq_lens[b] - n_b + qi, args.kv_cap - 1);   // last position read
  const int ns = qpos < 0 ? 0 : min(args.n_splits, qpos / args.split_len + 1);
  const int64_t orow = static_cast<int64_t>(tok) * args.num_q_heads + h;
  merge_rows<T, D>(args, args.ws_o + orow * args.n_splits * D, args.ws_ml + orow * args.n_splits * 2, 1, ns,
                   orow);
}

// Log-sum-exp merge of the decode segments of one unit: the slots unit + w
// of the waves w whose block ranges cut the unit.  Grid: (units, row
// groups); the 4-wave workgroup (u, y) folds rows y * kMergeRows + v,
// + 4, ... below (y + 1) * kMergeRows with wave v; units inside one wave's
// range were written final and exit at once.  One row block takes one row
// group; more row blocks (many query rows, few units, many segments each)
// spread each unit over 4 rows per workgroup.
template <int RBW>
constexpr int merge_rows_per_group() { return RBW == 1 ? 16 : 4; }

template <typename T, int D, int RBW>
__global__ __launch_bounds__(kThreads) void merge_segments_kernel(AttnArgs a, const int32_t* __restrict__ seq_blk) {
  constexpr int kRowsCap = 16 * RBW;
  constexpr int kMergeRows = merge_rows_per_group<RBW>();
  const int u = blockIdx.x;
  const int hkv = a.num_kv_heads;
  const int b = u / hkv;
  const int g = u - b * hkv;
  const int nb = seq_blk[b + 1] - seq_blk[b];
  if (nb == 0) return;
  const int per = decode_per(seq_blk[a.n_seqs] * hkv, a.waves, a.split_len);
  const int u0 = seq_blk[b] * hkv + g * nb;
  const int f = u0 / per;
  const int l = (u0 + nb - 1) / per;
  if (f == l) return;
  int q0, n_b, rows;
  decode_kv_end<RBW>(a, b, &q0, &n_b, &rows);
  const int r_end = min(rows, static_cast<int>(blockIdx.y + 1) * kMergeRows);
  for (int r = static_cast<int>(blockIdx.y) * kMergeRows + threadIdx.x / kWave; r < r_end; r += kThreads / kWave) {
    const int qi = r / a.group;
    const int tok = q0 + qi;
    if (tok >= a.total_q) continue;
    const int64_t orow = static_cast<int64_t>(tok) * a.num_q_heads + g * a.group + (r - qi * a.group);
    const int64_t row0 = static_cast<int64_t>(u + f) * kRowsCap + r;
    merge_rows<T, D>(a, a.ws_o + row0 * D, a.ws_ml + row0 * 2, kRowsCap, l - f + 1, orow);
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

// KV scatter into INT8 pages ("INT8 cache": quantization happens here, at
// write time, and a stored scale is never revised): kLpv = D / 8 consecutive lanes own one (token,
// KV head) vector of K or V, 8 bf16 each.  Its absolute maximum is reduced
// across those lanes; scale = max|x| / 127 and code = rint(x / scale), both
// IEEE fp32 divisions, codes clamped to [-127, 127]; a zero vector stores
// scale 0 and codes 0.  Each lane writes its 8 codes (8 bytes), the group's
// first lane the scale.
template <int D>
__global__ __launch_bounds__(kThreads) void store_kv_i8_kernel(
    char* __restrict__ k_pool, char* __restrict__ v_pool, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, const int64_t* __restrict__ slots, int32_t n_tokens, int32_t hkv,
    int32_t page_size, int32_t ps_shift, int64_t pool_slots, int32_t head_bytes) {
  constexpr int kLpv = D / 8;
  const int64_t per_pool = static_cast<int64_t>(n_tokens) * hkv;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  int64_t vec = gid / kLpv;                          // vector index over both pools
  const int part = static_cast<int>(gid % kLpv);
  const bool live = vec < 2 * per_pool;              // whole groups are live or not
  const bool is_v = vec >= per_pool;
  if (is_v) vec -= per_pool;
  if (!live) vec = 0;
  const uint16_t* src = (is_v ? v_new : k_new) + vec * D + part * 8;
  const u32x4 x = *reinterpret_cast<const u32x4*>(src);
  float f[8];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    f[2 * w] = __uint_as_float(x[w] << 16);
    f[2 * w + 1] = __uint_as_float(x[w] & 0xffff0000u);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
#pragma unroll
  for (int off = 1; off < kLpv; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float scale = amax / 127.f;
  uint32_t packed[2] = {0u, 0u};
  if (scale > 0.f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float c = fminf(fmaxf(rintf(f[i] / scale), -127.f), 127.f);
      packed[i >> 2] |= (static_cast<uint32_t>(static_cast<int32_t>(c)) & 0xffu) << (8 * (i & 3));
    }
  }
  if (!live) return;
  const int64_t t = vec / hkv;
  const int g = static_cast<int>(vec - t * hkv);
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= pool_slots) return;
  const int64_t page = ps_shift >= 0 ? (slot >> ps_shift) : slot / page_size;
  const int64_t off = slot - page * page_size;
  char* head = (is_v ? v_pool : k_pool) + (page * hkv + g) * static_cast<int64_t>(head_bytes);
  *reinterpret_cast<uint2*>(head + off * D + part * 8) = make_uint2(packed[0], packed[1]);
  if (part == 0) *reinterpret_cast<float*>(head + static_cast<int64_t>(page_size) * D + 4 * off) = scale;
}

// Page copy for copy-on-write.  A page is num_kv_heads contiguous (page, KV
// head) blocks, so a (source, destination) pair copies one contiguous run per
// pool.  Grid: x = pair (its page ids are scalar loads), y = a tile of
// kCopyPer * 256 of the pair's 16-byte chunks (K chunks, then V chunks); each
// thread issues its kCopyPer loads (non-temporal: 4,096 pairs copy in 88
// instead of 114 us) before its stores (plain: non-temporal stores were
// slower).
constexpr int kCopyPer = PKV_COPY_CHUNKS;
__global__ __launch_bounds__(kThreads) void copy_pages_kernel(char* __restrict__ k_pool, char* __restrict__ v_pool,
                                                              const int32_t* __restrict__ copies, int32_t page_chunks,
                                                              int32_t num_pages) {
  const int64_t pair = blockIdx.x;
  const int32_t src = copies[2 * pair];
  const int32_t dst = copies[2 * pair + 1];
  if (src < 0 || src >= num_pages || dst < 0 || dst >= num_pages || src == dst) return;
  const int c0 = static_cast<int>(blockIdx.y) * kThreads * kCopyPer + threadIdx.x;
  u32x4 x[kCopyPer];
#pragma unroll
  for (int j = 0; j < kCopyPer; ++j) {
    const int c = c0 + j * kThreads;
    if (c >= 2 * page_chunks) continue;
    const bool is_v = c >= page_chunks;
    const char* pool = is_v ? v_pool : k_pool;
    x[j] = ld_stream(reinterpret_cast<const u32x4*>(pool + (static_cast<int64_t>(src) * page_chunks + (is_v ? c - page_chunks : c)) * 16));
  }
#pragma unroll
  for (int j = 0; j < kCopyPer; ++j) {
    const int c = c0 + j * kThreads;
    if (c >= 2 * page_chunks) continue;
    const bool is_v = c >= page_chunks;
    char* pool = is_v ? v_pool : k_pool;
    *reinterpret_cast<u32x4*>(pool + (static_cast<int64_t>(dst) * page_chunks + (is_v ? c - page_chunks : c)) * 16) = x[j];
  }
}

// Group-wise low-bit codec of a prefix's K and V (the quantize / restore half
// of a KV handoff, ReKV section 2.2): groups of 64 elements along head_dim,
// one fp16 scale each, Q8 bytes or Q4 nibbles.  Four consecutive lanes own
// one group, 16 elements each; the payload holds the codes of K then V
// (position, KV head, element order), then the scales in the same order.
// Scale = fp16(max|x| / q_max); codes = rint(x * (1 / scale16)) clamped to
// [-q_max, q_max], with one IEEE fp32 reciprocal per group; a zero scale
// gives zero codes.  Restoring writes bf16(scale16 * code).
struct CodecArgs {
  const int32_t* block_table;
  int32_t n_positions;
  int32_t hkv;
  int32_t head_dim;
  int32_t page_size;
  int32_t ps_shift;
  int32_t num_pages;
  int64_t groups_per_tensor;   // n_positions * hkv * head_dim / 64
};

// Pool element offset of the 8 elements of (tensor-local) group gi, part;
// *valid is false when the block-table entry is not a page of the pool (the
// offset then names page 0, so address arithmetic never leaves the pool and
// takes no branch).  Index arithmetic is 32-bit: the host keeps
// 2 * groups_per_tensor * 8 below 2^31.  head_dim is 64 or 128, so a vector
// holds 1 or 2 groups.
__device__ __forceinline__ int64_t codec_pool_elem(const CodecArgs& a, int gi, int part, bool* valid) {
  const int gshift = a.head_dim == 128 ? 1 : 0;      // log2(groups per (position, head) vector)
  const int vec = gi >> gshift;
  const int d0 = (gi - (vec << gshift)) * 64 + part * 8;
  const int pos = static_cast<int>(static_cast<unsigned>(vec) / static_cast<unsigned>(a.hkv));
  const int head = vec - pos * a.hkv;
  const int blk = a.ps_shift >= 0 ? (pos >> a.ps_shift) : pos / a.page_size;
  const int off = pos - blk * a.page_size;
  const int entry = a.block_table[blk];
  *valid = entry >= 0 && entry < a.num_pages;
  const int page = *valid ? entry : 0;
  return ((static_cast<int64_t>(page) * a.hkv + head) * a.page_size + off) * a.head_dim + d0;
}

// Encode: four consecutive lanes own one group of 64 elements; lane p reads
// 16-byte chunks p and p + 4 (each load instruction of the four lanes covers
// 64 contiguous bytes), so the group's maximum takes two shuffles and the
// per-group work (address, scale, reciprocal) is shared by 16 elements.
// A code is rint(clamp(x / scale, -q_max, q_max)) with x / scale the
// correctly rounded fp32 quotient.  For a bf16 x and an fp16 scale that
// quotient never rounds onto a half-integer h unless x / scale is exactly h:
// a nonzero x - h * scale is at least 2^-12 relative to the scale, far above
// half an fp32 ulp of h (|h| < 128).  So the code is the exact quotient
// rounded to nearest, ties to even, and it is found without a division:
//  * c = rint(x * inv) with inv = 1 / scale rounded once per group; adding
//    1.5 * 2^23 to the clamped product rounds it to an integer (the low
//    bits of the sum are the two's complement code, its lowest bit the
//    parity), and c is within 1 of the answer;
//  * e = x - c * scale by one fma, exact (all terms are short multiples of a
//    common quantum); |e| > scale / 2 moves c one step toward e's sign, and
//    |e| = scale / 2 (an exact tie) moves it only when c is odd.
// The correction is needed only where the product lies within 2^-14 of a
// half-integer: it is within 1.5 * 2^-16 of the quotient for
// |x / scale| <= 128, so elsewhere rint(x * inv) is already the code.  It
// runs per element on a wave-wide vote (for N(0,1) bf16 groups about one
// element position in ten for Q4, whose ties are common, one in twenty for
// Q8).  Beyond q_max everything clamps to q_max.  With a zero scale inv is 1 and every element is below
// 2^-18 in magnitude (a nonzero max / q_max that rounds to fp16 zero is below
// 2^-25), so its code is 0.
constexpr int kCodecLanes = 4;   // lanes per group of 64, both directions

template <int kBits>
__global__ __launch_bounds__(kThreads) void codec_encode_kernel(CodecArgs a, const uint16_t* __restrict__ k_pool,
                                                                const uint16_t* __restrict__ v_pool,
                                                                uint8_t* __restrict__ codes,
                                                                uint16_t* __restrict__ scales) {
  constexpr float kQMax = kBits == 8 ? 127.f : 7.f;
  constexpr float kRound = 12582912.f;               // 1.5 * 2^23
  const int gid = static_cast<int>(blockIdx.x) * kThreads + static_cast<int>(threadIdx.x);
  const int gpt = static_cast<int>(a.groups_per_tensor);
  int group = gid >> 2;
  const int part = gid & 3;
  const bool live = group < 2 * gpt;                 // whole 4-lane groups are live or not
  if (!live) group = 0;
  const bool is_v = group >= gpt;
  const int gi = is_v ? group - gpt : group;
  bool valid;                                        // the 4 lanes of a group agree on it
  const uint16_t* src = (is_v ? v_pool : k_pool) + codec_pool_elem(a, gi, part, &valid);
  u32x4 x0 = *reinterpret_cast<const u32x4*>(src);              // elements 8 part ..
  u32x4 x1 = *reinterpret_cast<const u32x4*>(src + 32);         // elements 32 + 8 part ..
  if (!valid) x0 = x1 = u32x4{0u, 0u, 0u, 0u};       // a position off the pool encodes as zeros
  float f[16];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    f[2 * w] = __uint_as_float(x0[w] << 16);
    f[2 * w + 1] = __uint_as_float(x0[w] & 0xffff0000u);
    f[8 + 2 * w] = __uint_as_float(x1[w] << 16);
    f[8 + 2 * w + 1] = __uint_as_float(x1[w] & 0xffff0000u);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  const _Float16 s16 = static_cast<_Float16>(amax / kQMax);
  const float sf = static_cast<float>(s16);
  const float sd = sf > 0.f ? sf : 1.f;
  const float inv = 1.f / sd;                         // correctly rounded, once per lane
  const float half = 0.5f * sd;
  uint32_t c[16];                                     // low bits: the codes
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float y = __builtin_amdgcn_fmed3f(f[i] * inv, -kQMax, kQMax);
    const float r = y + kRound;
    c[i] = __float_as_uint(r);
    // Element i is corrected in every lane when any lane's product is near a
    // half-integer (a wave-uniform branch; the correction is exact in every
    // lane).  The test is exact: both terms are below 2^7.
    if (__builtin_amdgcn_ballot_w64(fabsf(y - (r - kRound)) > 0.5f - 0x1p-14f)) {
      const float cf = r - kRound;
      const float e = __builtin_fmaf(-cf, sd, f[i]);    // x - c * scale, exact
      const float ae = fabsf(e);
      const bool step = ae > half || (ae == half && (c[i] & 1u));
      const float cn = step ? cf + __builtin_copysignf(1.f, e) : cf;
      c[i] = __float_as_uint(__builtin_amdgcn_fmed3f(cn, -kQMax, kQMax) + kRound);
    }
  }
  if (!live) return;
  const int64_t e = static_cast<int64_t>(group) * 64;   // first element of the group in the payload
  if constexpr (kBits == 8) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t* q = c + 8 * h;
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo |= (q[i] & 0xffu) << (8 * i);
        hi |= (q[4 + i] & 0xffu) << (8 * i);
      }
      *reinterpret_cast<uint2*>(codes + e + 32 * h + 8 * part) = make_uint2(lo, hi);
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t w = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) w |= (c[8 * h + i] & 0xfu) << (4 * i);
      *reinterpret_cast<uint32_t*>(codes + e / 2 + 16 * h + 4 * part) = w;
    }
  }
  if (part == 0) scales[group] = __builtin_bit_cast(uint16_t, s16);
}

// Restore: kL consecutive lanes own one group; lane p writes the group's
// 16-byte chunks p, p + kL, ... (each store instruction of the kL lanes
// covers 16 kL contiguous bytes).
#ifndef PKV_RESTORE_LANES_Q8
#define PKV_RESTORE_LANES_Q8 8
#endif
#ifndef PKV_RESTORE_LANES_Q4
#define PKV_RESTORE_LANES_Q4 4
#endif
template <int kBits, int kL>
__global__ __launch_bounds__(kThreads) void codec_decode_kernel(CodecArgs a, uint16_t* __restrict__ k_pool,
                                                                uint16_t* __restrict__ v_pool,
                                                                const uint8_t* __restrict__ codes,
                                                                const uint16_t* __restrict__ scales) {
  static_assert(kL == 4 || kL == 8, "4 or 8 lanes per group");
  const int gid = static_cast<int>(blockIdx.x) * kThreads + static_cast<int>(threadIdx.x);
  const int gpt = static_cast<int>(a.groups_per_tensor);
  const int group = gid / kL;
  const int part = gid % kL;
  if (group >= 2 * gpt) return;
  const bool is_v = group >= gpt;
  const int gi = is_v ? group - gpt : group;
  const int64_t e = static_cast<int64_t>(group) * 64;   // first element of the group in the payload
  const float sf = static_cast<float>(__builtin_bit_cast(_Float16, scales[group]));
  // The payload loads do not depend on the table entry, so they are issued
  // together with it; only the stores wait for the validity test.
  constexpr int kIt = 8 / kL;
  uint32_t w[kIt][kBits == 8 ? 2 : 1];
#pragma unroll
  for (int h = 0; h < kIt; ++h) {
    const int chunk = part + kL * h;
    if constexpr (kBits == 8) {
      const uint2 x = *reinterpret_cast<const uint2*>(codes + e + 8 * chunk);
      w[h][0] = x.x;
      w[h][1] = x.y;
    } else {
      w[h][0] = *reinterpret_cast<const uint32_t*>(codes + e / 2 + 4 * chunk);
    }
  }
  bool valid;
  uint16_t* dst = (is_v ? v_pool : k_pool) + codec_pool_elem(a, gi, part, &valid);
  if (!valid) return;                                // a position off the pool is not written
#pragma unroll
  for (int h = 0; h < kIt; ++h) {
    int c[8];
    if constexpr (kBits == 8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[i] = static_cast<int8_t>(w[h][0] >> (8 * i));
        c[4 + i] = static_cast<int8_t>(w[h][1] >> (8 * i));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) c[i] = static_cast<int>(static_cast<int32_t>(w[h][0] << (28 - 4 * i)) >> 28);
    }
    f32x4 lo, hi;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo[i] = sf * static_cast<float>(c[i]);
      hi[i] = sf * static_cast<float>(c[4 + i]);
    }
    const uint2 plo = __builtin_bit_cast(uint2, pack_bf16x4(lo));
    const uint2 phi = __builtin_bit_cast(uint2, pack_bf16x4(hi));
    *reinterpret_cast<u32x4*>(dst + 8 * kL * h) = u32x4{plo.x, plo.y, phi.x, phi.y};
  }
}

// Streaming read of n16 16-byte chunks: a grid-stride loop, eight
// non-temporal loads in flight per thread (plain loads reach about a tenth
// less); workgroup i writes the sum modulo 2^32 of the words it read to
// sums[i].
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                                uint32_t* __restrict__ sums) {
  __shared__ uint32_t s_part[kThreads / kWave];
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = ld_stream(src + i + k * stride);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc += v[k][0] + v[k][1] + v[k][2] + v[k][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = src[i];
    acc += v[0] + v[1] + v[2] + v[3];
  }
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if ((threadIdx.x & (kWave - 1)) == 0) s_part[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
#pragma unroll
    for (int w = 0; w < kThreads / kWave; ++w) t += s_part[w];
    sums[blockIdx.x] = t;
  }
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
  if (d->dtype != PKV_F32 && d->dtype != PKV_BF16 && d->dtype != PKV_I8)
    return fail(PKV_ERR_UNSUPPORTED, std::string(fn) + ": dtype must be PKV_F32, PKV_BF16 or PKV_I8");
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

// Bytes of one (page, KV head) block of a pool of this descriptor.
int64_t head_block_bytes(const pkv_pool_desc* d) {
  if (d->dtype == PKV_I8) return i8_block_bytes(d->page_size, d->head_dim);
  return static_cast<int64_t>(d->page_size) * d->head_dim * (d->dtype == PKV_BF16 ? 2 : 4);
}

struct Plan {
  int max_q = 0;
  bool decode = false;  // decode path (few rows) vs a tile kernel
  bool prefill = false; // bf16 tiles: paged_prefill_kernel, else paged_attention_kernel
  bool pf_stream = false; // prefill: persistent workgroups over work-item records
  size_t rec_off = 0;     // prefill stream: the records in the workspace
  int64_t n_ids = 0;      // prefill stream: upper bound of the work-item ids
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
    // decode path: the units' 16-position blocks split evenly over at most
    // kDecodeWaves one-wave workgroups, each taking at least
    // PKV_DECODE_MIN_BLOCKS blocks.  Partial states: one slot per (unit,
    // wave) pair that can meet, at most units + waves.
    p->decode = true;
    p->rbw = static_cast<int>(std::max<int64_t>(1, (rows + 15) / 16));
    p->epi_rows = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(16, rows)));
    p->tile_rows = 16 * p->rbw;
    p->q_tiles = 1;
    const int64_t units = static_cast<int64_t>(n_seqs) * d->num_kv_heads;
    const int64_t blocks_max = units * ((static_cast<int64_t>(std::max(1, max_seq_len)) + 15) / 16);
    if (blocks_max > (int64_t{1} << 30)) return fail(PKV_ERR_UNSUPPORTED, std::string(fn) + ": too many KV blocks");
    p->split_len = PKV_DECODE_MIN_BLOCKS;
    const int64_t waves = d->dtype == PKV_I8 ? PKV_DECODE_WAVES_I8 : kDecodeWaves;
    p->grid = static_cast<int>(std::max<int64_t>(
        1, std::min<int64_t>(waves, (blocks_max + PKV_DECODE_MIN_BLOCKS - 1) / PKV_DECODE_MIN_BLOCKS)));
    p->n_splits = 2;   // partial slots are used
    p->items_off = 0;
    p->partial_off = (static_cast<size_t>(n_seqs + 1) * sizeof(int32_t) + 255) & ~size_t{255};
    const size_t slots = static_cast<size_t>(units) + p->grid;
    p->ws_bytes = p->partial_off + slots * (16 * p->rbw) * (d->head_dim + 2) * sizeof(float);
    return PKV_OK;
  }
  if (d->dtype == PKV_BF16 || d->dtype == PKV_I8) {
    // paged_prefill_kernel (256-row tiles) or the persistent kernel (contexts
    // up to kPfStreamCtx); KV splits only when the units' tiles alone cannot
    // fill the chip.
    p->prefill = true;
    p->pf_stream = max_seq_len <= kPfStreamCtx;
    const int keys = p->pf_stream ? kPfStreamKeys : kPfKeys;
    p->tile_rows = p->pf_stream ? 16 * kPfRb * kPfStreamWaves : kPfMaxRows;
    if (rows > (int64_t{1} << 28)) return fail(PKV_ERR_UNSUPPORTED, std::string(fn) + ": too many queries per sequence");
    const int64_t q_tiles = (rows + p->tile_rows - 1) / p->tile_rows;
    p->q_tiles = static_cast<int>(q_tiles);
    const int64_t units = static_cast<int64_t>(n_seqs) * d->num_kv_heads;
    p->n_blocks = static_cast<int>((units + 7) / 8);
    const int64_t max_tiles = (static_cast<int64_t>(max_seq_len) + keys - 1) / keys;
    int64_t want = (kTargetWorkgroups + units * q_tiles - 1) / (units * q_tiles);
    want = std::max<int64_t>(1, std::min<int64_t>(want, (max_seq_len + kMinSplitKeys - 1) / kMinSplitKeys));
    const int64_t tiles_per_split = std::max<int64_t>(1, (max_tiles + want - 1) / want);
    p->split_len = static_cast<int>(tiles_per_split * keys);
    p->n_splits = static_cast<int>(std::max<int64_t>(1, (max_tiles + tiles_per_split - 1) / tiles_per_split));
    const int64_t sched_rows = static_cast<int64_t>(p->n_blocks) * q_tiles * p->n_splits;
    if (sched_rows > (int64_t{1} << 27)) return fail(PKV_ERR_UNSUPPORTED, std::string(fn) + ": too many work items");
    p->items_off = 0;
    p->partial_off = (static_cast<size_t>(p->n_blocks + 1) * sizeof(int32_t) + 255) & ~size_t{255};
    if (p->pf_stream) {
      p->n_ids = sched_rows * 8;
      if (p->n_ids > (int64_t{1} << 24)) return fail(PKV_ERR_UNSUPPORTED, std::string(fn) + ": too many work items");
      p->rec_off = p->partial_off;
      p->partial_off = (p->rec_off + static_cast<size_t>(p->n_ids) * 8 * sizeof(int32_t) + 255) & ~size_t{255};
    }
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

template <typename T, int D, int RBW, bool kI8>
void launch_decode_t(const AttnArgs& a, const Plan& p, int n_seqs, char* ws, hipStream_t st) {
  int32_t* seq_blk = reinterpret_cast<int32_t*>(ws + p.items_off);
  constexpr int kLds = dec_lds_bytes<T, D, kI8>();
  if (a.ps_shift >= 4)
    paged_decode_kernel<T, D, RBW, 0, kI8><<<p.grid, dim3(kWave), kLds, st>>>(a, seq_blk, a.seq_lens, a.cu_q, a.block_tables);
  else if (a.ps_shift >= 0)
    paged_decode_kernel<T, D, RBW, 1, kI8><<<p.grid, dim3(kWave), kLds, st>>>(a, seq_blk, a.seq_lens, a.cu_q, a.block_tables);
  else
    paged_decode_kernel<T, D, RBW, 2, kI8><<<p.grid, dim3(kWave), kLds, st>>>(a, seq_blk, a.seq_lens, a.cu_q, a.block_tables);
  const dim3 merge_grid(static_cast<unsigned>(n_seqs * a.num_kv_heads),
                        static_cast<unsigned>(16 * RBW / merge_rows_per_group<RBW>()));
  merge_segments_kernel<T, D, RBW><<<merge_grid, dim3(kThreads), 0, st>>>(a, seq_blk);
}

// Upper bound on the prefill tile-rows the schedule kernel can list, from
// host scalars: a block's q-tiles are at most its units' sequences' q-tiles
// summed, and a sequence's units fall in at most hkv / 8 + 2 blocks.
int64_t prefill_grid(const Plan& p, int n_seqs, int hkv, int group, int total_q) {
  const int64_t tiles_all = (static_cast<int64_t>(total_q) * group + p.tile_rows - 1) / p.tile_rows + n_seqs;
  const int64_t per_seq_blocks = hkv % 8 == 0 ? hkv / 8 : hkv / 8 + 2;
  const int64_t rows = std::min<int64_t>(static_cast<int64_t>(p.n_blocks) * p.q_tiles, per_seq_blocks * tiles_all);
  return 8 * rows * p.n_splits;
}

template <int D, int kPageMode, int kWaves, int kKeys, bool kI8>
int launch_prefill_t(const AttnArgs& a, const Plan& p, char* ws, hipStream_t st) {
  constexpr int kLds = pf_lds_bytes<D, kKeys, kI8>();
  auto* kern = &paged_prefill_kernel<D, kPageMode, kWaves * kWave, kKeys, kI8>;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
  if (attr != hipSuccess) return fail(PKV_ERR_DEVICE, std::string("prefill: LDS attribute: ") + hipGetErrorString(attr));
  int32_t* row_off = reinterpret_cast<int32_t*>(ws + p.items_off);
  prefill_schedule_kernel<<<1, kSchedThreads, 0, st>>>(a, row_off, p.n_blocks, p.tile_rows, nullptr);
  const int64_t grid = prefill_grid(p, a.n_seqs, a.num_kv_heads, a.group, a.total_q);
  if (grid > INT32_MAX) return fail(PKV_ERR_UNSUPPORTED, "prefill: grid too large");
  if (grid > 0) kern<<<static_cast<int>(grid), dim3(kWaves * kWave), kLds, st>>>(a, row_off, p.n_blocks);
  if (p.n_splits > 1) {
    dim3 mg(a.num_q_heads, p.max_q, a.n_seqs);
    merge_chunks_kernel<uint16_t, D><<<mg, dim3(kWave), 0, st>>>(a);
  }
  return PKV_OK;
}

// Compute units of the current device (the stream launch fills each once).
int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  return cus;
}

template <int D, int kPageMode, int kWaves, int kKeys, bool kI8>
int launch_prefill_stream_t(const AttnArgs& a, const Plan& p, char* ws, hipStream_t st) {
  constexpr int kLds = pf_stream_lds_bytes<D, kKeys, kWaves * kWave, kI8, kPageMode>();
  static_assert(kLds <= 160 * 1024, "stream kernel LDS");
  auto* kern = &paged_prefill_stream_kernel<D, kPageMode, kWaves * kWave, kKeys, kI8>;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
  if (attr != hipSuccess) return fail(PKV_ERR_DEVICE, std::string("prefill: LDS attribute: ") + hipGetErrorString(attr));
  int32_t* row_off = reinterpret_cast<int32_t*>(ws + p.items_off);
  int32_t* rec = reinterpret_cast<int32_t*>(ws + p.rec_off);
  prefill_schedule_kernel<<<kSchedRecGroups, kSchedThreads, 0, st>>>(a, row_off, p.n_blocks, p.tile_rows, rec);
  // one workgroup per CU (two for 4-wave workgroups), a multiple of 8
  const int64_t per_cu = kWaves >= 8 ? 1 : 2;
  int64_t grid = std::min<int64_t>(device_cus() * per_cu, p.n_ids);
  grid = (grid + 7) / 8 * 8;
  if (grid > 0)
    kern<<<static_cast<int>(grid), dim3(kWaves * kWave), kLds, st>>>(a, row_off, p.n_blocks, rec);
  if (p.n_splits > 1) {
    dim3 mg(a.num_q_heads, p.max_q, a.n_seqs);
    merge_chunks_kernel<uint16_t, D><<<mg, dim3(kWave), 0, st>>>(a);
  }
  return PKV_OK;
}

template <int D, int kPageMode, bool kI8>
int launch_prefill_shape(const AttnArgs& a, const Plan& p, char* ws, hipStream_t st) {
  if (p.pf_stream) return launch_prefill_stream_t<D, kPageMode, kPfStreamWaves, kPfStreamKeys, kI8>(a, p, ws, st);
  return launch_prefill_t<D, kPageMode, kPfWaves, kPfKeys, kI8>(a, p, ws, st);
}

template <int D, bool kI8>
int launch_prefill_d(const AttnArgs& a, const Plan& p, char* ws, hipStream_t st) {
  const int mode = a.ps_shift < 0 ? 2 : a.page_size >= pf_wave_rows<D, kI8>() ? 0 : 1;
  return mode == 0 ? launch_prefill_shape<D, 0, kI8>(a, p, ws, st)
                   : mode == 1 ? launch_prefill_shape<D, 1, kI8>(a, p, ws, st) : launch_prefill_shape<D, 2, kI8>(a, p, ws, st);
}

template <typename T, int D, bool kI8 = false>
void launch_attention_d(const AttnArgs& a, const Plan& p, int n_seqs, int hkv, char* ws, hipStream_t st) {
  if (p.decode) {
    switch (p.rbw) {
      case 1: launch_decode_t<T, D, 1, kI8>(a, p, n_seqs, ws, st); break;
      case 2: launch_decode_t<T, D, 2, kI8>(a, p, n_seqs, ws, st); break;
      default: launch_decode_t<T, D, 3, kI8>(a, p, n_seqs, ws, st); break;
    }
    return;
  }
  if constexpr (kI8) return;   // INT8 pages: the decode and prefill kernels cover every plan
  launch_attention_t<T, D, 4, 1>(a, p, n_seqs, hkv, st);
  if (p.n_splits > 1) {
    dim3 grid(a.num_q_heads, p.max_q, n_seqs);
    merge_chunks_kernel<T, D><<<grid, dim3(kWave), 0, st>>>(a);
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
  a.waves = p.grid;
  a.head_bytes = static_cast<int32_t>(head_block_bytes(desc));
  a.kv_cap = static_cast<int32_t>(std::min<int64_t>(static_cast<int64_t>(bt_stride) * desc->page_size, max_seq_len));
  if (p.decode) {
    const size_t rows_out = (static_cast<size_t>(n_seqs) * desc->num_kv_heads + p.grid) * (16 * p.rbw);
    a.ws_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.partial_off);
    a.ws_ml = a.ws_o + rows_out * desc->head_dim;
  } else if (p.n_splits > 1) {
    const size_t rows_out = static_cast<size_t>(n_seqs) * max_q * hq * p.n_splits;
    a.ws_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.partial_off);
    a.ws_ml = a.ws_o + rows_out * desc->head_dim;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int hkv = desc->num_kv_heads;
  char* ws = static_cast<char*>(workspace);
  (void)hipGetLastError();
  const bool i8 = desc->dtype == PKV_I8;
  if (p.prefill) {
    if (desc->head_dim == 128)
      rc = i8 ? launch_prefill_d<128, true>(a, p, ws, st) : launch_prefill_d<128, false>(a, p, ws, st);
    else
      rc = i8 ? launch_prefill_d<64, true>(a, p, ws, st) : launch_prefill_d<64, false>(a, p, ws, st);
    if (rc != PKV_OK) return rc;
  } else if (i8) {
    if (desc->head_dim == 128)
      launch_attention_d<uint16_t, 128, true>(a, p, n_seqs, hkv, ws, st);
    else
      launch_attention_d<uint16_t, 64, true>(a, p, n_seqs, hkv, ws, st);
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

int codec_setup(const char* fn, const pkv_pool_desc* desc, const void* k_pool, const void* v_pool,
                const int32_t* block_table, int32_t n_positions, int32_t bits, const void* payload, CodecArgs* a,
                int64_t* groups) {
  int rc = check_desc(desc, fn);
  if (rc != PKV_OK) return rc;
  if (desc->dtype != PKV_BF16) return fail(PKV_ERR_UNSUPPORTED, std::string(fn) + ": bf16 pools only");
  if (bits != 4 && bits != 8) return fail(PKV_ERR_UNSUPPORTED, std::string(fn) + ": bits must be 4 or 8");
  if (n_positions < 0) return fail(PKV_ERR_INVALID_ARG, std::string(fn) + ": n_positions < 0");
  if (n_positions > 0 && (!k_pool || !v_pool || !block_table || !payload))
    return fail(PKV_ERR_INVALID_ARG, std::string(fn) + ": NULL device pointer");
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(payload))
    return fail(PKV_ERR_INVALID_ARG, std::string(fn) + ": pools and payload must be 16-byte aligned");
  a->block_table = block_table;
  a->n_positions = n_positions;
  a->hkv = desc->num_kv_heads;
  a->head_dim = desc->head_dim;
  a->page_size = desc->page_size;
  a->ps_shift = log2_exact(desc->page_size);
  a->num_pages = desc->num_pages;
  a->groups_per_tensor = static_cast<int64_t>(n_positions) * desc->num_kv_heads * (desc->head_dim / 64);
  if (2 * a->groups_per_tensor * 8 + kThreads > INT32_MAX)
    return fail(PKV_ERR_UNSUPPORTED, std::string(fn) + ": prefix too long");
  *groups = 2 * a->groups_per_tensor;   // K and V groups; each kernel sizes its grid by its lanes per group
  return PKV_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// Scratch of pkv_decode_noalloc: the decode kernels' workspace (the
// per-sequence block prefix and the split partial states) in a static device
// array, for callers that cannot allocate.  Each device holds its own copy
// from module load until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the
// symbol): the device address comes from hipGetSymbolAddress, taken once per
// device with that device current, and is kept per device.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device.
int scratch_address(const char* fn, void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return fail(PKV_ERR_DEVICE, std::string(fn) + ": hipGetDevice: " + hipGetErrorString(err));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PKV_ERR_UNSUPPORTED, std::string(fn) + ": device index " + std::to_string(dev) + " out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err != hipSuccess || !ptr)
      return fail(PKV_ERR_DEVICE, std::string(fn) + ": hipGetSymbolAddress(scratch): " + hipGetErrorString(err));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
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
  const int64_t pool_slots = static_cast<int64_t>(desc->num_pages) * desc->page_size;
  const int ps_shift = log2_exact(desc->page_size);
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (desc->dtype == PKV_I8) {
    // one group of head_dim / 8 lanes per (token, KV head) vector of K or V
    const int64_t threads = 2 * static_cast<int64_t>(n_tokens) * desc->num_kv_heads * (desc->head_dim / 8);
    const int64_t blocks = (threads + kThreads - 1) / kThreads;
    if (blocks > INT32_MAX) return fail(PKV_ERR_UNSUPPORTED, "pkv_store_kv: too many tokens");
    const int32_t hb = static_cast<int32_t>(head_block_bytes(desc));
    if (desc->head_dim == 128)
      store_kv_i8_kernel<128><<<dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, st>>>(
          static_cast<char*>(k_pool), static_cast<char*>(v_pool), static_cast<const uint16_t*>(k_new),
          static_cast<const uint16_t*>(v_new), slots, n_tokens, desc->num_kv_heads, desc->page_size, ps_shift,
          pool_slots, hb);
    else
      store_kv_i8_kernel<64><<<dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, st>>>(
          static_cast<char*>(k_pool), static_cast<char*>(v_pool), static_cast<const uint16_t*>(k_new),
          static_cast<const uint16_t*>(v_new), slots, n_tokens, desc->num_kv_heads, desc->page_size, ps_shift,
          pool_slots, hb);
  } else {
    const int es = desc->dtype == PKV_BF16 ? 2 : 4;
    const int64_t chunks = 2 * static_cast<int64_t>(n_tokens) * desc->num_kv_heads *
                           (desc->head_dim * es / 16);
    const int64_t blocks = (chunks + kThreads - 1) / kThreads;
    if (blocks > INT32_MAX) return fail(PKV_ERR_UNSUPPORTED, "pkv_store_kv: too many tokens");
    if (es == 2)
      store_kv_kernel<2><<<dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, st>>>(
                         static_cast<char*>(k_pool), static_cast<char*>(v_pool),
                         static_cast<const char*>(k_new), static_cast<const char*>(v_new), slots,
                         n_tokens, desc->num_kv_heads, desc->head_dim, desc->page_size, ps_shift, pool_slots);
    else
      store_kv_kernel<4><<<dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, st>>>(
                         static_cast<char*>(k_pool), static_cast<char*>(v_pool),
                         static_cast<const char*>(k_new), static_cast<const char*>(v_new), slots,
                         n_tokens, desc->num_kv_heads, desc->head_dim, desc->page_size, ps_shift, pool_slots);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess)
    return fail(PKV_ERR_DEVICE, std::string("pkv_store_kv: launch failed: ") + hipGetErrorString(err));
  return PKV_OK;
}

int pkv_copy_pages(const pkv_pool_desc* desc, void* k_pool, void* v_pool, const int32_t* copies,
                   int32_t n_copies, void* stream) {
  int rc = check_desc(desc, "pkv_copy_pages");
  if (rc != PKV_OK) return rc;
  if (n_copies < 0) return fail(PKV_ERR_INVALID_ARG, "pkv_copy_pages: n_copies < 0");
  if (n_copies == 0) return PKV_OK;
  if (!k_pool || !v_pool || !copies) return fail(PKV_ERR_INVALID_ARG, "pkv_copy_pages: NULL device pointer");
  if (!aligned16(k_pool) || !aligned16(v_pool) || (reinterpret_cast<uintptr_t>(copies) & 3u))
    return fail(PKV_ERR_INVALID_ARG, "pkv_copy_pages: misaligned device pointer");
  const int64_t page_bytes = head_block_bytes(desc) * desc->num_kv_heads;   // a multiple of 16
  const int64_t page_chunks = page_bytes / 16;
  const int64_t per_block = static_cast<int64_t>(kThreads) * kCopyPer;
  const int64_t tiles = (2 * page_chunks + per_block - 1) / per_block;
  if (page_chunks > INT32_MAX / 4 || tiles > 65535)
    return fail(PKV_ERR_UNSUPPORTED, "pkv_copy_pages: pages too large");
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  copy_pages_kernel<<<dim3(static_cast<unsigned>(n_copies), static_cast<unsigned>(tiles)), dim3(kThreads), 0, st>>>(
      static_cast<char*>(k_pool), static_cast<char*>(v_pool), copies, static_cast<int32_t>(page_chunks),
      desc->num_pages);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess)
    return fail(PKV_ERR_DEVICE, std::string("pkv_copy_pages: launch failed: ") + hipGetErrorString(err));
  return PKV_OK;
}

int pkv_stream_read(const void* buf, size_t bytes, uint32_t* partial_sums, int32_t n_partials, void* stream) {
  if (n_partials < 1 || n_partials > 65535)
    return fail(PKV_ERR_INVALID_ARG, "pkv_stream_read: n_partials must be in 1..65535");
  if (bytes % 16) return fail(PKV_ERR_INVALID_ARG, "pkv_stream_read: bytes must be a multiple of 16");
  if (!partial_sums || (bytes > 0 && !buf)) return fail(PKV_ERR_INVALID_ARG, "pkv_stream_read: NULL device pointer");
  if (!aligned16(buf) || (reinterpret_cast<uintptr_t>(partial_sums) & 3u))
    return fail(PKV_ERR_INVALID_ARG, "pkv_stream_read: misaligned device pointer");
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  stream_read_kernel<<<dim3(static_cast<unsigned>(n_partials)), dim3(kThreads), 0, st>>>(
      static_cast<const u32x4*>(buf), static_cast<int64_t>(bytes / 16), partial_sums);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess)
    return fail(PKV_ERR_DEVICE, std::string("pkv_stream_read: launch failed: ") + hipGetErrorString(err));
  return PKV_OK;
}

size_t pkv_codec_payload_bytes(int32_t n_positions, int32_t num_kv_heads, int32_t head_dim, int32_t bits) {
  if (n_positions < 0 || num_kv_heads < 1 || head_dim < 64 || head_dim % 64 || (bits != 4 && bits != 8)) return 0;
  const size_t elems = 2 * static_cast<size_t>(n_positions) * num_kv_heads * head_dim;
  return elems * bits / 8 + 2 * (elems / 64);
}


int pkv_codec_encode(const pkv_pool_desc* desc, const void* k_pool, const void* v_pool, const int32_t* block_table,
                     int32_t n_positions, int32_t bits, void* payload, void* stream) {
  CodecArgs a{};
  int64_t groups = 0;
  int rc = codec_setup("pkv_codec_encode", desc, k_pool, v_pool, block_table, n_positions, bits, payload, &a, &groups);
  if (rc != PKV_OK || n_positions == 0) return rc;
  uint8_t* codes = static_cast<uint8_t*>(payload);
  uint16_t* scales = reinterpret_cast<uint16_t*>(codes + 2 * a.groups_per_tensor * 64 * bits / 8);
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int64_t blocks = (groups * kCodecLanes + kThreads - 1) / kThreads;
  if (bits == 8)
    codec_encode_kernel<8><<<dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, st>>>(
        a, static_cast<const uint16_t*>(k_pool), static_cast<const uint16_t*>(v_pool), codes, scales);
  else
    codec_encode_kernel<4><<<dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, st>>>(
        a, static_cast<const uint16_t*>(k_pool), static_cast<const uint16_t*>(v_pool), codes, scales);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess)
    return fail(PKV_ERR_DEVICE, std::string("pkv_codec_encode: launch failed: ") + hipGetErrorString(err));
  return PKV_OK;
}

int pkv_codec_decode(const pkv_pool_desc* desc, void* k_pool, void* v_pool, const int32_t* block_table,
                     int32_t n_positions, int32_t bits, const void* payload, void* stream) {
  CodecArgs a{};
  int64_t groups = 0;
  int rc = codec_setup("pkv_codec_decode", desc, k_pool, v_pool, block_table, n_positions, bits, payload, &a, &groups);
  if (rc != PKV_OK || n_positions == 0) return rc;
  const uint8_t* codes = static_cast<const uint8_t*>(payload);
  const uint16_t* scales = reinterpret_cast<const uint16_t*>(codes + 2 * a.groups_per_tensor * 64 * bits / 8);
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (bits == 8)
    codec_decode_kernel<8, PKV_RESTORE_LANES_Q8>
        <<<dim3(static_cast<unsigned>((groups * PKV_RESTORE_LANES_Q8 + kThreads - 1) / kThreads)), dim3(kThreads), 0,
            st>>>(a, static_cast<uint16_t*>(k_pool), static_cast<uint16_t*>(v_pool), codes, scales);
  else
    codec_decode_kernel<4, PKV_RESTORE_LANES_Q4>
        <<<dim3(static_cast<unsigned>((groups * PKV_RESTORE_LANES_Q4 + kThreads - 1) / kThreads)), dim3(kThreads), 0,
            st>>>(a, static_cast<uint16_t*>(k_pool), static_cast<uint16_t*>(v_pool), codes, scales);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess)
    return fail(PKV_ERR_DEVICE, std::string("pkv_codec_decode: launch failed: ") + hipGetErrorString(err));
  return PKV_OK;
}

size_t pkv_i8_block_bytes(int32_t page_size, int32_t head_dim) {
  if (page_size < 1 || head_dim < 1) return 0;
  return static_cast<size_t>(i8_block_bytes(page_size, head_dim));
}

size_t pkv_pool_bytes(const pkv_pool_desc* desc) {
  if (check_desc(desc, "pkv_pool_bytes") != PKV_OK) return 0;
  return static_cast<size_t>(desc->num_pages) * desc->num_kv_heads * static_cast<size_t>(head_block_bytes(desc));
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

int pkv_decode_noalloc(const pkv_pool_desc* desc, const void* k_pool, const void* v_pool, const void* q,
                       int32_t n_seqs, int32_t num_q_heads, const int32_t* block_tables, int32_t bt_stride,
                       const int32_t* seq_lens, int32_t max_seq_len, float scale, void* out, void* stream) {
  const char* fn = "pkv_decode_noalloc";
  Plan p;
  int rc = make_plan(desc, n_seqs, num_q_heads, 1, max_seq_len, &p, fn);
  if (rc != PKV_OK) return rc;
  if (p.ws_bytes > PKV_NOALLOC_SCRATCH_BYTES)
    return fail(PKV_ERR_BUFFER_TOO_SMALL, std::string(fn) + ": this batch needs " + std::to_string(p.ws_bytes) +
                                              " bytes of scratch, above the static " +
                                              std::to_string(PKV_NOALLOC_SCRATCH_BYTES) +
                                              "; call pkv_decode with a workspace");
  void* ws = nullptr;
  if (p.ws_bytes > 0 && n_seqs > 0) {
    rc = scratch_address(fn, &ws);
    if (rc != PKV_OK) return rc;
  }
  return run_attention(fn, desc, k_pool, v_pool, q, n_seqs, nullptr, n_seqs, num_q_heads, block_tables,
                       bt_stride, seq_lens, 1, max_seq_len, scale, out, ws, ws ? PKV_NOALLOC_SCRATCH_BYTES : 0,
                       stream);
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
