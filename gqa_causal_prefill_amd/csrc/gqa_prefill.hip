// Causal grouped-query prefill attention for MI355X (gfx950, CDNA4).
//
// Pages cited by title and section:
//   [DCU report]  "DCU使用技术报告（中篇）" (DCU technical report, part 2)
//   [INT8 QK]     "gfx936 DCU上实现INT8 QK MMAC" (INT8 QK MMAC on gfx936)
//   [hybrid]      the hybrid-attention page whose section 五 is the wave64
//                 register staircase
//
// What is computed ([DCU report §1-§2], [INT8 QK §1, §4, §5.2]): for query i of
// a chunk (position kv_len - q_len + i) and query head h, the softmax over keys
// 0 .. kv_len - q_len + i of score = q·k/16 (or, with INT8 keys,
// int32(Qq·Kq)·sQ·sK/16), applied to V of KV head h/6, accumulated in FP32 and
// written as bf16.
//
// Work decomposition (designed for gfx950, not the pages' Triton tiling):
//   * a workgroup is 4 wave64s (one per SIMD) sharing one KV head g; every K/V
//     tile staged in LDS serves all its query rows ([DCU report §2, §4]: a
//     program covers tokens x heads of one GQA group, and the reuse of each K/V
//     tile grows with the rows per program). Each wave owns QB 16-column blocks
//     of the 16x16 MFMA output: block b = one query head, column c = one token
//     of a 16-token run. QB = 3: a workgroup is 32 tokens x all 6 heads of g
//     (192 rows); QB = 2: 64 tokens x a pair of g's heads (128 rows);
//   * scores are computed transposed (S^T = K·Q^T) so every lane holds keys of
//     ONE query column: the row maxima need two permlane swaps, and the lane's
//     S^T registers are directly the P^T operand of the P·V MFMA;
//   * KV tiles of 64 keys arrive by global_load_lds_dwordx4 (no staging
//     registers), double-buffered, stored chunk-major ([16-byte chunk][key]) so
//     that K fragments are one conflict-free ds_read_b128 and the V^T operand of
//     P·V is two ds_read_b64_tr_b16 transposing reads, all at immediate offsets;
//   * online softmax in the exp2 domain with a lazy rescale: the running max
//     used for the exponentials only moves when a tile raises it by more than
//     2^8, which keeps every exponent <= 2^8 and skips almost every rescale of
//     the accumulator registers (the result is the same softmax);
//   * P is rounded to bf16 for the MFMA and the row sums use the rounded values.
//     Workgroups whose first query sees fewer than 256 keys (short histories,
//     where few keys carry large weights) multiply with P split into a bf16
//     high part and a bf16 low part, keeping ~16 bits of P;
//   * with INT8 keys each query row is quantised in the prologue (once per row,
//     [INT8 QK §4]) and Q·K^T runs on v_mfma_i32_16x16x64_i8; the int32 score is
//     scaled by sK·sQ·log2(e)/16 per score before the softmax ([INT8 QK §1]).

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include "gqa_prefill.h"

#ifndef GQA_DEFAULT_QB
#define GQA_DEFAULT_QB 2
#endif

namespace {

constexpr int kHq = GQA_NUM_Q_HEADS;     // 24
constexpr int kHkv = GQA_NUM_KV_HEADS;   // 4
constexpr int kD = GQA_HEAD_DIM;         // 256
constexpr int kGroup = kHq / kHkv;       // 6
constexpr int kBs = GQA_BLOCK_SIZE;      // 16

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kKt = 64;                  // keys per KV tile
constexpr int kSplitBelow = 256;
constexpr float kTau = 8.0f;
constexpr float kLog2eOver16 = 1.4426950408889634f / 16.0f;

// LDS tiles are chunk-major: byte (chunk, key) at chunk * kChunkStride + key * 16.
constexpr int kChunkStride = kKt * 16;               // 1 KiB
constexpr int kKTileBf16 = (kD * 2 / 16) * kChunkStride;  // 32 chunks: 32 KiB
constexpr int kKTileI8 = (kD / 16) * kChunkStride;        // 16 chunks: 16 KiB
constexpr int kVTile = (kD * 2 / 16) * kChunkStride;      // 32 KiB
constexpr int kSkTile = kKt * 4;                          // 256 B of key scales

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

struct Params {
  const uint8_t* q;        // bf16 [q_len, 24, 256]
  const uint8_t* k;        // bf16 or int8, contiguous or paged
  const uint8_t* v;        // bf16, contiguous or paged
  const int32_t* bt;       // block table or null
  const float* ks;         // key scales [kv_len, 4] or null
  uint8_t* out;            // bf16 [q_len, 24, 256]
  int32_t num_blocks;
  int32_t q_len;
  int32_t kv_len;
  int32_t n_tblk;          // token blocks of the grid
};

// Workgroup shape for QB 16-column query blocks per wave.
template <int QB>
struct Shape {
  static constexpr int kTokenBlocks = (QB == 3) ? 2 : 4;            // 16-token runs per workgroup
  static constexpr int kHeadGroups = kWaves / kTokenBlocks;         // QB-head groups per workgroup
  static constexpr int kHeadsPerWg = QB * kHeadGroups;              // 6 or 2
  static constexpr int kTokPerWg = 16 * kTokenBlocks;               // 32 or 64
  static constexpr int kSplitsPerGroup = kGroup / kHeadsPerWg;      // 1 or 3 workgroups per (g, tokens)
};

__device__ __forceinline__ float wave_xor_max(float x, int mask) {
  return fmaxf(x, __shfl_xor(x, mask));
}
__device__ __forceinline__ float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One V^T operand of the P·V MFMA from a chunk-major V tile: two transposing reads,
// 16 keys apart (see the lane mapping at the call site). Issued as inline assembly
// so the compiler does not make them wait for the global->LDS copies into the
// other buffer; `vt_wait` must run before the registers are used.
struct VtFrag {
  uint2 lo, hi;
};

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

template <int OFF>
__device__ __forceinline__ void vt_issue(VtFrag& f, uint32_t addr) {
  asm volatile("ds_read_b64_tr_b16 %0, %2 offset:%3\n\tds_read_b64_tr_b16 %1, %2 offset:%4"
               : "=v"(f.lo), "=v"(f.hi)
               : "v"(addr), "i"(OFF), "i"(OFF + 256));
}

// Wait until at most N LDS operations of this wave are outstanding (LDS operations
// complete in order), tying the fragment's registers to the wait.
template <int N>
__device__ __forceinline__ void vt_wait(VtFrag& f) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(f.lo), "+v"(f.hi) : "i"(N));
}

__device__ __forceinline__ bf16x8 vt_value(const VtFrag& f) {
  const uint4 u = make_uint4(f.lo.x, f.lo.y, f.hi.x, f.hi.y);
  return __builtin_bit_cast(bf16x8, u);
}

// Element index of the row (key, kv head g) in the K/V arrays.
template <bool PAGED>
__device__ __forceinline__ size_t kv_row(int g, int key, int blk) {
  if constexpr (PAGED) {
    return ((size_t)(blk * kHkv + g) * kBs + (key & (kBs - 1))) * kD;
  } else {
    return ((size_t)key * kHkv + g) * kD;
  }
}

__device__ __forceinline__ int clamp_block(const Params& p, int blk) {
  return min(max(blk, 0), p.num_blocks - 1);
}

// Issue this wave's share of the global -> LDS copies for the KV tile at kbase.
// Lane t copies key kbase + t (clamped to the last key: keys past kv_len are
// finite duplicates that the causal mask hides); each instruction moves one
// 16-byte chunk column of the 64 keys. `blk` is the lane's physical block
// (paged caches only).
template <bool PAGED, bool INT8K>
__device__ __forceinline__ void issue_tile(const Params& p, int g, int kbase, int w, int lane,
                                           int blk, uint8_t* kbuf, uint8_t* vbuf, float* skbuf) {
  const int key = min(kbase + lane, p.kv_len - 1);
  const size_t row = kv_row<PAGED>(g, key, blk);
  const uint8_t* krow = p.k + row * (INT8K ? 1 : 2);
  const uint8_t* vrow = p.v + row * 2;
  constexpr int kKChunks = INT8K ? kD / 16 : kD * 2 / 16;
  constexpr int kKPerWave = kKChunks / kWaves;
#pragma unroll
  for (int i = 0; i < kKPerWave; ++i) {
    const int c = w * kKPerWave + i;
    __builtin_amdgcn_global_load_lds(krow + c * 16, kbuf + c * kChunkStride, 16, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = w * 8 + i;
    __builtin_amdgcn_global_load_lds(vrow + c * 16, vbuf + c * kChunkStride, 16, 0, 0);
  }
  if constexpr (INT8K) {
    if (w == 0) __builtin_amdgcn_global_load_lds(p.ks + (size_t)key * kHkv + g, skbuf, 4, 0, 0);
  }
}

// Physical block of the lane's key in the tile at kbase (paged caches).
template <bool PAGED>
__device__ __forceinline__ int tile_block(const Params& p, int kbase, int lane) {
  if constexpr (PAGED) {
    const int key = min(kbase + lane, p.kv_len - 1);
    return clamp_block(p, p.bt[key >> 4]);
  } else {
    return 0;
  }
}

__device__ __forceinline__ void wait_vm_all() {
  // s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima)
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Step N of O^T += V^T · P^T over a 64-key tile: N = 16 ks + db, ks = 32-key half,
// db = 16-feature block. Issues the transposing reads of step N + 1, waits for
// step N's, runs its MFMAs.
template <int N, int QB, bool SPLIT>
struct PvStep {
  static __device__ __forceinline__ void run(VtFrag (&vf)[2], uint32_t vaddr,
                                             const bf16x8 (&ph)[QB][2], const bf16x8 (&pl)[QB][2],
                                             f32x4 (&o)[16][QB]) {
    constexpr int ks = N >> 4, db = N & 15;
    if constexpr (N + 1 < 32) {
      constexpr int ks1 = (N + 1) >> 4, db1 = (N + 1) & 15;
      vt_issue<db1 * 2 * kChunkStride + 32 * ks1 * 16>(vf[(N + 1) & 1], vaddr);
      vt_wait<2>(vf[N & 1]);
    } else {
      vt_wait<0>(vf[N & 1]);
    }
    const bf16x8 v = vt_value(vf[N & 1]);
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      o[db][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v, ph[b][ks], o[db][b], 0, 0, 0);
      if constexpr (SPLIT)
        o[db][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v, pl[b][ks], o[db][b], 0, 0, 0);
    }
    if constexpr (N + 1 < 32) PvStep<N + 1, QB, SPLIT>::run(vf, vaddr, ph, pl, o);
  }
};

template <bool PAGED, bool INT8K, int QB>
struct Tile {
  // S^T for 64 keys x (QB x 16) columns, P and the running softmax state
  template <bool SPLIT>
  static __device__ __forceinline__ void compute(const uint8_t* kbuf, const uint8_t* vbuf,
                                                 const float* skbuf, int kbase, int L, int c,
                                                 int lane, bool diag, int limit,
                                                 const bf16x8 (&qf)[INT8K ? 1 : QB][INT8K ? 1 : 8],
                                                 const i32x4 (&qq)[INT8K ? QB : 1][INT8K ? 4 : 1],
                                                 const float (&qs)[QB], float (&m)[QB],
                                                 float (&l)[QB], f32x4 (&o)[16][QB]) {
    // ---- S^T = K · Q^T ----
    float sc[QB][16];   // [query block][key slot 4 kb + r] for key 16 kb + 4 L + r
    const int koff = L * kChunkStride + c * 16;
    if constexpr (!INT8K) {
      f32x4 acc[QB][4];
#pragma unroll
      for (int b = 0; b < QB; ++b)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) acc[b][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      // K fragments for step s + 1 are read while the MFMAs of step s run
      bf16x8 kf[2][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        kf[0][kb] = *reinterpret_cast<const bf16x8*>(kbuf + koff + kb * 256);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        if (s + 1 < 8) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
            kf[(s + 1) & 1][kb] = *reinterpret_cast<const bf16x8*>(
                kbuf + koff + 4 * (s + 1) * kChunkStride + kb * 256);
        }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int b = 0; b < QB; ++b)
            acc[b][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s & 1][kb], qf[b][s], acc[b][kb],
                                                                 0, 0, 0);
      }
#pragma unroll
      for (int b = 0; b < QB; ++b)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[b][4 * kb + r] = acc[b][kb][r] * kLog2eOver16;
    } else {
      i32x4 acc[QB][4];
#pragma unroll
      for (int b = 0; b < QB; ++b)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) acc[b][kb] = i32x4{0, 0, 0, 0};
      i32x4 kf[2][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        kf[0][kb] = *reinterpret_cast<const i32x4*>(kbuf + koff + kb * 256);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (s + 1 < 4) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
            kf[(s + 1) & 1][kb] = *reinterpret_cast<const i32x4*>(
                kbuf + koff + 4 * (s + 1) * kChunkStride + kb * 256);
        }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int b = 0; b < QB; ++b)
            acc[b][kb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kf[s & 1][kb], qq[b][s], acc[b][kb],
                                                               0, 0, 0);
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const f32x4 sk = *reinterpret_cast<const f32x4*>(skbuf + 16 * kb + 4 * L);
#pragma unroll
        for (int b = 0; b < QB; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[b][4 * kb + r] = (float)acc[b][kb][r] * sk[r] * qs[b];
      }
    }

    // ---- causal mask (only tiles that reach past the workgroup's first query) ----
    if (diag) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kbase + 16 * kb + 4 * L + r;
          if (key > limit) {
#pragma unroll
            for (int b = 0; b < QB; ++b) sc[b][4 * kb + r] = -__builtin_inff();
          }
        }
    }

    // ---- online softmax (exp2 domain, lazy rescale) ----
    float mnew[QB];
    bool need = false;
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      float mx = sc[b][0];
#pragma unroll
      for (int e = 1; e < 16; ++e) mx = fmaxf(mx, sc[b][e]);
      mx = xor16_max(mx);
      mx = xor32_max(mx);
      mnew[b] = fmaxf(m[b], mx);
      need = need || (mnew[b] > m[b] + kTau);
    }
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        const float alpha = __builtin_amdgcn_exp2f(m[b] - mnew[b]);
        m[b] = mnew[b];
        l[b] *= alpha;
#pragma unroll
        for (int db = 0; db < 16; ++db) o[db][b] *= alpha;
      }
    }
    // P^T operands: k-step ks covers keys 32 ks .. 32 ks + 31; a lane's 8 elements are
    // keys 32 ks + 4 L + {0..3} and 32 ks + 16 + 4 L + {0..3} = its S^T slots 8 ks .. 8 ks + 7
    bf16x8 ph[QB][2], pl[QB][2];
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      float sum = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        f32x8 pv;
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = __builtin_amdgcn_exp2f(sc[b][8 * ks + e] - m[b]);
        ph[b][ks] = __builtin_convertvector(pv, bf16x8);
        const f32x8 hi = __builtin_convertvector(ph[b][ks], f32x8);
        if constexpr (SPLIT) {
          pl[b][ks] = __builtin_convertvector(pv - hi, bf16x8);
          const f32x8 lo = __builtin_convertvector(pl[b][ks], f32x8);
#pragma unroll
          for (int e = 0; e < 8; ++e) sum += hi[e] + lo[e];
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) sum += hi[e];
        }
      }
      l[b] += sum;
    }

    // ---- O^T += V^T · P^T ----
    // transposing read: lane i of 16-lane group L fetches features 16 db + 4 (i & 3) .. +3 of
    // key 32 ks + 16 h + 4 L + (i >> 2); after the transpose lane (L, c) holds
    // V[32 ks + 16 h + 4 L + k][16 db + c] for k = 0..3
    const int voff = ((c & 3) >> 1) * kChunkStride + (4 * L + (c >> 2)) * 16 + 8 * (c & 1);
    // V^T fragments for step n + 1 (n = 16 ks + db) are read while the MFMAs of step n run
    VtFrag vf[2];
    const uint32_t vaddr = lds_addr(vbuf) + voff;
    vt_issue<0>(vf[0], vaddr);
    PvStep<0, QB, SPLIT>::run(vf, vaddr, ph, pl, o);
  }
};

template <bool PAGED, bool INT8K, int QB>
constexpr int stage_bytes() {
  return (INT8K ? kKTileI8 : kKTileBf16) + kVTile + (INT8K ? kSkTile : 0);
}

// The whole workgroup program. SPLIT selects the P·V form (see the file header); it
// is fixed per workgroup, so each form is a separate straight-line program.
template <bool PAGED, bool INT8K, int QB, bool SPLIT>
__device__ __forceinline__ void run(const Params& p, uint8_t* smem) {
  using S = Shape<QB>;
  constexpr int kKTile = INT8K ? kKTileI8 : kKTileBf16;
  constexpr int kStage = stage_bytes<PAGED, INT8K, QB>();

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int L = lane >> 4;      // k-group of the MFMA operands / row group of the output
  const int c = lane & 15;      // query column (token) inside a 16-column block
  const int tw = w % S::kTokenBlocks;
  const int hw = w / S::kTokenBlocks;

  // Workgroup id -> (KV head, head subset, token block). id % 4 is the KV head, so
  // workgroups dispatched round-robin over the 8 XCDs keep one KV head per XCD (its
  // K/V stream shares that XCD's L2); token blocks go longest first.
  const int id = blockIdx.x;
  const int g = id & (kHkv - 1);
  const int rest = id >> 2;
  const int hsel = rest % S::kSplitsPerGroup;
  const int tblk = p.n_tblk - 1 - rest / S::kSplitsPerGroup;
  const int t0 = tblk * S::kTokPerWg;
  const int off = p.kv_len - p.q_len;
  const int head0 = kGroup * g + hsel * S::kHeadsPerWg + hw * QB;   // head of query block 0

  // query column (b, c) of this lane: token t0 + 16 tw + c, head head0 + b
  const int tok = t0 + 16 * tw + c;
  const bool tok_ok = tok < p.q_len;
  const int limit = off + tok;   // last visible key of this column

  const int last_tok = min(t0 + S::kTokPerWg, p.q_len);
  const int ntiles = (off + last_tok + kKt - 1) / kKt;

  // start the first tile's copies before the Q prologue
  int blk = tile_block<PAGED>(p, 0, lane);
  issue_tile<PAGED, INT8K>(p, g, 0, w, lane, blk, smem, smem + kKTile,
                           reinterpret_cast<float*>(smem + kKTile + kVTile));
  if (ntiles > 1) blk = tile_block<PAGED>(p, kKt, lane);

  // ---- prologue: Q fragments (B operand of S^T = K·Q^T) ----
  bf16x8 qf[INT8K ? 1 : QB][INT8K ? 1 : 8];
  i32x4 qq[INT8K ? QB : 1][INT8K ? 4 : 1];
  float qs[QB];
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    const uint8_t* qrow = p.q + ((size_t)tok * kHq + head0 + b) * kD * 2;
    if constexpr (!INT8K) {
      qs[b] = kLog2eOver16;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        uint4 raw = tok_ok ? *reinterpret_cast<const uint4*>(qrow + (32 * s + 8 * L) * 2)
                           : make_uint4(0, 0, 0, 0);
        qf[b][s] = __builtin_bit_cast(bf16x8, raw);
      }
    } else {
      // each lane holds features 64 s + 16 L .. +15 (s = 0..3) of its query row;
      // the four lanes L = 0..3 of column c hold the whole row
      float x[4][16];
      float amax = 0.0f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          uint4 raw = tok_ok ? *reinterpret_cast<const uint4*>(qrow + (64 * s + 16 * L + 8 * h2) * 2)
                             : make_uint4(0, 0, 0, 0);
          bf16x8 vv = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            x[s][8 * h2 + e] = (float)vv[e];
            amax = fmaxf(amax, fabsf(x[s][8 * h2 + e]));
          }
        }
      }
      amax = xor16_max(amax);
      amax = xor32_max(amax);
      const float sq = amax / 127.0f;
      qs[b] = sq * kLog2eOver16;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        uint32_t wv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t packed = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float r = (sq == 0.0f) ? 0.0f : __builtin_rintf(x[s][4 * j + e] / sq);
            r = fminf(fmaxf(r, -127.0f), 127.0f);
            packed |= ((uint32_t)((int)r) & 0xffu) << (8 * e);
          }
          wv[j] = packed;
        }
        qq[b][s] = i32x4{(int)wv[0], (int)wv[1], (int)wv[2], (int)wv[3]};
      }
    }
  }

  // ---- accumulators: O^T blocks [feature block db][query block b] ----
  f32x4 o[16][QB];
#pragma unroll
  for (int db = 0; db < 16; ++db)
#pragma unroll
    for (int b = 0; b < QB; ++b) o[db][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[QB], l[QB];
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    m[b] = -__builtin_inff();
    l[b] = 0.0f;
  }

  using T = Tile<PAGED, INT8K, QB>;
  for (int j = 0; j < ntiles; ++j) {
    const int kbase = j * kKt;
    uint8_t* cur = smem + (j & 1) * kStage;
    uint8_t* nxt = smem + ((j + 1) & 1) * kStage;
    wait_vm_all();
    __syncthreads();   // tile j is in `cur`; everyone is done with `nxt` (tile j - 1)
    if (j + 1 < ntiles) {
      issue_tile<PAGED, INT8K>(p, g, kbase + kKt, w, lane, blk, nxt, nxt + kKTile,
                               reinterpret_cast<float*>(nxt + kKTile + kVTile));
      if (j + 2 < ntiles) blk = tile_block<PAGED>(p, kbase + 2 * kKt, lane);
    }
    T::template compute<SPLIT>(cur, cur + kKTile, reinterpret_cast<const float*>(cur + kKTile + kVTile),
                               kbase, L, c, lane, kbase + kKt - 1 > off + t0, limit, qf, qq, qs, m,
                               l, o);
  }

  // ---- epilogue: O / l -> bf16 ----
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    float lt = l[b];
    lt = xor16_sum(lt);
    lt = xor32_sum(lt);
    const float inv = 1.0f / lt;
    if (tok_ok) {
      uint8_t* orow = p.out + ((size_t)tok * kHq + head0 + b) * kD * 2;
#pragma unroll
      for (int db = 0; db < 16; ++db) {
        const f32x4 y = o[db][b] * inv;
        const bf16x4 yb = __builtin_convertvector(y, bf16x4);
        *reinterpret_cast<bf16x4*>(orow + (16 * db + 4 * L) * 2) = yb;
      }
    }
  }
}

template <bool PAGED, bool INT8K, int QB>
__global__ __launch_bounds__(kThreads, 1) void gqa_prefill_kernel(const Params p) {
  using S = Shape<QB>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * stage_bytes<PAGED, INT8K, QB>()];
  const int rest = blockIdx.x >> 2;
  const int t0 = (p.n_tblk - 1 - rest / S::kSplitsPerGroup) * S::kTokPerWg;
  if (p.kv_len - p.q_len + t0 + 1 < kSplitBelow)
    run<PAGED, INT8K, QB, true>(p, smem);
  else
    run<PAGED, INT8K, QB, false>(p, smem);
}

// ---- standalone row quantiser: one wave per 256-element row ----
__global__ __launch_bounds__(256) void quantize_rows_kernel(const uint8_t* x, int64_t rows,
                                                            int8_t* xq, float* scale) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint2 raw = *reinterpret_cast<const uint2*>(x + (row * kD + 4 * lane) * 2);
  const bf16x4 v = __builtin_bit_cast(bf16x4, raw);
  float f[4];
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[e] = (float)v[e];
    amax = fmaxf(amax, fabsf(f[e]));
  }
#pragma unroll
  for (int mask = 32; mask >= 1; mask >>= 1) amax = wave_xor_max(amax, mask);
  const float s = amax / 127.0f;
  uint32_t packed = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float r = (s == 0.0f) ? 0.0f : __builtin_rintf(f[e] / s);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    packed |= ((uint32_t)((int)r) & 0xffu) << (8 * e);
  }
  *reinterpret_cast<uint32_t*>(xq + row * kD + 4 * lane) = packed;
  if (lane == 0) scale[row] = s;
}

// ---- host side ----

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_prefill_lengths(int32_t q_len, int32_t kv_len) {
  if (q_len < 0 || kv_len < 0 || q_len > kv_len || kv_len > GQA_MAX_LEN) return GQA_ERR_BAD_LENGTH;
  return GQA_OK;
}

struct Launch {
  const char* name;
  int qb;
  int n_tblk;
  int workgroups;
  int threads;
  int lds_bytes;
};

constexpr int kDefaultQB = GQA_DEFAULT_QB;

template <int QB>
Launch shape_launch(int32_t q_len, bool int8k) {
  using S = Shape<QB>;
  const int n_tblk = (q_len + S::kTokPerWg - 1) / S::kTokPerWg;
  Launch lc;
  lc.qb = QB;
  lc.n_tblk = n_tblk;
  lc.workgroups = n_tblk * kHkv * S::kSplitsPerGroup;
  lc.threads = kThreads;
  lc.lds_bytes = 2 * ((int8k ? kKTileI8 : kKTileBf16) + kVTile + (int8k ? kSkTile : 0));
  return lc;
}

// Dispatch rule (the analogue of the pages' q_len/kv_len-gated variant choice): one
// kernel family; the query-block count per wave is the only shape parameter.
Launch plan_for(int32_t q_len, int32_t kv_len, bool paged, bool int8k) {
  (void)kv_len;
  Launch lc = shape_launch<kDefaultQB>(q_len, int8k);
  if (int8k)
    lc.name = kDefaultQB == 3 ? "int8k_contiguous_t32h6_kt64" : "int8k_contiguous_t64h2_kt64";
  else if (paged)
    lc.name = kDefaultQB == 3 ? "bf16_paged_t32h6_kt64" : "bf16_paged_t64h2_kt64";
  else
    lc.name = kDefaultQB == 3 ? "bf16_contiguous_t32h6_kt64" : "bf16_contiguous_t64h2_kt64";
  return lc;
}

}  // namespace

extern "C" {

int gqa_abi_version(void) { return GQA_ABI_VERSION; }

const char* gqa_status_string(int status) {
  switch (status) {
    case GQA_OK: return "ok";
    case GQA_ERR_NULL_ARG: return "a required pointer is NULL";
    case GQA_ERR_BAD_LENGTH: return "invalid length (need 0 <= q_len <= kv_len <= GQA_MAX_LEN, rows >= 0, enough blocks)";
    case GQA_ERR_MISALIGNED: return "a tensor pointer is misaligned";
    case GQA_ERR_UNSUPPORTED: return "unsupported combination (paged caches with INT8 keys)";
    case GQA_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int gqa_attn_prefill_plan(int32_t q_len, int32_t kv_len, int paged, int int8k, char* buf, size_t n) {
  if (buf == nullptr || n == 0) return GQA_ERR_NULL_ARG;
  int st = check_prefill_lengths(q_len, kv_len);
  if (st == GQA_OK && paged && int8k) st = GQA_ERR_UNSUPPORTED;
  if (st != GQA_OK) {
    snprintf(buf, n, "error: %s", gqa_status_string(st));
    return st;
  }
  const Launch lc = plan_for(q_len, kv_len, paged != 0, int8k != 0);
  snprintf(buf, n, "variant=%s workgroups=%d threads=%d lds_bytes=%d", lc.name, lc.workgroups,
           lc.threads, lc.lds_bytes);
  return GQA_OK;
}

int gqa_attn_prefill(const void* q, const void* k, const void* v, const int32_t* block_table,
                     int32_t num_blocks, const float* k_scale, int32_t q_len, int32_t kv_len,
                     void* out, void* stream) {
  int st = check_prefill_lengths(q_len, kv_len);
  if (st != GQA_OK) return st;
  if (q_len == 0) return GQA_OK;
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return GQA_ERR_NULL_ARG;
  const bool paged = block_table != nullptr;
  const bool int8k = k_scale != nullptr;
  if (paged && int8k) return GQA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return GQA_ERR_MISALIGNED;
  if (paged && !aligned(block_table, 4)) return GQA_ERR_MISALIGNED;
  if (int8k && !aligned(k_scale, 4)) return GQA_ERR_MISALIGNED;
  if (paged) {
    const int64_t need = ((int64_t)kv_len + kBs - 1) / kBs;
    if (num_blocks < need || num_blocks <= 0) return GQA_ERR_BAD_LENGTH;
  }

  Params p;
  p.q = static_cast<const uint8_t*>(q);
  p.k = static_cast<const uint8_t*>(k);
  p.v = static_cast<const uint8_t*>(v);
  p.bt = block_table;
  p.ks = k_scale;
  p.out = static_cast<uint8_t*>(out);
  p.num_blocks = paged ? num_blocks : 0;
  p.q_len = q_len;
  p.kv_len = kv_len;

  const Launch lc = plan_for(q_len, kv_len, paged, int8k);
  p.n_tblk = lc.n_tblk;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(lc.workgroups), block(lc.threads);
  if (int8k)
    hipLaunchKernelGGL((gqa_prefill_kernel<false, true, kDefaultQB>), grid, block, 0, s, p);
  else if (paged)
    hipLaunchKernelGGL((gqa_prefill_kernel<true, false, kDefaultQB>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((gqa_prefill_kernel<false, false, kDefaultQB>), grid, block, 0, s, p);
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

int gqa_quantize_rows_int8(const void* x, int64_t rows, void* xq, float* scale, void* stream) {
  if (rows < 0 || rows > (int64_t)GQA_MAX_LEN * GQA_NUM_Q_HEADS) return GQA_ERR_BAD_LENGTH;
  if (rows == 0) return GQA_OK;
  if (x == nullptr || xq == nullptr || scale == nullptr) return GQA_ERR_NULL_ARG;
  if (!aligned(x, 16) || !aligned(xq, 4) || !aligned(scale, 4)) return GQA_ERR_MISALIGNED;
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  hipLaunchKernelGGL(quantize_rows_kernel, grid, block, 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint8_t*>(x), rows, static_cast<int8_t*>(xq), scale);
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

}  // extern "C"
