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
//     of a 16-token run. QB = 3 (the default): a workgroup is 32 tokens x all 6
//     heads of g (192 rows); QB = 2: 64 tokens x a pair of g's heads (128 rows);
//     QB = 1, for chunks of at most 4 tokens (decode): a wave is one token and
//     column c is head 6 g + c ([INT8 QK §5.1]: 6 live columns of 16);
//   * long histories with few query rows are cut into KV segments whose partial
//     results a second kernel merges by the log-sum-exp rule ([INT8 QK §4]);
//   * scores are computed transposed (S^T = K·Q^T) so every lane holds keys of
//     ONE query column, and the lane's S^T registers are directly the P^T operand
//     of the P·V MFMA;
//   * KV tiles of 64 keys arrive by buffer loads that write LDS directly (no
//     staging registers), double-buffered, issued one or two per MFMA step of the
//     Q·K^T part of an iteration; rows are stored in 128-byte segments with an XOR swizzle so
//     that K fragments are conflict-free ds_read_b128 and the V^T operand of P·V
//     is two conflict-free ds_read_b64_tr_b16 transposing reads;
//   * software pipeline: iteration j turns S(j) into P(j) while the MFMAs of
//     S(j+1) run, then accumulates O += V(j)·P(j); one barrier per tile;
//   * softmax in the exp2 domain against a fixed reference maximum per column
//     (tile 0's maximum), so no accumulator is ever rescaled; if a column's
//     running sum of exponentials passes 2^32 the workgroup restarts with the
//     exact column maxima (the result is the same softmax);
//   * P is rounded to bf16 for the MFMA and the row sums (an MFMA against ones)
//     use the rounded values. Workgroups whose first query sees fewer than 256
//     keys (short histories, where few keys carry large weights) multiply with P
//     split into a bf16 high part and a bf16 low part, keeping ~16 bits of P;
//   * the output accumulator lives in the accumulation registers (AGPRs), scores,
//     P and fragments in the architectural VGPRs;
//   * with INT8 keys each query row is quantised in the prologue (once per row,
//     [INT8 QK §4]) unless the caller hands in its codes, and Q·K^T runs on
//     v_mfma_i32_16x16x64_i8; the int32 score is scaled by sK·sQ·log2(e)/16 per
//     score before the softmax ([INT8 QK §1]), for the next tile during the P·V
//     steps of the current one.
//   * with INT8 values as well ([INT8 QK §6] names INT8 PV and defines nothing more; the
//     reading taken: V codes per (KV head, feature) over the sequence, stored feature-major
//     by the producer, and P codes round(127 * 2^(y - max)) against each column's exact
//     maximum), a first sweep over the history finds those maxima, then one pass forms the
//     P codes in place of bf16 P and runs P·V on v_mfma_i32_16x16x64_i8 into int32
//     accumulators; the V^T tile is laid out so that each lane's 16 keys of a feature are
//     one ds_read_b128.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "gqa_prefill.h"

// Device memory of gqa_attn_prefill_noalloc, for callers that cannot allocate: the
// KV-segment partials (unnormalised O, reference maxima and row sums) that
// gqa_attn_prefill_ws keeps in the caller's workspace. One copy per GPU, held for the
// life of the process. In host code `scratch` names a host-side stand-in, never the
// device memory: the host takes the address of each GPU's copy with
// hipGetSymbolAddress (scratch_on) and passes that pointer to the kernels.
static __device__ __align__(256) uint8_t scratch[GQA_NOALLOC_SCRATCH_BYTES];

#ifndef GQA_DEFAULT_QB
#define GQA_DEFAULT_QB 3
#endif

namespace {

constexpr int kHq = GQA_NUM_Q_HEADS;     // 24
constexpr int kHkv = GQA_NUM_KV_HEADS;   // 4
constexpr int kD = GQA_HEAD_DIM;         // 256
constexpr int kGroup = kHq / kHkv;       // 6
constexpr int kBs = GQA_BLOCK_SIZE;      // 16

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
// Keys per KV tile: 64 (the library). 32 is built only to compare the two (a build with
// -DGQA_KT=32 serves contiguous K/V and refuses paged caches).
#ifndef GQA_KT
#define GQA_KT 64
#endif
constexpr int kKt = GQA_KT;              // keys per KV tile
static_assert(kKt == 64 || kKt == 32, "KV tile of 32 or 64 keys");
constexpr int kHalves = kKt / 32;        // 32-key halves per tile (Q·K^T units)
constexpr int kKb = kKt / 16;            // 16-key blocks per tile (MFMA rows of S^T)
constexpr int kWaveKeys = kKt / 4;       // keys of a tile each of the 4 waves copies
constexpr int kPvSteps = 16 * kHalves;   // P·V steps per tile (32 keys x 16 features each)
constexpr int kSplitBelow = 256;
// Pass 0 restarts once a column's running sum of exponentials exceeds 2^32: every
// exponential is then still at most 2^32 (finite in bf16 and fp32 with ample margin
// for the fp32 accumulation of up to 2^24 keys), and a sum that overflowed is inf,
// which compares greater too.
constexpr float kOverSum = 4294967296.0f;
constexpr float kLog2eOver16 = 1.4426950408889634f / 16.0f;
// INT8 values: P codes are 127 * 2^(y - max), the exponent shifted by log2(127)
constexpr float kLog2Of127 = 6.988684686772166f;

// key scales of a tile: a 256-byte area per wave, [KV head][16 key slots] (a 32-key tile
// uses 8 of the 16 slots of each wave)
constexpr int kSkTile = 4 * kHkv * 16 * 4;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

struct Params {
  const uint8_t* q;        // bf16 [q_len, 24, 256], or int8 codes of Q when qsc is set
  const float* qsc;        // INT8 keys, Q quantised beforehand: sQ [q_len, 24]; else null
  const uint8_t* k;        // bf16 or int8, contiguous or paged
  const uint8_t* v;        // bf16, contiguous or paged; INT8 values: codes [4, 256, v_ld]
  const int32_t* bt;       // block table or null
  const float* ks;         // key scales [kv_len, 4] or null
  uint8_t* out;            // bf16 [q_len, 24, 256]
  int32_t num_blocks;
  int32_t q_len;
  int32_t kv_len;
  int32_t n_tblk;          // token blocks of the grid
  int32_t n_seg;           // KV segments per split (KV head, token block); 1 = none split
  int32_t n_plain;         // n_seg > 1: the shortest token blocks 0 .. n_plain - 1 run whole
  float* ws_o;             // n_seg > 1: unnormalised O [n_seg, split rows, 24, 256]
  float* ws_ml;            // n_seg > 1: (reference maximum, row sum) [n_seg, split rows, 24, 2]
  const float* vs;         // INT8 values: sV [4, 256]; else null
  int32_t v_ld;            // INT8 values: tokens per stored feature row of V
};

// Workgroup shape for QB 16-column query blocks per wave. QB = 3 and QB = 2 map a
// column to a token (16-token runs) and a block to a query head. QB = 1 is the decode
// shape: one token per wave, and column c of its single block is query head 6 g + c of
// the GQA group (6 of the 16 columns are live). The pages make the same choice for
// decode, where one new token cannot fill the 16 output rows of the matrix instruction
// and the rows come from the group's query heads ("gfx936 DCU上实现INT8 QK MMAC" §5.1).
template <int QB>
struct Shape {
  static constexpr bool kDecode = QB == 1;
  static constexpr int kTokenBlocks = (QB == 3) ? 2 : 4;            // 16-token runs per workgroup
  static constexpr int kHeadGroups = kDecode ? 1 : kWaves / kTokenBlocks;   // QB-head groups
  static constexpr int kHeadsPerWg = kDecode ? kGroup : QB * kHeadGroups;   // 6, 6 or 2
  static constexpr int kTokPerWg = kDecode ? kWaves : 16 * kTokenBlocks;    // 4, 32 or 64
  static constexpr int kSplitsPerGroup = kGroup / kHeadsPerWg;      // 1 or 3 workgroups per (g, tokens)
};

// What one workgroup computes. The grid is 4 x (work units): id % 4 is the KV head, and
// the units run in this order: first the token blocks n_plain - 1 .. 0 whole (longest
// first), then the longer token blocks n_tblk - 1 .. n_plain, each cut into n_seg KV
// segments (segment fastest). Only the split token blocks' rows (tokens from
// n_plain * tokens-per-workgroup on) pass through the workspace and the merge.
struct Unit {
  int g, seg, nseg, hsel, tblk;
};
template <int QB>
__device__ __forceinline__ Unit unit_of(const Params& p, int id) {
  using S = Shape<QB>;
  Unit u;
  u.g = id & (kHkv - 1);
  const int k = id >> 2;
  const int plain = p.n_plain * S::kSplitsPerGroup;
  int rest;
  if (k < plain) {
    u.seg = 0;
    u.nseg = 1;
    rest = k;
    u.tblk = p.n_plain - 1 - rest / S::kSplitsPerGroup;
  } else {
    u.seg = (k - plain) % p.n_seg;
    u.nseg = p.n_seg;
    rest = (k - plain) / p.n_seg;
    u.tblk = p.n_tblk - 1 - rest / S::kSplitsPerGroup;
  }
  u.hsel = rest % S::kSplitsPerGroup;
  return u;
}

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

// Element index of the row (key, kv head g) in the K/V arrays.
template <bool PAGED>
__device__ __forceinline__ size_t kv_row(int g, int key, int blk) {
  if constexpr (PAGED) {
    return ((size_t)(blk * kHkv + g) * kBs + (key & (kBs - 1))) * kD;
  } else {
    return ((size_t)key * kHkv + g) * kD;
  }
}

// ---- LDS tile layout ----
// A tile holds 64 keys. Each key row (512 B of bf16 K or V, 256 B of int8 K) is cut
// into 128-byte segments and segment `sg` of all 64 keys is stored contiguously:
//   byte(key, piece) = (piece >> 3) * kSegStride + key * 128 + (((piece & 7) ^ swz(key)) << 4)
// with `piece` the 16-byte piece index inside the row and a per-tensor XOR swizzle
//   K: swz = key & 7         (the 8 lanes of a ds_read_b128 phase read 8 keys at one
//                             piece and hit 8 different 16-byte bank groups)
//   V: swz = ((key >> 1) & 3) << 1
//                            (a transposing read serves 32 lanes per LDS cycle: 8 keys
//                             x 32 bytes; keys of equal parity share the 128-byte half
//                             of the 256-byte bank row and this swizzle spreads the
//                             four of each parity over its four 32-byte bank groups)
// A global->LDS copy instruction moves 8 keys x one 128-byte segment: every lane
// group of 8 reads one whole 128-byte line of a key row.
//
// Paged INT8 K (the split-d cache below) keeps the cache's own page order instead:
// the 16 keys of a 16-key block kb form one 4 KiB page, chunk (16 features) ch of key
// k at kb * 4096 + ch * 256 + (k & 15) * 16. A copy instruction is then 1 KiB of a
// page, contiguous on both sides, and a fragment read (16 keys x one chunk per lane
// group) is 1 KiB of consecutive LDS, conflict-free without a swizzle.
constexpr int kSegStride = kKt * 128;   // 8 KiB
constexpr int kPageBytes = kBs * kD;    // 4 KiB: 16 keys x 256 int8 features

template <bool V>
__device__ __forceinline__ int tile_swizzle(int key) {
  return V ? (((key >> 1) & 3) << 1) : (key & 7);
}

// ---- global -> LDS tile copies ----
// Each wave copies its 16 keys (keys 16w .. 16w + 15 of a tile) of a tensor with
// buffer loads that write LDS directly. The wave's keys lie in one 16-key block, so a
// wave-uniform buffer descriptor starts at its first row (or its physical block) and
// every lane offset is a constant of the kernel. The descriptor's size ends right
// after the last row before kv_len: rows past it are out of range, and such buffer
// loads write zeros into LDS (finite rows that the causal mask hides). A tile past the
// end therefore costs no memory traffic at all.
typedef __attribute__((address_space(3))) void lds_void;

// f(std::integral_constant<int, I>) for I = LO .. HI - 1
template <int LO, int HI, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (LO < HI) {
    f(std::integral_constant<int, LO>{});
    static_for<LO + 1, HI>(f);
  }
}

__device__ __forceinline__ lds_void* lds_ptr(uint32_t addr) {
  return (lds_void*)(uintptr_t)addr;
}

// SPLITD: the paged INT8 K cache of "gfx936 DCU上实现INT8 QK MMAC" §3, laid out
// [block, kv_head, 256 / 16, 16 slots, 16]: a (block, head) page is 16 chunks of 16
// features, each holding that chunk for all 16 slots (chunk c of slot k at c * 256 +
// k * 16). The wave copies its page as it is, 1 KiB per instruction, into the
// page-major tile above. The slots of a page are interleaved, so the descriptor covers
// the whole 4 KiB page; slots past kv_len hold whatever the cache holds (finite int8
// codes) and their scales, which are zeroed (ScaleCopy), make their scores 0 before the
// causal mask hides them.
template <bool PAGED, int ROW_BYTES, bool V, bool SPLITD = false>
struct WaveCopy {
  static_assert(!SPLITD || (PAGED && ROW_BYTES == kD), "the split-d layout is the paged INT8 K cache");
  static constexpr int kNseg = ROW_BYTES / 128;                      // 128-byte segments per row
  static constexpr int kInsts = (kWaveKeys / 8) * kNseg;            // 8 keys x one segment each
  static constexpr int kStride = PAGED ? ROW_BYTES : kHkv * ROW_BYTES;   // bytes between keys

  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t lds;   // LDS address of the wave's first row, segment 0, in the destination tile

  // Source offset of lane (kr = lane / 8, physical piece pp = lane % 8) for key half `half`:
  // the lane fetches the logical piece that the tile swizzle stores at position pp
  // (SPLITD: byte 16 lane of each KiB of the page).
  static __device__ __forceinline__ uint32_t lane_offset(int lane, int half) {
    if constexpr (SPLITD) {
      (void)half;
      return (uint32_t)(lane * 16);
    } else {
      const int kr = lane >> 3, pp = lane & 7;
      const int piece = pp ^ tile_swizzle<V>(kr);
      return (uint32_t)((8 * half + kr) * kStride + (piece << 4));
    }
  }

  // first = kbase + 16 w (wave-uniform); blk = the physical block holding it (paged);
  // lds_rows = the wave's first row (segment 0) in the destination tile, or (SPLITD) its
  // page
  __device__ __forceinline__ WaveCopy(const Params& p, const uint8_t* base, int g, int first,
                                      int blk, uint32_t lds_rows) {
    const int n = min(max(p.kv_len - first, 0), 16);   // rows of this wave before kv_len
    int bytes;
    if constexpr (SPLITD)
      bytes = n > 0 ? kBs * ROW_BYTES : 0;
    else
      bytes = n > 0 ? (n - 1) * kStride + ROW_BYTES : 0;
    // (uniform; readfirstlane keeps the whole descriptor in scalar registers)
    const int nrec = __builtin_amdgcn_readfirstlane(bytes);
    const uint8_t* wb;
    if constexpr (PAGED) {
      wb = base + (size_t)(blk * kHkv + g) * kBs * ROW_BYTES + (SPLITD ? 0 : (first & (kBs - 1)) * ROW_BYTES);
    } else {
      (void)blk;
      wb = base + ((size_t)first * kHkv + g) * ROW_BYTES;   // not dereferenced when n == 0
    }
    rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(wb), (short)0, nrec, 0x00020000);
    lds = lds_rows;
  }

  // Instruction I: key half I / kNseg, segment I % kNseg; SPLITD: KiB I of the page.
  template <int I>
  __device__ __forceinline__ void issue(const uint32_t (&voff)[2]) const {
    if constexpr (SPLITD) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, lds_ptr(lds + I * 1024), 16, voff[0], I * 1024,
                                               0, 0);
    } else {
      constexpr int half = I / kNseg, sg = I % kNseg;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, lds_ptr(lds + half * 1024 + sg * kSegStride), 16,
                                               voff[half], sg * 128, 0, 0);
    }
  }
};

// INT8 key scales: each wave copies the scales of its 16 keys for all 4 KV heads into
// a 1 KiB slot laid out [16-key block][KV head][16 keys] (lane = 16 head + key).
// Contiguous scales are [kv_len, 4]; paged ones [block, 4, 16], the 256 bytes of a
// block in lane order. Scales of keys past kv_len arrive as 0: out of the descriptor's
// range (contiguous), or through an out-of-range lane offset (paged, where a block's
// slots are interleaved by head).
template <bool PAGED>
struct ScaleCopy {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t lds;
  int n;   // keys of this wave before kv_len
  __device__ __forceinline__ ScaleCopy() = default;
  static __device__ __forceinline__ uint32_t lane_offset(int lane) {
    if constexpr (PAGED)
      return (uint32_t)(lane * 4);
    else
      return (uint32_t)((lane & 15) * kHkv * 4 + (lane >> 4) * 4);
  }
  __device__ __forceinline__ ScaleCopy(const Params& p, int first, int blk, uint32_t lds_block) {
    n = __builtin_amdgcn_readfirstlane(min(max(p.kv_len - first, 0), kWaveKeys));
    const uint8_t* wb;
    int bytes;
    if constexpr (PAGED) {
      wb = reinterpret_cast<const uint8_t*>(p.ks) + (size_t)blk * kHkv * kBs * 4;
      bytes = n > 0 ? kHkv * kBs * 4 : 0;
    } else {
      (void)blk;
      wb = reinterpret_cast<const uint8_t*>(p.ks) + (size_t)first * kHkv * 4;
      bytes = n * kHkv * 4;
    }
    rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(wb), (short)0,
                                             __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
    lds = lds_block;
  }
  // voff = lane_offset(lane); key = lane % 16
  __device__ __forceinline__ void issue(uint32_t voff, int key) const {
    if constexpr (PAGED) voff = key < n ? voff : 0x40000000u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, lds_ptr(lds), 4, voff, 0, 0, 0);
  }
};

// INT8 values: the producer stores the codes feature-major, [4, 256, ld] with the token
// index fastest, so a tile (64 keys of all 256 features of KV head g) is one 64-byte run
// per feature. In LDS each feature f is a 64-byte row; its 16-byte slot s holds, as dwords
// kb = 0..3, the keys 16 kb + 4 L .. 16 kb + 4 L + 3 with L = s ^ ((f >> 1) & 3). Lane
// (L, c) of the P·V step needs for feature c of a 16-feature block exactly the 16 keys whose
// scores its S^T registers hold (keys 16 kb + 4 L + r, r = 0..3), in that order: one
// ds_read_b128 of slot L ^ ((c >> 1) & 3). A 16-byte read is served 8 lanes at a time
// from a 128-byte bank row (the K reads' pattern is conflict-free by that rule, and a swizzle
// on f >> 2 measured 2-way conflicts); rows c = 0..7 of a lane group fall at 64 (c & 1)
// modulo 128, and the XOR on c >> 1 gives the four rows of each parity four different
// slots. A copy instruction fills 4 feature rows (256 B, lane l writing dword l), one dword
// (4 keys) per lane; wave w copies features 64 w .. 64 w + 63 in 16 instructions. Feature
// 64 w + 4 I + (l >> 4) of instruction I has swizzle (2 I + (l >> 5)) & 3, so a lane needs
// 2 source offsets, for even and odd I. The descriptor covers the wave's 64 rows up to the
// tile's last key, cut at the end of the array; a tile at or past kv_len has no range at all.
struct VtCopy {
  static constexpr int kInsts = 16;
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t lds;   // LDS address of the wave's first feature row in the destination tile
  uint32_t ld;    // bytes between feature rows

  // source offset of lane l for the instructions I with I % 2 == P
  static __device__ __forceinline__ uint32_t lane_offset(int lane, int P, int ld) {
    const int d = lane & 15;   // destination dword in the feature row: slot d >> 2, key block d & 3
    const int swz = (2 * P + (lane >> 5)) & 3;
    return (uint32_t)((lane >> 4) * ld + 16 * (d & 3) + 4 * ((d >> 2) ^ swz));
  }
  __device__ __forceinline__ VtCopy(const Params& p, int g, int kbase, int w, uint32_t lds_tile) {
    const int n = min(max(p.kv_len - kbase, 0), kKt);
    const int64_t row0 = (int64_t)g * kD + 64 * w;
    const int64_t first = row0 * p.v_ld + kbase;
    const int64_t left = (int64_t)kHkv * kD * p.v_ld - first;   // bytes from the first to the end
    const int64_t span = (int64_t)63 * p.v_ld + kKt;
    const int bytes = n > 0 ? (int)min(span, left) : 0;
    rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.v + first), (short)0,
                                             __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
    lds = lds_tile + 64 * w * kKt;
    ld = (uint32_t)p.v_ld;
  }
  // the whole offset goes into the lane's offset, which the range check covers
  template <int I>
  __device__ __forceinline__ void issue(const uint32_t (&vto)[2]) const {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, lds_ptr(lds + I * 256), 4, vto[I & 1] + (4 * I) * ld,
                                             0, 0, 0);
  }
};

// ---- phase clock: a measurement build only (-DGQA_PHASE_CLOCK=1 or 2; the library has none of it) ----
// Each wave adds up the shader cycles (s_memtime) of the phases of its tile loop and reads
// the 100 MHz real-time counter (s_memrealtime) around the loop, so that cycles over real
// time give the shader clock under load. Slots per wave: Q·K^T + softmax, P·V, copy wait
// and barrier (unmasked tiles), unmasked tiles, masked-tile cycles, masked tiles, the
// INT8-value maximum sweep's cycles and tiles, loop cycles, loop real-time ticks.
#ifdef GQA_PHASE_CLOCK
constexpr int kPhaseWaves = 8192 * 4;
constexpr int kPhaseSlots = 10;
__device__ unsigned long long phase_clock[kPhaseWaves * kPhaseSlots];
struct PhaseClock {
  unsigned long long qk = 0, pv = 0, sync = 0, n = 0, masked = 0, n_masked = 0, sweep = 0, n_sweep = 0,
                     c0 = 0, r0 = 0;
  // GQA_PHASE_CLOCK=2 also pins every read in the instruction order (a scheduling barrier on
  // each side), so the phases are exact for that order, which then differs from the library's
  static __device__ __forceinline__ unsigned long long cycles() {
#if GQA_PHASE_CLOCK >= 2
    __builtin_amdgcn_sched_barrier(0);
    const unsigned long long t = __builtin_readcyclecounter();
    __builtin_amdgcn_sched_barrier(0);
    return t;
#else
    return __builtin_readcyclecounter();
#endif
  }
  static __device__ __forceinline__ unsigned long long ticks() { return __builtin_amdgcn_s_memrealtime(); }
};
#define GQA_PC(...) __VA_ARGS__
#else
#define GQA_PC(...)
#endif

__device__ __forceinline__ void wait_vm_all() {
  // s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima)
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// s_waitcnt vmcnt(N): a wave's vector memory operations complete in order, so at most N
// outstanding means all but its N most recent are done
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// ---- explicit LDS reads ----
// K fragments are read with inline assembly too, so the prefetch distance is the one
// written here (the compiler, short of VGPRs, would otherwise serialise each read with
// its first use). LDS operations of a wave complete in order, so waiting until at most
// N are outstanding makes every older read's registers valid; the waits tie the
// registers they guard so no consumer is scheduled above them.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

template <int OFF>
__device__ __forceinline__ u32x4 lds_read_b128(uint32_t addr) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}

template <int N>
__device__ __forceinline__ void lds_wait4(u32x4& a, u32x4& b, u32x4& c, u32x4& d) {
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d) : "i"(N));
}

// ---- S^T = K · Q^T for one 64-key tile ----
// Lane (L, c) reads K fragment (kb, s) = key 16 kb + c, piece 4 s + L:
//   (s >> 1) * kSegStride + kb * 2048 + c * 128 + (((4 (s & 1) + L) ^ (c & 7)) << 4)
// i.e. one of two per-lane bases (s even / odd) plus an immediate offset.
template <bool INT8K, int QB, bool PM = false>
struct QK {
  static_assert(!PM || INT8K, "the page-major K tile holds INT8 keys");
  using Acc = typename std::conditional<INT8K, i32x4, f32x4>::type;
  using Frag = typename std::conditional<INT8K, i32x4, bf16x8>::type;
  static constexpr int kSteps = INT8K ? 4 : 8;
  // K steps whose fragments are read ahead of the step being multiplied. bf16 keys: 2
  // (against 1, same-box A/B with outputs bitwise equal: 0.7% faster on 4096 x 32768, 1.0%
  // on 3072 x 16384 and on the paged 512 x 32768 tail; 8 more VGPRs, no spills). INT8 keys
  // keep 1: 2 took 1.3% more loop cycles a tile and 0.4% more time on 3072 x 16384.
  static constexpr int kDepth = INT8K ? 1 : 2;

  // Fragments kb = KB0, KB0 + 1 of K step s; `base` = the lane's even- or odd-step base.
  // PM (page-major tile): lane (L, c) reads chunk 4 s + L of key 16 kb + c at
  // kb * 4096 + s * 1024 + L * 256 + c * 16, one base for every step.
  template <int S, int KB0>
  static __device__ __forceinline__ void issue(u32x4 (&f)[2], uint32_t base_even, uint32_t base_odd) {
    if constexpr (PM) {
      f[0] = lds_read_b128<S * 1024 + (KB0 + 0) * kPageBytes>(base_even);
      f[1] = lds_read_b128<S * 1024 + (KB0 + 1) * kPageBytes>(base_even);
    } else {
      const uint32_t base = (S & 1) ? base_odd : base_even;
      f[0] = lds_read_b128<(S >> 1) * kSegStride + (KB0 + 0) * 2048>(base);
      f[1] = lds_read_b128<(S >> 1) * kSegStride + (KB0 + 1) * 2048>(base);
    }
  }

  static __device__ __forceinline__ Acc mfma(const u32x4& k, const Frag& q, const Acc& c) {
    if constexpr (INT8K)
      return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, k), q, c, 0, 0, 0);
    else
      return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k), q, c, 0, 0, 0);
  }
};

template <int N>
__device__ __forceinline__ void lds_wait2(u32x4& a, u32x4& b) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "i"(N));
}

// One K step S over key blocks KB0, KB0 + 1 (32 keys): issue the reads of step S + D
// (D = QK::kDepth steps ahead), wait for step S's 2 fragments (the reads of the up to D
// steps after it may stay in flight), run its 2 x QB MFMAs, then `extra(S)`. The
// fragments of step s live in kf[s % (D + 1)].
template <bool INT8K, int QB, bool PM, int KB0, int S, class KF, class Extra>
__device__ __forceinline__ void qk_half(KF& kf, uint32_t be, uint32_t bo,
                                        const typename QK<INT8K, QB>::Frag (&qf)[QB][QK<INT8K, QB>::kSteps],
                                        typename QK<INT8K, QB>::Acc (&acc)[QB][kKb], Extra&& extra) {
  using Q = QK<INT8K, QB, PM>;
  constexpr int D = Q::kDepth;
  static_assert(std::is_same<KF, u32x4[D + 1][2]>::value, "a ring of D + 1 fragment pairs");
  if constexpr (S + D < Q::kSteps) Q::template issue<S + D, KB0>(kf[(S + D) % (D + 1)], be, bo);
  constexpr int kAhead = (Q::kSteps - 1 - S) < D ? (Q::kSteps - 1 - S) : D;   // steps in flight after S
  lds_wait2<2 * kAhead>(kf[S % (D + 1)][0], kf[S % (D + 1)][1]);
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int b = 0; b < QB; ++b)
      acc[b][KB0 + kk] = Q::mfma(kf[S % (D + 1)][kk], qf[b][S], acc[b][KB0 + kk]);
  extra(std::integral_constant<int, S>{});
  if constexpr (S + 1 < Q::kSteps) qk_half<INT8K, QB, PM, KB0, S + 1>(kf, be, bo, qf, acc, extra);
}

// All K steps over key blocks KB0, KB0 + 1 of the tile at LDS address `kbuf`.
template <bool INT8K, int QB, bool PM, int KB0, class Extra>
__device__ __forceinline__ void qk_pair(uint32_t kbuf, int kb_even, int kb_odd,
                                        const typename QK<INT8K, QB>::Frag (&qf)[QB][QK<INT8K, QB>::kSteps],
                                        typename QK<INT8K, QB>::Acc (&acc)[QB][kKb], Extra&& extra) {
  using Q = QK<INT8K, QB, PM>;
  u32x4 kf[Q::kDepth + 1][2];
  static_for<0, (Q::kDepth < Q::kSteps ? Q::kDepth : Q::kSteps)>([&](auto ic) {
    constexpr int I = decltype(ic)::value;
    Q::template issue<I, KB0>(kf[I], kbuf + kb_even, kbuf + kb_odd);
  });
  qk_half<INT8K, QB, PM, KB0, 0>(kf, kbuf + kb_even, kbuf + kb_odd, qf, acc, extra);
}

// ---- O^T += V^T · P^T (and l += 1 · P^T) ----
// Transposing read: lane i of 16-lane group L fetches features 16 db + 4 (i & 3) .. +3 of
// key 32 ks + 16 h + 4 L + (i >> 2); after the transpose lane (L, c) holds
// V[32 ks + 16 h + 4 L + k][16 db + c], k = 0..3, exactly its P^T operand's keys.
struct VtFrag {
  uint2 lo, hi;
};

// Issued as inline assembly so the compiler does not make these reads wait for the
// global->LDS copies into other buffers; vt_wait must run before the registers are used.
template <int OFF>
__device__ __forceinline__ void vt_issue(VtFrag& f, uint32_t addr) {
  asm volatile("ds_read_b64_tr_b16 %0, %2 offset:%3\n\tds_read_b64_tr_b16 %1, %2 offset:%4"
               : "=v"(f.lo), "=v"(f.hi)
               : "v"(addr), "i"(OFF), "i"(OFF + 16 * 128));
}

// Wait until at most N LDS operations of this wave are outstanding (LDS operations
// complete in order), tying the fragment's registers to the wait.
template <int N>
__device__ __forceinline__ void vt_wait(VtFrag& f) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(f.lo), "+v"(f.hi) : "i"(N));
}

__device__ __forceinline__ bf16x8 vt_value(const VtFrag& f) {
  return __builtin_bit_cast(bf16x8, make_uint4(f.lo.x, f.lo.y, f.hi.x, f.hi.y));
}

// Step N = 16 ks + db: ks = 32-key half of the tile, db = 16-feature block.
// V^T fragment (ks, db) sits at vbase[db & 3] + (db >> 2) * kSegStride + ks * 4096.
// Fragments travel in a ring of kVtDepth + 1: step N issues the reads of step
// N + kVtDepth, then waits for its own (2 reads per step).
// Depth 3 measured fastest on every cell of the pages' grid of chunk shapes against 2 and
// 4 (the other depths are built only to compare them).
#ifndef GQA_VT_DEPTH
#define GQA_VT_DEPTH 3
#endif
constexpr int kVtDepth = GQA_VT_DEPTH;
// at most 2 (kVtDepth + 1) reads in flight, plus the 4 key-scale reads of INT8 keys, and
// lgkmcnt counts to 15
static_assert(kVtDepth >= 1 && 2 * (kVtDepth + 1) + 4 <= 15, "V^T read ring depth");

template <int N>
__device__ __forceinline__ void vt_issue_step(VtFrag& f, const uint32_t (&vbase)[4]) {
  constexpr int ks = N >> 4, db = N & 15;
  vt_issue<(db >> 2) * kSegStride + ks * 4096>(f, vbase[db & 3]);
}

// O^T += V^T · P^T with the accumulator pinned to the accumulation registers (AGPRs).
// Written as inline assembly so that the compiler keeps all output blocks there and
// leaves the architectural VGPRs to scores, P and fragments. The compiler does not see
// into the assembly, so the hazards it would otherwise cover are covered here:
//  * an MFMA may read a VGPR only 2 wait states after a vector ALU instruction wrote
//    it: FIRST marks a tile's first MFMA on each P register (P is written by the
//    vector ALU), and the assembly then starts with s_nop 1. That statement also lists P
//    as an operand it rewrites (it does not), so that every other reader of P depends on
//    it and the compiler cannot move one ahead of it; without this it reorders the
//    independent statements of a tile's second key half and puts another before the
//    first, one wait state after the conversion that wrote P;
//  * V^T fragments come from LDS reads whose wait precedes the call;
//  * consecutive MFMAs on the same accumulator need no wait states;
//  * vector ALU accesses to the accumulators (zeroing, the epilogue) are separated
//    from the MFMAs by agpr_fence below.
template <bool FIRST>
__device__ __forceinline__ void mfma_pv(f32x4& acc, const bf16x8& v, bf16x8& p) {
  if constexpr (FIRST)
    asm("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %2, %1, %0 ; carry %1" : "+a"(acc), "+v"(p) : "v"(v));
  else
    asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(v), "v"(p));
}

// Orders every access to the output accumulators: each block is tied to a volatile
// assembly statement (these keep their program order), and the first statement carries
// NOPS wait states. Before the accumulators are zeroed or read by the vector ALU after
// MFMAs, 24 wait states cover the longest MFMA-write to vector-access distance of the
// 16x16x32 MFMAs; after zeroing, 2 cover the vector-write to MFMA-read distance.
template <int NOPS, int QB, class T>
__device__ __forceinline__ void agpr_fence(T (&o)[16][QB]) {
  static_assert(NOPS == 2 || NOPS == 24, "wait states");
  if constexpr (NOPS == 2)
    asm volatile("s_nop 1" : "+a"(o[0][0]));
  else
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(o[0][0]));
#pragma unroll
  for (int db = 0; db < 16; ++db)
#pragma unroll
    for (int b = 0; b < QB; ++b)
      if (db != 0 || b != 0) asm volatile("" : "+a"(o[db][b]));
}

// mfma_pv carrying one to three 32-bit registers through the statement as operands the
// instruction does not touch (named in an assembly comment, for the ISA check of the
// package). Vector work that reads a carried register after the
// statement, or whose result a later statement carries, stays between the two statements:
// the compiler orders them by these operands, and tracks the hazards of that vector work
// itself, since it is not inside the assembly.
template <bool FIRST>
__device__ __forceinline__ void mfma_pv_carry(f32x4& acc, const bf16x8& v, bf16x8& p, uint32_t& a) {
  if constexpr (FIRST)
    asm("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %[o], %[v], %[p], %[o] ; carry %[p] %[ca]"
        : [o] "+a"(acc), [p] "+v"(p), [ca] "+v"(a) : [v] "v"(v));
  else
    asm("v_mfma_f32_16x16x32_bf16 %[o], %[v], %[p], %[o] ; carry %[ca]" : [o] "+a"(acc), [ca] "+v"(a) : [v] "v"(v), [p] "v"(p));
}
template <bool FIRST>
__device__ __forceinline__ void mfma_pv_carry(f32x4& acc, const bf16x8& v, bf16x8& p, uint32_t& a,
                                              uint32_t& b) {
  if constexpr (FIRST)
    asm("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %[o], %[v], %[p], %[o] ; carry %[p] %[ca] %[cb]"
        : [o] "+a"(acc), [p] "+v"(p), [ca] "+v"(a), [cb] "+v"(b) : [v] "v"(v));
  else
    asm("v_mfma_f32_16x16x32_bf16 %[o], %[v], %[p], %[o] ; carry %[ca] %[cb]"
        : [o] "+a"(acc), [ca] "+v"(a), [cb] "+v"(b) : [v] "v"(v), [p] "v"(p));
}
template <bool FIRST>
__device__ __forceinline__ void mfma_pv_carry(f32x4& acc, const bf16x8& v, bf16x8& p, uint32_t& a,
                                              uint32_t& b, uint32_t& c) {
  if constexpr (FIRST)
    asm("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %[o], %[v], %[p], %[o] ; carry %[p] %[ca] %[cb] %[cc]"
        : [o] "+a"(acc), [p] "+v"(p), [ca] "+v"(a), [cb] "+v"(b), [cc] "+v"(c) : [v] "v"(v));
  else
    asm("v_mfma_f32_16x16x32_bf16 %[o], %[v], %[p], %[o] ; carry %[ca] %[cb] %[cc]"
        : [o] "+a"(acc), [ca] "+v"(a), [cb] "+v"(b), [cc] "+v"(c) : [v] "v"(v), [p] "v"(p));
}

// Registers one P·V MFMA statement carries for the scaling of the next tile's scores
// placed between the statements (at most 3): a score's key scale (SK), float(S) (C), the
// product of the scales (T), the finished exponent (Y) or, with bf16 keys, the maximum of
// the score's column (M).
struct CarryPlan {
  enum { kSK, kC, kT, kY, kM };
  int n = 0;
  int kind[3] = {0, 0, 0};
  int score[3] = {0, 0, 0};
};

// Placement of the INT8-key scaling among a tile's P·V MFMA statements 0 .. STMTS - 1:
// the 3 instructions of score i (op 3i: float(S); 3i + 1: sK * sQ'; 3i + 2: the FMA) go
// to gaps FIRST .. STMTS - 2 in order, evenly (gap g follows statement g). An instruction
// is held after statement g by carrying its operand through g (the key scale, or a result
// of an earlier gap), and before statement g + 1 by carrying its result through g + 1.
// The int32 score is never carried: the Q·K^T MFMA that writes it may still be in flight
// (the compiler moves the last ones into the P·V steps), and a statement that lists it as
// an output would hide that write from the compiler, which would then let the conversion
// read the register without the MFMA's wait states. The conversion is held only by its
// result.
template <int STMTS, int FIRST, int SCORES>
struct ScaleSchedule {
  static constexpr int kScores = SCORES;
  static constexpr int kOps = 3 * SCORES;
  static constexpr int kGaps = STMTS - 1 - FIRST;
  static_assert(kGaps >= kScores, "room for the scaling");
  static constexpr int gap(int j) { return FIRST + (j * kGaps) / kOps; }
  // first op in gap g (ops are in gap order)
  static constexpr int first_op(int g) {
    int j = 0;
    while (j < kOps && gap(j) < g) ++j;
    return j;
  }
  static constexpr CarryPlan carries(int k) {
    CarryPlan cp;
    auto add = [&cp](int kind, int i) {
      cp.kind[cp.n] = kind;
      cp.score[cp.n] = i;
      ++cp.n;
    };
    for (int i = 0; i < kScores; ++i) {
      const int gc = gap(3 * i), gm = gap(3 * i + 1), gf = gap(3 * i + 2);
      if (gm == k) add(CarryPlan::kSK, i);
      if (gf > gc && (gc + 1 == k || (gf > gc + 1 && gf == k))) add(CarryPlan::kC, i);
      if (gf > gm && (gm + 1 == k || (gf > gm + 1 && gf == k))) add(CarryPlan::kT, i);
      if (gf + 1 == k) add(CarryPlan::kY, i);
    }
    return cp;
  }
};

// Placement of the bf16-key exponent FMAs of the next tile's first key half (one a
// score) among the last TAIL gaps of a tile's STMTS P·V MFMA statements (gap g follows
// statement g), at most two a gap: after the last V reads those MFMAs run back to back
// and leave the vector ALU idle. Score i's FMA is held after statement g by carrying its
// column's maximum through g (the score itself, written by a Q·K^T MFMA, is never
// carried) and before statement g + 1 by carrying its result through g + 1.
template <int STMTS, int TAIL, int SCORES>
struct ExpSchedule {
  static constexpr int kScores = SCORES;
  static constexpr int kFirst = STMTS - 1 - TAIL;
  static_assert(kFirst >= 0 && 2 * TAIL >= kScores, "room for the FMAs, two a gap");
  static constexpr int gap(int i) { return kFirst + (i * TAIL) / kScores; }
  static constexpr int first_op(int g) {
    int i = 0;
    while (i < kScores && gap(i) < g) ++i;
    return i;
  }
  static constexpr CarryPlan carries(int k) {
    CarryPlan cp;
    auto add = [&cp](int kind, int i) {
      cp.kind[cp.n] = kind;
      cp.score[cp.n] = i;
      ++cp.n;
    };
    int last_u = -1;   // one maximum per 4-score unit (the unit's scores share a column)
    for (int i = 0; i < kScores; ++i) {
      if (gap(i) == k && i / 4 != last_u) {
        add(CarryPlan::kM, i);
        last_u = i / 4;
      }
      if (gap(i) + 1 == k) add(CarryPlan::kY, i);
    }
    return cp;
  }
};

// Step N of P·V: the MFMA statements go through `mf`, called with the statement's index
// in the tile (N * QB (* 2 with the low part) + its place in the step), whether it is the
// first on its P register, and the operands.
template <int N, int QB, bool SPLIT>
struct PvStep {
  template <class Extra, class Mf>
  static __device__ __forceinline__ void run(VtFrag (&vf)[kVtDepth + 1], const uint32_t (&vbase)[4],
                                             bf16x8 (&ph)[QB][2], bf16x8 (&pl)[QB][2],
                                             const bf16x8& ones, f32x4 (&o)[16][QB],
                                             f32x4 (&lacc)[QB], Extra&& extra, Mf&& mf) {
    constexpr int ks = N >> 4, db = N & 15;
    constexpr int kMf = SPLIT ? 2 : 1;
    extra(std::integral_constant<int, N>{});
    constexpr int kAhead = (kPvSteps - 1 - N) < kVtDepth ? (kPvSteps - 1 - N) : kVtDepth;  // steps in flight after N
    if constexpr (N + kVtDepth < kPvSteps) vt_issue_step<N + kVtDepth>(vf[(N + kVtDepth) % (kVtDepth + 1)], vbase);
    vt_wait<2 * kAhead>(vf[N % (kVtDepth + 1)]);
    const bf16x8 v = vt_value(vf[N % (kVtDepth + 1)]);
    static_for<0, QB>([&](auto bc) {
      constexpr int b = decltype(bc)::value;
      mf(std::integral_constant<int, (N * QB + b) * kMf>{}, std::bool_constant<db == 0>{}, o[db][b], v,
         ph[b][ks]);
      if constexpr (SPLIT)
        mf(std::integral_constant<int, (N * QB + b) * kMf + 1>{}, std::bool_constant<db == 0>{}, o[db][b], v,
           pl[b][ks]);
    });
    if constexpr (db == 0) {
      // row sums from the same bf16 P the P·V product uses
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        lacc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, ph[b][ks], lacc[b], 0, 0, 0);
        if constexpr (SPLIT)
          lacc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pl[b][ks], lacc[b], 0, 0, 0);
      }
    }
    if constexpr (N + 1 < kPvSteps) PvStep<N + 1, QB, SPLIT>::run(vf, vbase, ph, pl, ones, o, lacc, extra, mf);
  }
};

// ---- INT8 values: O^T += Vq^T · Pq^T in int32 ----
// The V^T operand of 16 features x 64 keys is one ds_read_b128 per lane (see VtCopy), so a
// step is one read and QB MFMAs of v_mfma_i32_16x16x64_i8 over the whole 64-key tile; the
// same hazards as mfma_pv apply (FIRST: P was written by the vector ALU).
template <bool FIRST>
__device__ __forceinline__ void mfma_pv_i8(i32x4& acc, const i32x4& v, i32x4& p) {
  if constexpr (FIRST)
    asm("s_nop 1\n\tv_mfma_i32_16x16x64_i8 %0, %2, %1, %0 ; carry %1" : "+a"(acc), "+v"(p) : "v"(v));
  else
    asm("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(acc) : "v"(v), "v"(p));
}

template <int N>
__device__ __forceinline__ void vt8_wait(u32x4& f) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(f) : "i"(N));
}

// Step N = feature block db (16 features) of the 16 steps of a tile; V^T fragment db at
// vbase + db * 1024 (16 rows of 64 B). Fragments travel in a ring of kVtDepth + 1 reads.
template <int N, int QB>
struct PvStepI8 {
  static constexpr int kSteps = kD / 16;
  template <class Extra>
  static __device__ __forceinline__ void run(u32x4 (&vf)[kVtDepth + 1], uint32_t vbase,
                                             i32x4 (&pq)[QB], const i32x4& ones,
                                             i32x4 (&o)[16][QB], i32x4 (&lacc)[QB], Extra&& extra) {
    extra(std::integral_constant<int, N>{});
    constexpr int kAhead = (kSteps - 1 - N) < kVtDepth ? (kSteps - 1 - N) : kVtDepth;
    if constexpr (N + kVtDepth < kSteps)
      vf[(N + kVtDepth) % (kVtDepth + 1)] = lds_read_b128<(N + kVtDepth) * 1024>(vbase);
    vt8_wait<kAhead>(vf[N % (kVtDepth + 1)]);
    const i32x4 v = __builtin_bit_cast(i32x4, vf[N % (kVtDepth + 1)]);
#pragma unroll
    for (int b = 0; b < QB; ++b) mfma_pv_i8<N == 0>(o[N][b], v, pq[b]);
    if constexpr (N == 0) {
      // row sums from the same codes
#pragma unroll
      for (int b = 0; b < QB; ++b) lacc[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ones, pq[b], lacc[b], 0, 0, 0);
    }
    if constexpr (N + 1 < kSteps) PvStepI8<N + 1, QB>::run(vf, vbase, pq, ones, o, lacc, extra);
  }
};

template <bool PAGED, bool INT8K, int QB>
constexpr int k_tile_bytes() {
  return (INT8K ? 2 : 4) * kSegStride;
}

// bytes of a V tile: 64 keys x 256 features of bf16, or of INT8 codes
template <bool INT8V>
constexpr int v_tile_bytes() {
  return (INT8V ? 2 : 4) * kSegStride;
}

// key-scale slots: a ring of 3 in the main loop; INT8 values add a fourth for the
// maximum sweep, which keeps three tiles in flight
template <bool INT8K, bool INT8V>
constexpr int sk_slots() {
  return INT8V ? 4 : (INT8K ? 3 : 0);
}

// LDS: two K tiles, two V tiles, (INT8 keys) the ring of key-scale rows, and two slots of
// one restart flag per wave.
template <bool PAGED, bool INT8K, int QB, bool INT8V = false>
constexpr int lds_bytes() {
  return 2 * k_tile_bytes<PAGED, INT8K, QB>() + 2 * v_tile_bytes<INT8V>() +
         sk_slots<INT8K, INT8V>() * kSkTile + 32;
}

// The whole workgroup program. SPLIT selects the P·V form (see the file header); it
// is fixed per workgroup, so each form is a separate straight-line program.
//
// Software pipeline over KV tiles: iteration j holds S(j) from the previous
// iteration, computes P(j) while the MFMAs of S(j+1) = K(j+1)·Q^T run, then
// O += V(j)·P(j). LDS holds K(j+1) and V(j) while K(j+2) and V(j+1) are copied in.
template <bool PAGED, bool INT8K, int QB, bool SPLIT, bool INT8V = false>
__device__ __forceinline__ void run(const Params& p, uint8_t* smem) {
  static_assert(!INT8V || (INT8K && !PAGED && !SPLIT && QB > 1 && kKt == 64),
                "INT8 values: contiguous INT8 keys, prefill shapes, 64-key tiles");
  using S = Shape<QB>;
  constexpr bool kPM = PAGED && INT8K;   // page-major K tiles (the split-d cache)
  using Q = QK<INT8K, QB, kPM>;
  using Acc = typename Q::Acc;
  constexpr int kKTile = k_tile_bytes<PAGED, INT8K, QB>();
  constexpr int kVTile = v_tile_bytes<INT8V>();
  constexpr int kVOff = 2 * kKTile;                    // V tiles follow the two K tiles
  constexpr int kSkOff = kVOff + 2 * kVTile;           // then the key-scale ring
  constexpr int kFlagOff = kSkOff + sk_slots<INT8K, INT8V>() * kSkTile;   // then the restart flags

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
  const int L = lane >> 4;      // k-group of the MFMA operands / row group of the output
  const int c = lane & 15;      // query column (token) inside a 16-column block
  const int tw = w % S::kTokenBlocks;
  const int hw = w / S::kTokenBlocks;
  GQA_PC(PhaseClock pc;)

  // Workgroup id -> (KV head, KV segment, head subset, token block) by unit_of. id % 4 is
  // the KV head, so workgroups dispatched round-robin over the 8 XCDs keep one KV head per
  // XCD (its K/V stream shares that XCD's L2); whole token blocks go longest first, then
  // the segments of the cut ones.
  const Unit unit = unit_of<QB>(p, blockIdx.x);
  const int g = unit.g;
  const int seg = unit.seg;
  const int hsel = unit.hsel;
  const int t0 = unit.tblk * S::kTokPerWg;
  // workspace rows of a split token block: [segment][token - q0][head]
  const int q0 = p.n_plain * S::kTokPerWg;
  const size_t ws_rows = (size_t)(p.q_len - q0);
  const int off = p.kv_len - p.q_len;
  const int head0 = S::kDecode ? kGroup * g + min(c, kGroup - 1)
                                : kGroup * g + hsel * S::kHeadsPerWg + hw * QB;   // head of block 0

  // query column (b, c) of this lane: token t0 + 16 tw + c, head head0 + b; in the decode
  // shape token t0 + w, head 6 g + c for c < 6 (head0 + b below always names the head)
  const int tok = S::kDecode ? t0 + w : t0 + 16 * tw + c;
  const bool tok_ok = tok < p.q_len && (!S::kDecode || c < kGroup);
  const int limit = off + tok;   // last visible key of this column

  const int last_tok = min(t0 + S::kTokPerWg, p.q_len);
  const int ntiles = (off + last_tok + kKt - 1) / kKt;   // tiles of the whole history
  // This workgroup's KV segment: tiles [j0, j1). The host makes every segment at least
  // 8 tiles long, so each segment starts at or before the workgroup's first query and
  // its first key is visible to every query of the workgroup (the pass-0 reference
  // below is then a real score of every column).
  const int j0 = (int)(((int64_t)ntiles * seg) / unit.nseg);
  const int j1 = (int)(((int64_t)ntiles * (seg + 1)) / unit.nseg);
  if (j0 >= j1) {   // empty segment (not produced by the host's plans): weight 0 in the merge
    if (tok_ok && L == 0) {
#pragma unroll
      for (int b = 0; b < QB; ++b)
        *reinterpret_cast<float2*>(p.ws_ml + ((seg * ws_rows + (tok - q0)) * kHq + head0 + b) * 2) =
            make_float2(-__builtin_inff(), 0.0f);
    }
    return;
  }

  // ---- tile copies (this wave's 16 keys of each tile) ----
  using KCopy = WaveCopy<PAGED, INT8K ? kD : 2 * kD, false, PAGED && INT8K>;
  using SCopy = ScaleCopy<PAGED>;
  using VCopy = typename std::conditional<INT8V, VtCopy, WaveCopy<PAGED, 2 * kD, true>>::type;
  const uint32_t smem_addr = lds_addr(smem);
  const uint32_t sk_addr = smem_addr + kSkOff;   // key-scale ring (INT8 keys)
  const uint32_t kvo[2] = {KCopy::lane_offset(lane, 0), KCopy::lane_offset(lane, kHalves - 1)};
  uint32_t vvo[2];
  if constexpr (INT8V) {
    vvo[0] = VtCopy::lane_offset(lane, 0, p.v_ld);
    vvo[1] = VtCopy::lane_offset(lane, 1, p.v_ld);
  } else {
    vvo[0] = VCopy::lane_offset(lane, 0);
    vvo[1] = VCopy::lane_offset(lane, kHalves - 1);
  }
  const uint32_t svo = SCopy::lane_offset(lane);
  const int skey = lane & 15;   // the key whose scales this lane copies
  // Paged: the physical block of this wave's 16 keys of the tile at kbase (an entry
  // outside [0, num_blocks) is clamped into it); 0 when contiguous. The block table is
  // read-only for the whole launch, so it is read as constant memory: a scalar load
  // into a scalar register, which a loop-carried value can wait in until its use.
  auto block_of = [&](int kbase) -> int {
    if constexpr (PAGED) {
      const int first = __builtin_amdgcn_readfirstlane(min(kbase + kWaveKeys * w, p.kv_len - 1));
      const int entry = *(const __attribute__((address_space(4))) int32_t*)(p.bt + (first >> 4));
      return min(max(entry, 0), p.num_blocks - 1);
    } else {
      (void)kbase;
      return 0;
    }
  };
  auto kcopy = [&](int kbase, int buf, int blk) {
    return KCopy(p, p.k, g, kbase + kWaveKeys * w, blk,
                 smem_addr + buf * kKTile + (kPM ? w * kPageBytes : kWaveKeys * w * 128));
  };
  auto vcopy = [&](int kbase, int buf, int blk) {
    if constexpr (INT8V) {
      (void)blk;
      return VCopy(p, g, kbase, w, smem_addr + kVOff + buf * kVTile);
    } else {
      return VCopy(p, p.v, g, kbase + kWaveKeys * w, blk,
                   smem_addr + kVOff + buf * kVTile + kWaveKeys * w * 128);
    }
  };
  auto scopy = [&](int kbase, int slot, int blk) {
    return SCopy(p, kbase + kWaveKeys * w, blk, sk_addr + slot * kSkTile + w * 256);
  };
  // whole-tile copies outside the pipelined loop
  auto copy_k_all = [&](int kbase, int buf, int slot) {
    const int blk = block_of(kbase);
    const KCopy kc = kcopy(kbase, buf, blk);
    static_for<0, KCopy::kInsts>([&](auto ic) { kc.template issue<decltype(ic)::value>(kvo); });
    if constexpr (INT8K) scopy(kbase, slot, blk).issue(svo, skey);
  };
  auto copy_v_all = [&](int kbase, int buf) {
    const VCopy vc = vcopy(kbase, buf, block_of(kbase));
    static_for<0, VCopy::kInsts>([&](auto ic) { vc.template issue<decltype(ic)::value>(vvo); });
  };

  // INT8 values: the maximum sweep below runs first, over every tile of the history, with
  // three tiles of K in flight in the four K and V buffers and the four key-scale slots
  constexpr int kSweepDepth = 3;
  constexpr int kSweepPerTile = KCopy::kInsts + 1;   // this wave's copies per sweep tile
  static_assert(!INT8V || 2 * kSweepPerTile < 16, "sweep copies in flight");
  if constexpr (INT8V) {
    static_assert(kVTile == kKTile, "the sweep uses the V buffers as K buffers");
    for (int t = 0; t < min(kSweepDepth, ntiles); ++t) copy_k_all(t * kKt, t & 3, t & 3);
  } else {
    // start the first copies before the Q prologue
    copy_k_all(j0 * kKt, j0 & 1, j0 % 3);
    copy_v_all(j0 * kKt, j0 & 1);
    if (j1 - j0 > 1) copy_k_all((j0 + 1) * kKt, (j0 + 1) & 1, (j0 + 1) % 3);
  }

  // ---- prologue: Q fragments (B operand of S^T = K·Q^T) ----
  typename Q::Frag qf[QB][Q::kSteps];
  float qs[QB];   // log2(e)/16, times sQ with INT8 keys
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
    } else if (p.qsc != nullptr) {
      // Q quantised beforehand: the fragment is bytes 64 s + 16 L .. + 15 of the row's
      // codes, the same one the quantising form below packs
      const uint8_t* crow = p.q + ((size_t)tok * kHq + head0 + b) * kD;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint4 raw = tok_ok ? *reinterpret_cast<const uint4*>(crow + 64 * s + 16 * L)
                                 : make_uint4(0, 0, 0, 0);
        qf[b][s] = __builtin_bit_cast(i32x4, raw);
      }
      const float sq = tok_ok ? p.qsc[(size_t)tok * kHq + head0 + b] : 0.0f;
      qs[b] = sq * kLog2eOver16;
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
        qf[b][s] = i32x4{(int)wv[0], (int)wv[1], (int)wv[2], (int)wv[3]};
      }
    }
  }

  // ---- per-lane LDS bases ----
  const int kb_even = kPM ? L * 256 + c * 16 : c * 128 + ((L ^ (c & 7)) << 4);
  const int kb_odd = kPM ? kb_even : c * 128 + (((L ^ (c & 7)) ^ 4) << 4);
  uint32_t vbase_off[4];
  const int vsw = tile_swizzle<true>(4 * L + (c >> 2)) >> 1;   // V swizzle of this lane's key
#pragma unroll
  for (int jj = 0; jj < 4; ++jj)
    vbase_off[jj] = (4 * L + (c >> 2)) * 128 + ((2 * (jj ^ vsw) + ((c & 3) >> 1)) << 4) +
                    8 * (c & 1);
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;
  // INT8 values: lane (L, c) reads slot L ^ ((c >> 1) & 3) of feature row c of each
  // 16-feature block (VtCopy)
  const uint32_t vt8_off = c * kKt + 16 * (L ^ ((c >> 1) & 3));
  const i32x4 ones8 = {0x01010101, 0x01010101, 0x01010101, 0x01010101};

  // ---- accumulators: O^T blocks [feature block db][query block b], row sums ----
  using OAcc = typename std::conditional<INT8V, i32x4, f32x4>::type;   // int32 with INT8 values
  OAcc o[16][QB];
  OAcc lacc[QB];
  float m[QB];   // reference maximum per column (log2 units), fixed during a pass
  Acc sacc[QB][kKb];
  int* const flags = reinterpret_cast<int*>(smem + kFlagOff);

  // S^T of the tile in K buffer `kbuf` into sacc
  auto qk_tile = [&](uint32_t kbuf) {
#pragma unroll
    for (int b = 0; b < QB; ++b)
#pragma unroll
      for (int kb = 0; kb < kKb; ++kb) sacc[b][kb] = Acc{0, 0, 0, 0};
    qk_pair<INT8K, QB, kPM, 0>(kbuf, kb_even, kb_odd, qf, sacc, [](auto) {});
    if constexpr (kHalves > 1) qk_pair<INT8K, QB, kPM, 2>(kbuf, kb_even, kb_odd, qf, sacc, [](auto) {});
  };
  // INT8 keys: sacc holds int32 dot products until scale_unit turns them, in place, into
  // float scores in log2 units (their bit patterns): y = float(S) * (sK * sQ * log2(e)/16),
  // or, inside the tile loop where the pass's reference maximum m is fixed, the exponent
  // y - m itself as one fused multiply-add. Both forms are written out explicitly (no
  // contraction left to the compiler), so every build rounds every score the same way.
  // The scales of keys 16 kb + 4 L .. + 3 for KV head g come from one 16-byte LDS read
  // per 16-key block kb.
  // (32-key tiles: keys 4 L .. 4 L + 3 of block kb were copied by wave 2 kb + L / 2)
  auto sk_read = [&](uint32_t sk_slot, u32x4 (&sr)[4]) {
    if constexpr (kKt == 64) {
      const uint32_t a = sk_slot + g * 64 + 16 * L;
      sr[0] = lds_read_b128<0>(a);
      sr[1] = lds_read_b128<256>(a);
      sr[2] = lds_read_b128<512>(a);
      sr[3] = lds_read_b128<768>(a);
    } else {
      const uint32_t a = sk_slot + g * 64 + 16 * (L & 1) + 256 * (L >> 1);
      sr[0] = lds_read_b128<0>(a);
      sr[1] = lds_read_b128<512>(a);
      sr[2] = sr[0];   // unused
      sr[3] = sr[1];
    }
  };
  auto scale_unit = [&](auto kb_c, auto b_c, const u32x4 (&sr)[4], auto minus_m_c) {
#pragma clang fp contract(off)
    constexpr int kb = decltype(kb_c)::value, b = decltype(b_c)::value;
    f32x4 skv = __builtin_bit_cast(f32x4, sr[kb]);
    // Empty volatile statements on the key scales and on the result hold this unit's
    // scaling at the P·V step that calls it: volatile statements keep their order among
    // themselves, and each step's LDS wait is one. Without them the compiler sinks all of
    // a tile's scaling past the tile barrier (the restart exit does not need it), where it
    // runs with no MFMA to overlap. The int32 scores are not held: the Q·K^T MFMA that
    // writes them may still be in flight, and a statement that lists them as outputs would
    // hide that write from the compiler, which then omits the MFMA's wait states before
    // the conversion reads them.
    if constexpr (decltype(minus_m_c)::value) asm volatile("; hold %0" : "+v"(skv));
    f32x4 y;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (decltype(minus_m_c)::value)
        y[r] = __builtin_fmaf((float)sacc[b][kb][r], skv[r] * qs[b], -m[b]);
      else
        y[r] = (float)sacc[b][kb][r] * (skv[r] * qs[b]);
    }
    if constexpr (decltype(minus_m_c)::value) asm volatile("; hold %0" : "+v"(y));
    sacc[b][kb] = __builtin_bit_cast(Acc, y);
  };
  // the whole tile at once (outside the pipelined loop)
  auto scale_tile = [&](uint32_t sk_slot) {
    if constexpr (INT8K) {
      u32x4 sr[4];
      sk_read(sk_slot, sr);
      lds_wait4<0>(sr[0], sr[1], sr[2], sr[3]);
      static_for<0, kKb * QB>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        scale_unit(std::integral_constant<int, u / QB>{}, std::integral_constant<int, u % QB>{}, sr,
                   std::false_type{});
      });
    }
  };
  // the first tile of a pass: y -> y - m once m is known
  auto shift_tile = [&]() {
    if constexpr (INT8K) {
#pragma clang fp contract(off)
#pragma unroll
      for (int b = 0; b < QB; ++b)
#pragma unroll
        for (int kb = 0; kb < kKb; ++kb) {
          f32x4 y = __builtin_bit_cast(f32x4, sacc[b][kb]);
#pragma unroll
          for (int r = 0; r < 4; ++r) y[r] = y[r] - m[b];
          sacc[b][kb] = __builtin_bit_cast(Acc, y);
        }
    } else {   // bf16 keys: the first key half's exponents s * log2(e)/16 - m, which the
               // tile loop forms for the next tile during the P·V steps
#pragma clang fp contract(off)
#pragma unroll
      for (int b = 0; b < QB; ++b)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)   // key blocks 0, 1
#pragma unroll
          for (int r = 0; r < 4; ++r) sacc[b][kb][r] = __builtin_fmaf(sacc[b][kb][r], kLog2eOver16, -m[b]);
    }
  };
  // scores of key blocks 2h, 2h + 1 (keys kbase + 32 h .. + 31) from sacc, in log2 units
  // once multiplied by scale[b] (bf16: raw dot products, but inside the tile loop the
  // first key half already holds its exponents; INT8 keys: already scaled), causal mask
  // applied. sc[b][e]: e = 0..3 keys 32 h + 4 L + e, e = 4..7 keys 32 h + 16 + 4 L + e - 4
  auto half_scores = [&](auto mask_c, int kbase, int h, float (&sc)[QB][8], float (&scale)[QB]) {
    constexpr bool kMask = decltype(mask_c)::value;
    if constexpr (!INT8K) {
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        scale[b] = kLog2eOver16;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[b][4 * kk + r] = sacc[b][2 * h + kk][r];
      }
    } else {   // already scaled: y for the maxima of a first tile, else y - m, which
               // the softmax takes as the exponent (bit-cast whole vectors: a cast of
               // one vector element by reference would not name that element)
#pragma unroll
      for (int b = 0; b < QB; ++b)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const f32x4 sf = __builtin_bit_cast(f32x4, sacc[b][2 * h + kk]);
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[b][4 * kk + r] = sf[r];
        }
#pragma unroll
      for (int b = 0; b < QB; ++b) scale[b] = 1.0f;
    }
    if constexpr (kMask) {   // tiles that reach past the workgroup's first query
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kbase + 16 * (2 * h + kk) + 4 * L + r;
          if (key > limit) {
#pragma unroll
            for (int b = 0; b < QB; ++b) sc[b][4 * kk + r] = -__builtin_inff();
          }
        }
    }
  };
  // this lane's maximum of each column (not yet reduced over the 4 lanes of a column)
  auto lane_max = [&](const float (&sc)[QB][8], int b) {
    float mx = sc[b][0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sc[b][e]);
    return mx;
  };
  // column maxima of the whole tile in sacc (reduced over the 4 lanes of a column)
  auto tile_max = [&](int kbase, float (&mx)[QB]) {
    float sc0[QB][8], sc1[QB][8], scale[QB];
    half_scores(std::true_type{}, kbase, 0, sc0, scale);
    if constexpr (kHalves > 1) half_scores(std::true_type{}, kbase, 1, sc1, scale);
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      const float lm = kHalves > 1 ? fmaxf(lane_max(sc0, b), lane_max(sc1, b)) : lane_max(sc0, b);
      mx[b] = xor32_max(xor16_max(lm)) * scale[b];
    }
  };

  // Pass 0 takes each column's maximum over tile 0 as the reference (tile 0 holds key
  // 0, which every query sees, so the reference is a real score of the column and its
  // sum of exponentials is at least 1). If a column's running sum exceeds kOverSum
  // (some later score lies far above the reference) the whole workgroup starts again
  // (pass 1) with the exact column maxima over all its keys, found by a max-only
  // sweep. Either way no accumulator is ever rescaled.
  // (two instantiations, not a loop, so nothing of pass 1 is hoisted into pass 0)
  auto main_pass = [&](auto pass_c) -> bool {
    constexpr int pass = decltype(pass_c)::value;
    if constexpr (pass > 0) {
      copy_k_all(j0 * kKt, j0 & 1, j0 % 3);
      copy_v_all(j0 * kKt, j0 & 1);
      if (j1 - j0 > 1) copy_k_all((j0 + 1) * kKt, (j0 + 1) & 1, (j0 + 1) % 3);
    }
    if constexpr (pass > 0) agpr_fence<24>(o);   // after the MFMAs of pass 0
#pragma unroll
    for (int b = 0; b < QB; ++b) {
#pragma unroll
      for (int db = 0; db < 16; ++db) o[db][b] = OAcc{0, 0, 0, 0};
      lacc[b] = OAcc{0, 0, 0, 0};
    }
    agpr_fence<2>(o);
    if (pass == 0 && tid < 8) flags[tid] = 0;
    wait_vm_all();
    __syncthreads();
    qk_tile(smem_addr + (j0 & 1) * kKTile);   // S(j0)
    scale_tile(sk_addr + (j0 % 3) * kSkTile);
    if (pass == 0) tile_max(j0 * kKt, m);
    shift_tile();
    __syncthreads();   // every wave is done with K(j0) before K(j0+2) overwrites it

    // Tiles that end at or before the workgroup's first query need no causal mask; the
    // rest (one or two per workgroup) run the masked form of the same body. The body
    // is one basic block: copies past the last tile re-read the clamped last key into a
    // buffer nothing reads again, and the restart flag is rewritten every tile.
    const int n_plain = min(j1, (off + t0 + 1) / kKt);
    int flag_seen = 0;   // flags read after the previous tile's barrier
    // first key of the tile that iteration j copies (K and scales of tile j + 2, V of tile
    // j + 1); a tile past the segment is fetched from kv_len on: no rows, no traffic
    auto copy_base = [&](int tile) { return tile < j1 ? tile * kKt : p.kv_len; };
    // Paged: block-table entries are read one iteration before their copies (the value
    // for iteration j + 1's K copy is loaded at the start of iteration j), so a copy never
    // waits for its block-table read.
    int blk_v = block_of(copy_base(j0 + 1));   // V copy of the current iteration
    int blk_k = block_of(copy_base(j0 + 2));   // K and scale copies of the current iteration
    // returns true when pass 0 must restart
    auto body = [&](int j, auto mask_c) -> bool {
      GQA_PC(const unsigned long long tp0 = PhaseClock::cycles();)
      const int kbase = j * kKt;
      const uint8_t* knext = smem + ((j + 1) & 1) * kKTile;             // K(j+1) (stale on the last tile)
      const uint8_t* vcur = smem + kVOff + (j & 1) * kVTile;   // V(j)
      // copies of K(j+2) and V(j+1), spread evenly over the K steps of both halves (one
      // per step for bf16 keys): the vector memory path moves about 64 B per clock per CU,
      // so the 64 KiB of a tile need a good part of the iteration, and issuing them in a
      // burst would stall the waves on a full address queue; the P·V steps, three MFMAs
      // each, leave too little time between copies (measured)
      const int kb2 = copy_base(j + 2);
      const int kb1 = copy_base(j + 1);
      const int blk_next = block_of(copy_base(j + 3));
      const KCopy kc = kcopy(kb2, j & 1, blk_k);
      const VCopy vc = vcopy(kb1, (j + 1) & 1, blk_v);
      SCopy scp;
      if constexpr (INT8K) scp = scopy(kb2, (j + 2) % 3, blk_k);
      blk_v = blk_k;
      blk_k = blk_next;
      constexpr int kCopies = KCopy::kInsts + VCopy::kInsts + (INT8K ? 1 : 0);
      auto copy_issue = [&](auto ic) {
        constexpr int I = decltype(ic)::value;
        if constexpr (I < KCopy::kInsts)
          kc.template issue<I>(kvo);
        else if constexpr (I < KCopy::kInsts + VCopy::kInsts)
          vc.template issue<I - KCopy::kInsts>(vvo);
        else
          scp.issue(svo, skey);
      };
      constexpr int kSlots = kHalves * Q::kSteps;   // issue slots: the K steps of the halves
      // the copies whose slot (I * kSlots) / kCopies is SLOT
      auto copies_at = [&](auto slot_c) {
        constexpr int kSlot = decltype(slot_c)::value;
        static_for<0, kCopies>([&](auto ic) {
          constexpr int I = decltype(ic)::value;
          if constexpr ((I * kSlots) / kCopies == kSlot) copy_issue(ic);
        });
      };

      // ---- P(j) from S(j), interleaved with S(j+1) = K(j+1) · Q^T, one 32-key half at a
      // time: the half of S(j) being turned into P is copied out of the accumulators
      // before the MFMAs of S(j+1) overwrite them ----
      bf16x8 ph[QB][2], pl[QB][2];
      uint32_t pq8[QB][4];   // INT8 values: P codes, dword kb = keys 16 kb + 4 L .. + 3
      // INT8 keys, bf16 P without a low part: P of the second key half is formed during
      // the first 16 P·V steps (which do not read it) instead of after the last Q·K^T
      // MFMAs, where its exponentials would have no MFMA to overlap
      constexpr bool kLateP = INT8K && !INT8V && !SPLIT && kHalves == 2;
      float scl[QB][8];      // the second half's exponents (y - m), kept for those steps
      const uint32_t kn = lds_addr(knext);
      auto half = [&](auto hc) {
        constexpr int H = decltype(hc)::value;
        float sc[QB][8], scale[QB];
        half_scores(mask_c, kbase, H, sc, scale);
        if constexpr (!INT8K && H > 0) {
          // bf16 keys, second key half: the exponent s * log2(e)/16 - m at once, reading
          // the accumulators before this half's MFMAs reuse them, so the scores need no
          // copy (the first half's exponents were formed during the previous tile's last
          // P·V steps)
#pragma clang fp contract(off)
#pragma unroll
          for (int b = 0; b < QB; ++b) {
            const float nm = -m[b];
#pragma unroll
            for (int e = 0; e < 8; ++e) sc[b][e] = __builtin_fmaf(sc[b][e], scale[b], nm);
          }
        }
        if constexpr (kLateP && H == 1) {
#pragma unroll
          for (int b = 0; b < QB; ++b)
#pragma unroll
            for (int e = 0; e < 8; ++e) scl[b][e] = sc[b][e];
        }
#pragma unroll
        for (int b = 0; b < QB; ++b) sacc[b][2 * H] = sacc[b][2 * H + 1] = Acc{0, 0, 0, 0};
        // P for query block b after K step ((b + 1) * steps) / QB - 1 of this half
        auto softmax_part = [&](auto st_c) {
          constexpr int st = decltype(st_c)::value;
          copies_at(std::integral_constant<int, H * Q::kSteps + st>{});
          if constexpr (kLateP && H == 1) return;
#pragma unroll
          for (int b = 0; b < QB; ++b) {
            if (st == ((b + 1) * Q::kSteps) / QB - 1) {
              if constexpr (INT8V) {
                // Pq = round(127 * 2^(y - max)): the exponent already holds + log2(127); the
                // clamp keeps a code that rounding lifts past 127 at 127
                uint32_t wv[2] = {0u, 0u};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                  const float x = fminf(__builtin_amdgcn_exp2f(sc[b][e]), 127.0f);
                  wv[e >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_rintf(x), e & 3, wv[e >> 2]);
                }
                pq8[b][2 * H] = wv[0];
                pq8[b][2 * H + 1] = wv[1];
              } else {
                f32x8 pv;   // the exponents are ready (bf16 keys: the second half's computed
                            // above, the first half's during the previous tile's P·V steps)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                  pv[e] = __builtin_amdgcn_exp2f(sc[b][e]);
                ph[b][H] = __builtin_convertvector(pv, bf16x8);
                if constexpr (SPLIT)
                  pl[b][H] = __builtin_convertvector(pv - __builtin_convertvector(ph[b][H], f32x8), bf16x8);
              }
            }
          }
        };
        qk_pair<INT8K, QB, kPM, 2 * H>(kn, kb_even, kb_odd, qf, sacc, softmax_part);
      };
      half(std::integral_constant<int, 0>{});
      if constexpr (kHalves > 1) half(std::integral_constant<int, 1>{});
      GQA_PC(const unsigned long long tp1 = PhaseClock::cycles();)

      // ---- O^T += V^T(j) · P^T(j); INT8 keys: S(j+1) is scaled between the steps, where
      // the vector ALU has room (the Q·K^T halves above are short on it: half as many
      // MFMAs as with bf16 keys for the same softmax work) ----
      if constexpr (INT8V) {
        u32x4 sr[4];   // scales of tile j + 1 (copied two iterations ago)
        sk_read(sk_addr + ((j + 1) % 3) * kSkTile, sr);
        const uint32_t vb = lds_addr(vcur) + vt8_off;
        u32x4 vf[kVtDepth + 1];
        static_for<0, kVtDepth>([&](auto nc) {   // the first kVtDepth steps' reads
          constexpr int N = decltype(nc)::value;
          vf[N] = lds_read_b128<N * 1024>(vb);
        });
        i32x4 pqv[QB];
#pragma unroll
        for (int b = 0; b < QB; ++b)
          pqv[b] = i32x4{(int)pq8[b][0], (int)pq8[b][1], (int)pq8[b][2], (int)pq8[b][3]};
        PvStepI8<0, QB>::run(vf, vb, pqv, ones8, o, lacc, [&](auto nc) {
          constexpr int N = decltype(nc)::value;
          // at step 1 only the kVtDepth reads of steps 1 .. kVtDepth are younger than the
          // scale reads: the wait costs nothing and marks them valid
          if constexpr (N == 1) lds_wait4<kVtDepth>(sr[0], sr[1], sr[2], sr[3]);
          if constexpr (N >= 2 && N - 2 < kKb * QB) {
            constexpr int u = N - 2;
            scale_unit(std::integral_constant<int, u / QB>{}, std::integral_constant<int, u % QB>{}, sr,
                       std::true_type{});
          }
        });
      } else {
        u32x4 sr[4];   // scales of tile j + 1 (copied two iterations ago)
        if constexpr (INT8K) sk_read(sk_addr + ((j + 1) % 3) * kSkTile, sr);
        uint32_t vbase[4];
        const uint32_t v0 = lds_addr(vcur);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) vbase[jj] = v0 + vbase_off[jj];
        VtFrag vf[kVtDepth + 1];
        static_for<0, kVtDepth>([&](auto nc) {   // the first kVtDepth steps' reads
          vt_issue_step<decltype(nc)::value>(vf[decltype(nc)::value], vbase);
        });
        // INT8 keys: the scores of S(j+1) are turned into exponents y - m between the P·V
        // MFMAs (the arithmetic of scale_unit), one vector instruction at a time: the
        // conversion, the product of the scales and the FMA of each score are spread evenly
        // over the gaps between the tile's MFMA statements from step 2 on (the scale reads
        // are waited for at step 1), one or two per gap. Each instruction is held in its gap
        // by carrying registers through the statements around it (ScaleSchedule). Measured
        // against whole 4-score units every other step: 3.4% faster on 3072 x 16384; against
        // one score's three instructions per gap: 1.3%.
        using SS = ScaleSchedule<kPvSteps * QB * (SPLIT ? 2 : 1), 2 * QB * (SPLIT ? 2 : 1), 4 * kKb * QB>;
        float cvt[SS::kScores], prod[SS::kScores];   // per score: float(S), sK * sQ'
        float plf[QB][8];      // kLateP: exponentials of the second key half
        uint32_t plw[QB][4];   // kLateP: their bf16 pairs
        PvStep<0, QB, SPLIT>::run(
            vf, vbase, ph, pl, ones, o, lacc,
            [&](auto nc) {
              constexpr int N = decltype(nc)::value;
              // at step 1 only the 2 kVtDepth reads of steps 1 .. kVtDepth are younger
              // than the scale reads: the wait costs nothing and marks them valid
              if constexpr (INT8K && N == 1) lds_wait4<2 * kVtDepth>(sr[0], sr[1], sr[2], sr[3]);
              if constexpr (kLateP && N <= 16) {
                // step N takes exponents i0 .. i1 - 1 of the 8 QB (score i: block i / 8,
                // key i % 8); empty volatile statements at the starts of steps N and N + 1
                // hold each step's work between them (they keep their order with the
                // steps' LDS waits and reads). Only values the vector ALU wrote are held
                // (the exponents come from the scaling of the previous iteration).
                // Measured against forming them after the Q·K^T MFMAs: 1.2% faster on
                // 3072 x 16384, 1.8% on the paged 512 x 32768 tail.
                constexpr int kN = 8 * QB;
                if constexpr (N > 0) {   // results of step N - 1
                  constexpr int j0 = ((N - 1) * kN) / 16, j1 = (N * kN) / 16;
                  static_for<j0, j1>([&](auto ic) {
                    constexpr int i = decltype(ic)::value;
                    // (a reference first: this compiler does not capture a variable that a
                    // nested lambda names only in an asm operand)
                    if constexpr (i & 1) {
                      uint32_t& w = plw[i / 8][(i % 8) >> 1];
                      asm volatile("; hold %0" : "+v"(w));
                    } else {
                      float& x = plf[i / 8][i % 8];
                      asm volatile("; hold %0" : "+v"(x));
                    }
                  });
                }
                if constexpr (N == 16) {
#pragma unroll
                  for (int b = 0; b < QB; ++b)
                    ph[b][1] = __builtin_bit_cast(bf16x8, u32x4{plw[b][0], plw[b][1], plw[b][2], plw[b][3]});
                } else {
                  constexpr int i0 = (N * kN) / 16, i1 = ((N + 1) * kN) / 16;
                  static_for<i0, i1>([&](auto ic) {
                    constexpr int i = decltype(ic)::value;
                    float& x = scl[i / 8][i % 8];
                    asm volatile("; hold %0" : "+v"(x));
                  });
                  static_for<i0, i1>([&](auto ic) {
                    constexpr int i = decltype(ic)::value, b = i / 8, e = i % 8;
                    plf[b][e] = __builtin_amdgcn_exp2f(scl[b][e]);
                    if constexpr (e & 1) {
                      typedef float f32x2 __attribute__((ext_vector_type(2)));
                      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
                      const f32x2 two = {plf[b][e - 1], plf[b][e]};
                      plw[b][e >> 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(two, bf16x2));
                    }
                  });
                }
              }
            },
            [&](auto kc, auto first_c, f32x4& acc, const bf16x8& v, bf16x8& pp) {
              constexpr bool kF = decltype(first_c)::value;
              constexpr int k = decltype(kc)::value;
              if constexpr (!INT8K) {
                // bf16 keys: the exponents of S(j+1)'s first key half over the last 16
                // gaps (ExpSchedule; one or two FMAs a gap with 3 query blocks). Measured in
                // loop cycles a tile against forming them before that half's first Q·K^T
                // MFMA, where they ran with no MFMA to overlap: 1.7% fewer on 4096 x 32768,
                // 1.5% on 3072 x 16384, 0.2% on the paged 512 x 32768 tail (12 gaps, two a
                // gap: 1.5% and 1.2% fewer, 0.3% more; 24 gaps, one a gap: 0.5% and 0.4%
                // fewer, 1.2% more; all 48 FMAs spread over the steps from step 2: 0.5%
                // slower in time on 4096 x 32768). In time the gain is smaller (0.1-1.2%,
                // same-box A/B): the chip holds the denser loop at a lower clock.
                constexpr int kStmts = kPvSteps * QB * (SPLIT ? 2 : 1);
                using ES = ExpSchedule<kStmts, (kStmts - 1 < 16 ? kStmts - 1 : 16), 8 * QB>;
                constexpr CarryPlan cp = ES::carries(k);
                auto load = [&](auto ic) -> uint32_t {
                  constexpr int kind = cp.kind[decltype(ic)::value], i = cp.score[decltype(ic)::value];
                  constexpr int u = i / 4, kb = u / QB, b = u % QB, r = i % 4;
                  // (the element read into a scalar first: this compiler's bit cast of a
                  // vector element reads the vector's first element instead)
                  const float x = kind == CarryPlan::kY ? sacc[b][kb][r] : m[b];
                  return __builtin_bit_cast(uint32_t, x);
                };
                auto store = [&](auto ic, uint32_t w) {
                  constexpr int kind = cp.kind[decltype(ic)::value], i = cp.score[decltype(ic)::value];
                  constexpr int u = i / 4, kb = u / QB, b = u % QB, r = i % 4;
                  if constexpr (kind == CarryPlan::kY) sacc[b][kb][r] = __builtin_bit_cast(float, w);
                  else m[b] = __builtin_bit_cast(float, w);
                };
                using I0 = std::integral_constant<int, 0>;
                using I1 = std::integral_constant<int, 1>;
                using I2 = std::integral_constant<int, 2>;
                if constexpr (cp.n == 0) {
                  mfma_pv<kF>(acc, v, pp);
                } else if constexpr (cp.n == 1) {
                  uint32_t a = load(I0{});
                  mfma_pv_carry<kF>(acc, v, pp, a);
                  store(I0{}, a);
                } else if constexpr (cp.n == 2) {
                  uint32_t a = load(I0{}), b = load(I1{});
                  mfma_pv_carry<kF>(acc, v, pp, a, b);
                  store(I0{}, a);
                  store(I1{}, b);
                } else {
                  static_assert(cp.n == 3, "at most 3 registers carried per statement");
                  uint32_t a = load(I0{}), b = load(I1{}), c = load(I2{});
                  mfma_pv_carry<kF>(acc, v, pp, a, b, c);
                  store(I0{}, a);
                  store(I1{}, b);
                  store(I2{}, c);
                }
                static_for<ES::first_op(k), ES::first_op(k + 1)>([&](auto ic) {
#pragma clang fp contract(off)
                  constexpr int i = decltype(ic)::value;
                  constexpr int u = i / 4, kb = u / QB, b = u % QB, r = i % 4;
                  sacc[b][kb][r] = __builtin_fmaf(sacc[b][kb][r], kLog2eOver16, -m[b]);
                });
              } else {
                constexpr CarryPlan cp = SS::carries(k);
                auto load = [&](auto ic) -> uint32_t {
                  constexpr int kind = cp.kind[decltype(ic)::value], i = cp.score[decltype(ic)::value];
                  constexpr int u = i / 4, kb = u / QB, b = u % QB, r = i % 4;
                  if constexpr (kind == CarryPlan::kY) return sacc[b][kb][r];
                  else if constexpr (kind == CarryPlan::kSK) return sr[kb][r];
                  else if constexpr (kind == CarryPlan::kC) return __builtin_bit_cast(uint32_t, cvt[i]);
                  else return __builtin_bit_cast(uint32_t, prod[i]);
                };
                auto store = [&](auto ic, uint32_t w) {
                  constexpr int kind = cp.kind[decltype(ic)::value], i = cp.score[decltype(ic)::value];
                  constexpr int u = i / 4, kb = u / QB, b = u % QB, r = i % 4;
                  if constexpr (kind == CarryPlan::kY) sacc[b][kb][r] = w;
                  else if constexpr (kind == CarryPlan::kSK) sr[kb][r] = w;
                  else if constexpr (kind == CarryPlan::kC) cvt[i] = __builtin_bit_cast(float, w);
                  else prod[i] = __builtin_bit_cast(float, w);
                };
                using I0 = std::integral_constant<int, 0>;
                using I1 = std::integral_constant<int, 1>;
                using I2 = std::integral_constant<int, 2>;
                if constexpr (cp.n == 0) {
                  mfma_pv<kF>(acc, v, pp);
                } else if constexpr (cp.n == 1) {
                  uint32_t a = load(I0{});
                  mfma_pv_carry<kF>(acc, v, pp, a);
                  store(I0{}, a);
                } else if constexpr (cp.n == 2) {
                  uint32_t a = load(I0{}), b = load(I1{});
                  mfma_pv_carry<kF>(acc, v, pp, a, b);
                  store(I0{}, a);
                  store(I1{}, b);
                } else {
                  static_assert(cp.n == 3, "at most 3 registers carried per statement");
                  uint32_t a = load(I0{}), b = load(I1{}), c = load(I2{});
                  mfma_pv_carry<kF>(acc, v, pp, a, b, c);
                  store(I0{}, a);
                  store(I1{}, b);
                  store(I2{}, c);
                }
                // this gap's instructions, in order
                static_for<SS::first_op(k), SS::first_op(k + 1)>([&](auto jc) {
#pragma clang fp contract(off)
                  constexpr int jj = decltype(jc)::value, i = jj / 3;
                  constexpr int u = i / 4, kb = u / QB, b = u % QB, r = i % 4;
                  if constexpr (jj % 3 == 0) {
                    cvt[i] = (float)sacc[b][kb][r];
                  } else if constexpr (jj % 3 == 1) {
                    // the element read into a scalar first: this compiler's __builtin_bit_cast
                    // of a vector element reads the vector's first element instead
                    const uint32_t skr = sr[kb][r];
                    prod[i] = __builtin_bit_cast(float, skr) * qs[b];
                  } else {
                    sacc[b][kb][r] = __builtin_bit_cast(int, __builtin_fmaf(cvt[i], prod[i], -m[b]));
                  }
                });
              }
            });
      }

      GQA_PC(const unsigned long long tp2 = PhaseClock::cycles();)
      // Flags are double-buffered by tile parity: the write for tile j + 2 happens only
      // after every wave has passed barrier j + 1, i.e. after it read tile j's slot, so
      // all waves read the same value and leave the loop on the same tile. A wave's
      // condition never clears once raised (the running sums only grow), so rewriting
      // the flag every tile keeps it raised.
      if (pass == 0) {
        bool over = false;
#pragma unroll
        for (int b = 0; b < QB; ++b) over = over || !(lacc[b][0] <= kOverSum);
        flags[4 * (j & 1) + w] = __builtin_amdgcn_ballot_w64(over) != 0;
      }
      wait_vm_all();
      __syncthreads();   // K(j+2), V(j+1) landed; everyone is done with K(j+1) and V(j)
      GQA_PC(const unsigned long long tp3 = PhaseClock::cycles();
             if constexpr (decltype(mask_c)::value) {
               pc.masked += tp3 - tp0;
               pc.n_masked += 1;
             } else {
               pc.qk += tp1 - tp0;
               pc.pv += tp2 - tp1;
               pc.sync += tp3 - tp2;
               pc.n += 1;
             })
      if (pass == 0) {
        // act on the flags of the tile before (one tile late, so the read is off the
        // critical path; the extra tile's garbage is discarded by the restart)
        if (flag_seen != 0) return true;
        const i32x4 f = *reinterpret_cast<const i32x4*>(flags + 4 * (j & 1));
        flag_seen = f[0] | f[1] | f[2] | f[3];
      }
      return false;
    };
    bool restart = false;
    int j = j0;
    GQA_PC(pc.qk = pc.pv = pc.sync = pc.n = pc.masked = pc.n_masked = 0;
           pc.c0 = PhaseClock::cycles(); pc.r0 = PhaseClock::ticks();)
    for (; j < n_plain && !restart; ++j) restart = body(j, std::false_type{});
    for (; j < j1 && !restart; ++j) restart = body(j, std::true_type{});
    if (pass == 0 && !restart && flag_seen != 0) restart = true;   // raised on the last tile
    GQA_PC(if (lane == 0 && blockIdx.x < kPhaseWaves / 4) {
             unsigned long long* slot = phase_clock + ((size_t)blockIdx.x * 4 + w) * kPhaseSlots;
             const unsigned long long c1 = PhaseClock::cycles(), r1 = PhaseClock::ticks();
             slot[0] = pc.qk; slot[1] = pc.pv; slot[2] = pc.sync; slot[3] = pc.n;
             slot[4] = pc.masked; slot[5] = pc.n_masked; slot[6] = pc.sweep; slot[7] = pc.n_sweep;
             slot[8] = c1 - pc.c0; slot[9] = r1 - pc.r0;
           })
    return restart;
  };

  if constexpr (INT8V) {
    // ---- exact column maxima over every visible key of the whole history, then the one
    // pass, with the maxima as reference (no restart: every exponent is at most log2 127) ----
    const int n_unmasked = (off + t0 + 1) / kKt;   // tiles before the first query's diagonal
    float lm[QB];
#pragma unroll
    for (int b = 0; b < QB; ++b) lm[b] = -__builtin_inff();
    GQA_PC(const unsigned long long ts0 = PhaseClock::cycles();)
    for (int t = 0; t < ntiles; ++t) {
      const int ahead = min(ntiles - 1 - t, kSweepDepth - 1);   // tiles copied after t so far
      if (ahead >= 2)
        wait_vm<2 * kSweepPerTile>();
      else if (ahead == 1)
        wait_vm<kSweepPerTile>();
      else
        wait_vm<0>();
      __syncthreads();   // tile t landed for every wave; every wave is done with tile t - 1
      if (t + kSweepDepth < ntiles)
        copy_k_all((t + kSweepDepth) * kKt, (t + kSweepDepth) & 3, (t + kSweepDepth) & 3);
      qk_tile(smem_addr + (t & 3) * kKTile);
      scale_tile(sk_addr + (t & 3) * kSkTile);
      float sc0[QB][8], sc1[QB][8], scale[QB];
      if (t < n_unmasked) {
        half_scores(std::false_type{}, t * kKt, 0, sc0, scale);
        half_scores(std::false_type{}, t * kKt, 1, sc1, scale);
      } else {
        half_scores(std::true_type{}, t * kKt, 0, sc0, scale);
        half_scores(std::true_type{}, t * kKt, 1, sc1, scale);
      }
#pragma unroll
      for (int b = 0; b < QB; ++b) lm[b] = fmaxf(lm[b], fmaxf(lane_max(sc0, b), lane_max(sc1, b)));
    }
#pragma unroll
    for (int b = 0; b < QB; ++b) m[b] = xor32_max(xor16_max(lm[b])) - kLog2Of127;
    __syncthreads();   // every wave is done with the sweep's buffers
    GQA_PC(pc.sweep = PhaseClock::cycles() - ts0; pc.n_sweep = ntiles;)
    main_pass(std::integral_constant<int, 1>{});
  } else if (main_pass(std::integral_constant<int, 0>{})) {
    // ---- exact column maxima over every visible key (max-only sweep), then pass 1 ----
#pragma unroll
    for (int b = 0; b < QB; ++b) m[b] = -__builtin_inff();
    for (int t = j0; t < j1; ++t) {
      copy_k_all(t * kKt, 0, 0);
      wait_vm_all();
      __syncthreads();
      qk_tile(smem_addr);
      scale_tile(sk_addr);
      float mx[QB];
      tile_max(t * kKt, mx);
#pragma unroll
      for (int b = 0; b < QB; ++b) m[b] = fmaxf(m[b], mx[b]);
      __syncthreads();
    }
    main_pass(std::integral_constant<int, 1>{});
  }

  agpr_fence<24>(o);
  if constexpr (INT8V) {
    // ---- epilogue: O = sV * (Vq^T Pq^T) / l -> bf16 ----
    float inv[QB];
#pragma unroll
    for (int b = 0; b < QB; ++b) inv[b] = 1.0f / (float)lacc[b][0];
    if (tok_ok) {
#pragma unroll
      for (int db = 0; db < 16; ++db) {
        const f32x4 sv = *reinterpret_cast<const f32x4*>(p.vs + g * kD + 16 * db + 4 * L);
#pragma unroll
        for (int b = 0; b < QB; ++b) {
          f32x4 y;
#pragma unroll
          for (int r = 0; r < 4; ++r) y[r] = (float)o[db][b][r] * sv[r] * inv[b];
          uint8_t* orow = p.out + ((size_t)tok * kHq + head0 + b) * kD * 2;
          *reinterpret_cast<bf16x4*>(orow + (16 * db + 4 * L) * 2) = __builtin_convertvector(y, bf16x4);
        }
      }
    }
  } else {
    if (unit.nseg > 1) {
      // ---- epilogue of one KV segment: unnormalised O, the reference maximum (log2
      // units, scale included) and the row sum, merged by merge_segments_kernel ----
      if (tok_ok) {
        const size_t row0 = (seg * ws_rows + (tok - q0)) * kHq + head0;
#pragma unroll
        for (int b = 0; b < QB; ++b) {
          float* orow = p.ws_o + (row0 + b) * kD;
#pragma unroll
          for (int db = 0; db < 16; ++db) *reinterpret_cast<f32x4*>(orow + 16 * db + 4 * L) = o[db][b];
          if (L == 0) *reinterpret_cast<float2*>(p.ws_ml + (row0 + b) * 2) = make_float2(m[b], lacc[b][0]);
        }
      }
      return;
    }
    // ---- epilogue: O / l -> bf16 ----
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      const float inv = 1.0f / lacc[b][0];
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
}

template <bool PAGED, bool INT8K, int QB, bool INT8V = false>
__global__ __launch_bounds__(kThreads, 1) void gqa_prefill_kernel(const Params p) {
  using S = Shape<QB>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[lds_bytes<PAGED, INT8K, QB, INT8V>()];
  if constexpr (INT8V) {
    run<false, true, QB, false, true>(p, smem);   // P codes carry no low part
  } else {
    const int t0 = unit_of<QB>(p, blockIdx.x).tblk * S::kTokPerWg;
    if (p.kv_len - p.q_len + t0 + 1 < kSplitBelow)
      run<PAGED, INT8K, QB, true>(p, smem);
    else
      run<PAGED, INT8K, QB, false>(p, smem);
  }
}

// ---- merge of KV segments ----
// Each segment took its exponentials against its own reference maximum m_s (log2
// units) and left unnormalised O_s and the row sum l_s. With M the largest m_s,
//   out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s,
// the softmax over the whole history (a segment with l_s = 0 has no keys and weight 0).
// Long histories are cut into segments the same way for decode attention and for
// chunked prefill on the pages ("gfx936 DCU上实现INT8 QK MMAC" §4).
//
// Grid (output row = (token, head), 64-feature quarter of the row); the 4 waves of a
// workgroup take every 4th segment, a lane one feature, so even a single decode token
// (24 rows, up to 64 segments) keeps 384 waves loading independently; the waves' sums
// meet in LDS. Loads are unconditional (the workspace holds n_seg full rows) and an
// empty segment's contribution is dropped by a select, so whatever its O_s holds never
// reaches the result.
constexpr int kMergeBatch = 16;   // segments per wave loaded at once (up to 64 segments)
__global__ __launch_bounds__(256) void merge_segments_kernel(const float* ws_o, const float* ws_ml,
                                                             int n_seg, int64_t rows, uint8_t* out) {
  const int64_t row = blockIdx.x;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int f = blockIdx.y * 64 + lane;
  const float2* ml = reinterpret_cast<const float2*>(ws_ml);
  float mmax = -__builtin_inff();
  float acc = 0.0f, lsum = 0.0f;
  if (n_seg <= 4 * kMergeBatch) {
    // every load of the workgroup issued before any arithmetic (one round trip to memory
    // instead of one per batch of the loop below), then the same sums in the same order;
    // indices past n_seg load segment 0 and are not used
    float2 mv[kMergeBatch];
    float ov[kMergeBatch];
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      const int sg = wv + 4 * i < n_seg ? wv + 4 * i : 0;
      mv[i] = ml[sg * rows + row];
      ov[i] = ws_o[(size_t)(sg * rows + row) * kD + f];
    }
    const float2 vm = ml[(lane < n_seg ? lane : 0) * rows + row];
    if (lane < n_seg) mmax = vm.y > 0.0f ? fmaxf(mmax, vm.x) : mmax;
    for (int x = 32; x >= 1; x >>= 1) mmax = fmaxf(mmax, __shfl_xor(mmax, x));
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      if (wv + 4 * i < n_seg) {
        const float2 v = mv[i];
        const float o = ov[i];
        const bool used = v.y > 0.0f;
        const float wgt = __builtin_amdgcn_exp2f(v.x - mmax);
        acc += used ? wgt * o : 0.0f;
        lsum += used ? wgt * v.y : 0.0f;
      }
    }
  } else {
    for (int sg = lane; sg < n_seg; sg += 64) {
      const float2 v = ml[sg * rows + row];
      mmax = v.y > 0.0f ? fmaxf(mmax, v.x) : mmax;
    }
    for (int x = 32; x >= 1; x >>= 1) mmax = fmaxf(mmax, __shfl_xor(mmax, x));
#pragma unroll 4
    for (int sg = wv; sg < n_seg; sg += 4) {
      const float2 v = ml[sg * rows + row];
      const float o = ws_o[(size_t)(sg * rows + row) * kD + f];
      const bool used = v.y > 0.0f;
      const float wgt = __builtin_amdgcn_exp2f(v.x - mmax);
      acc += used ? wgt * o : 0.0f;
      lsum += used ? wgt * v.y : 0.0f;
    }
  }
  __shared__ float part[4][64];
  __shared__ float lpart[4];
  part[wv][lane] = acc;
  if (lane == 0) lpart[wv] = lsum;
  __syncthreads();
  if (wv == 0) {
    const float total = part[0][lane] + part[1][lane] + part[2][lane] + part[3][lane];
    const float l = lpart[0] + lpart[1] + lpart[2] + lpart[3];
    reinterpret_cast<__bf16*>(out)[(size_t)row * kD + f] = (__bf16)(total * (1.0f / l));
  }
}

// The same merge for many output rows (a prefill chunk cut into a few segments), where a
// workgroup per row quarter would spend more time starting than loading: one wave per
// row, a lane four features, so each segment's part of the row is one contiguous KiB.
// The segments are summed in order.
__global__ __launch_bounds__(256) void merge_rows_kernel(const float* ws_o, const float* ws_ml,
                                                         int n_seg, int64_t rows, uint8_t* out) {
  const int64_t row = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float2* ml = reinterpret_cast<const float2*>(ws_ml);
  float mmax = -__builtin_inff();
  for (int sg = 0; sg < n_seg; ++sg) {
    const float2 v = ml[sg * rows + row];
    mmax = v.y > 0.0f ? fmaxf(mmax, v.x) : mmax;
  }
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  float lsum = 0.0f;
  for (int sg = 0; sg < n_seg; ++sg) {
    const float2 v = ml[sg * rows + row];
    const f32x4 o = *reinterpret_cast<const f32x4*>(ws_o + (size_t)(sg * rows + row) * kD + 4 * lane);
    const bool used = v.y > 0.0f;
    const float wgt = __builtin_amdgcn_exp2f(v.x - mmax);
    acc += used ? wgt * o : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    lsum += used ? wgt * v.y : 0.0f;
  }
  const bf16x4 y = __builtin_convertvector(acc * (1.0f / lsum), bf16x4);
  *reinterpret_cast<bf16x4*>(out + ((size_t)row * kD + 4 * lane) * 2) = y;
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

// ---- standalone V quantiser for INT8 values: codes per (KV head, feature) column ----
// The per-row rule of the Q/K quantiser (float32 max|x| / 127 by IEEE division,
// round-half-even of x / s, clamp to [-127, 127], a zero column gives s = 0) applied to
// each column of V along the tokens. A workgroup per (KV head, 64-feature block): the
// column maxima over all tokens (wave w takes every 4th token, a lane one feature), then
// the codes, written feature-major [4, 256, ld] through an LDS tile of 64 tokens x 64
// features so that each feature row is written 16 bytes at a time; positions kv_len ..
// ld - 1 get code 0. A producer-side step, outside the attention call.
__global__ __launch_bounds__(256) void quantize_v_kernel(const uint8_t* v, int32_t kv_len, int32_t ld,
                                                         int8_t* vq, float* vs) {
  const int g = blockIdx.x >> 2, fb = blockIdx.x & 3;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int f = 64 * fb + lane;
  const __bf16* vb = reinterpret_cast<const __bf16*>(v);
  __shared__ float part[4][64];
  __shared__ __attribute__((aligned(16))) int8_t tile[64][80];
  float amax = 0.0f;
  for (int t = w; t < kv_len; t += 4) amax = fmaxf(amax, fabsf((float)vb[((size_t)t * kHkv + g) * kD + f]));
  part[w][lane] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(part[0][lane], part[1][lane]), fmaxf(part[2][lane], part[3][lane]));
  const float s = amax / 127.0f;
  if (w == 0) vs[g * kD + f] = s;
  const int r = threadIdx.x >> 2, qd = threadIdx.x & 3;   // writer: feature row r, 16-token chunk qd
  for (int t0 = 0; t0 < ld; t0 += 64) {
#pragma unroll 4
    for (int i = 0; i < 16; ++i) {
      const int t = t0 + 16 * w + i;
      const float x = t < kv_len ? (float)vb[((size_t)t * kHkv + g) * kD + f] : 0.0f;
      float c = (s == 0.0f) ? 0.0f : __builtin_rintf(x / s);
      c = fminf(fmaxf(c, -127.0f), 127.0f);
      tile[lane][16 * w + i] = (int8_t)(int)c;
    }
    __syncthreads();
    const int t = t0 + 16 * qd;
    if (t < ld)
      *reinterpret_cast<uint4*>(vq + ((size_t)g * kD + 64 * fb + r) * ld + t) =
          *reinterpret_cast<const uint4*>(&tile[r][16 * qd]);
    __syncthreads();
  }
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
  int tok_per_wg;
  int n_tblk;
  int per_tblk;      // workgroups per (KV head, token block): 1, or 3 with 2 heads each
  int workgroups;
  int threads;
  int lds_bytes;
};

constexpr int kDefaultQB = GQA_DEFAULT_QB;

template <int QB>
Launch shape_launch(int32_t q_len, bool int8k, bool int8v = false) {
  using S = Shape<QB>;
  const int n_tblk = (q_len + S::kTokPerWg - 1) / S::kTokPerWg;
  Launch lc;
  lc.qb = QB;
  lc.tok_per_wg = S::kTokPerWg;
  lc.n_tblk = n_tblk;
  lc.per_tblk = S::kSplitsPerGroup;
  lc.workgroups = n_tblk * kHkv * S::kSplitsPerGroup;
  lc.threads = kThreads;
  lc.lds_bytes = int8v ? lds_bytes<false, true, QB, true>()
                      : (int8k ? lds_bytes<false, true, QB>() : lds_bytes<false, false, QB>());
  return lc;
}

constexpr int kCUs = 256;        // compute units of an MI355X
constexpr int kMinSegTiles = 512 / kKt;  // shortest KV segment (512 keys)
constexpr double kTileSeconds = 2.4e-6 * kKt / 64;   // about one workgroup's time per tile

// Estimated run time, in tile times (one workgroup through one 64-key tile), of a launch
// that cuts every (KV head, token block) into n_seg KV segments. The workgroups run
// longest first, one per compute unit, so they go in rounds of kCUs and each round
// lasts about as long as its first (longest) workgroup; each workgroup also pays about
// two tile times of prologue and epilogue; and a split launch moves n_seg partial rows
// of 1 KiB + 8 B per output row through memory twice (written, then read by the merge)
// at about 5 TB/s, against the ~2.4 us a workgroup spends on one tile.
double plan_cost(int32_t q_len, int32_t kv_len, int tok, int n_tblk, int n_seg) {
  constexpr double kWgTiles = 2.0;
  const int64_t pieces = (int64_t)kHkv * n_tblk * n_seg;
  double t = 0.0;
  for (int64_t first = 0; first < pieces; first += kCUs) {
    const int64_t tblk = n_tblk - 1 - first / n_seg / kHkv;   // grid order: longest first
    const int64_t last = std::min<int64_t>((tblk + 1) * tok, q_len);
    const int64_t T = ((int64_t)kv_len - q_len + last + kKt - 1) / kKt;
    t += (double)((T + n_seg - 1) / n_seg) + kWgTiles;
  }
  if (n_seg > 1) t += 2.0 * n_seg * (double)q_len * kHq * (kD + 2) * 4 / (5e12 * kTileSeconds);
  return t;
}

// KV segments per (KV head, token block) for a small grid: when the grid has fewer
// workgroups than the 256 CUs, every token block is cut the same way, into the count
// with the lowest plan_cost among those that keep every segment at least kMinSegTiles
// long in the shortest (first) token block.
int uniform_segments(int32_t q_len, int32_t kv_len, const Launch& lc) {
  const int tok = lc.tok_per_wg;
  const int n_tblk = lc.n_tblk;
  const int64_t t_min = ((int64_t)kv_len - q_len + std::min(q_len, tok) + kKt - 1) / kKt;
  int best = 1;
  double best_cost = plan_cost(q_len, kv_len, tok, n_tblk, 1);
  static const int kCandidates[] = {2, 3, 4, 5, 6, 8, 10, 12, 16, 24, 32, 48, 64};
  for (int n : kCandidates) {
    if (t_min / n < kMinSegTiles) break;
    const double c = plan_cost(q_len, kv_len, tok, n_tblk, n);
    if (c < 0.97 * best_cost) {   // split only for a clear gain
      best = n;
      best_cost = c;
    }
  }
  return best;
}

// How a call with a workspace is cut: every token block at or past n_plain into n_seg
// KV segments (n_seg = 1: nothing is cut).
struct SegPlan {
  int n_seg = 1;
  int n_plain = 0;
};

int64_t tblk_tiles(int32_t q_len, int32_t kv_len, int tok, int64_t t) {
  const int64_t last = std::min<int64_t>((t + 1) * tok, q_len);
  return ((int64_t)kv_len - q_len + last + kKt - 1) / kKt;
}

// Estimated run time of a plan for a grid of at least one workgroup per CU, in tile
// times. Workgroups go round-robin to the 8 XCDs (workgroup id mod 8), so the two XCDs
// that serve a KV head (id mod 4) take its work units alternately, and inside an XCD
// each unit starts on the first of the 32 CUs to become free, in grid order. Each
// workgroup adds about two tile times of prologue and epilogue, and the split rows pass
// through the workspace and the merge (as in plan_cost).
double plan_makespan(int32_t q_len, int32_t kv_len, const Launch& lc, const SegPlan& sp) {
  constexpr int kCUsPerXcd = 32;
  constexpr double kWgTiles = 2.0;
  double free_at[2][kCUsPerXcd] = {};
  double span = 0.0;
  int64_t k = 0;
  auto place = [&](double len) {
    double* cu = free_at[k & 1];
    int first = 0;
    for (int i = 1; i < kCUsPerXcd; ++i)
      if (cu[i] < cu[first]) first = i;
    cu[first] += len + kWgTiles;
    span = std::max(span, cu[first]);
    ++k;
  };
  const int tok = lc.tok_per_wg;
  const int64_t whole = sp.n_seg > 1 ? sp.n_plain : lc.n_tblk;   // token blocks run whole
  for (int64_t t = whole - 1; t >= 0; --t)
    for (int h = 0; h < lc.per_tblk; ++h) place((double)tblk_tiles(q_len, kv_len, tok, t));
  if (sp.n_seg > 1) {
    for (int64_t t = lc.n_tblk - 1; t >= sp.n_plain; --t) {
      const int64_t T = tblk_tiles(q_len, kv_len, tok, t);
      for (int h = 0; h < lc.per_tblk; ++h)
        for (int sg = 0; sg < sp.n_seg; ++sg)
          place((double)(T * (sg + 1) / sp.n_seg - T * sg / sp.n_seg));
    }
    const int64_t split_rows = (int64_t)q_len - (int64_t)sp.n_plain * tok;
    span += 2.0 * sp.n_seg * (double)split_rows * kHq * (kD + 2) * 4 / (5e12 * kTileSeconds);
  }
  return span;
}

// The cut for a call that has a workspace. A grid with fewer workgroups than CUs is cut
// uniformly (uniform_segments). A larger grid whose last round of workgroups would
// leave CUs idle (384 workgroups on 256 CUs run in 1.5 rounds) has its longest token
// blocks cut into 2 to 4 segments, as many as make the work units a whole number of
// rounds (64 per KV head), when plan_makespan says that is clearly faster. Every
// segment is at least kMinSegTiles long and every segment of a split token block starts
// at or before the block's first query (its first key is visible to every query).
SegPlan segments_for(int32_t q_len, int32_t kv_len, const Launch& lc) {
  SegPlan best;
  if (q_len == 0) return best;
  if (lc.workgroups < kCUs) {
    best.n_seg = uniform_segments(q_len, kv_len, lc);
    return best;
  }
  constexpr int kUnitsPerRound = kCUs / kHkv;   // work units of one KV head per round
  const int64_t units = (int64_t)lc.n_tblk * lc.per_tblk;
  if (units % kUnitsPerRound == 0 || lc.n_tblk > 512) return best;
  double best_cost = plan_makespan(q_len, kv_len, lc, best);
  const int64_t k0 = (units + kUnitsPerRound - 1) / kUnitsPerRound;
  for (int S = 2; S <= 4; ++S) {
    for (int64_t k = k0; k <= k0 + 2; ++k) {
      // units - n_split * per_tblk + n_split * per_tblk * S = k rounds
      const int64_t extra = k * kUnitsPerRound - units;
      const int64_t step = (int64_t)(S - 1) * lc.per_tblk;
      if (extra % step != 0) continue;
      const int64_t n_split = extra / step;
      if (n_split < 1 || n_split >= lc.n_tblk) continue;
      SegPlan sp;
      sp.n_seg = S;
      sp.n_plain = (int)(lc.n_tblk - n_split);
      // the shortest split token block: segments long enough, and starting in the history
      const int64_t T = tblk_tiles(q_len, kv_len, lc.tok_per_wg, sp.n_plain);
      const int64_t first_query = (int64_t)kv_len - q_len + (int64_t)sp.n_plain * lc.tok_per_wg;
      if (T / S < kMinSegTiles || (T * (S - 1) / S) * kKt > first_query) continue;
      const double c = plan_makespan(q_len, kv_len, lc, sp);
      if (c < 0.97 * best_cost) {
        best = sp;
        best_cost = c;
      }
    }
  }
  return best;
}

// Output rows from which the merge runs a wave per row (merge_rows_kernel: 256 rows
// already give every compute unit a workgroup) instead of a workgroup per row quarter.
constexpr int64_t kMergeRowsMin = 1024;

// Tokens of a call whose rows pass through the workspace (those of the split token blocks).
int64_t split_tokens(int32_t q_len, const Launch& lc, const SegPlan& sp) {
  return sp.n_seg > 1 ? (int64_t)q_len - (int64_t)sp.n_plain * lc.tok_per_wg : 0;
}

size_t workspace_bytes_for(int32_t q_len, const Launch& lc, const SegPlan& sp) {
  if (sp.n_seg <= 1) return 0;
  return (size_t)sp.n_seg * split_tokens(q_len, lc, sp) * kHq * (kD + 2) * sizeof(float);
}

int64_t grid_workgroups(const Launch& lc, const SegPlan& sp) {
  return (int64_t)kHkv * lc.per_tblk *
         (sp.n_plain + (int64_t)(lc.n_tblk - sp.n_plain) * sp.n_seg);
}

// Chunks of at most this many query tokens run the decode shape (4 tokens x 6 heads
// per workgroup, a token per wave) instead of 32 tokens x 6 heads.
constexpr int kDecodeMaxQ = 4;

// Dispatch rule (the analogue of the pages' q_len/kv_len-gated variant choice, and of
// their separate decode and prefill row mappings): one kernel family; the shape of the
// query block is the only parameter.
Launch plan_for(int32_t q_len, int32_t kv_len, bool paged, bool int8k) {
  (void)kv_len;
  const bool dec = q_len <= kDecodeMaxQ;
  Launch lc = dec ? shape_launch<1>(q_len, int8k) : shape_launch<kDefaultQB>(q_len, int8k);
#define GQA_KT_NAME_(x) "_kt" #x
#define GQA_KT_NAME(x) GQA_KT_NAME_(x)
  static const char* const kNames[4][3] = {
      // decode, 32 tokens x 6 heads, 64 tokens x 2 heads
      {"bf16_contiguous_decode_t4h6" GQA_KT_NAME(GQA_KT), "bf16_contiguous_t32h6" GQA_KT_NAME(GQA_KT),
       "bf16_contiguous_t64h2" GQA_KT_NAME(GQA_KT)},
      {"bf16_paged_decode_t4h6" GQA_KT_NAME(GQA_KT), "bf16_paged_t32h6" GQA_KT_NAME(GQA_KT),
       "bf16_paged_t64h2" GQA_KT_NAME(GQA_KT)},
      {"int8k_contiguous_decode_t4h6" GQA_KT_NAME(GQA_KT), "int8k_contiguous_t32h6" GQA_KT_NAME(GQA_KT),
       "int8k_contiguous_t64h2" GQA_KT_NAME(GQA_KT)},
      {"int8k_paged_splitd_decode_t4h6" GQA_KT_NAME(GQA_KT), "int8k_paged_splitd_t32h6" GQA_KT_NAME(GQA_KT),
       "int8k_paged_splitd_t64h2" GQA_KT_NAME(GQA_KT)}};
  lc.name = kNames[(int8k ? 2 : 0) + (paged ? 1 : 0)][dec ? 0 : (lc.qb == 3 ? 1 : 2)];
  return lc;
}

// INT8 values: contiguous INT8 keys, the prefill shape at every q_len (no decode shape),
// the whole history in one piece
Launch plan_int8kv(int32_t q_len) {
  Launch lc = shape_launch<kDefaultQB>(q_len, true, true);
  lc.name = lc.qb == 3 ? "int8kv_contiguous_t32h6" GQA_KT_NAME(GQA_KT) : "int8kv_contiguous_t64h2" GQA_KT_NAME(GQA_KT);
  return lc;
}

int check_int8kv_lengths(int32_t q_len, int32_t kv_len) {
  const int st = check_prefill_lengths(q_len, kv_len);
  if (st != GQA_OK) return st;
  if (kKt != 64 || kv_len > GQA_INT8KV_MAX_KV) return GQA_ERR_UNSUPPORTED;
  return GQA_OK;
}

int scratch_on(hipStream_t stream, void** ptr);

// Shared by the entry points; `allow_split` is false for the call without a workspace,
// `q_scale` is set (and q holds int8 codes) only for the call with Q quantised beforehand,
// `noalloc` takes the workspace from the library's scratch array instead of the caller
// (after every argument check, so a refused call touches no device).
int prefill(const void* q, const float* q_scale, const void* k, const void* v,
            const int32_t* block_table, int32_t num_blocks, const float* k_scale, int32_t q_len,
            int32_t kv_len, void* out, void* workspace, size_t workspace_bytes, bool allow_split,
            void* stream, bool noalloc = false) {
  int st = check_prefill_lengths(q_len, kv_len);
  if (st != GQA_OK) return st;
  if (q_len == 0) return GQA_OK;
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return GQA_ERR_NULL_ARG;
  const bool paged = block_table != nullptr;
  const bool int8k = k_scale != nullptr;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return GQA_ERR_MISALIGNED;
  if (paged && !aligned(block_table, 4)) return GQA_ERR_MISALIGNED;
  if (kKt != 64 && paged && int8k) return GQA_ERR_UNSUPPORTED;   // page-major INT8 tiles are 64 keys
  if (int8k && !aligned(k_scale, 4)) return GQA_ERR_MISALIGNED;
  if (q_scale != nullptr && !aligned(q_scale, 4)) return GQA_ERR_MISALIGNED;
  if (paged) {
    const int64_t need = ((int64_t)kv_len + kBs - 1) / kBs;
    if (num_blocks < need || num_blocks <= 0) return GQA_ERR_BAD_LENGTH;
  }
  const Launch lc = plan_for(q_len, kv_len, paged, int8k);
  const SegPlan sp = allow_split ? segments_for(q_len, kv_len, lc) : SegPlan{};
  const int n_seg = sp.n_seg;
  const size_t ws_need = workspace_bytes_for(q_len, lc, sp);
  if (noalloc && n_seg > 1) {
    if (ws_need > (size_t)GQA_NOALLOC_SCRATCH_BYTES) return GQA_ERR_SCRATCH;
    st = scratch_on(static_cast<hipStream_t>(stream), &workspace);
    if (st != GQA_OK) return st;
    workspace_bytes = GQA_NOALLOC_SCRATCH_BYTES;
  }
  if (n_seg > 1) {
    if (workspace == nullptr || workspace_bytes < ws_need) return GQA_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return GQA_ERR_MISALIGNED;
  }

  Params p;
  p.q = static_cast<const uint8_t*>(q);
  p.qsc = q_scale;
  p.k = static_cast<const uint8_t*>(k);
  p.v = static_cast<const uint8_t*>(v);
  p.bt = block_table;
  p.ks = k_scale;
  p.out = static_cast<uint8_t*>(out);
  p.num_blocks = paged ? num_blocks : 0;
  p.q_len = q_len;
  p.kv_len = kv_len;
  p.n_tblk = lc.n_tblk;
  p.n_seg = n_seg;
  p.n_plain = sp.n_plain;
  const int64_t split_tok = split_tokens(q_len, lc, sp);
  p.ws_o = n_seg > 1 ? static_cast<float*>(workspace) : nullptr;
  p.ws_ml = n_seg > 1 ? p.ws_o + (size_t)n_seg * split_tok * kHq * kD : nullptr;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)grid_workgroups(lc, sp)), block(lc.threads);
  auto launch = [&](auto qb_c) {
    constexpr int QB = decltype(qb_c)::value;
    if (int8k && paged)
      hipLaunchKernelGGL((gqa_prefill_kernel<true, true, QB>), grid, block, 0, s, p);
    else if (int8k)
      hipLaunchKernelGGL((gqa_prefill_kernel<false, true, QB>), grid, block, 0, s, p);
    else if (paged)
      hipLaunchKernelGGL((gqa_prefill_kernel<true, false, QB>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((gqa_prefill_kernel<false, false, QB>), grid, block, 0, s, p);
  };
  if (lc.qb == 1)
    launch(std::integral_constant<int, 1>{});
  else
    launch(std::integral_constant<int, kDefaultQB>{});
  if (hipGetLastError() != hipSuccess) return GQA_ERR_HIP;
  if (n_seg > 1) {
    // the split token blocks' rows: the last split_tok tokens of the chunk
    const int64_t rows = split_tok * kHq;
    uint8_t* out_split = p.out + (size_t)(q_len - split_tok) * kHq * kD * 2;
    if (rows >= kMergeRowsMin)
      hipLaunchKernelGGL(merge_rows_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s,
                         p.ws_o, p.ws_ml, n_seg, rows, out_split);
    else
      hipLaunchKernelGGL(merge_segments_kernel, dim3((unsigned)rows, kD / 64), dim3(256), 0, s,
                         p.ws_o, p.ws_ml, n_seg, rows, out_split);
    if (hipGetLastError() != hipSuccess) return GQA_ERR_HIP;
  }
  return GQA_OK;
}

// The address of the GPU's copy of `scratch` for a call on `stream` (its device; the
// current device for the null stream). Taken once per device, with that device current,
// and kept: the array lives as long as the process.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_on(hipStream_t stream, void** ptr) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return GQA_ERR_HIP;
  int dev = cur;
  if (stream != nullptr && hipStreamGetDevice(stream, &dev) != hipSuccess) return GQA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return GQA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return GQA_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return GQA_ERR_HIP;
    if (e != hipSuccess || p == nullptr) return GQA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return GQA_OK;
}

}  // namespace

extern "C" {

#ifdef GQA_PHASE_CLOCK
// the measurement build's per-wave phase clock of the last launch, copied to host memory
int gqa_phase_clock_read(void* host, size_t bytes) {
  if (host == nullptr || bytes > sizeof(phase_clock)) return GQA_ERR_BAD_LENGTH;
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(phase_clock), bytes, 0, hipMemcpyDeviceToHost) == hipSuccess
             ? GQA_OK
             : GQA_ERR_HIP;
}
#endif

int gqa_abi_version(void) { return GQA_ABI_VERSION; }

const char* gqa_status_string(int status) {
  switch (status) {
    case GQA_OK: return "ok";
    case GQA_ERR_NULL_ARG: return "a required pointer is NULL";
    case GQA_ERR_BAD_LENGTH: return "invalid length (need 0 <= q_len <= kv_len <= GQA_MAX_LEN, rows >= 0, enough blocks)";
    case GQA_ERR_MISALIGNED: return "a tensor pointer is misaligned";
    case GQA_ERR_UNSUPPORTED: return "unsupported combination of arguments";
    case GQA_ERR_HIP: return "HIP launch failed";
    case GQA_ERR_WORKSPACE: return "workspace missing or smaller than gqa_attn_prefill_workspace_size()";
    case GQA_ERR_SCRATCH:
      return "gqa_attn_prefill_noalloc: the call needs more than GQA_NOALLOC_SCRATCH_BYTES of scratch";
    default: return "unknown status";
  }
}

int gqa_attn_prefill_plan(int32_t q_len, int32_t kv_len, int paged, int int8k, char* buf, size_t n) {
  if (buf == nullptr || n == 0) return GQA_ERR_NULL_ARG;
  int st = check_prefill_lengths(q_len, kv_len);
  if (st != GQA_OK) {
    snprintf(buf, n, "error: %s", gqa_status_string(st));
    return st;
  }
  if (int8k == 2) {   // INT8 values: contiguous only, one piece
    st = paged ? GQA_ERR_UNSUPPORTED : check_int8kv_lengths(q_len, kv_len);
    if (st != GQA_OK) {
      snprintf(buf, n, "error: %s", gqa_status_string(st));
      return st;
    }
    const Launch lc = plan_int8kv(q_len);
    snprintf(buf, n,
             "variant=%s workgroups=%d threads=%d lds_bytes=%d segments=1 whole_token_blocks=%d "
             "workspace_bytes=0",
             lc.name, lc.workgroups, lc.threads, lc.lds_bytes, lc.n_tblk);
    return GQA_OK;
  }
  const Launch lc = plan_for(q_len, kv_len, paged != 0, int8k != 0);
  const SegPlan sp = segments_for(q_len, kv_len, lc);
  snprintf(buf, n,
           "variant=%s workgroups=%lld threads=%d lds_bytes=%d segments=%d whole_token_blocks=%d "
           "workspace_bytes=%zu",
           lc.name, (long long)grid_workgroups(lc, sp), lc.threads, lc.lds_bytes, sp.n_seg,
           sp.n_seg > 1 ? sp.n_plain : lc.n_tblk, workspace_bytes_for(q_len, lc, sp));
  return GQA_OK;
}

size_t gqa_attn_prefill_workspace_size(int32_t q_len, int32_t kv_len, int paged, int int8k) {
  if (check_prefill_lengths(q_len, kv_len) != GQA_OK || int8k == 2) return 0;
  const Launch lc = plan_for(q_len, kv_len, paged != 0, int8k != 0);
  return workspace_bytes_for(q_len, lc, segments_for(q_len, kv_len, lc));
}

int gqa_attn_prefill(const void* q, const void* k, const void* v, const int32_t* block_table,
                     int32_t num_blocks, const float* k_scale, int32_t q_len, int32_t kv_len,
                     void* out, void* stream) {
  return prefill(q, nullptr, k, v, block_table, num_blocks, k_scale, q_len, kv_len, out, nullptr, 0,
                 false, stream);
}

int gqa_attn_prefill_ws(const void* q, const void* k, const void* v, const int32_t* block_table,
                        int32_t num_blocks, const float* k_scale, int32_t q_len, int32_t kv_len,
                        void* out, void* workspace, size_t workspace_bytes, void* stream) {
  return prefill(q, nullptr, k, v, block_table, num_blocks, k_scale, q_len, kv_len, out, workspace,
                 workspace_bytes, true, stream);
}

int gqa_attn_prefill_noalloc(const void* q, const void* k, const void* v,
                             const int32_t* block_table, int32_t num_blocks, const float* k_scale,
                             int32_t q_len, int32_t kv_len, void* out, void* stream) {
  return prefill(q, nullptr, k, v, block_table, num_blocks, k_scale, q_len, kv_len, out, nullptr, 0,
                 true, stream, /*noalloc=*/true);
}

int gqa_attn_prefill_qint8(const void* q_codes, const float* q_scale, const void* k, const void* v,
                           const int32_t* block_table, int32_t num_blocks, const float* k_scale,
                           int32_t q_len, int32_t kv_len, void* out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  const int st = check_prefill_lengths(q_len, kv_len);
  if (st != GQA_OK || q_len == 0) return st;
  if (q_scale == nullptr || k_scale == nullptr) return GQA_ERR_NULL_ARG;
  return prefill(q_codes, q_scale, k, v, block_table, num_blocks, k_scale, q_len, kv_len, out,
                 workspace, workspace_bytes, true, stream);
}

int gqa_attn_prefill_int8kv(const void* q, const float* q_scale, const void* k, const float* k_scale,
                            const void* v_codes, const float* v_scale, int32_t v_ld, int32_t q_len,
                            int32_t kv_len, void* out, void* stream) {
  int st = check_prefill_lengths(q_len, kv_len);
  if (st != GQA_OK) return st;
  if (q_len == 0) return GQA_OK;
  if (v_ld < kv_len || v_ld > GQA_MAX_LEN || (v_ld & 15) != 0) return GQA_ERR_BAD_LENGTH;
  if (q == nullptr || k == nullptr || k_scale == nullptr || v_codes == nullptr || v_scale == nullptr ||
      out == nullptr)
    return GQA_ERR_NULL_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v_codes, 16) || !aligned(out, 16) ||
      !aligned(k_scale, 4) || !aligned(v_scale, 16) || (q_scale != nullptr && !aligned(q_scale, 4)))
    return GQA_ERR_MISALIGNED;
  st = check_int8kv_lengths(q_len, kv_len);
  if (st != GQA_OK) return st;
  const Launch lc = plan_int8kv(q_len);
  Params p;
  p.q = static_cast<const uint8_t*>(q);
  p.qsc = q_scale;
  p.k = static_cast<const uint8_t*>(k);
  p.v = static_cast<const uint8_t*>(v_codes);
  p.bt = nullptr;
  p.ks = k_scale;
  p.out = static_cast<uint8_t*>(out);
  p.num_blocks = 0;
  p.q_len = q_len;
  p.kv_len = kv_len;
  p.n_tblk = lc.n_tblk;
  p.n_seg = 1;
  p.n_plain = 0;
  p.ws_o = nullptr;
  p.ws_ml = nullptr;
  p.vs = v_scale;
  p.v_ld = v_ld;
  if constexpr (kKt == 64) {   // the INT8-value kernel is built for 64-key tiles only
    hipLaunchKernelGGL((gqa_prefill_kernel<false, true, kDefaultQB, true>), dim3((unsigned)lc.workgroups),
                       dim3(lc.threads), 0, static_cast<hipStream_t>(stream), p);
    return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_HIP;
  } else {
    return GQA_ERR_UNSUPPORTED;
  }
}

int gqa_quantize_v_int8(const void* v, int32_t kv_len, int32_t v_ld, void* v_codes, float* v_scale,
                        void* stream) {
  if (kv_len < 0 || kv_len > GQA_MAX_LEN || v_ld < kv_len || v_ld > GQA_MAX_LEN || (v_ld & 15) != 0)
    return GQA_ERR_BAD_LENGTH;
  if (v_codes == nullptr || v_scale == nullptr || (kv_len > 0 && v == nullptr)) return GQA_ERR_NULL_ARG;
  if (!aligned(v, 16) || !aligned(v_codes, 16) || !aligned(v_scale, 4)) return GQA_ERR_MISALIGNED;
  hipLaunchKernelGGL(quantize_v_kernel, dim3(kHkv * kD / 64), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint8_t*>(v), kv_len, v_ld, static_cast<int8_t*>(v_codes), v_scale);
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
