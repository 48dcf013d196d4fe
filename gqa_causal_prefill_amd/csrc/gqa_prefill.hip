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
// Work decomposition (one design for gfx950, not the pages' Triton tiling):
//   * one workgroup = 4 wave64s = one KV head g x a pair of its query heads x
//     64 query tokens (128 query rows), so every K/V tile staged in LDS serves
//     128 rows of the GQA group ([DCU report §2, §4]: a program covers tokens x
//     heads of one group and the reuse of each K/V tile grows with the rows per
//     program). The three head pairs of a group are three workgroups;
//   * each wave owns 16 tokens x 2 heads = 32 rows, as two 16-column blocks of
//     the 16x16 MFMA output (block b = head, column c = token); scores are
//     computed transposed (S^T = K·Q^T) so every lane holds keys of ONE query
//     column and the softmax reductions are mostly lane-local;
//   * the loop walks KV tiles of 32 keys; K is staged row-major with an XOR
//     swizzle, V is staged transposed (V^T) so it can feed the A operand of the
//     P·V MFMA, both double-buffered through registers;
//   * online softmax in the exp2 domain with a lazy rescale: the running max
//     used for the exponentials only moves when a tile raises it by more than
//     2^8, which keeps every exponent <= 2^8 and skips almost every rescale of
//     the 192 accumulator registers (the result is the same softmax);
//   * P is rounded to bf16 for the MFMA and the row sums use the rounded values.
//     Workgroups whose first query sees fewer than 256 keys (short histories,
//     where few keys carry large weights) multiply with P split into a bf16
//     high part and a bf16 low part, keeping ~16 bits of P.
//   * with INT8 keys each query row is quantised in the prologue (once per row,
//     [INT8 QK §4]) and Q·K^T runs on v_mfma_i32_16x16x64_i8; the int32 score is
//     scaled by sQ·sK·log2(e)/16 per score before the softmax ([INT8 QK §1]).

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include "gqa_prefill.h"

namespace {

constexpr int kHq = GQA_NUM_Q_HEADS;     // 24
constexpr int kHkv = GQA_NUM_KV_HEADS;   // 4
constexpr int kD = GQA_HEAD_DIM;         // 256
constexpr int kGroup = kHq / kHkv;       // 6
constexpr int kBs = GQA_BLOCK_SIZE;      // 16

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTokPerWave = 16;                   // x 2 heads = 32 rows per wave
constexpr int kTokPerWg = kTokPerWave * kWaves;   // 64 tokens per workgroup
constexpr int kHeadsPerWg = 2;                    // query heads per workgroup
constexpr int kPairs = kGroup / kHeadsPerWg;      // 3 workgroups per (KV head, token block)
constexpr int kQB = kHeadsPerWg;                  // 16-column query blocks per wave
constexpr int kKt = 32;                           // keys per KV tile
constexpr int kSplitBelow = 256;
constexpr float kTau = 8.0f;
constexpr float kLog2eOver16 = 1.4426950408889634f / 16.0f;

// LDS layout (bytes)
constexpr int kKTileBf16 = kKt * kD * 2;          // 16 KiB
constexpr int kKTileI8 = kKt * kD;                // 8 KiB
constexpr int kVTile = kKt * kD * 2;              // 16 KiB (V^T)
constexpr int kSkTile = kKt * 4;                  // 128 B of key scales

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

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
  int32_t n_tblk;          // ceil(q_len / 64)
};

__device__ __forceinline__ float wave_xor_max(float x, int mask) {
  return fmaxf(x, __shfl_xor(x, mask));
}

__device__ __forceinline__ uint32_t perm_b32(uint32_t hi_src, uint32_t lo_src, uint32_t sel) {
  return __builtin_amdgcn_perm(hi_src, lo_src, sel);
}

// Byte offset of K row chunk (16 B) `chunk` of key `key` inside a staged K tile.
// XOR swizzle on the low three chunk bits: the 8 lanes of one ds_read_b128 phase
// read 8 different keys at the same logical chunk and land in 8 different
// 16-byte bank groups.
template <int ROW_BYTES>
__device__ __forceinline__ int k_lds_off(int key, int chunk) {
  return key * ROW_BYTES + ((chunk ^ (key & 7)) << 4);
}

// Byte offset of the 16-byte group `grp` (keys {4grp..4grp+3, 16+4grp..16+4grp+3})
// of V^T row `d`. Within a row (64 B = the tile's 32 keys of one feature), group
// grp holds keys 4grp..4grp+3 then 16+4grp..16+4grp+3: exactly the 8 keys one
// lane feeds to the P·V MFMA, in the order its S^T registers hold them. The
// group index is XOR-swizzled by (d >> 1) & 3 so the 8 lanes of a read phase
// (8 consecutive d) hit 8 different bank groups.
__device__ __forceinline__ int vt_lds_off(int d, int grp) {
  return d * 64 + ((grp ^ ((d >> 1) & 3)) << 4);
}

template <bool PAGED>
__device__ __forceinline__ size_t kv_row_elem(const Params& p, int g, int key, int blk) {
  if constexpr (PAGED) {
    return ((size_t)(blk * kHkv + g) * kBs + (key & (kBs - 1))) * kD;
  } else {
    return ((size_t)key * kHkv + g) * kD;
  }
}

template <bool PAGED, bool INT8K>
struct Stage {
  uint4 kreg[INT8K ? 2 : 4];
  uint2 vreg[2][4];
  float sk;
};

// Global -> registers for KV tile starting at key `kbase`.
template <bool PAGED, bool INT8K>
__device__ __forceinline__ void stage_load(const Params& p, int g, int kbase, int tid,
                                           Stage<PAGED, INT8K>& st) {
  int blk0 = 0, blk1 = 0;
  if constexpr (PAGED) {
    const int tb = kbase >> 4;
    blk0 = p.bt[tb];
    blk1 = (kbase + kBs < p.kv_len) ? p.bt[tb + 1] : blk0;
    blk0 = min(max(blk0, 0), p.num_blocks - 1);
    blk1 = min(max(blk1, 0), p.num_blocks - 1);
  }
  // K: bf16 rows are 32 chunks of 16 B (4 per thread); int8 rows are 16 chunks (2 per thread)
  constexpr int kChunks = INT8K ? 16 : 32;
  constexpr int kShift = INT8K ? 4 : 5;
  constexpr int kPer = INT8K ? 2 : 4;
  constexpr int kElem = INT8K ? 1 : 2;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int u = tid + kThreads * i;
    const int key = u >> kShift;
    const int chunk = u & (kChunks - 1);
    const int kk = kbase + key;
    if (kk < p.kv_len) {
      const size_t e = kv_row_elem<PAGED>(p, g, kk, key < kBs ? blk0 : blk1);
      st.kreg[i] = *reinterpret_cast<const uint4*>(p.k + e * kElem + chunk * 16);
    } else {
      st.kreg[i] = make_uint4(0, 0, 0, 0);
    }
  }
  // V: 2 units of 4 keys x 4 features per thread
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int kq = tid & 7;
    const int dq = (tid >> 3) + 32 * i;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = 4 * kq + r;
      const int kk = kbase + key;
      if (kk < p.kv_len) {
        const size_t e = kv_row_elem<PAGED>(p, g, kk, key < kBs ? blk0 : blk1);
        st.vreg[i][r] = *reinterpret_cast<const uint2*>(p.v + (e + 4 * dq) * 2);
      } else {
        st.vreg[i][r] = make_uint2(0, 0);
      }
    }
  }
  if constexpr (INT8K) {
    st.sk = 0.0f;
    if (tid < kKt && kbase + tid < p.kv_len) st.sk = p.ks[(size_t)(kbase + tid) * kHkv + g];
  }
}

// Registers -> LDS (K swizzled, V transposed).
template <bool PAGED, bool INT8K>
__device__ __forceinline__ void stage_store(uint8_t* kbuf, uint8_t* vtbuf, float* skbuf, int tid,
                                            const Stage<PAGED, INT8K>& st) {
  constexpr int kChunks = INT8K ? 16 : 32;
  constexpr int kShift = INT8K ? 4 : 5;
  constexpr int kPer = INT8K ? 2 : 4;
  constexpr int kRow = INT8K ? kD : 2 * kD;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int u = tid + kThreads * i;
    const int key = u >> kShift;
    const int chunk = u & (kChunks - 1);
    *reinterpret_cast<uint4*>(kbuf + k_lds_off<kRow>(key, chunk)) = st.kreg[i];
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int kq = tid & 7;
    const int dq = (tid >> 3) + 32 * i;
    const int grp = kq & 3;
    const int half = kq >> 2;
    const uint2* r = st.vreg[i];
    // 4x4 transpose of bf16: row r = key 4kq+r holding features 4dq..4dq+3
    uint2 col[4];
    col[0] = make_uint2(perm_b32(r[1].x, r[0].x, 0x05040100u), perm_b32(r[3].x, r[2].x, 0x05040100u));
    col[1] = make_uint2(perm_b32(r[1].x, r[0].x, 0x07060302u), perm_b32(r[3].x, r[2].x, 0x07060302u));
    col[2] = make_uint2(perm_b32(r[1].y, r[0].y, 0x05040100u), perm_b32(r[3].y, r[2].y, 0x05040100u));
    col[3] = make_uint2(perm_b32(r[1].y, r[0].y, 0x07060302u), perm_b32(r[3].y, r[2].y, 0x07060302u));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = 4 * dq + j;
      *reinterpret_cast<uint2*>(vtbuf + vt_lds_off(d, grp) + half * 8) = col[j];
    }
  }
  if constexpr (INT8K) {
    if (tid < kKt) skbuf[tid] = st.sk;
  }
}

template <bool PAGED, bool INT8K>
__global__ __launch_bounds__(kThreads, 1) void gqa_prefill_kernel(const Params p) {
  constexpr int kKTile = INT8K ? kKTileI8 : kKTileBf16;
  constexpr int kSk = INT8K ? kSkTile : 0;
  constexpr int kStage = kKTile + kVTile + kSk;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int L = lane >> 4;      // k-group of the MFMA operands / row group of the output
  const int c = lane & 15;      // query column (token) inside a 16-column block

  // Workgroup id -> (KV head, head pair, token block). id % 4 is the KV head, so
  // workgroups dispatched round-robin over the 8 XCDs keep one KV head per XCD
  // (its K/V stream shares that XCD's L2); token blocks go longest first.
  const int id = blockIdx.x;
  const int g = id & (kHkv - 1);
  const int rest = id >> 2;
  const int hp = rest % kPairs;
  const int tblk = p.n_tblk - 1 - rest / kPairs;
  const int t0 = tblk * kTokPerWg;
  const int off = p.kv_len - p.q_len;

  // query column (b, c) of this lane: token t0 + 16w + c, head 6g + 2hp + b
  const int tok = t0 + kTokPerWave * w + c;
  const bool tok_ok = tok < p.q_len;
  const int limit = off + tok;   // last visible key of this column

  const int last_tok = min(t0 + kTokPerWg, p.q_len);
  const int n_keys = off + last_tok;
  const int ntiles = (n_keys + kKt - 1) / kKt;
  const bool split = (off + t0 + 1) < kSplitBelow;

  // ---- prologue: Q fragments (B operand of S^T = K·Q^T) ----
  bf16x8 qf[INT8K ? 1 : kQB][INT8K ? 1 : 8];
  i32x4 qq[INT8K ? kQB : 1][INT8K ? 4 : 1];
  float qs[kQB];
#pragma unroll
  for (int b = 0; b < kQB; ++b) {
    const int head = kGroup * g + kHeadsPerWg * hp + b;
    const uint8_t* qrow = p.q + ((size_t)tok * kHq + head) * kD * 2;
    if constexpr (!INT8K) {
      qs[b] = kLog2eOver16;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        uint4 raw = tok_ok ? *reinterpret_cast<const uint4*>(qrow + (32 * s + 8 * L) * 2)
                           : make_uint4(0, 0, 0, 0);
        qf[b][s] = __builtin_bit_cast(bf16x8, raw);
      }
    } else {
      // each lane holds features 64s + 16L .. +15 (s = 0..3) of its query row;
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
      amax = wave_xor_max(amax, 16);
      amax = wave_xor_max(amax, 32);
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
  f32x4 o[16][kQB];
#pragma unroll
  for (int db = 0; db < 16; ++db)
#pragma unroll
    for (int b = 0; b < kQB; ++b) o[db][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[kQB], l[kQB];
#pragma unroll
  for (int b = 0; b < kQB; ++b) {
    m[b] = -__builtin_inff();
    l[b] = 0.0f;
  }

  // ---- first tile ----
  Stage<PAGED, INT8K> st;
  stage_load<PAGED, INT8K>(p, g, 0, tid, st);
  stage_store<PAGED, INT8K>(smem, smem + kKTile, reinterpret_cast<float*>(smem + kKTile + kVTile),
                            tid, st);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int kbase = j * kKt;
    uint8_t* kbuf = smem + (j & 1) * kStage;
    uint8_t* vtbuf = kbuf + kKTile;
    const float* skbuf = reinterpret_cast<const float*>(vtbuf + kVTile);
    const bool more = (j + 1) < ntiles;
    if (more) stage_load<PAGED, INT8K>(p, g, kbase + kKt, tid, st);

    // ---- S^T = K · Q^T for 32 keys x 32 query columns ----
    float sc[kQB][8];   // [query block][key slot: 4 keys of block kb=0, then 4 of kb=1]
    if constexpr (!INT8K) {
      f32x4 acc[kQB][2];
#pragma unroll
      for (int b = 0; b < kQB; ++b) acc[b][0] = acc[b][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(
              kbuf + k_lds_off<2 * kD>(16 * kb + c, 4 * s + L));
#pragma unroll
          for (int b = 0; b < kQB; ++b)
            acc[b][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[b][s], acc[b][kb], 0, 0, 0);
        }
      }
#pragma unroll
      for (int b = 0; b < kQB; ++b)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[b][4 * kb + r] = acc[b][kb][r] * kLog2eOver16;
    } else {
      i32x4 acc[kQB][2];
#pragma unroll
      for (int b = 0; b < kQB; ++b) acc[b][0] = acc[b][1] = i32x4{0, 0, 0, 0};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const i32x4 kf = *reinterpret_cast<const i32x4*>(
              kbuf + k_lds_off<kD>(16 * kb + c, 4 * s + L));
#pragma unroll
          for (int b = 0; b < kQB; ++b)
            acc[b][kb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kf, qq[b][s], acc[b][kb], 0, 0, 0);
        }
      }
      const f32x4 sk0 = *reinterpret_cast<const f32x4*>(skbuf + 4 * L);
      const f32x4 sk1 = *reinterpret_cast<const f32x4*>(skbuf + 16 + 4 * L);
#pragma unroll
      for (int b = 0; b < kQB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sc[b][r] = (float)acc[b][0][r] * sk0[r] * qs[b];
          sc[b][4 + r] = (float)acc[b][1][r] * sk1[r] * qs[b];
        }
    }

    // ---- causal mask (only tiles that reach past the workgroup's first query) ----
    if (kbase + kKt - 1 > off + t0) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kbase + 16 * kb + 4 * L + r;
          if (key > limit) {
#pragma unroll
            for (int b = 0; b < kQB; ++b) sc[b][4 * kb + r] = -__builtin_inff();
          }
        }
    }

    // ---- online softmax (exp2 domain, lazy rescale) ----
    float mnew[kQB];
    bool need = false;
#pragma unroll
    for (int b = 0; b < kQB; ++b) {
      float mx = sc[b][0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sc[b][e]);
      mx = wave_xor_max(mx, 16);
      mx = wave_xor_max(mx, 32);
      mnew[b] = fmaxf(m[b], mx);
      need = need || (mnew[b] > m[b] + kTau);
    }
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
      for (int b = 0; b < kQB; ++b) {
        const float alpha = __builtin_amdgcn_exp2f(m[b] - mnew[b]);
        m[b] = mnew[b];
        l[b] *= alpha;
#pragma unroll
        for (int db = 0; db < 16; ++db) o[db][b] *= alpha;
      }
    }
    bf16x8 ph[kQB], pl[kQB];
#pragma unroll
    for (int b = 0; b < kQB; ++b) {
      f32x8 pv;
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = __builtin_amdgcn_exp2f(sc[b][e] - m[b]);
      ph[b] = __builtin_convertvector(pv, bf16x8);
      const f32x8 hi = __builtin_convertvector(ph[b], f32x8);
      float sum = 0.0f;
      if (split) {
        pl[b] = __builtin_convertvector(pv - hi, bf16x8);
        const f32x8 lo = __builtin_convertvector(pl[b], f32x8);
#pragma unroll
        for (int e = 0; e < 8; ++e) sum += hi[e] + lo[e];
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) sum += hi[e];
      }
      l[b] += sum;
    }

    // ---- O^T += V^T · P^T ----
#pragma unroll
    for (int db = 0; db < 16; ++db) {
      const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vtbuf + vt_lds_off(16 * db + c, L));
#pragma unroll
      for (int b = 0; b < kQB; ++b)
        o[db][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, ph[b], o[db][b], 0, 0, 0);
    }
    if (split) {
#pragma unroll
      for (int db = 0; db < 16; ++db) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vtbuf + vt_lds_off(16 * db + c, L));
#pragma unroll
        for (int b = 0; b < kQB; ++b)
          o[db][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pl[b], o[db][b], 0, 0, 0);
      }
    }

    if (more) {
      uint8_t* nk = smem + ((j + 1) & 1) * kStage;
      stage_store<PAGED, INT8K>(nk, nk + kKTile, reinterpret_cast<float*>(nk + kKTile + kVTile),
                                tid, st);
    }
    __syncthreads();
  }

  // ---- epilogue: O / l -> bf16 ----
#pragma unroll
  for (int b = 0; b < kQB; ++b) {
    float lt = l[b];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const float inv = 1.0f / lt;
    if (tok_ok) {
      const int head = kGroup * g + kHeadsPerWg * hp + b;
      uint8_t* orow = p.out + ((size_t)tok * kHq + head) * kD * 2;
#pragma unroll
      for (int db = 0; db < 16; ++db) {
        const f32x4 y = o[db][b] * inv;
        const bf16x4 yb = __builtin_convertvector(y, bf16x4);
        *reinterpret_cast<bf16x4*>(orow + (16 * db + 4 * L) * 2) = yb;
      }
    }
  }
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
  int workgroups;
  int threads;
  int lds_bytes;
};

Launch plan_for(int32_t q_len, int32_t kv_len, bool paged, bool int8k) {
  (void)kv_len;
  const int n_tblk = (q_len + kTokPerWg - 1) / kTokPerWg;
  Launch lc;
  lc.workgroups = n_tblk * kHkv * kPairs;
  lc.threads = kThreads;
  lc.lds_bytes = 2 * ((int8k ? kKTileI8 : kKTileBf16) + kVTile + (int8k ? kSkTile : 0));
  if (int8k)
    lc.name = "int8k_contiguous_t64h2_kt32";
  else
    lc.name = paged ? "bf16_paged_t64h2_kt32" : "bf16_contiguous_t64h2_kt32";
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
  p.n_tblk = (q_len + kTokPerWg - 1) / kTokPerWg;

  const Launch lc = plan_for(q_len, kv_len, paged, int8k);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(lc.workgroups), block(lc.threads);
  if (int8k)
    hipLaunchKernelGGL((gqa_prefill_kernel<false, true>), grid, block, 0, s, p);
  else if (paged)
    hipLaunchKernelGGL((gqa_prefill_kernel<true, false>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((gqa_prefill_kernel<false, false>), grid, block, 0, s, p);
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
