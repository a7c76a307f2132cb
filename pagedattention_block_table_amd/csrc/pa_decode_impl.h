// Paged-attention decode kernels for gfx950 (CDNA4, wave64).
//
// What is computed (pages cited by title and section):
//   [P1] "突破GPU内存瓶颈：vLLM与PagedAttention技术深度解析" §2 — K/V are stored in
//        fixed-size blocks; a block table maps a sequence's logical blocks to physical
//        ones; only the last block is partly filled; blocks may be shared.
//   [P2] vLLM architecture deep-dive §1.1 — scores are q.K^T / sqrt(d); the kernel
//        loads on demand the blocks named by the table. §3.3 / §4.1 — a split-context
//        second kernel for long text. §4.2 — FP8 KV cache.
//   [P3] "内存优化：KV Cache管理、PagedAttention原理与内存池配置" — decode scores the
//        current query against every cached K/V of the sequence.
//
// Work decomposition. A work unit is (KV head g, sequence s, partition p); one
// workgroup of NW waves runs it. The unit's blocks are dealt to the waves in chunks of
// U consecutive logical blocks, round robin. Within a wave, lane `lane` owns the 16
// bytes at column c = lane % LPT of token row r = lane / LPT of each wave load, where
// LPT = head_dim * elem_bytes / 16 lanes cover one token row. One wave load therefore
// reads TPL = 64 / LPT consecutive token rows = 1 KiB of contiguous tile memory.
// A K/V tile (one physical block, one KV head) is BS * D * e contiguous bytes, so the
// NL = BS / TPL loads of a tile stream one contiguous run.
//
// Arithmetic (all fp32): each lane-row group keeps its own online-softmax state
// (running max m, running sum l, output accumulator) for the G query heads of the
// group, over the tokens it reads, with scores in log2 units (scale * log2(e) folded
// into q, and k_scale too for fp8). Every chunk: scores by per-lane dot products reduced
// across the LPT lanes of the row with DPP; m' = max(m, chunk max); rescale by
// exp2(m - m'); accumulate exp2(z - m') * V. Tokens past the end are excluded by select
// (their score is -inf and their rows are never loaded), never by multiplying by zero.
// At the end the row states of a wave are merged with cross-lane shuffles and the wave
// states of the workgroup through LDS, with the same max/rescale/sum rule.
//
// The order of arithmetic depends only on logical token positions, never on physical
// block ids, so results are bitwise identical under any physical placement or sharing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

enum : int { kF32 = PA_F32, kF16 = PA_F16, kBF16 = PA_BF16, kFP8 = PA_FP8_E4M3 };

constexpr float kLog2e = 1.4426950408889634f;

template <int T> struct ElemBytes;
template <> struct ElemBytes<kF32> { static constexpr int value = 4; };
template <> struct ElemBytes<kF16> { static constexpr int value = 2; };
template <> struct ElemBytes<kBF16> { static constexpr int value = 2; };
template <> struct ElemBytes<kFP8> { static constexpr int value = 1; };

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Arguments shared by every decode kernel instance (passed by value).
struct DecodeArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;
  float* ws;             // partitioned mode: m [S*H*NP], l [S*H*NP], o [S*H*NP*D]
  void* dbg_k;           // debug: raw K rows [S][Hkv][dbg_max_ctx][D]
  void* dbg_v;
  int32_t* dbg_counts;   // debug: [S][Hkv][dbg_max_ctx]
  int32_t* dbg_block_reads;  // debug (grouped kernel): 16-token loads per [block][Hkv], or null
  int num_seqs;
  int max_blocks_per_seq;
  int num_blocks;
  int num_heads;
  int num_kv_heads;
  int part_tokens;       // tokens per partition (multiple of BS)
  int num_parts;         // partitions per (s, g) in the grid
  int max_ctx;           // context lengths are clamped to [0, max_ctx]
  int dbg_max_ctx;
  int32_t* counters;     // balanced mode: arrivals per (KV head, sequence); zero between calls
  int nwg;               // balanced mode: workgroups sharing the chunks
  float q_mul;           // scale * log2(e) (* k_scale for fp8)
  float out_mul;         // v_scale for fp8, else 1
  int ordered;           // longest-first dispatch: unit ranks map to sequences by length
  int order_hpx;         // ordered mode: KV heads per XCD share of the units (0: not whole)
  int wave_parts;        // split-context streaming kernel: partitions per wave (at most)
  int wave_chunks;       // ... and runs per (sequence, KV head)
  int wave_interleave;   // run c takes partitions c, c + wave_chunks, ... (else consecutive)
  int wave_merge;        // ... and each workgroup merges its units' partitions itself
  // grouped kernel over the new tokens of short queries (extend): when set, a group is one
  // sequence and its members are its query_start_loc[s + 1] - query_start_loc[s] new tokens
  const int32_t* query_start_loc;
};

// ---------------------------------------------------------------------------------
// storage conversions
// ---------------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// 16 bytes of KV storage -> 16 / elem_bytes fp32 values, in memory order.
template <int T> __device__ __forceinline__ void widen16(const uint4& r, float* f);

template <> __device__ __forceinline__ void widen16<kF32>(const uint4& r, float* f) {
  f[0] = __builtin_bit_cast(float, r.x);
  f[1] = __builtin_bit_cast(float, r.y);
  f[2] = __builtin_bit_cast(float, r.z);
  f[3] = __builtin_bit_cast(float, r.w);
}

template <> __device__ __forceinline__ void widen16<kF16>(const uint4& r, float* f) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f16x2 h = __builtin_bit_cast(f16x2, w[i]);
    f[2 * i] = (float)h.x;
    f[2 * i + 1] = (float)h.y;
  }
}

template <> __device__ __forceinline__ void widen16<kBF16>(const uint4& r, float* f) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __builtin_bit_cast(float, w[i] << 16);
    f[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
  }
}

// gfx950 converts OCP e4m3 pairs in hardware; word_sel picks bytes {0,1} or {2,3}.
template <> __device__ __forceinline__ void widen16<kFP8>(const uint4& r, float* f) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
    f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
    f[4 * i + 0] = lo.x;
    f[4 * i + 1] = lo.y;
    f[4 * i + 2] = hi.x;
    f[4 * i + 3] = hi.y;
  }
}

template <int IO> __device__ __forceinline__ float load_io(const void* p, int64_t i) {
  if constexpr (IO == kF32) {
    return ((const float*)p)[i];
  } else if constexpr (IO == kF16) {
    return (float)((const _Float16*)p)[i];
  } else {
    return bf16_to_f32(((const uint16_t*)p)[i]);
  }
}

template <int IO> __device__ __forceinline__ void store_io(void* p, int64_t i, float v) {
  if constexpr (IO == kF32) {
    ((float*)p)[i] = v;
  } else if constexpr (IO == kF16) {
    ((_Float16*)p)[i] = (_Float16)v;
  } else {
    ((uint16_t*)p)[i] = f32_to_bf16_rne(v);
  }
}

// ---------------------------------------------------------------------------------
// cross-lane reductions
// ---------------------------------------------------------------------------------

template <int CTRL> __device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                                0xF, 0xF, false));
}

// DPP controls (gfx9): quad_perm = s0 | s1 << 2 | s2 << 4 | s3 << 6; row_ror n = 0x120 + n;
// row_half_mirror = 0x141.
constexpr int kQuadXor1 = 1 | (0 << 2) | (3 << 4) | (2 << 6);
constexpr int kQuadXor2 = 2 | (3 << 2) | (0 << 4) | (1 << 6);
constexpr int kRowHalfMirror = 0x141;

// Sum over aligned groups of N consecutive lanes; every lane receives its group's sum.
template <int N> __device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group");
  if constexpr (N == 1) {
    return x;
  } else if constexpr (N == 2) {
    return x + dpp<kQuadXor1>(x);
  } else if constexpr (N == 4) {
    x += dpp<kQuadXor1>(x);
    return x + dpp<kQuadXor2>(x);
  } else if constexpr (N == 8) {
    // lane i (of 8) + lane 7-i, then the quad sum covers all eight.
    x += dpp<kRowHalfMirror>(x);
    x += dpp<kQuadXor1>(x);
    return x + dpp<kQuadXor2>(x);
  } else if constexpr (N == 16) {
    x += dpp<0x128>(x);  // row_ror 8
    x += dpp<0x124>(x);  // row_ror 4
    x += dpp<0x122>(x);  // row_ror 2
    return x + dpp<0x121>(x);  // row_ror 1
  } else if constexpr (N == 32) {
    x = group_sum<16>(x);
    return x + __shfl_xor(x, 16);
  } else {
    x = group_sum<16>(x);
    x += __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
  }
}

// Lane pairs l, l ^ 16 and l, l ^ 32: gfx950's v_permlane16_swap / v_permlane32_swap exchange rows
// between two registers in one vector instruction, leaving each lane its own value and
// that of lane l ^ 16 (resp. l ^ 32), with no LDS traffic. Max and + are commutative, so
// both lanes of a pair get the same bits. The second register starts as a copy of the
// first; the empty asm keeps the optimizer from treating the two as one value. The pair's
// elements are copied into plain integers before any bit cast (a bit cast taken straight
// from an element of the returned pair read element 0 for both).
__device__ __forceinline__ void rows_pair16(float x, float& a, float& b) {
  unsigned u = __builtin_bit_cast(unsigned, x), w = u;
  asm volatile("" : "+v"(w));
  const auto p = __builtin_amdgcn_permlane16_swap(u, w, false, false);
  const unsigned p0 = p[0], p1 = p[1];
  a = __builtin_bit_cast(float, p0);
  b = __builtin_bit_cast(float, p1);
}
__device__ __forceinline__ void rows_pair32(float x, float& a, float& b) {
  unsigned u = __builtin_bit_cast(unsigned, x), w = u;
  asm volatile("" : "+v"(w));
  const auto p = __builtin_amdgcn_permlane32_swap(u, w, false, false);
  const unsigned p0 = p[0], p1 = p[1];
  a = __builtin_bit_cast(float, p0);
  b = __builtin_bit_cast(float, p1);
}
// A lane's value and that of lane l ^ K: the pair exchanges above for K = 16 and 32 (no
// LDS traffic), a lane shuffle below 16.
template <int K> __device__ __forceinline__ void lane_pair(float x, float& a, float& b) {
  if constexpr (K == 16) {
    rows_pair16(x, a, b);
  } else if constexpr (K == 32) {
    rows_pair32(x, a, b);
  } else {
    a = x;
    b = __shfl_xor(x, K);
  }
}

// Reduce across the row groups of a wave: lanes that differ only in bits >= log2(STRIDE).
// Both lanes of a pair combine the same two values (max and + commute), so every lane of
// a row-group set ends with the same bits.
template <int STRIDE> __device__ __forceinline__ float rows_max(float x) {
  if constexpr (STRIDE < 64) {
    float a, b;
    lane_pair<STRIDE>(x, a, b);
    return rows_max<2 * STRIDE>(fmaxf(a, b));
  } else {
    return x;
  }
}
template <int STRIDE> __device__ __forceinline__ float rows_sum(float x) {
  if constexpr (STRIDE < 64) {
    float a, b;
    lane_pair<STRIDE>(x, a, b);
    return rows_sum<2 * STRIDE>(a + b);
  } else {
    return x;
  }
}

// ---------------------------------------------------------------------------------
// XCD-aware unit order
// ---------------------------------------------------------------------------------

// Workgroups are dispatched round robin over the 8 XCDs (each with its own L2).
// Map workgroup i to unit v so that each XCD receives one contiguous range of units;
// units are ordered KV-head-major, so the sequences that share prefix blocks of one KV
// head read them through the same L2.
__device__ __forceinline__ int xcd_unit(int i, int n) {
  constexpr int X = 8;
  const int xcd = i % X;
  const int k = i / X;
  const int per = n / X;
  const int rem = n % X;
  return xcd * per + min(xcd, rem) + k;
}

// Length classes of the longest-first order: four per doubling of the context length
// (4 floor(log2 L) plus the next two bits of L).
constexpr int kOrderClasses = 128;

__device__ __forceinline__ int length_class(int L) {
  if (L <= 1) return 0;
  const int e = 31 - __builtin_clz((unsigned)L);
  const int frac = e >= 2 ? (L >> (e - 2)) & 3 : (L << (2 - e)) & 3;
  return min(4 * e + frac, kOrderClasses - 1);
}

// Sequence s and KV head g of unit index sg (the partition already factored out), KV-head
// major with the sequences in index order.
__device__ __forceinline__ void unit_seq_head(const DecodeArgs& a, int sg, int& s, int& g) {
  s = sg % a.num_seqs;
  g = sg / a.num_seqs;
}

// The same, sequence major (the KV heads of one sequence consecutive): each XCD's range
// then reads whole blocks, all heads, instead of a few heads' pieces of every block.
__device__ __forceinline__ void unit_seq_major(const DecodeArgs& a, int sg, int& s, int& g) {
  s = sg / a.num_kv_heads;
  g = sg % a.num_kv_heads;
}

// Longest-first dispatch: rank and KV head of unit index sg. When each XCD's contiguous
// share of the units is a whole number of KV heads (order_hpx of them), rank major inside
// the share, so that every XCD starts its longest sequences first; else KV-head major with
// the sequences taken by rank.
__device__ __forceinline__ void unit_rank_head(const DecodeArgs& a, int sg, int& rank, int& g) {
  const int S = a.num_seqs;
  if (a.order_hpx > 0) {
    const int per = S * a.order_hpx;
    const int blk = sg / per;
    const int l = sg - blk * per;
    rank = l / a.order_hpx;
    g = blk * a.order_hpx + (l - rank * a.order_hpx);
  } else {
    rank = sg % S;
    g = sg / S;
  }
}

// Longest-first dispatch is taken for batches up to this many sequences, whose length
// classes stay in LDS for the selection. Every workgroup reads all S lengths, so the
// selection costs O(S) per workgroup; for larger batches that outweighs the tail it removes
// (4096 sequences of 128 tokens: 628 us ordered against 247 us in index order, even with
// the selection reading the lengths in segments), and they are dispatched in index order.
constexpr int kOrderLdsSeqs = 2048;

// LDS of the in-launch ordering: class counts, the result, and the classes of the batch.
struct OrderLds {
  int cnt[kOrderClasses];
  int res[3];  // class, place in the class, sequence
  unsigned char cls[kOrderLdsSeqs];
};

// The sequence of rank `rank` in the longest-first order (length class descending, then
// sequence index ascending), found by the workgroup from the context lengths alone, so
// every workgroup agrees on the order without a separate sorting launch: a class histogram
// in LDS (each wave adds its lanes of one class with one atomic; the classes kept in LDS
// too), one wave's exclusive prefix sums from the top class down to find the rank's class
// and its place in it, then that wave walks the classes 64 at a time and picks the class
// member of that place with a ballot. Requires num_seqs <= kOrderLdsSeqs. Called by every
// thread of the workgroup (it holds barriers).
template <int NTH>
__device__ __forceinline__ int ordered_seq(const DecodeArgs& a, int rank, OrderLds& sm) {
  static_assert(NTH % 64 == 0, "whole waves");
  const int S = a.num_seqs;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  for (int i = tid; i < kOrderClasses; i += NTH) sm.cnt[i] = 0;
  __syncthreads();
  // wave-uniform trip count: every lane of a wave takes part in the ballots
  for (int q0 = tid - lane; q0 < S; q0 += NTH) {
    const int q = q0 + lane;
    const bool valid = q < S;
    const int c = valid ? length_class(min(max(a.context_lens[q], 0), a.max_ctx)) : 0;
    if (valid) sm.cls[q] = (unsigned char)c;
    bool pending = valid;
    for (unsigned long long left = __ballot(pending); left != 0ull; left = __ballot(pending)) {
      const int lead = __ffsll((long long)left) - 1;
      const int lc = __shfl(c, lead);
      const bool same = pending && c == lc;
      const unsigned long long m = __ballot(same);
      if (lane == lead) atomicAdd(&sm.cnt[lc], __popcll(m));
      pending = pending && !same;
    }
  }
  __syncthreads();
  if (tid < 64) {
    static_assert(kOrderClasses == 128, "two classes per lane of one wave");
    const int hi = kOrderClasses - 1 - 2 * tid;  // lane l: classes 127 - 2l and 126 - 2l
    const int c0 = sm.cnt[hi];
    const int c1 = sm.cnt[hi - 1];
    int v = c0 + c1;
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) {
      const int y = __shfl_up(v, k);
      if (tid >= k) v += y;
    }
    const int excl = v - c0 - c1;
    if (rank >= excl && rank < excl + c0) {
      sm.res[0] = hi;
      sm.res[1] = rank - excl;
    } else if (rank >= excl + c0 && rank < excl + c0 + c1) {
      sm.res[0] = hi - 1;
      sm.res[1] = rank - excl - c0;
    }
  }
  __syncthreads();
  if (tid < 64) {
    const int want = sm.res[0];
    const int place = sm.res[1];
    int seen = 0;
    for (int base = 0; base < S; base += 64) {
      const int q = base + tid;
      const int c = q < S ? (int)sm.cls[q] : -1;
      const bool hit = c == want;
      const unsigned long long mask = __ballot(hit);
      const int n = __popcll(mask);
      if (place < seen + n) {
        if (hit && __popcll(mask & ((1ull << tid) - 1ull)) == place - seen) sm.res[2] = q;
        break;
      }
      seen += n;
    }
  }
  __syncthreads();
  return sm.res[2];
}

// Sequence and KV head of unit index sg for either dispatch (every thread of the workgroup
// calls it: the ordered form holds barriers). SEQ_MAJOR: index order sequence major.
template <int NTH, bool SEQ_MAJOR = false>
__device__ __forceinline__ void unit_seq(const DecodeArgs& a, int sg, OrderLds& sm_ord, int& s, int& g) {
  if (a.ordered && a.num_seqs <= kOrderLdsSeqs) {
    int rank;
    unit_rank_head(a, sg, rank, g);
    s = ordered_seq<NTH>(a, rank, sm_ord);
  } else if constexpr (SEQ_MAJOR) {
    unit_seq_major(a, sg, s, g);
  } else {
    unit_seq_head(a, sg, s, g);
  }
}

// ---------------------------------------------------------------------------------
// the decode kernel
// ---------------------------------------------------------------------------------

// Tokens per wave step of the vector kernel, the same for every block size (the token
// order of a wave, and hence the result, does not depend on the block size).
#ifndef PA_CHUNK_TOKENS
#define PA_CHUNK_TOKENS 32
#endif
// Steps whose loads a wave of the vector kernel keeps in flight.
#ifndef PA_VEC_DEPTH
#define PA_VEC_DEPTH 1
#endif
constexpr int kVecDepth = PA_VEC_DEPTH;
// Steps in flight per wave in the streaming split-context kernel with one query head per KV
// head. Its grid holds about four waves per compute unit (one per SIMD), so registers are
// not what limits its occupancy and the loads of the next step can be issued before the
// current one is consumed (more query heads keep one: their states fill the registers).
#ifndef PA_STREAM_DEPTH
#define PA_STREAM_DEPTH 2
#endif
constexpr int kStreamDepth = PA_STREAM_DEPTH;

// Blocks larger than SB tokens (32, or 16 / 8 for 512- / 1024-byte rows) are walked as
// SB-token sub-blocks: sub-block j covers tokens SB j .. SB j + SB - 1, lies in logical
// block j / SPB at row SB (j % SPB), and is itself one contiguous run of its tile.
template <int KV, int D, int BS, int G_>
struct Geometry {
  static constexpr int E = ElemBytes<KV>::value;
  static constexpr int VEC = 16 / E;           // elements per lane load
  static constexpr int LPT = D / VEC;          // lanes per token row
  static constexpr int TPL = 64 / LPT;         // token rows per wave load
  // tokens per (sub-)block step: at most PA_CHUNK_TOKENS, and at most 8 wave loads
  // (head_dim 256)
  static constexpr int SB_MAX = 8 * TPL < PA_CHUNK_TOKENS ? 8 * TPL : PA_CHUNK_TOKENS;
  static constexpr int SB = BS < SB_MAX ? BS : SB_MAX;
  static constexpr int SPB = BS / SB;          // sub-blocks per block
  static constexpr int NL = SB / TPL;          // wave loads per sub-block
  static constexpr int ROW_BYTES = D * E;
  static constexpr int TILE = BS * D * E;      // bytes of one (block, kv-head) tile
  static constexpr bool ok = (LPT >= 1) && (LPT <= 64) && (TPL >= 1) && (SB % TPL == 0) && (BS % SB == 0);
};

template <int G, int VEC> struct RowState {
  float m[G];
  float l[G];
  float acc[G][VEC];
};

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte K/V load. NT: marked non-temporal (the cache is not to keep the line), for
// streams that read each byte once: the split-context stream over long contexts reads
// 4.3 GB in 630 instead of 699 us that way, and the one-workgroup-per-head kernel in 632
// instead of 698 us with only its K loads so marked. Where the cache serves repeats
// (prefix blocks shared by several sequences) plain loads are faster (matrix-core engine
// on a shared-prefix batch: 34.0 against 38.3 us), and on a small batch (LLaMA-7B, 4K
// contexts) non-temporal V loads cost 7% while non-temporal K loads cost nothing.
template <bool NT = false>
__device__ __forceinline__ uint4 load16(const char* p) {
  if constexpr (NT) {
    const u32x4_t r = __builtin_nontemporal_load((const u32x4_t*)p);
    return make_uint4(r.x, r.y, r.z, r.w);
  } else {
    return *(const uint4*)p;
  }
}

// K/V registers of one wave step: U consecutive (sub-)blocks, NL wave loads each.
template <int KV, int D, int BS, int G, int U>
struct StepBuf {
  using Geo = Geometry<KV, D, BS, G>;
  uint4 kr[U][Geo::NL];
  uint4 vr[U][Geo::NL];
};

// Issue the K/V loads of the step whose first (sub-)block is j0, with bid[u] the physical
// block of (sub-)block j0 + u. A lane whose row is at or past t_end reads row j0 * SB
// instead (finite data of this step; the score of such a row is excluded by select, so its
// probability is exactly 0; with t_end <= j0 * SB every lane reads that row). Every load is unconditional:
// loads under a branch make the compiler wait for every outstanding load, those of the
// next step included, before the step's data is used.
// NTK / NTV: K / V loads marked non-temporal.
template <int KV, int D, int BS, int G, int U, bool NTK = false, bool NTV = NTK>
__device__ __forceinline__ void issue_step(StepBuf<KV, D, BS, G, U>& b, const char* kbase, const char* vbase,
                                           int64_t blk_stride, const int (&bid)[U], int j0, int t_end,
                                           int r, int c) {
  using Geo = Geometry<KV, D, BS, G>;
  constexpr int NL = Geo::NL, TPL = Geo::TPL, SB = Geo::SB, SPB = Geo::SPB;
  const uint32_t lane_off = (uint32_t)(r * Geo::ROW_BYTES + c * 16);
  const int64_t sub0 = SPB > 1 ? (int64_t)(j0 % SPB) * SB * Geo::ROW_BYTES : 0;
  const int64_t first = (int64_t)bid[0] * blk_stride + sub0 + c * 16;  // row j0 * SB
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t sub = SPB > 1 ? (int64_t)((j0 + u) % SPB) * SB * Geo::ROW_BYTES : 0;
    const int64_t tile = (int64_t)bid[u] * blk_stride + sub;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int t = (j0 + u) * SB + i * TPL + r;
      const int64_t off = t < t_end ? tile + lane_off + i * TPL * Geo::ROW_BYTES : first;
      b.kr[u][i] = load16<NTK>(kbase + off);
      b.vr[u][i] = load16<NTV>(vbase + off);
    }
  }
}

// Scores, online-softmax update and V accumulation of one loaded step (first (sub-)block
// j0). TAIL: the step reaches past t_end; those rows get score -inf by select.
template <int IO, int KV, int D, int BS, int G, int U, bool TAIL, bool DBG>
__device__ __forceinline__ void consume_step(const DecodeArgs& a, const StepBuf<KV, D, BS, G, U>& b, int j0,
                                             int t_end, int r, int c, int s, int g,
                                             const float (&qf)[G][16 / ElemBytes<KV>::value],
                                             RowState<G, 16 / ElemBytes<KV>::value>& st) {
  using Geo = Geometry<KV, D, BS, G>;
  constexpr int VEC = Geo::VEC, NL = Geo::NL, TPL = Geo::TPL, LPT = Geo::LPT, SB = Geo::SB;

  if constexpr (DBG) {
    const int Hkv = a.num_kv_heads;
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int t = (j0 + u) * SB + i * TPL + r;
        if (t < t_end) {
          const int64_t row = ((int64_t)s * Hkv + g) * a.dbg_max_ctx + t;
          *(uint4*)((char*)a.dbg_k + row * Geo::ROW_BYTES + c * 16) = b.kr[u][i];
          *(uint4*)((char*)a.dbg_v + row * Geo::ROW_BYTES + c * 16) = b.vr[u][i];
          if (c == 0) atomicAdd(a.dbg_counts + row, 1);
        }
      }
    }
  }

  // scores (log2 units)
  float z[U][NL][G];
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      float kf[VEC];
      widen16<KV>(b.kr[u][i], kf);
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc = fmaf(qf[gi][e], kf[e], acc);
        acc = group_sum<LPT>(acc);
        if (TAIL) {
          const int t = (j0 + u) * SB + i * TPL + r;
          acc = (t < t_end) ? acc : -INFINITY;
        }
        z[u][i][gi] = acc;
      }
    }
  }

  // online softmax update
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    float mx = st.m[gi];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < NL; ++i) mx = fmaxf(mx, z[u][i][gi]);
    const float alpha = __builtin_amdgcn_exp2f(st.m[gi] - mx);
    st.m[gi] = mx;
    st.l[gi] *= alpha;
#pragma unroll
    for (int e = 0; e < VEC; ++e) st.acc[gi][e] *= alpha;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      float vf[VEC];
      widen16<KV>(b.vr[u][i], vf);
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        const float p = __builtin_amdgcn_exp2f(z[u][i][gi] - st.m[gi]);
        st.l[gi] += p;
#pragma unroll
        for (int e = 0; e < VEC; ++e) st.acc[gi][e] = fmaf(p, vf[e], st.acc[gi][e]);
      }
    }
  }
}

// Physical blocks of the (sub-)blocks j0 .. j0+U-1 of a step (j0 < j_end): scalar loads
// of the table row; (sub-)blocks past the end take the step's first block (their rows
// are never used). Ids are clamped into the pool so that a bad table never reads outside
// it (contract: 0 <= id < num_blocks).
template <int KV, int D, int BS, int G, int U>
__device__ __forceinline__ void step_blocks(const DecodeArgs& a, const int32_t* bt, int j0, int j_end,
                                            int (&bid)[U]) {
  constexpr int SPB = Geometry<KV, D, BS, G>::SPB;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = j0 + u < j_end ? j0 + u : j0;
    const int b = __builtin_amdgcn_readfirstlane(bt[j / SPB]);
    bid[u] = min(max(b, 0), a.num_blocks - 1);
  }
}

// Physical blocks of a wave's steps, fetched ahead with vector loads. Lane l of window w
// holds the table entries of the wave's step 64 w + l, whose (sub-)blocks are
// j_first + (64 w + l) j_stride + u, u < U; the wave takes a step's ids with readlane.
// Window 0 is requested before the context length is known (it needs only the unit's
// first block), together with it, so the first K/V loads wait for one memory round trip
// instead of two; window w + 1 is requested when the wave enters window w, 64 steps
// ahead of its use. A table read that depended on the previous step would sit between
// that step's compute and the next step's loads, and once the device streams at full
// rate every such read waits behind the queued K/V requests. Entries are read inside the
// table row (indices clamped to it); entries of steps past the wave's last step are read
// but never used, and ids are clamped into the pool when taken, so that a bad table never
// reads outside it (contract: 0 <= id < num_blocks). A refill is issued right before a
// step's K/V loads, so waiting for those loads covers it in order.
template <int U, int SPB>
struct StepWindow {
  int win[2][U];
  int cur;
  const int32_t* bt;
  int last, j_first, j_stride, spp, jump;

  // first (sub-)block of step k: j_first + (k / spp) jump + (k % spp) j_stride
  __device__ __forceinline__ int step_first(int k) const { return j_first + (k / spp) * jump + (k % spp) * j_stride; }
  __device__ __forceinline__ void load(int w, int (&dst)[U]) const {
    const int j = step_first(64 * w + (int)(threadIdx.x & 63));
#pragma unroll
    for (int u = 0; u < U; ++u) dst[u] = bt[min((j + u) / SPB, last)];
  }
  // steps k at j_first + k j_stride, or, with spp > 0, groups of spp such steps jump apart
  __device__ __forceinline__ void begin(const int32_t* bt_row, int row_len, int j_first_, int j_stride_,
                                        int spp_ = 0, int jump_ = 0) {
    bt = bt_row;
    last = row_len - 1;
    j_first = j_first_;
    j_stride = j_stride_;
    spp = spp_ > 0 ? spp_ : 0x7fffffff;
    jump = jump_;
    cur = 0;
    load(0, win[0]);
    load(1, win[1]);
  }
  // ids of step k (k never decreases between calls)
  __device__ __forceinline__ void ids(int k, int num_blocks, int (&bid)[U]) {
    if ((k >> 6) != cur) {
      cur = k >> 6;
#pragma unroll
      for (int u = 0; u < U; ++u) win[0][u] = win[1][u];
      load(cur + 1, win[1]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int b = __builtin_amdgcn_readlane(win[0][u], k & 63);
      bid[u] = min(max(b, 0), num_blocks - 1);
    }
  }
};

// One step of U consecutive (sub-)blocks starting at j0, loaded and consumed at once.
template <int IO, int KV, int D, int BS, int G, int U, bool TAIL, bool DBG>
__device__ __forceinline__ void process_chunk(const DecodeArgs& a, const int32_t* bt,
                                              const char* kbase, const char* vbase,
                                              int64_t blk_stride, int j0, int j_end, int t_end,
                                              int r, int c, int s, int g,
                                              const float (&qf)[G][16 / ElemBytes<KV>::value],
                                              RowState<G, 16 / ElemBytes<KV>::value>& st) {
  int bid[U];
  step_blocks<KV, D, BS, G, U>(a, bt, j0, j_end, bid);
  StepBuf<KV, D, BS, G, U> buf;
  issue_step<KV, D, BS, G, U>(buf, kbase, vbase, blk_stride, bid, j0, t_end, r, c);
  consume_step<IO, KV, D, BS, G, U, TAIL, DBG>(a, buf, j0, t_end, r, c, s, g, qf, st);
}

template <int IO, int KV, int D, int BS, int G, int NW, int U, bool DBG>
__global__ void __launch_bounds__(NW * 64)
decode_kernel(const DecodeArgs a) {
  using Geo = Geometry<KV, D, BS, G>;
  static_assert(Geo::ok, "unsupported geometry");
  constexpr int VEC = Geo::VEC, LPT = Geo::LPT;

  __shared__ float sm_m[NW][G];
  __shared__ float sm_l[NW][G];
  __shared__ float sm_o[NW][G][D];

  __shared__ OrderLds sm_ord;
  const int unit = xcd_unit((int)blockIdx.x, (int)gridDim.x);
  const int part = unit % a.num_parts;
  const int sg = unit / a.num_parts;
  int s, g;
  // One query head per KV head: sequence-major index order (LLaMA-7B batch 26.9 -> 25.1 us,
  // 32 x 2K-token batch 168 -> 161; 8 x 32K 633 -> 641). With more heads per KV head the
  // units of one KV head stay together, so that sequences sharing prefix blocks meet in one
  // L2 (shared-prefix batch 31.9 against 35.2 us sequence major).
  unit_seq<NW * 64, G == 1>(a, sg, sm_ord, s, g);

  constexpr int SB = Geo::SB;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t_begin = part * a.part_tokens;
  const int j_begin = t_begin / SB;
  // this wave's steps k start at (sub-)block j_begin + (wave + k NW) U; their table
  // entries are requested together with the context length
  const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  StepWindow<U, Geo::SPB> tw;
  tw.begin(bt, a.max_blocks_per_seq, j_begin + wave * U, NW * U);

  int L = a.context_lens[s];
  L = min(max(L, 0), a.max_ctx);
  if (part > 0 && t_begin >= L) return;  // nothing in this partition (whole workgroup)
  const int t_end = min(L, t_begin + a.part_tokens);
  const int j_end = (t_end + SB - 1) / SB;

  const int lane = threadIdx.x & 63;
  const int r = lane / LPT;
  const int c = lane % LPT;
  const int H = a.num_heads;

  // q of the G heads of this group, this lane's VEC columns, pre-scaled to log2 units
  float qf[G][VEC];
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    const int64_t base = ((int64_t)s * H + (int64_t)g * G + gi) * D + c * VEC;
#pragma unroll
    for (int e = 0; e < VEC; ++e) qf[gi][e] = load_io<IO>(a.q, base + e) * a.q_mul;
  }

  RowState<G, VEC> st;
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    st.m[gi] = -3.0e38f;
    st.l[gi] = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) st.acc[gi][e] = 0.f;
  }

  const int64_t blk_stride = (int64_t)a.num_kv_heads * Geo::TILE;
  const char* kbase = (const char*)a.k_pool + (int64_t)g * Geo::TILE;
  const char* vbase = (const char*)a.v_pool + (int64_t)g * Geo::TILE;

  // This wave's steps k = 0 .. nwc-1 start at (sub-)block j_begin + (wave + k NW) U; the
  // loads of kVecDepth steps are in flight. Past the last step the issue reads the first
  // row of step nwc - 1 (never consumed), so that the loop issues unconditionally.
  const int steps = (j_end - j_begin + U - 1) / U;
  const int nwc = wave < steps ? (steps - wave + NW - 1) / NW : 0;
  if (nwc > 0) {
    using Buf = StepBuf<KV, D, BS, G, U>;
    auto j0_of = [&](int k) { return j_begin + (wave + min(k, nwc - 1) * NW) * U; };
    auto consume = [&](const Buf& b, int k) {
      const int j0 = j0_of(k);
      if ((j0 + U) * SB <= t_end) {
        consume_step<IO, KV, D, BS, G, U, false, DBG>(a, b, j0, t_end, r, c, s, g, qf, st);
      } else {
        consume_step<IO, KV, D, BS, G, U, true, DBG>(a, b, j0, t_end, r, c, s, g, qf, st);
      }
    };
    auto issue = [&](Buf& b, int k) {
      int bid[U];
      tw.ids(min(k, nwc - 1), a.num_blocks, bid);
      // a step past the wave's last is never consumed: its lanes all read the step's first
      // row (one row instead of the step, so that non-temporal loads fetch no step twice)
      issue_step<KV, D, BS, G, U, true, false>(b, kbase, vbase, blk_stride, bid, j0_of(k), k < nwc ? t_end : 0,
                                               r, c);
    };
    Buf buf[kVecDepth];
#pragma unroll
    for (int d = 0; d < kVecDepth; ++d) issue(buf[d], d);
    int k = 0;
    for (; k + kVecDepth <= nwc; k += kVecDepth) {
#pragma unroll
      for (int d = 0; d < kVecDepth; ++d) {
        consume(buf[d], k + d);
        issue(buf[d], k + d + kVecDepth);
      }
    }
#pragma unroll
    for (int d = 0; d < kVecDepth - 1; ++d)
      if (k + d < nwc) consume(buf[d], k + d);
  }

  // merge the row groups of this wave
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    const float M = rows_max<LPT>(st.m[gi]);
    const float f = __builtin_amdgcn_exp2f(st.m[gi] - M);
    st.m[gi] = M;
    st.l[gi] = rows_sum<LPT>(st.l[gi] * f);
#pragma unroll
    for (int e = 0; e < VEC; ++e) st.acc[gi][e] = rows_sum<LPT>(st.acc[gi][e] * f);
  }
  if (r == 0) {
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) sm_o[wave][gi][c * VEC + e] = st.acc[gi][e];
      if (c == 0) {
        sm_m[wave][gi] = st.m[gi];
        sm_l[wave][gi] = st.l[gi];
      }
    }
  }
  __syncthreads();

  // merge the waves and write
  const int n_parts_s = (L + a.part_tokens - 1) / a.part_tokens;
  const bool write_out = n_parts_s <= 1;
  for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
    const int gi = idx / D;
    const int d = idx % D;
    float M = sm_m[0][gi];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, sm_m[w][gi]);
    float o = 0.f, lsum = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = __builtin_amdgcn_exp2f(sm_m[w][gi] - M);
      o = fmaf(f, sm_o[w][gi][d], o);
      lsum = fmaf(f, sm_l[w][gi], lsum);
    }
    const int h = g * G + gi;
    if (write_out) {
      const float v = lsum > 0.f ? (o / lsum) * a.out_mul : 0.f;
      store_io<IO>(a.out, ((int64_t)s * H + h) * D + d, v);
    } else {
      const int64_t NPH = (int64_t)a.num_seqs * H * a.num_parts;
      const int64_t slot = ((int64_t)s * H + h) * a.num_parts + part;
      a.ws[2 * NPH + slot * D + d] = o * a.out_mul;
      if (d == 0) {
        a.ws[slot] = M;
        a.ws[NPH + slot] = lsum;
      }
    }
  }
}

// Split-context decode, streaming form. Each wave takes a run of a.wave_parts consecutive
// partitions of one (sequence, KV head) and streams their tokens as one wave does in
// decode_kernel, in steps of U (sub-)blocks with the next steps' loads in flight; at the
// end of every partition it merges its row groups, writes that partition's state (or the
// output, for a sequence of one partition) and starts the next partition from a fresh
// state, while the loads of the next partition's first steps are already in flight. The
// host picks wave_parts so that the grid holds a few waves per SIMD: each wave then has a
// long, unbroken stream (a whole 4K-token run at 512-token partitions of 32K contexts)
// instead of one partition between a dependent prologue and a write. Partitions are whole
// steps (the partition size is a multiple of the step, U * SB tokens), so a step never
// spans two partitions and only the context end is masked.
// Partition states a wave of the streaming kernel buffers before writing them: about
// 8 KiB of LDS per wave (16 states of one head at head_dim 128), at least one.
__host__ __device__ constexpr int stream_states(int G, int D) {
  return (2080 / (G * (D + 2))) > 0 ? (2080 / (G * (D + 2))) : 1;
}
template <int G, int D>
constexpr int kStreamStates = stream_states(G, D);

template <int IO, int KV, int D, int BS, int G, int NW, int U, bool DBG>
__global__ void __launch_bounds__(NW * 64)
decode_stream_kernel(const DecodeArgs a) {
  using Geo = Geometry<KV, D, BS, G>;
  static_assert(Geo::ok, "unsupported geometry");
  constexpr int VEC = Geo::VEC, LPT = Geo::LPT, SB = Geo::SB;
  constexpr int ST = U * SB;  // tokens per step
  constexpr int SD = G == 1 ? kStreamDepth : 1;  // steps in flight (more heads: registers)

  const int hw_wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gw = xcd_unit((int)blockIdx.x, (int)gridDim.x) * NW + hw_wave;

  // Partition states go to a per-wave LDS buffer and reach the workspace in batches, with
  // full-wave stores, when the buffer is full or the run is done. Stores retire in order
  // with the loads on the same counter, so a store issued at every partition end would
  // hold up the consumption of every load issued after it; batched, the wave issues them
  // once per buffer (at the end of the run for runs that fit). When every (sequence, KV
  // head) is run by the waves of one workgroup and fits their buffers (wave_merge), the
  // workgroup merges the states itself and writes the output: no workspace traffic and
  // no second launch.
  constexpr int SBUF = kStreamStates<G, D>;
  __shared__ __align__(16) float sm_st[NW][SBUF][G][D];
  __shared__ float sm_ml[NW][2][SBUF][G];
  __shared__ int sm_cnt[NW];
  const bool wmerge = a.wave_merge != 0;
  int nbuf = 0, pbuf = 0;  // states buffered, partition of the first one

  auto run = [&]() {
  const int cps = a.wave_chunks;
  if (gw >= a.num_seqs * a.num_kv_heads * cps) return;  // past the last run (this wave)
  const int chunk = gw % cps;
  int s, g;
  unit_seq_head(a, gw / cps, s, g);

  // the run's partitions: pf, pf + ps, pf + 2 ps, ... (consecutive, or every cps-th)
  const int P = a.part_tokens;
  const int pf = a.wave_interleave ? chunk : chunk * a.wave_parts;
  const int ps = a.wave_interleave ? cps : 1;
  const int spp = P / ST;  // steps per partition
  const int psb = P / SB;  // (sub-)blocks per partition
  // step k starts at (sub-)block (pf + (k / spp) ps) psb + (k % spp) U; the first steps'
  // table entries are requested together with the context length
  const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  StepWindow<U, Geo::SPB> tw;
  tw.begin(bt, a.max_blocks_per_seq, pf * psb, U, spp, ps * psb);

  int L = a.context_lens[s];
  L = min(max(L, 0), a.max_ctx);
  if (chunk > 0 && pf * P >= L) return;  // nothing in this run
  const int n_parts_s = (L + P - 1) / P;
  const bool write_out = n_parts_s <= 1;
  // partitions of the run inside the context, and the steps of its last one
  const int n_run = a.wave_interleave ? (n_parts_s > pf ? (n_parts_s - pf + ps - 1) / ps : 0)
                                      : min(a.wave_parts, n_parts_s - pf);
  const int p_last = pf + (max(n_run, 1) - 1) * ps;
  const int last_steps = (min(L, (p_last + 1) * P) - p_last * P + ST - 1) / ST;
  const int nsteps = n_run > 0 ? (n_run - 1) * spp + last_steps : 0;

  const int lane = threadIdx.x & 63;
  const int r = lane / LPT;
  const int c = lane % LPT;
  const int H = a.num_heads;
  const int64_t NPH = (int64_t)a.num_seqs * H * a.num_parts;

  float qf[G][VEC];
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    const int64_t base = ((int64_t)s * H + (int64_t)g * G + gi) * D + c * VEC;
#pragma unroll
    for (int e = 0; e < VEC; ++e) qf[gi][e] = load_io<IO>(a.q, base + e) * a.q_mul;
  }
  RowState<G, VEC> st;
  auto reset = [&]() {
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      st.m[gi] = -3.0e38f;
      st.l[gi] = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) st.acc[gi][e] = 0.f;
    }
  };
  float (*wst)[G][D] = sm_st[hw_wave];
  auto flush = [&]() {
    if (nbuf == 0) return;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // buffered state j is partition pbuf + j * ps; its row for head gi is contiguous (8-byte
    // pieces: the output rows start 8 * NPH bytes into the workspace)
    for (int idx = lane; idx < nbuf * G * (D / 2); idx += 64) {
      const int j = idx / (G * (D / 2));
      const int gi = (idx / (D / 2)) % G;
      const int d2 = idx % (D / 2);
      const int64_t slot = ((int64_t)s * H + (int64_t)g * G + gi) * a.num_parts + pbuf + j * ps;
      *(float2*)(a.ws + 2 * NPH + slot * D + 2 * d2) = *(const float2*)&wst[j][gi][2 * d2];
    }
    for (int idx = lane; idx < nbuf * G; idx += 64) {
      const int j = idx / G;
      const int gi = idx % G;
      const int64_t slot = ((int64_t)s * H + (int64_t)g * G + gi) * a.num_parts + pbuf + j * ps;
      a.ws[slot] = sm_ml[hw_wave][0][j][gi];
      a.ws[NPH + slot] = sm_ml[hw_wave][1][j][gi];
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    nbuf = 0;
  };
  // merge the row groups of the wave, then lanes of row group 0 write their columns of
  // the output (a sequence of one partition) or buffer partition `part`'s state
  auto finish = [&](int part) {
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      const float M = rows_max<LPT>(st.m[gi]);
      const float f = __builtin_amdgcn_exp2f(st.m[gi] - M);
      st.m[gi] = M;
      st.l[gi] = rows_sum<LPT>(st.l[gi] * f);
#pragma unroll
      for (int e = 0; e < VEC; ++e) st.acc[gi][e] = rows_sum<LPT>(st.acc[gi][e] * f);
    }
    if (write_out) {
      if (r == 0) {
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
          const int h = g * G + gi;
#pragma unroll
          for (int e = 0; e < VEC; ++e)
            store_io<IO>(a.out, ((int64_t)s * H + h) * D + c * VEC + e,
                         st.l[gi] > 0.f ? (st.acc[gi][e] / st.l[gi]) * a.out_mul : 0.f);
        }
      }
      return;
    }
    if (nbuf == SBUF) flush();
    if (nbuf == 0) pbuf = part;
    if (r == 0) {
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) wst[nbuf][gi][c * VEC + e] = st.acc[gi][e] * a.out_mul;
        if (c == 0) {
          sm_ml[hw_wave][0][nbuf][gi] = st.m[gi];
          sm_ml[hw_wave][1][nbuf][gi] = st.l[gi];
        }
      }
    }
    ++nbuf;
  };
  reset();
  if (nsteps <= 0) {  // empty sequence: its output is zero
    finish(pf);
    return;
  }

  const int64_t blk_stride = (int64_t)a.num_kv_heads * Geo::TILE;
  const char* kbase = (const char*)a.k_pool + (int64_t)g * Geo::TILE;
  const char* vbase = (const char*)a.v_pool + (int64_t)g * Geo::TILE;

  using Buf = StepBuf<KV, D, BS, G, U>;
  auto j0_of = [&](int k) { return tw.step_first(min(k, nsteps - 1)); };
  auto consume = [&](const Buf& b, int k) {
    const int j0 = j0_of(k);
    if ((j0 + U) * SB <= L) {
      consume_step<IO, KV, D, BS, G, U, false, DBG>(a, b, j0, L, r, c, s, g, qf, st);
    } else {
      consume_step<IO, KV, D, BS, G, U, true, DBG>(a, b, j0, L, r, c, s, g, qf, st);
    }
  };
  // after step k's successor loads are issued: close the partition if step k ended it
  auto close = [&](int k) {
    if ((k + 1) % spp == 0 || k + 1 == nsteps) {
      finish(pf + (k / spp) * ps);
      reset();
    }
  };
  auto issue = [&](Buf& b, int k) {
    int bid[U];
    tw.ids(min(k, nsteps - 1), a.num_blocks, bid);
    // each K/V byte of the run is read once: non-temporal loads; a step past the run's
    // last (never consumed) reads only its first row
    issue_step<KV, D, BS, G, U, true>(b, kbase, vbase, blk_stride, bid, j0_of(k), k < nsteps ? L : 0, r, c);
  };
  Buf buf[SD];
#pragma unroll
  for (int d = 0; d < SD; ++d) issue(buf[d], d);
  int k = 0;
  for (; k + SD <= nsteps; k += SD) {
#pragma unroll
    for (int d = 0; d < SD; ++d) {
      consume(buf[d], k + d);
      issue(buf[d], k + d + SD);
      close(k + d);
    }
  }
#pragma unroll
  for (int d = 0; d < SD - 1; ++d)
    if (k + d < nsteps) {
      consume(buf[d], k + d);
      close(k + d);
    }
  if (!wmerge) flush();
  };
  run();
  if (!wmerge) return;

  // log-sum-exp merge of the partition states of this workgroup's (sequence, KV head)
  // units ([P2] §3.3 / §4.1), from the waves' buffers
  if ((threadIdx.x & 63) == 0) sm_cnt[hw_wave] = nbuf;
  __syncthreads();
  const int cpu = a.wave_chunks;  // waves (runs) per unit
  const int unit0 = (gw - hw_wave) / cpu;
  const int P = a.part_tokens;
  for (int idx = threadIdx.x; idx < (NW / cpu) * G * D; idx += NW * 64) {
    const int ul = idx / (G * D);
    const int gi = (idx / D) % G;
    const int d = idx % D;
    const int unit = unit0 + ul;
    if (unit >= a.num_seqs * a.num_kv_heads) continue;
    int s, g;
    unit_seq_head(a, unit, s, g);
    const int L = min(max(a.context_lens[s], 0), a.max_ctx);
    if ((L + P - 1) / P <= 1) continue;  // one partition: its run wrote the output
    float M = -3.0e38f;
    for (int w = ul * cpu; w < (ul + 1) * cpu; ++w)
      for (int j = 0; j < sm_cnt[w]; ++j) M = fmaxf(M, sm_ml[w][0][j][gi]);
    float num = 0.f, den = 0.f;
    for (int w = ul * cpu; w < (ul + 1) * cpu; ++w)
      for (int j = 0; j < sm_cnt[w]; ++j) {
        const float f = __builtin_amdgcn_exp2f(sm_ml[w][0][j][gi] - M);
        num = fmaf(f, sm_st[w][j][gi][d], num);
        den = fmaf(f, sm_ml[w][1][j][gi], den);
      }
    store_io<IO>(a.out, ((int64_t)s * a.num_heads + (int64_t)g * G + gi) * D + d, den > 0.f ? num / den : 0.f);
  }
}

// The vector path as an engine of the chunk schedulers (the balanced grid): the same
// process_chunk math on chunks of ValuEngine::CT tokens counted from token `base`,
// chunk k0 + rotated(wave + k*nw, rot, len) for the wave's k-th step.
template <int IO, int KV, int D, int BS, int G, bool DBG>
struct ValuEngine {
  using Geo = Geometry<KV, D, BS, G>;
  static constexpr int VEC = Geo::VEC, LPT = Geo::LPT, SB = Geo::SB;
  static constexpr int U = SB >= Geo::SB_MAX ? 1 : Geo::SB_MAX / SB;  // (sub-)blocks per step
  static constexpr int CT = U * SB;                                      // SB_MAX tokens
  static_assert(Geo::ok, "unsupported geometry");

  int lane, r, c;
  int s, g, t_end, j_end, base, k0, len, rot, wave, nw;
  const int32_t* bt;
  const char* kbase;
  const char* vbase;
  int64_t blk_stride;
  float qf[G][VEC];
  RowState<G, VEC> st;

  __device__ __forceinline__ explicit ValuEngine(int l) : lane(l), r(l / LPT), c(l % LPT) {}

  __device__ __forceinline__ void begin(const DecodeArgs& a, int s_, int g_, int t_end_, int base_,
                                        int k0_, int len_, int rot_, int wave_, int nw_) {
    s = s_;
    g = g_;
    t_end = t_end_;
    j_end = (t_end + SB - 1) / SB;
    base = base_;
    k0 = k0_;
    len = len_;
    rot = rot_;
    wave = wave_;
    nw = nw_;
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      const int64_t qb = ((int64_t)s * a.num_heads + (int64_t)g * G + gi) * D + c * VEC;
#pragma unroll
      for (int e = 0; e < VEC; ++e) qf[gi][e] = load_io<IO>(a.q, qb + e) * a.q_mul;
      st.m[gi] = -3.0e38f;
      st.l[gi] = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) st.acc[gi][e] = 0.f;
    }
    bt = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
    blk_stride = (int64_t)a.num_kv_heads * Geo::TILE;
    kbase = (const char*)a.k_pool + (int64_t)g * Geo::TILE;
    vbase = (const char*)a.v_pool + (int64_t)g * Geo::TILE;
  }

  __device__ __forceinline__ void run(const DecodeArgs& a) {
    const int nwc = wave < len ? (len - wave + nw - 1) / nw : 0;
    for (int k = 0; k < nwc; ++k) {
      int ci = wave + k * nw + rot;
      ci = ci >= len ? ci - len : ci;
      const int j0 = (base + CT * (k0 + ci)) / SB;
      if ((j0 + U) * SB <= t_end) {
        process_chunk<IO, KV, D, BS, G, U, false, DBG>(a, bt, kbase, vbase, blk_stride, j0, j_end, t_end, r, c,
                                                       s, g, qf, st);
      } else {
        process_chunk<IO, KV, D, BS, G, U, true, DBG>(a, bt, kbase, vbase, blk_stride, j0, j_end, t_end, r, c,
                                                      s, g, qf, st);
      }
    }
  }

  template <int NW>
  __device__ __forceinline__ void finish(float (&sm_m)[NW][G], float (&sm_l)[NW][G],
                                         float (&sm_o)[NW][G][D]) {
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      const float M = rows_max<LPT>(st.m[gi]);
      const float f = __builtin_amdgcn_exp2f(st.m[gi] - M);
      st.m[gi] = M;
      st.l[gi] = rows_sum<LPT>(st.l[gi] * f);
#pragma unroll
      for (int e = 0; e < VEC; ++e) st.acc[gi][e] = rows_sum<LPT>(st.acc[gi][e] * f);
    }
    if (r == 0) {
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) sm_o[wave][gi][c * VEC + e] = st.acc[gi][e];
        if (c == 0) {
          sm_m[wave][gi] = st.m[gi];
          sm_l[wave][gi] = st.l[gi];
        }
      }
    }
  }
};

}  // namespace pa

#include "pa_mfma_decode.h"
#include "pa_group_decode.h"

namespace pa {

// Per-(io, kv) launcher; defined in one translation unit per dtype pair.
struct LaunchSpec {
  DecodeArgs args;
  int head_dim;
  int block_size;
  int group;
  bool debug;
  bool balanced;   // balanced_decode_kernel (MFMA shapes only)
  bool grouped;        // grouped_decode_kernel (shared prefixes; grid = Hkv x groups x splits)
  bool stream_kernel;  // split-context: the streaming kernel if the shape takes the vector kernel
  int stream_waves;    // its grid, in waves
  int grid;            // units (workgroups of the balanced kernel)
  hipStream_t stream;
};

#ifndef PA_MFMA
#define PA_MFMA 1
#endif
#ifndef PA_WAVES
#define PA_WAVES 4
#endif
// Waves per workgroup of the one-unit-per-workgroup matrix-core kernel.
#ifndef PA_MFMA_WAVES
#define PA_MFMA_WAVES PA_WAVES
#endif

template <int IO, int KV, int D, int BS, int G>
constexpr int pick_unroll() {
  // Consecutive (sub-)blocks per wave iteration: SB_MAX tokens (at most PA_CHUNK_TOKENS
  // and at most 8 wave loads of K), whatever the block size, so that the token order of a
  // wave and hence the result does not depend on the block size.
  using Geo = Geometry<KV, D, BS, G>;
  constexpr int CT = Geo::SB_MAX < PA_CHUNK_TOKENS ? Geo::SB_MAX : PA_CHUNK_TOKENS;
  return Geo::SB >= CT ? 1 : CT / Geo::SB;
}

template <int IO, int KV, int D, int BS, int G>
int launch_one(const LaunchSpec& ls) {
  if constexpr (!Geometry<KV, D, BS, G>::ok) {
    return PA_ERR_UNSUPPORTED;
  } else {
    constexpr int NW = PA_WAVES;
    constexpr int U = pick_unroll<IO, KV, D, BS, G>();
    if (ls.balanced) {
      if constexpr (mfma_supported<IO, KV, D, G>()) {
        if (ls.debug) {
          hipLaunchKernelGGL((balanced_decode_kernel<IO, KV, D, BS, G, NW, true>), dim3(ls.grid),
                             dim3(NW * 64), 0, ls.stream, ls.args);
        } else {
          hipLaunchKernelGGL((balanced_decode_kernel<IO, KV, D, BS, G, NW, false>), dim3(ls.grid),
                             dim3(NW * 64), 0, ls.stream, ls.args);
        }
        return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
      } else {
        return PA_ERR_UNSUPPORTED;
      }
    }
    if (ls.grouped) {
      if constexpr (GroupShape<IO, KV, D, BS, G, NW, false>::ok) {
        if (ls.debug) {
          hipLaunchKernelGGL((grouped_decode_kernel<IO, KV, D, BS, G, NW, true>), dim3(ls.grid), dim3(NW * 64), 0,
                             ls.stream, ls.args);
        } else {
          hipLaunchKernelGGL((grouped_decode_kernel<IO, KV, D, BS, G, NW, false>), dim3(ls.grid), dim3(NW * 64), 0,
                             ls.stream, ls.args);
        }
        return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
      } else {
        return PA_ERR_UNSUPPORTED;
      }
    }
    // one workgroup per unit: the matrix-core kernel when query heads share a KV head; for
    // one query head per KV head the vector kernel (whole 1 KiB rows per wave load) is faster
    if constexpr (PA_MFMA && G >= 2 && mfma_supported<IO, KV, D, G>()) {
      constexpr int NWM = PA_MFMA_WAVES;
      if (ls.debug) {
        hipLaunchKernelGGL((mfma_decode_kernel<IO, KV, D, BS, G, NWM, true>), dim3(ls.grid),
                           dim3(NWM * 64), 0, ls.stream, ls.args);
      } else {
        hipLaunchKernelGGL((mfma_decode_kernel<IO, KV, D, BS, G, NWM, false>), dim3(ls.grid),
                           dim3(NWM * 64), 0, ls.stream, ls.args);
      }
      return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
    }
    if (ls.stream_kernel && ls.args.part_tokens % (U * Geometry<KV, D, BS, G>::SB) == 0) {
      const int grid = (ls.stream_waves + NW - 1) / NW;
      if (ls.debug) {
        hipLaunchKernelGGL((decode_stream_kernel<IO, KV, D, BS, G, NW, U, true>), dim3(grid), dim3(NW * 64), 0,
                           ls.stream, ls.args);
      } else {
        hipLaunchKernelGGL((decode_stream_kernel<IO, KV, D, BS, G, NW, U, false>), dim3(grid), dim3(NW * 64), 0,
                           ls.stream, ls.args);
      }
      return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
    }
    if (ls.debug) {
      hipLaunchKernelGGL((decode_kernel<IO, KV, D, BS, G, NW, U, true>), dim3(ls.grid), dim3(NW * 64),
                         0, ls.stream, ls.args);
    } else {
      hipLaunchKernelGGL((decode_kernel<IO, KV, D, BS, G, NW, U, false>), dim3(ls.grid), dim3(NW * 64),
                         0, ls.stream, ls.args);
    }
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
  }
}

template <int IO, int KV, int D, int BS>
int launch_g(const LaunchSpec& ls) {
  switch (ls.group) {
    case 1: return launch_one<IO, KV, D, BS, 1>(ls);
    case 2: return launch_one<IO, KV, D, BS, 2>(ls);
    case 4: return launch_one<IO, KV, D, BS, 4>(ls);
    case 8: return launch_one<IO, KV, D, BS, 8>(ls);
    default: return PA_ERR_UNSUPPORTED;
  }
}

// LARGE: blocks of 64 .. 512 tokens, else 8 .. 32 (two translation units per dtype pair)
template <int IO, int KV, int D, bool LARGE>
int launch_bs(const LaunchSpec& ls) {
  if constexpr (LARGE) {
    switch (ls.block_size) {
      case 64: return launch_g<IO, KV, D, 64>(ls);
      case 128: return launch_g<IO, KV, D, 128>(ls);
      case 256: return launch_g<IO, KV, D, 256>(ls);
      case 512: return launch_g<IO, KV, D, 512>(ls);
      default: return PA_ERR_UNSUPPORTED;
    }
  } else {
    switch (ls.block_size) {
      case 8: return launch_g<IO, KV, D, 8>(ls);
      case 16: return launch_g<IO, KV, D, 16>(ls);
      case 32: return launch_g<IO, KV, D, 32>(ls);
      default: return PA_ERR_UNSUPPORTED;
    }
  }
}

template <int IO, int KV, bool LARGE>
int launch_decode(const LaunchSpec& ls) {
  switch (ls.head_dim) {
    case 64: return launch_bs<IO, KV, 64, LARGE>(ls);
    case 128: return launch_bs<IO, KV, 128, LARGE>(ls);
    case 256: return launch_bs<IO, KV, 256, LARGE>(ls);
    default: return PA_ERR_UNSUPPORTED;
  }
}

// Explicit per-pair entry points (one translation unit each, compiled in parallel); the
// _large ones take block sizes 64 .. 512.
int launch_f32_f32(const LaunchSpec&);
int launch_f16_f16(const LaunchSpec&);
int launch_bf16_bf16(const LaunchSpec&);
int launch_f32_fp8(const LaunchSpec&);
int launch_f16_fp8(const LaunchSpec&);
int launch_bf16_fp8(const LaunchSpec&);
int launch_f32_f32_large(const LaunchSpec&);
int launch_f16_f16_large(const LaunchSpec&);
int launch_bf16_bf16_large(const LaunchSpec&);
int launch_f32_fp8_large(const LaunchSpec&);
int launch_f16_fp8_large(const LaunchSpec&);
int launch_bf16_fp8_large(const LaunchSpec&);

}  // namespace pa
