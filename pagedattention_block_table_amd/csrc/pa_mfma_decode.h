// Decode kernels for gfx950 with both products on the matrix cores.
//
// Same computation as decode_kernel (pages cited there): for a KV head g and the G query
// heads that share it (G = 2, 4 or 8), scores z = scale * q.K^T over the cached tokens,
// online softmax, and the softmax-weighted sum of V rows, accumulated in fp32.
//
// MFMA operand layout (wave64): for v_mfma_f32_16x16x32, lane l supplies row l%16 of A
// and column l%16 of B, each as the 8 consecutive k values 8*(l/16) .. 8*(l/16)+7, and
// receives D[4*(l/16) + r][l%16] in result register r; the 16x16x16 form takes four k
// values per lane (4*(l/16) .. +3) with the same result layout. The k order inside a
// product is free, so each lane feeds the score product straight from its own 16-byte
// K loads: lane (n = l%16, lg = l/16) loads the 16-byte chunks 4i + lg of token n's row.
//
// The per-wave engine (MfmaTEngine below) computes the scores transposed, S^T = K Q^T,
// so that each lane receives the scores of one query row for four tokens of a 16-token
// tile: exactly its B operand of O^T += V^T P^T after the softmax. V^T comes from the
// wave's LDS copy of the tile, read transposed.
//
// Softmax: each query row keeps a running max in log2 units, raised only when a tile's
// max exceeds it by more than kLazyRescale; in between the probabilities exp2(z - m) stay
// <= 2^kLazyRescale, and the final normalisation by the running sum makes the result
// independent of which m was used.
//
// Work is cut into chunks of 16 * NT tokens. Chunks are dealt round robin to the waves of
// a workgroup, so the order of arithmetic depends only on logical token positions:
// results are bitwise identical under any block size, physical placement or sharing.
// Each wave fetches the table entries of its chunks ahead, 64 at a time, and keeps the
// next chunk's K/V loads in flight while it computes the current one.
//
// Two schedulers drive the engines (the vector engine ValuEngine for one query head per
// KV head in the balanced grid):
//   mfma_decode_kernel      one workgroup per (KV head, sequence, partition), its waves
//                           taking the chunks round robin and merging through LDS;
//   balanced_decode_kernel  a fixed grid of workgroups splits the total chunk count of
//                           the batch evenly; a (KV head, sequence) whose chunks span
//                           several workgroups is merged by the last one to finish it.
#pragma once

#include <type_traits>

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

// log2-unit headroom of the lazy running-max update (probabilities stay <= 2^8)
constexpr float kLazyRescale = 8.0f;

#ifndef PA_STAGGER
#define PA_STAGGER 1
#endif

// Fixed work of one segment of the balanced scheduler (engine set-up, wave merge, write),
// counted in chunks when the batch is split evenly over the workgroups: without it a
// workgroup whose range holds many short sequences does more work than the others.
#ifndef PA_SEG_COST
#define PA_SEG_COST 8
#endif
constexpr int kSegCost = PA_SEG_COST;

// Largest batch the balanced scheduler takes (its chunk prefix sums live in LDS).
constexpr int kMaxBalancedSeqs = 4096;

template <int MT> struct Mma;
template <> struct Mma<kF16> {
  typedef f16x8_t vec;
  static __device__ __forceinline__ f32x4_t mma(const vec& a, const vec& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mma<kBF16> {
  typedef bf16x8_t vec;
  static __device__ __forceinline__ f32x4_t mma(const vec& a, const vec& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

// Eight e4m3 codes (two dwords) -> eight MFMA operands of type MT, exactly: every e4m3
// value has at most 4 significant bits and an exponent inside the f16 and bf16 ranges.
// gfx950 converts a pair of codes straight to f16 or bf16 (v_cvt_scalef32_pk_*_fp8 with a
// scale of 1.0, which is exact); word_sel picks bytes {0,1} or {2,3} of the dword, the
// lower code going to the lower half.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
template <int MT, bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_mt(uint32_t w) {
  if constexpr (MT == kBF16) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
  }
}

template <int MT>
__device__ __forceinline__ typename Mma<MT>::vec fp8x8_operand(uint32_t w0, uint32_t w1) {
  uint4 r;
  r.x = fp8x2_to_mt<MT, false>(w0);
  r.y = fp8x2_to_mt<MT, true>(w0);
  r.z = fp8x2_to_mt<MT, false>(w1);
  r.w = fp8x2_to_mt<MT, true>(w1);
  return __builtin_bit_cast(typename Mma<MT>::vec, r);
}

template <int MT, int KV>
__device__ __forceinline__ typename Mma<MT>::vec k_operand(const uint4& r, int half) {
  if constexpr (KV == kFP8) {
    return half == 0 ? fp8x8_operand<MT>(r.x, r.y) : fp8x8_operand<MT>(r.z, r.w);
  } else {
    return __builtin_bit_cast(typename Mma<MT>::vec, r);
  }
}

template <int KV, int D>
struct MfmaGeo {
  static constexpr int E = ElemBytes<KV>::value;
  static constexpr int VEC = 16 / E;         // values per 16-byte chunk
  static constexpr int RB = D * E;           // bytes of one token row
  static constexpr int CPR = RB / 16;        // chunks per row
  static constexpr int CPL = CPR / 4;        // K chunks per lane per row
  static constexpr int VPL = CPL / 2;        // V chunks per lane per token (two tokens)
  static constexpr int NST = D / 32;         // MFMA steps over head_dim
  static constexpr bool ok = (KV != kF32) && (CPR % 4 == 0) && (CPL >= 2) && (CPL % 2 == 0);
};

// Shapes the MFMA kernels take: 1, 2, 4 or 8 query heads per KV head (8 only with the V
// product on the matrix cores), io f16/bf16, KV = io or fp8, head_dim 64 or 128 and at
// least 128 bytes per token row.
template <int IO, int KV, int D, int G>
constexpr bool mfma_supported() {
  return (G == 1 || G == 2 || G == 4 || G == 8) && (IO == kF16 || IO == kBF16) && (KV == IO || KV == kFP8) &&
         D <= 128 && MfmaGeo<KV, D>::ok;
}

// Chunks a wave keeps in flight: the loads of chunks k+1 .. k+kPipeDepth-1 are
// outstanding while chunk k is computed.
#ifndef PA_PIPE_DEPTH
#define PA_PIPE_DEPTH 2
#endif
constexpr int kPipeDepth = PA_PIPE_DEPTH;

// Drive an engine's issue / consume over a wave's nwc chunks with kPipeDepth register
// buffers (the buffer index is a compile-time constant after unrolling). The steady-state
// loop issues unconditionally: past the last chunk it issues chunk nwc - 1 again with
// live = false, for which the engine reads only the chunk's first row (never consumed).
// With every path into the loop header issuing the same loads in the same order, the
// compiler waits only for the buffer being consumed; a conditional issue would make it
// wait for the loads of the following chunks as well.
template <class Eng>
__device__ __forceinline__ void run_pipelined(Eng& eng, const DecodeArgs& a, int nwc) {
  if (nwc <= 0) return;
  typename Eng::Buf b[kPipeDepth];
#pragma unroll
  for (int d = 0; d < kPipeDepth; ++d) eng.issue(a, b[d], min(d, nwc - 1), d < nwc);
  int k = 0;
  for (; k + kPipeDepth <= nwc; k += kPipeDepth) {
#pragma unroll
    for (int d = 0; d < kPipeDepth; ++d) {
      eng.consume(a, b[d], k + d);
      const int kn = k + d + kPipeDepth;
      eng.issue(a, b[d], min(kn, nwc - 1), kn < nwc);
    }
  }
#pragma unroll
  for (int d = 0; d < kPipeDepth - 1; ++d)
    if (k + d < nwc) eng.consume(a, b[d], k + d);
}

// Order in which a wave visits the `len` chunks of a segment: from a per-sequence
// rotation, so that workgroups that share prefix blocks do not all start on the same
// block at the same time.
__device__ __forceinline__ int rotated(int idx, int rot, int len) {
  const int c = idx + rot;
  return c >= len ? c - len : c;
}

// Lane roles inside a wave: n = token of a 16-token tile, lg = lane group (which
// 16-byte chunks of a row), hh = half of the tile the lane pairs with for V.
struct LaneIds {
  int lane, n, lg, hh;
  __device__ __forceinline__ explicit LaneIds(int l) : lane(l), n(l & 15), lg(l >> 4), hh((l & 15) >> 3) {}
};

// Query operands of (sequence s, KV head g): row n of A is head g*G + n%G, and the k
// index (lg, e) of step i*VEC/8 + hf is column VEC*(4i+lg) + 8*hf + e.
template <int IO, int KV, int D, int G>
__device__ __forceinline__ void load_q(const DecodeArgs& a, int s, int g, const LaneIds& li,
                                       typename Mma<IO>::vec (&qa)[MfmaGeo<KV, D>::NST]) {
  using Geo = MfmaGeo<KV, D>;
  const uint16_t* qrow = (const uint16_t*)a.q + ((int64_t)s * a.num_heads + g * G + (li.n % G)) * D;
#pragma unroll
  for (int i = 0; i < Geo::CPL; ++i) {
    const int col = Geo::VEC * (4 * i + li.lg);
#pragma unroll
    for (int hf = 0; hf < Geo::VEC / 8; ++hf) {
      const uint4 w = *(const uint4*)(qrow + col + 8 * hf);
      qa[i * (Geo::VEC / 8) + hf] = __builtin_bit_cast(typename Mma<IO>::vec, w);
    }
  }
}

// 16x16x16 products for the V side: A = probabilities, B = V^T tile read transposed
// from LDS. Operands are four 16-bit values per lane: lane l supplies row l%16 of A and
// column l%16 of B for k = 4*(l/16) .. 4*(l/16)+3; the result layout is that of the
// 16x16x32 product.
template <int MT> struct Mma16;
template <> struct Mma16<kF16> {
  typedef _Float16 elem;
  typedef _Float16 v4 __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ f32x4_t mma(const v4& a, const v4& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
  // p = hi + lo + (error <= 2^-22 |p|): both halves as f16 codes
  static __device__ __forceinline__ void split(float p, uint16_t& hi, uint16_t& lo) {
    const _Float16 h = (_Float16)p;
    hi = __builtin_bit_cast(uint16_t, h);
    lo = __builtin_bit_cast(uint16_t, (_Float16)(p - (float)h));
  }
};
template <> struct Mma16<kBF16> {
  typedef short elem;
  typedef short v4 __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ f32x4_t mma(const v4& a, const v4& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
  // p = hi + lo + (error <= 2^-16 |p|): hi is p truncated to bf16, lo the truncated rest
  static __device__ __forceinline__ void split(float p, uint16_t& hi, uint16_t& lo) {
    const uint32_t u = __builtin_bit_cast(uint32_t, p);
    hi = (uint16_t)(u >> 16);
    const float rest = p - __builtin_bit_cast(float, u & 0xffff0000u);
    lo = (uint16_t)(__builtin_bit_cast(uint32_t, rest) >> 16);
  }
};

// V registers of one 16-token chunk in flight, in memory order: instruction i of lane l
// holds bytes 1024*i + 16*l .. +15 of the chunk's 16 V rows.
template <int KV, int D>
struct VTileRegs {
  static constexpr int NV = 16 * D * ElemBytes<KV>::value / 1024;
  uint4 v[NV > 0 ? NV : 1];
};

// Reductions over the four 16-lane rows of a wave (lanes l, l ^ 16, l ^ 32, l ^ 48), every
// lane receiving the result (pair exchanges rows_pair16 / rows_pair32).
__device__ __forceinline__ float rows4_max(float x) {
  float a, b;
  rows_pair16(x, a, b);
  rows_pair32(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float rows4_sum(float x) {
  float a, b;
  rows_pair16(x, a, b);
  rows_pair32(a + b, a, b);
  return a + b;
}

// Per-wave engine with both products on the matrix cores in transposed form, for G = 2, 4
// or 8 query heads per KV head (any supported KV type). Scores run as S^T = K Q^T
// (16x16x32: A = the chunk's K rows straight from the lanes' 16-byte loads, B = the query
// rows; row rho of the 16 holds head rho % G), so that lane l receives the scores of query
// row l % 16 for tokens 4 (l / 16) .. +3 of each 16-token tile: after the softmax these are
// exactly its B operand of O^T += V^T P^T (16x16x16, A = V^T read transposed from the
// wave's LDS copy of the V tile: ds_read_b64_tr_b16 gives lane i of a 16-lane group
// column i of four rows). The
// probabilities never leave the registers (high and low 16-bit halves, fp32 accuracy), and
// each lane keeps the running max and exp-sum of its own row; the four lanes of a row take
// identical decisions. The lazy raise of the running max is decided per row, so a row's
// arithmetic depends only on its own scores. fp8 K is converted to the MFMA type in
// registers and fp8 V while it is written to LDS (both exact). Chunks are NT 16-token tiles.
template <int IO, int KV, int D, int BS, int G, int NT, bool DBG>
struct MfmaTEngine {
  using Geo = MfmaGeo<KV, D>;
  static constexpr int CT = 16 * NT;
  static constexpr int NBC = CT >= BS ? CT / BS : 1;
  static constexpr int RB = Geo::RB;
  static constexpr int TILE_BYTES = BS * RB;
  static constexpr int NDT = D / 16;
  static constexpr int NV = VTileRegs<KV, D>::NV;  // V loads per lane per 16-token tile
  // 16-bit elements per LDS tile row: rows padded by 32 B spread the transposed reads of
  // four rows over the banks (other pads measured the same or worse for fp8 KV)
  static constexpr int VT_ROW = D + 16;
  static constexpr int VT_BYTES = 16 * VT_ROW * 2;
  // Type of the V product. bf16 V keeps bf16 with the probabilities split into a high and
  // a low half (fp32 accuracy). f16 V, and fp8 V widened to f16 (exact: every e4m3 value is
  // an f16 value), take the probabilities rounded to f16 in one product: relative error at
  // most 2^-12 per weight, below 1.2e-3 of the largest |V| in the output.
  static constexpr int PVT = KV == kBF16 ? kBF16 : kF16;
  static constexpr bool SPLIT_P = PVT == kBF16;
  static constexpr int kLdsBytes = NT * VT_BYTES;
  // K staging (blocks of at least 16 tokens, so a tile's 16 rows are contiguous): K is
  // loaded as whole 1 KiB runs of the tile, as V is, and put into the MFMA layout (lane
  // (n, lg): row n, chunks 4i + lg) through the wave's LDS tile, whose rows are padded by
  // 16 bytes so that each 16-lane quarter of a read or write meets 16 distinct 16-byte bank
  // groups. Loaded row by row instead, every K load instruction touched 16 half-used
  // 128-byte lines: the shared-prefix batch, whose K rows mostly come from L2, took 32.0
  // instead of 26.5 us that way.
  static constexpr bool KSTAGE = BS >= 16;
  static constexpr int KT_ROW = RB + 16;  // bytes per staged K row
  static_assert(!KSTAGE || 16 * KT_ROW <= VT_BYTES, "K tile fits the V tile's LDS");
  using vec = typename Mma<IO>::vec;
  using M16 = Mma16<PVT>;
  using v4 = typename M16::v4;
  static_assert(G == 2 || G == 4 || G == 8, "group");
  static_assert(mfma_supported<IO, KV, D, G>(), "unsupported MFMA decode geometry");
  static_assert(NV >= 1 && 16 * RB % 1024 == 0, "V tile of whole wave loads");
  static_assert(CT % BS == 0 || BS % CT == 0, "chunks and blocks nest");

  struct Buf {
    uint4 kr[NT][Geo::CPL];
    VTileRegs<KV, D> vt[NT];
  };

  LaneIds li;
  int s, g, t_end, j_end;
  int base, k0, len, rot, wave, nw;
  const int32_t* bt;
  const char* kbase;
  const char* vbase;
  int64_t blk_stride;
  int win[2][NBC];
  int cur_win;
  vec qa[Geo::NST];
  float m, l;       // running max (log2 units) of row li.n, this lane's part of its exp-sum
  f32x4_t o[NDT];   // O^T: register r of tile dt holds column 16 dt + 4 lg + r of row li.n
  char* lds;        // this wave's V tiles

  __device__ __forceinline__ MfmaTEngine(int lane, char* wave_lds) : li(lane), lds(wave_lds) {}

  __device__ __forceinline__ int chunk_token(int k) const {
    return base + CT * (k0 + rotated(wave + k * nw, rot, len));
  }

  // Raw table entries of the wave's chunks 64w .. 64w+63 (lane l: chunk 64w + l); entries
  // of chunks or blocks past the end read entry 0 of the row instead (never used for a
  // valid token). Ids are clamped into the pool when they are taken (block_off).
  __device__ __forceinline__ void load_window(const DecodeArgs& a, int w, int (&dst)[NBC]) {
    const int k = 64 * w + li.lane;
    const bool live = wave + k * nw < len;
    const int j = live ? chunk_token(k) / BS : 0;
#pragma unroll
    for (int u = 0; u < NBC; ++u) dst[u] = bt[live && j + u < j_end ? j + u : 0];
  }

  // Byte offset of the u-th block of chunk k (k in the current window), its id clamped
  // into the pool so that a bad table never reads outside it (contract: 0 <= id < num_blocks).
  __device__ __forceinline__ int64_t block_off(const DecodeArgs& a, int u, int k) const {
    const int b = __builtin_amdgcn_readlane(win[0][u], k & 63);
    return (int64_t)min(max(b, 0), a.num_blocks - 1) * blk_stride;
  }

  __device__ __forceinline__ void begin(const DecodeArgs& a, int s_, int g_, int t_end_, int base_,
                                        int k0_, int len_, int rot_, int wave_, int nw_) {
    s = s_;
    g = g_;
    t_end = t_end_;
    j_end = (t_end + BS - 1) / BS;
    base = base_;
    k0 = k0_;
    len = len_;
    rot = rot_;
    wave = wave_;
    nw = nw_;
    bt = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
    blk_stride = (int64_t)a.num_kv_heads * TILE_BYTES;
    kbase = (const char*)a.k_pool + (int64_t)g * TILE_BYTES;
    vbase = (const char*)a.v_pool + (int64_t)g * TILE_BYTES;
    load_window(a, 0, win[0]);
    load_window(a, 1, win[1]);
    cur_win = 0;
    load_q<IO, KV, D, G>(a, s, g, li, qa);
    m = -3.0e38f;
    l = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // Block offset of token t of the chunk starting at c0 (jb = c0 / BS).
  __device__ __forceinline__ int64_t tok_block(const int64_t (&off)[NBC], int t, int jb) const {
    int64_t bo = off[0];
#pragma unroll
    for (int u = 1; u < NBC; ++u) bo = t / BS - jb == u ? off[u] : bo;
    return bo;
  }

  // live = false: the chunk is not consumed and every lane reads its first row
  __device__ __forceinline__ void issue(const DecodeArgs& a, Buf& b, int k, bool live) {
    if ((k >> 6) != cur_win) {
      cur_win = k >> 6;
#pragma unroll
      for (int u = 0; u < NBC; ++u) win[0][u] = win[1][u];
      load_window(a, cur_win + 1, win[1]);
    }
    int64_t off[NBC];
#pragma unroll
    for (int u = 0; u < NBC; ++u) off[u] = block_off(a, u, k);
    const int c0 = chunk_token(k);
    const int jb = c0 / BS;
    // Rows at or past t_end read token c0's row instead (finite data already being
    // fetched; their scores are excluded by select): every load is unconditional. V loads
    // are non-temporal, K loads plain: the mixed fp8 batch takes 196 instead of 213 us and
    // the 8-head batch 99 instead of 108, while the shared-prefix batch, whose K rows L2
    // serves to every sequence, keeps its time (non-temporal K: 38.7 against 34.6 us).
    const int te = live ? t_end : 0;
#pragma unroll
    for (int tau = 0; tau < NT; ++tau) {
      if constexpr (KSTAGE) {
        // K: instruction i covers bytes 1024 i .. of the tile's 16 rows (rows at or past
        // t_end read the tile's first row)
        const int t0 = c0 + 16 * tau;
        const char* ktile = kbase + tok_block(off, t0, jb) + (t0 % BS) * RB;
#pragma unroll
        for (int i = 0; i < Geo::CPL; ++i) {
          const int byte = 1024 * i + 16 * li.lane;
          b.kr[tau][i] = load16(ktile + (t0 + byte / RB < te ? byte : byte % RB));
        }
      } else {
        int to = c0 + 16 * tau + li.n;  // K: lane (n, lg) loads chunks 4i + lg of token n
        to = to < te ? to : c0;
        const char* krow = kbase + tok_block(off, to, jb) + (to % BS) * RB;
#pragma unroll
        for (int i = 0; i < Geo::CPL; ++i) b.kr[tau][i] = load16(krow + 16 * (4 * i + li.lg));
      }
#pragma unroll
      for (int i = 0; i < NV; ++i) {  // V: instruction i covers bytes 1024 i .. of the tile's 16 rows
        const int byte = 1024 * i + 16 * li.lane;
        int t = c0 + 16 * tau + byte / RB;
        t = t < te ? t : c0;
        b.vt[tau].v[i] = load16<true>(vbase + tok_block(off, t, jb) + (t % BS) * RB + byte % RB);
      }
    }
  }

  __device__ __forceinline__ void trace(const DecodeArgs& a, const Buf& b, int c0) {
    const int Hkv = a.num_kv_heads;
    const int64_t row0 = ((int64_t)s * Hkv + g) * a.dbg_max_ctx;
#pragma unroll
    for (int tau = 0; tau < NT; ++tau) {
      if constexpr (KSTAGE) {
#pragma unroll
        for (int i = 0; i < Geo::CPL; ++i) {
          const int byte = 1024 * i + 16 * li.lane;
          const int t = c0 + 16 * tau + byte / RB;
          if (t < t_end) {
            *(uint4*)((char*)a.dbg_k + (row0 + t) * RB + byte % RB) = b.kr[tau][i];
            if (byte % RB == 0) atomicAdd(a.dbg_counts + row0 + t, 1);
          }
        }
      } else {
        const int to = c0 + 16 * tau + li.n;
        if (to < t_end) {
#pragma unroll
          for (int i = 0; i < Geo::CPL; ++i)
            *(uint4*)((char*)a.dbg_k + (row0 + to) * RB + 16 * (4 * i + li.lg)) = b.kr[tau][i];
          if (li.lg == 0) atomicAdd(a.dbg_counts + row0 + to, 1);
        }
      }
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int byte = 1024 * i + 16 * li.lane;
        const int t = c0 + 16 * tau + byte / RB;
        if (t < t_end) *(uint4*)((char*)a.dbg_v + (row0 + t) * RB + byte % RB) = b.vt[tau].v[i];
      }
    }
  }

  // Lanes of one wave exchange data through LDS: a wave-scope fence keeps the compiler
  // from moving a lane's LDS reads above other lanes' writes (the hardware executes one
  // wave's LDS instructions in order).
  static __device__ __forceinline__ void lds_exchange() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }

  __device__ __forceinline__ void consume(const DecodeArgs& a, const Buf& b, int k) {
    const int c0 = chunk_token(k);
    if constexpr (DBG) trace(a, b, c0);

    // the previous chunk's transposed reads of the tiles come before these writes
    lds_exchange();
    // K in the MFMA layout: staged through the tiles (read back before V overwrites them)
    uint4 kr[NT][Geo::CPL];
    if constexpr (KSTAGE) {
#pragma unroll
      for (int tau = 0; tau < NT; ++tau) {
        char* kt = lds + tau * VT_BYTES;
#pragma unroll
        for (int i = 0; i < Geo::CPL; ++i) {
          const int byte = 1024 * i + 16 * li.lane;
          *(uint4*)(kt + (byte / RB) * KT_ROW + byte % RB) = b.kr[tau][i];
        }
      }
      lds_exchange();
#pragma unroll
      for (int tau = 0; tau < NT; ++tau) {
        const char* kt = lds + tau * VT_BYTES;
#pragma unroll
        for (int i = 0; i < Geo::CPL; ++i) kr[tau][i] = *(const uint4*)(kt + li.n * KT_ROW + 16 * (4 * i + li.lg));
      }
      lds_exchange();
    } else {
#pragma unroll
      for (int tau = 0; tau < NT; ++tau)
#pragma unroll
        for (int i = 0; i < Geo::CPL; ++i) kr[tau][i] = b.kr[tau][i];
    }
#pragma unroll
    for (int tau = 0; tau < NT; ++tau) {
      uint16_t* vt = (uint16_t*)(lds + tau * VT_BYTES);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int byte = 1024 * i + 16 * li.lane;
        const int t = byte / RB;
        const int col = (byte % RB) / ElemBytes<KV>::value;
        if constexpr (KV == kFP8) {
          const uint4 r = b.vt[tau].v[i];
          const uint32_t w[4] = {r.x, r.y, r.z, r.w};
          uint32_t packed[8];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            packed[2 * q] = fp8x2_to_mt<PVT, false>(w[q]);
            packed[2 * q + 1] = fp8x2_to_mt<PVT, true>(w[q]);
          }
          *(uint4*)(vt + t * VT_ROW + col) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
          *(uint4*)(vt + t * VT_ROW + col + 8) = make_uint4(packed[4], packed[5], packed[6], packed[7]);
        } else {
          *(uint4*)(vt + t * VT_ROW + col) = b.vt[tau].v[i];
        }
      }
    }
    // the tiles are read back by other lanes of the wave (transposed)
    lds_exchange();

    // S^T: lane l gets row li.n's scores of tokens 4 lg + r of each tile (log2 units)
    float z[NT][4];
    float mx = -INFINITY;
#pragma unroll
    for (int tau = 0; tau < NT; ++tau) {
      f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < Geo::CPL; ++i)
#pragma unroll
        for (int hf = 0; hf < Geo::VEC / 8; ++hf)
          c = Mma<IO>::mma(k_operand<IO, KV>(kr[tau][i], hf), qa[i * (Geo::VEC / 8) + hf], c);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = c0 + 16 * tau + 4 * li.lg + r < t_end;
        z[tau][r] = ok ? c[r] * a.q_mul : -INFINITY;
        mx = fmaxf(mx, z[tau][r]);
      }
    }
    // the row's maximum over its four lanes
    mx = rows4_max(mx);
    const bool raise = mx > m + kLazyRescale;
    if (__any(raise)) {
      const float mn = raise ? mx : m;
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      m = mn;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[dt][r] *= alpha;
    }

    // probabilities as the B operand (bf16: high and low halves), then O^T += V^T P^T
    const int vrow = 4 * li.lg + (li.n >> 2);
    const int vcol = 4 * (li.n & 3);
    using elem = typename M16::elem;
#pragma unroll
    for (int tau = 0; tau < NT; ++tau) {
      v4 phi, plo;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(z[tau][r] - m);
        l += p;
        if constexpr (SPLIT_P) {
          uint16_t hi, lo;
          M16::split(p, hi, lo);
          phi[r] = __builtin_bit_cast(elem, hi);
          plo[r] = __builtin_bit_cast(elem, lo);
        } else {
          phi[r] = (_Float16)p;
        }
      }
      const uint16_t* vt = (const uint16_t*)(lds + tau * VT_BYTES);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const v4 av = __builtin_bit_cast(
            v4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) i16x4_t*)(vt + vrow * VT_ROW + 16 * dt + vcol)));
        o[dt] = M16::mma(av, phi, o[dt]);
        if constexpr (SPLIT_P) o[dt] = M16::mma(av, plo, o[dt]);
      }
    }
  }

  __device__ __forceinline__ void run(const DecodeArgs& a) {
    const int nwc = wave < len ? (len - wave + nw - 1) / nw : 0;
    run_pipelined(*this, a, nwc);
  }

  // Row li.n < G is head li.n: its four lanes store their columns; lane lg 0 the max and sum.
  template <int NW>
  __device__ __forceinline__ void finish(float (&sm_m)[NW][G], float (&sm_l)[NW][G],
                                         float (&sm_o)[NW][G][D]) {
    const float lt = rows4_sum(l);
    if (li.n < G) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) sm_o[wave][li.n][16 * dt + 4 * li.lg + r] = o[dt][r];
      if (li.lg == 0) {
        sm_m[wave][li.n] = m;
        sm_l[wave][li.n] = lt;
      }
    }
  }
};

// Engine used for a shape: one query head per KV head takes the vector engine (whole
// 1 KiB rows per wave load, no matrix-core rows wasted); 2, 4 or 8 take the transposed
// matrix-core engine.
#ifndef PA_T_TILES
#define PA_T_TILES 1
#endif
#ifndef PA_T_TILES_FP8
#define PA_T_TILES_FP8 1
#endif
template <int IO, int KV, int D, int BS, int G, bool DBG>
struct EngineFor {
  static constexpr bool valu = G == 1;
  static constexpr int TNT = KV == kFP8 ? PA_T_TILES_FP8 : PA_T_TILES;
  using type = typename std::conditional<valu, ValuEngine<IO, KV, D, BS, G, DBG>,
                                         MfmaTEngine<IO, KV, D, BS, (valu ? 2 : G), TNT, DBG>>::type;
  static constexpr int lds_bytes = valu ? 16 : MfmaTEngine<IO, KV, D, BS, (valu ? 2 : G), TNT, DBG>::kLdsBytes;
};

template <class Eng> struct EngineMaker;  // builds an engine with or without its LDS tile
template <int IO, int KV, int D, int BS, int G, bool DBG>
struct EngineMaker<ValuEngine<IO, KV, D, BS, G, DBG>> {
  static __device__ __forceinline__ ValuEngine<IO, KV, D, BS, G, DBG> make(int lane, char*) {
    return ValuEngine<IO, KV, D, BS, G, DBG>(lane);
  }
};
template <int IO, int KV, int D, int BS, int G, int NT, bool DBG>
struct EngineMaker<MfmaTEngine<IO, KV, D, BS, G, NT, DBG>> {
  static __device__ __forceinline__ MfmaTEngine<IO, KV, D, BS, G, NT, DBG> make(int lane, char* lds) {
    return MfmaTEngine<IO, KV, D, BS, G, NT, DBG>(lane, lds);
  }
};

// Merge of the NW wave states in LDS for element (head gi, column d): running max M,
// sum of exp2(m - M) * l and of exp2(m - M) * o.
template <int NW, int G, int D>
__device__ __forceinline__ void merge_waves(const float (&sm_m)[NW][G], const float (&sm_l)[NW][G],
                                            const float (&sm_o)[NW][G][D], int gi, int d, float& Mx,
                                            float& lsum, float& o) {
  Mx = sm_m[0][gi];
#pragma unroll
  for (int w = 1; w < NW; ++w) Mx = fmaxf(Mx, sm_m[w][gi]);
  o = 0.f;
  lsum = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const float f = __builtin_amdgcn_exp2f(sm_m[w][gi] - Mx);
    o = fmaf(f, sm_o[w][gi][d], o);
    lsum = fmaf(f, sm_l[w][gi], lsum);
  }
}

template <int IO, int KV, int D, int BS, int G, int NW, bool DBG>
__global__ void __launch_bounds__(NW * 64)
mfma_decode_kernel(const DecodeArgs a) {
  using Sel = EngineFor<IO, KV, D, BS, G, DBG>;
  using Eng = typename Sel::type;
  constexpr int CT = Eng::CT;

  __shared__ __align__(16) char sm_eng[NW][Sel::lds_bytes];
  __shared__ float sm_m[NW][G];
  __shared__ float sm_l[NW][G];
  __shared__ float sm_o[NW][G][D];

  __shared__ OrderLds sm_ord;
  const int unit = xcd_unit((int)blockIdx.x, (int)gridDim.x);
  const int part = unit % a.num_parts;
  const int sg = unit / a.num_parts;
  int s, g;
  unit_seq<NW * 64>(a, sg, sm_ord, s, g);

  int L = a.context_lens[s];
  L = min(max(L, 0), a.max_ctx);
  const int t_begin = part * a.part_tokens;
  if (part > 0 && t_begin >= L) return;  // nothing in this partition (whole workgroup)
  const int t_end = min(L, t_begin + a.part_tokens);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  Eng eng = EngineMaker<Eng>::make(threadIdx.x & 63, sm_eng[wave]);
  const int nch = (t_end - t_begin + CT - 1) / CT;
  const int rot = PA_STAGGER ? (s * 5) % max(nch, 1) : 0;
  eng.begin(a, s, g, t_end, t_begin, 0, nch, rot, wave, NW);
  eng.run(a);
  eng.template finish<NW>(sm_m, sm_l, sm_o);
  __syncthreads();

  // merge the waves and write
  const int H = a.num_heads;
  const int n_parts_s = (L + a.part_tokens - 1) / a.part_tokens;
  const bool write_out = n_parts_s <= 1;
  for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
    const int gi = idx / D;
    const int d = idx % D;
    float Mx, lsum, o;
    merge_waves<NW, G, D>(sm_m, sm_l, sm_o, gi, d, Mx, lsum, o);
    const int h = g * G + gi;
    if (write_out) {
      const float v = lsum > 0.f ? (o / lsum) * a.out_mul : 0.f;
      store_io<IO>(a.out, ((int64_t)s * H + h) * D + d, v);
    } else {
      const int64_t NPH = (int64_t)a.num_seqs * H * a.num_parts;
      const int64_t slot = ((int64_t)s * H + h) * a.num_parts + part;
      a.ws[2 * NPH + slot * D + d] = o * a.out_mul;
      if (d == 0) {
        a.ws[slot] = Mx;
        a.ws[NPH + slot] = lsum;
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// balanced scheduler
// ---------------------------------------------------------------------------------

// First chunk of logical workgroup w when C chunks are shared by nwg workgroups.
__device__ __forceinline__ int64_t chunk_begin(int64_t w, int64_t C, int64_t nwg) {
  return w * C / nwg;
}
// Logical workgroup whose range holds chunk x (every range is non-empty when nwg <= C).
__device__ __forceinline__ int64_t chunk_owner(int64_t x, int64_t C, int64_t nwg) {
  return ((x + 1) * nwg - 1) / C;
}

// Floats per partial-state slot: m[G], l[G], o[G][D].
template <int G, int D> constexpr int slot_floats() { return G * (D + 2); }

// At least two waves per SIMD (the default grid is two workgroups per CU): the register
// allocator must fit VGPRs and AGPRs together into 256 per lane.
template <int IO, int KV, int D, int BS, int G, int NW, bool DBG>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
balanced_decode_kernel(const DecodeArgs a) {
  using Sel = EngineFor<IO, KV, D, BS, G, DBG>;
  using Eng = typename Sel::type;
  constexpr int CT = Eng::CT;
  constexpr int NTH = NW * 64;
  constexpr int SLOT = slot_floats<G, D>();

  __shared__ float sm_m[NW][G];
  __shared__ float sm_l[NW][G];
  __shared__ float sm_o[NW][G][D];
  __shared__ int sm_pref[kMaxBalancedSeqs + 1];  // exclusive prefix sums of chunk counts
  __shared__ int sm_wsum[NW];
  __shared__ int sm_last;
  __shared__ __align__(16) char sm_eng[NW][Sel::lds_bytes];

  const int S = a.num_seqs;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;

  // 1. cost of each sequence in chunk units: kSegCost for the fixed work of a segment
  //    (set-up, wave merge, write) plus its chunks (at least one, so that empty sequences
  //    get their zero output written); exclusive prefix sums of the costs, thread t owning
  //    a contiguous run of S/NTH sequences. Real chunk k of sequence s sits at cost
  //    position sm_pref[s] + kSegCost + k.
  const int per = (S + NTH - 1) / NTH;
  const int i0 = min(S, tid * per);
  const int i1 = min(S, i0 + per);
  int local = 0;
  for (int i = i0; i < i1; ++i) {
    const int L = min(max(a.context_lens[i], 0), a.max_ctx);
    local += kSegCost + max(1, (L + CT - 1) / CT);
  }
  int incl = local;  // inclusive scan over the wave
#pragma unroll
  for (int k = 1; k < 64; k <<= 1) {
    const int y = __shfl_up(incl, k);
    if (lane >= k) incl += y;
  }
  if (lane == 63) sm_wsum[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += sm_wsum[w];
  int run = base + incl - local;
  for (int i = i0; i < i1; ++i) {
    sm_pref[i] = run;
    const int L = min(max(a.context_lens[i], 0), a.max_ctx);
    run += kSegCost + max(1, (L + CT - 1) / CT);
  }
  if (tid == NTH - 1) {
    int tot = 0;
    for (int w = 0; w < NW; ++w) tot += sm_wsum[w];
    sm_pref[S] = tot;
  }
  __syncthreads();

  // 2. this workgroup's range [cb, ce) of the C = Hkv * Cg cost positions (KV-head major)
  const int Cg = sm_pref[S];
  const int64_t C = (int64_t)a.num_kv_heads * Cg;
  const int64_t nwg = min((int64_t)a.nwg, C);
  const int64_t v = xcd_unit((int)blockIdx.x, (int)gridDim.x);
  if (v >= nwg) return;  // more workgroups than cost positions (whole workgroup)
  const int64_t cb = chunk_begin(v, C, nwg);
  const int64_t ce = chunk_begin(v + 1, C, nwg);

  Eng eng = EngineMaker<Eng>::make(lane, sm_eng[wave]);
  const int H = a.num_heads;
  int64_t c = cb;
  while (c < ce) {
    const int g = (int)(c / Cg);
    const int r = (int)(c - (int64_t)g * Cg);
    // sequence s with sm_pref[s] <= r < sm_pref[s + 1] (prefix sums strictly increase)
    int lo = 0, hi = S;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (sm_pref[mid] <= r) lo = mid; else hi = mid;
    }
    const int s = lo;
    const int u0 = sm_pref[s] + kSegCost;  // cost position of real chunk 0
    const int nch = sm_pref[s + 1] - u0;
    const int64_t seg_end = min((int64_t)g * Cg + sm_pref[s + 1], ce);
    const int k0 = max(0, r - u0);
    const int k1 = (int)max((int64_t)0, seg_end - (int64_t)g * Cg - u0);
    c = seg_end;
    if (k1 <= k0) continue;  // only the fixed-cost part of this sequence is in the range
    const int len = k1 - k0;
    const int L = min(max(a.context_lens[s], 0), a.max_ctx);

    const int rot = PA_STAGGER ? (s * 5) % len : 0;
    eng.begin(a, s, g, L, 0, k0, len, rot, wave, NW);
    eng.run(a);
    eng.template finish<NW>(sm_m, sm_l, sm_o);
    __syncthreads();

    if (k0 == 0 && k1 == nch) {
      // the whole (sequence, KV head) is here: normalise and write
      for (int idx = tid; idx < G * D; idx += NTH) {
        const int gi = idx / D;
        const int d = idx % D;
        float Mx, lsum, o;
        merge_waves<NW, G, D>(sm_m, sm_l, sm_o, gi, d, Mx, lsum, o);
        const float val = lsum > 0.f ? (o / lsum) * a.out_mul : 0.f;
        store_io<IO>(a.out, ((int64_t)s * H + g * G + gi) * D + d, val);
      }
    } else {
      // a piece: store (m, l, o) in one of this workgroup's two slots, then count the
      // arrival. Slot 0 holds the piece of the (sequence, KV head) that began at or before
      // the start of the workgroup's range (cb >= ub), slot 1 the piece of the one that
      // begins inside the range and runs past its end (at most one of each).
      const int64_t ub = (int64_t)g * Cg + u0;  // cost position of this (s, g)'s first chunk
      float* slot = a.ws + ((int64_t)v * 2 + (cb >= ub ? 0 : 1)) * SLOT;
      for (int idx = tid; idx < G * D; idx += NTH) {
        const int gi = idx / D;
        const int d = idx % D;
        float Mx, lsum, o;
        merge_waves<NW, G, D>(sm_m, sm_l, sm_o, gi, d, Mx, lsum, o);
        __hip_atomic_store(slot + 2 * G + gi * D + d, o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (d == 0) {
          __hip_atomic_store(slot + gi, Mx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(slot + G + gi, lsum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      // Hand-off between workgroups, which may run on different XCDs (each with its own
      // L2). Every slot store above and every slot load below is an agent-scope atomic,
      // performed at the device's coherence point rather than in an XCD's L2 (sc1). Each
      // wave waits until its slot stores have completed (vmcnt 0) before the barrier, so
      // all of this workgroup's stores are done before its arrival is counted; the last
      // arriver reads the slots only after its own arrival returned, and only with
      // agent-scope atomic loads. No access to the slots goes through a non-coherent
      // cache, so no cache write-back or invalidation is needed. (An agent-scope release
      // fence and acquire fence in their place write back and invalidate the whole L2 of
      // the XCD for every piece: the mixed fp8 batch took 420 instead of 218 us.)
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      const int64_t w0 = chunk_owner(ub, C, nwg);
      const int64_t w1 = chunk_owner(ub + nch - 1, C, nwg);
      int32_t* counter = a.counters + (int64_t)g * S + s;
      if (tid == 0) {
        const int old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sm_last = old == (int)(w1 - w0);
      }
      __syncthreads();
      if (sm_last) {
        // last piece to arrive: merge all pieces of (s, g) and write the output
        for (int idx = tid; idx < G * D; idx += NTH) {
          const int gi = idx / D;
          const int d = idx % D;
          float Mx = -3.0e38f;
          for (int64_t w = w0; w <= w1; ++w) {
            const int pos = chunk_begin(w, C, nwg) >= ub ? 0 : 1;
            const float* ps = a.ws + (w * 2 + pos) * SLOT;
            Mx = fmaxf(Mx, __hip_atomic_load(ps + gi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
          }
          float o = 0.f, lsum = 0.f;
          for (int64_t w = w0; w <= w1; ++w) {
            const int pos = chunk_begin(w, C, nwg) >= ub ? 0 : 1;
            const float* ps = a.ws + (w * 2 + pos) * SLOT;
            const float m = __hip_atomic_load(ps + gi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const float f = __builtin_amdgcn_exp2f(m - Mx);
            lsum = fmaf(f, __hip_atomic_load(ps + G + gi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), lsum);
            o = fmaf(f, __hip_atomic_load(ps + 2 * G + gi * D + d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), o);
          }
          const float val = lsum > 0.f ? (o / lsum) * a.out_mul : 0.f;
          store_io<IO>(a.out, ((int64_t)s * H + g * G + gi) * D + d, val);
        }
        // leave the counter at zero for the next call
        if (tid == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();  // LDS is reused by the next segment
  }
}

}  // namespace pa
