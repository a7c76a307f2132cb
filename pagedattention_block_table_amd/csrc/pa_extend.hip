// Paged attention for several new query tokens per sequence (prefill / extend).
//
// Pages cited by title and section:
//   [P2] vLLM architecture deep-dive §2.1 — the engine runs prefill (the prompt), decode
//        and extend (long texts); §2.2 — the attention metadata holds block tables,
//        context lengths and query lengths.
//   [P1] "突破GPU内存瓶颈：vLLM与PagedAttention技术深度解析" §2 — the block table maps a
//        sequence's logical blocks to physical blocks of the pool.
//   [P3] "内存优化：KV Cache管理、PagedAttention原理与内存池配置" — tokens attend over the
//        cached keys and values of their request.
//
// Sequence s has L = context_lens[s] cached tokens, the last Q of them new, with queries
// q[query_start_loc[s] + i], i < Q. New token i sits at position p = L - Q + i and
// attends over positions 0 .. p (causal), through the block table.
//
// One workgroup (4 waves) takes 64 query rows of one (sequence, KV head): 64 / G new
// tokens times the G query heads of the group. Wave w owns rows 16w .. 16w+15 (row r is
// token r / G, head r % G of the tile). The workgroup walks the keys in 32-token chunks:
// all 256 lanes copy a chunk's K and V rows (looked up through the block table, fp8
// widened exactly to the 16-bit MFMA type, rows past L zeroed) into LDS, double
// buffered, with the next chunk's global loads in flight during the current one.
//
// Both products run on the matrix cores as v_mfma_f32_16x16x32 in the transposed
// orientation, which keeps the probabilities in the registers that computed them:
//   S^T[token][row] = K[token][:] . Q[row][:]   A = K rows from LDS, B = Q^T (registers)
//   O^T[d][row]    += V^T[d][token] P^T[token][row]
// Lane (n = l%16, q = l/16) receives S^T rows 4q + r of both 16-token halves of the
// chunk for query row n: tokens 4q + r and 16 + 4q + r. The k order inside an MFMA is
// free, so k = 8q + j stands for token 4q + j (j < 4) and 16 + 4q + j - 4 (j >= 4) in
// both operands: the lane's own eight probabilities form its B operand, and its A
// operand (V^T, row d = n) is two transposed LDS reads (ds_read_b64_tr_b16) of rows
// 4q .. 4q+3 and 16+4q .. 16+4q+3. fp8 V is widened to f16 (exact) and takes the
// probabilities rounded to f16 in one product (relative error <= 2^-12 per weight). Online
// softmax per query row in log2 units, the running max shared by the row's four lanes and
// raised lazily.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>

#include "pa.h"
#include "pa_decode_impl.h"

namespace pa {
namespace {

struct ExtendArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start_loc;
  void* out;
  int num_seqs;
  int max_blocks_per_seq;
  int num_blocks;
  int num_heads;
  int num_kv_heads;
  int bs_shift;   // log2(block_size)
  int q_tiles;    // workgroups per (sequence, KV head)
  float q_mul;    // scale * log2(e) * k_scale
  float v_scale;
  int skip_q;     // sequences with at most this many new tokens run elsewhere (0: none)
};

// max of three scores in one instruction, without the canonicalizing moves fmaxf adds
// (scores are finite dot products or the -inf of a masked slot for finite inputs)
__device__ __forceinline__ float max3(float x, float y, float z) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(y), "v"(z));
  return r;
}

constexpr int kExtWaves = 4;
constexpr int kExtRows = 16 * kExtWaves;  // query rows per workgroup
constexpr int kExtChunk = 32;             // key tokens per step

template <int IO, int KV, int D>
struct ExtGeo {
  static constexpr int E = ElemBytes<KV>::value;
  static constexpr int PPR = D * E / 16;                           // 16-byte pieces per row
  static constexpr int PIECES = kExtChunk * PPR;                   // per chunk, K (and V)
  static constexpr int NPT = (PIECES + kExtWaves * 64 - 1) / (kExtWaves * 64);  // per thread
  static constexpr int VPP = 16 / E;                               // values per piece
  static constexpr int KROW = D + 8;     // LDS K row, 16-bit elements (16-byte pad)
  static constexpr int VROW = D + 16;    // LDS V row (32-byte pad: transposed reads spread)
  static constexpr int K_BYTES = kExtChunk * KROW * 2;
  static constexpr int V_BYTES = kExtChunk * VROW * 2;
  static constexpr int BUF_BYTES = K_BYTES + V_BYTES;
  static constexpr int NKS = D / 32;     // k-steps of the score product
  static constexpr int NDT = D / 16;     // 16-column tiles of head_dim
};

// one 16-byte global piece -> LDS row slot in the MFMA type (fp8 widened exactly)
template <int IO, int KV>
__device__ __forceinline__ void put_piece(uint16_t* dst, const uint4& r) {
  if constexpr (KV == kFP8) {
    const uint4 lo = __builtin_bit_cast(uint4, fp8x8_operand<IO>(r.x, r.y));
    const uint4 hi = __builtin_bit_cast(uint4, fp8x8_operand<IO>(r.z, r.w));
    *(uint4*)dst = lo;
    *(uint4*)(dst + 8) = hi;
  } else {
    *(uint4*)dst = r;
  }
}

template <int IO, int KV, int D, int G>
__global__ void __launch_bounds__(kExtWaves * 64) extend_kernel(const ExtendArgs a) {
  using Geo = ExtGeo<IO, KV, D>;
  using vec = typename Mma<IO>::vec;
  // Type of the V product: fp8 V widened to f16 (exact: every e4m3 value is an f16 value)
  // with the probabilities rounded to f16 in one product (relative error <= 2^-12 per
  // weight); bf16 V keeps bf16 with the probabilities split in high and low halves.
  constexpr int PVT = KV == kFP8 ? kF16 : IO;
  using pvec = typename Mma<PVT>::vec;
  using M16 = Mma16<PVT>;
  constexpr int QT = kExtRows / G;  // new tokens per workgroup
  static_assert(kExtRows % G == 0 && 16 % G == 0, "group");

  __shared__ __attribute__((aligned(16))) char lds[2 * Geo::BUF_BYTES];

  // units: (sequence, KV head, query tile), tiles of one (s, g) adjacent (same XCD),
  // heaviest tile (last tokens: longest causal range) first
  const int unit = xcd_unit((int)blockIdx.x, (int)gridDim.x);
  const int qt = a.q_tiles - 1 - unit % a.q_tiles;
  const int sg = unit / a.q_tiles;
  // KV-head-major: each XCD's contiguous range of units holds a few KV heads of every
  // sequence (balanced however the context lengths differ); the query tiles of one
  // (sequence, KV head) stay together and share the chunks through that XCD's L2
  const int s = sg % a.num_seqs;
  const int g = sg / a.num_seqs;
  if (g >= a.num_kv_heads) return;

  const int q0 = a.query_start_loc[s];
  const int Q = a.query_start_loc[s + 1] - q0;
  const int i0 = qt * QT;
  // whole workgroup: no query rows here, or a short query the grouped decode kernel takes
  if (Q <= 0 || i0 >= Q || Q <= a.skip_q) return;
  const int cap = a.max_blocks_per_seq << a.bs_shift;
  const int L = min(max(a.context_lens[s], 0), cap);
  const int i_end = min(Q, i0 + QT);
  const int p0 = L - Q;                      // position of new token 0
  const int p_last = p0 + i_end - 1;         // last position any row of the tile attends to
  const int nch = p_last >= 0 ? p_last / kExtChunk + 1 : 0;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 15;
  const int lq = lane >> 4;

  // this lane's query row (column n of the wave's 16)
  const int row = 16 * wave + n;
  const int ti = i0 + row / G;
  const int h = g * G + row % G;
  const bool row_ok = ti < i_end;
  const int pos = p0 + ti;                   // may be < 0 outside the contract
  // the wave's position range (uniform)
  const int w_first = i0 + (16 * wave) / G;
  const int w_last = min(i_end, i0 + (16 * wave + 15) / G + 1) - 1;
  const bool wave_live = w_first < i_end;
  const int wp_min = p0 + w_first;
  const int wp_max = p0 + w_last;

  // Q^T operand: lane (n, lq) holds row n's head_dim values 32ks + 8lq .. +7
  vec qv[Geo::NKS];
  {
    const int64_t base = ((int64_t)(q0 + (row_ok ? ti : 0)) * a.num_heads + h) * D;
#pragma unroll
    for (int ks = 0; ks < Geo::NKS; ++ks) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (row_ok) w = *(const uint4*)((const char*)a.q + (base + 32 * ks + 8 * lq) * 2);
      qv[ks] = __builtin_bit_cast(vec, w);
    }
  }

  const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  const int bs_mask = (1 << a.bs_shift) - 1;
  const int64_t row_bytes = (int64_t)D * Geo::E;
  const int64_t tile_bytes = row_bytes << a.bs_shift;
  const int64_t blk_stride = tile_bytes * a.num_kv_heads;
  const char* kb = (const char*)a.k_pool + (int64_t)g * tile_bytes;
  const char* vb = (const char*)a.v_pool + (int64_t)g * tile_bytes;

  uint4 kreg[Geo::NPT], vreg[Geo::NPT];
  auto load_chunk = [&](int c) {
#pragma unroll
    for (int u = 0; u < Geo::NPT; ++u) {
      const int piece = tid + u * kExtWaves * 64;
      const int r = piece / Geo::PPR;
      const int col = piece % Geo::PPR;
      const int t = c * kExtChunk + r;
      uint4 kk = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (piece < Geo::PIECES && t < L) {
        // contract: 0 <= b < num_blocks; clamp so that a bad table never reads outside
        const int b = min(max(bt[t >> a.bs_shift], 0), a.num_blocks - 1);
        const int64_t off = (int64_t)b * blk_stride + (int64_t)(t & bs_mask) * row_bytes + 16 * col;
        kk = *(const uint4*)(kb + off);
        vv = *(const uint4*)(vb + off);
      }
      kreg[u] = kk;
      vreg[u] = vv;
    }
  };
  auto store_chunk = [&](int buf) {
    uint16_t* kt = (uint16_t*)(lds + buf * Geo::BUF_BYTES);
    uint16_t* vt = (uint16_t*)(lds + buf * Geo::BUF_BYTES + Geo::K_BYTES);
#pragma unroll
    for (int u = 0; u < Geo::NPT; ++u) {
      const int piece = tid + u * kExtWaves * 64;
      if (piece < Geo::PIECES) {
        const int r = piece / Geo::PPR;
        const int col = (piece % Geo::PPR) * Geo::VPP;
        put_piece<IO, KV>(kt + r * Geo::KROW + col, kreg[u]);
        put_piece<PVT, KV>(vt + r * Geo::VROW + col, vreg[u]);
      }
    }
  };

  // probabilities as f16 keep 11 significant bits; bf16 keeps 8, so there they go as
  // high + low halves
  constexpr bool SPLIT = PVT == kBF16;
  float m = -3.0e38f;  // running max of row n (log2 units), same in the row's 4 lanes
  f32x4_t lacc = f32x4_t{0.f, 0.f, 0.f, 0.f};  // softmax denominator of row n
  constexpr uint32_t kOne2 = PVT == kF16 ? 0x3C003C00u : 0x3F803F80u;  // two 16-bit 1.0
  const pvec ones = __builtin_bit_cast(pvec, make_uint4(kOne2, kOne2, kOne2, kOne2));
  f32x4_t o[Geo::NDT];
#pragma unroll
  for (int dt = 0; dt < Geo::NDT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (nch > 0) {
    load_chunk(0);
    store_chunk(0);
  }
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    if (c + 1 < nch) load_chunk(c + 1);
    const int t0 = c * kExtChunk;
    if (wave_live && t0 <= wp_max) {
      const uint16_t* kt = (const uint16_t*)(lds + (c & 1) * Geo::BUF_BYTES);
      const uint16_t* vt = (const uint16_t*)(lds + (c & 1) * Geo::BUF_BYTES + Geo::K_BYTES);
      // scores: S^T of the two 16-token halves
      f32x4_t acc[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        acc[hf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < Geo::NKS; ++ks) {
          const vec kop = *(const vec*)(kt + (16 * hf + n) * Geo::KROW + 32 * ks + 8 * lq);
          acc[hf] = Mma<IO>::mma(kop, qv[ks], acc[hf]);
        }
      }
      // z[j]: token t0 + 4lq + j (j < 4) and t0 + 16 + 4lq + j - 4 (j >= 4), raw dot
      // products (the scale is folded into the exponent; q_mul > 0)
      float z[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) z[j] = acc[j >> 2][j & 3];
      if (t0 + kExtChunk - 1 > wp_min) {  // uniform: only chunks that reach the diagonal
        asm volatile("" ::: "memory");
        const int lim = pos - t0 - 4 * lq;
#pragma unroll
        for (int j = 0; j < 8; ++j) z[j] = 16 * (j >> 2) + (j & 3) <= lim ? z[j] : -INFINITY;
      }
      // the row's four lanes exchange maxima only when one of them would raise the
      // row's max past the lazy-rescale threshold
      float mx = max3(max3(z[0], z[1], z[2]), max3(z[3], z[4], z[5]), fmaxf(z[6], z[7])) * a.q_mul;
      if (__builtin_amdgcn_ballot_w64(mx > m + kLazyRescale) != 0) {
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const bool raise = mx > m + kLazyRescale;
        const float mn = raise ? mx : m;
        const float alpha = __builtin_amdgcn_exp2f(m - mn);
        m = mn;
#pragma unroll
        for (int r = 0; r < 4; ++r) lacc[r] *= alpha;
#pragma unroll
        for (int dt = 0; dt < Geo::NDT; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[dt][r] *= alpha;
      }
      float p[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) p[j] = __builtin_amdgcn_exp2f(fmaf(z[j], a.q_mul, -m));
      pvec bhi, blo;
      if constexpr (SPLIT) {
        uint16_t phi[8], plo[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) M16::split(p[j], phi[j], plo[j]);
        uint4 bh, bl;
        bh.x = phi[0] | ((uint32_t)phi[1] << 16);
        bh.y = phi[2] | ((uint32_t)phi[3] << 16);
        bh.z = phi[4] | ((uint32_t)phi[5] << 16);
        bh.w = phi[6] | ((uint32_t)phi[7] << 16);
        bl.x = plo[0] | ((uint32_t)plo[1] << 16);
        bl.y = plo[2] | ((uint32_t)plo[3] << 16);
        bl.z = plo[4] | ((uint32_t)plo[5] << 16);
        bl.w = plo[6] | ((uint32_t)plo[7] << 16);
        bhi = __builtin_bit_cast(pvec, bh);
        blo = __builtin_bit_cast(pvec, bl);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) bhi[j] = (_Float16)p[j];
      }
      // the softmax denominator as one more tile with V^T = 1
      lacc = Mma<PVT>::mma(ones, bhi, lacc);
      if constexpr (SPLIT) lacc = Mma<PVT>::mma(ones, blo, lacc);
      // V^T operand: row d = 16dt + n, tokens 4lq .. 4lq+3 and 16+4lq .. 16+4lq+3
      const int vr = 4 * lq + (n >> 2);
      const int vc = 4 * (n & 3);
#pragma unroll
      for (int dt = 0; dt < Geo::NDT; ++dt) {
        const i16x4_t x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4_t*)(vt + vr * Geo::VROW + 16 * dt + vc));
        const i16x4_t x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4_t*)(vt + (16 + vr) * Geo::VROW + 16 * dt + vc));
        const uint2 w0 = __builtin_bit_cast(uint2, x0);
        const uint2 w1 = __builtin_bit_cast(uint2, x1);
        const pvec av = __builtin_bit_cast(pvec, make_uint4(w0.x, w0.y, w1.x, w1.y));
        o[dt] = Mma<PVT>::mma(av, bhi, o[dt]);
        if constexpr (SPLIT) o[dt] = Mma<PVT>::mma(av, blo, o[dt]);
      }
    }
    if (c + 1 < nch) store_chunk((c + 1) & 1);
    __syncthreads();
  }

  if (!row_ok) return;
  const float lt = lacc[0];
  // lane (n, lq) holds O^T[16dt + 4lq + r][row n]
  const float inv = pos >= 0 && lt > 0.f ? a.v_scale / lt : 0.f;
  const int64_t obase = ((int64_t)(q0 + ti) * a.num_heads + h) * D;
#pragma unroll
  for (int dt = 0; dt < Geo::NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) store_io<IO>(a.out, obase + 16 * dt + 4 * lq + r, o[dt][r] * inv);
}

// ---------------------------------------------------------------------------------
// 16-bit KV: direct-to-LDS loads into a ring of chunk buffers, 128 query rows per workgroup
// ---------------------------------------------------------------------------------
//
// A workgroup takes 128 query rows: with head_dim 128, eight waves of one 16-row tile
// (four waves per SIMD); with head_dim 64, four waves of two tiles, each K / V operand
// read from LDS feeding two MFMAs. K and V chunks go from HBM straight into LDS with
// global_load_lds_dwordx4 (lane l of an instruction lands 16 * l bytes past the
// instruction's LDS base), up to three chunks ahead of the one being computed. The copies are
// issued from inline assembly so that the compiler, which cannot tell which LDS bytes
// they write, does not wait for all of them before every LDS read; the kernel waits
// for exactly the chunk it is about to use (s_waitcnt vmcnt) and then synchronises the
// workgroup. Rows past the end of the context load the last valid row instead (finite
// data; their probability is zero), so every lane issues every copy and the count of
// outstanding copies is known. Block ids come from a per-lane window of 64 chunks.
//
// LDS rows are unpadded (the copies fill 1 KiB runs); 16-byte pieces are XOR-swizzled
// per row so that the K operand reads (16 rows, same column) and the transposed V reads
// (4 rows, 2 pieces) hit distinct banks.
//
// Per chunk a wave runs the softmax of the chunk's scores (computed one step earlier),
// then the next chunk's scores and this chunk's V product together, so the vector unit
// and the matrix cores overlap. The vector work is kept small: the scale is folded into
// the exponent (one fma per score), the causal mask is applied only on chunks that
// reach the diagonal, the four lanes of a query row exchange their maxima only when one
// of them would raise the row's max past the lazy-rescale threshold, and the softmax
// denominator is one more MFMA tile (V^T = 1) instead of a per-lane sum.

#ifndef PA_EXT_STAGES
#define PA_EXT_STAGES 4
#endif
constexpr int kDmaStages = PA_EXT_STAGES;  // chunks in the LDS ring (kDmaStages - 1 in flight)
#ifndef PA_EXT_ROWS
#define PA_EXT_ROWS 128
#endif
constexpr int kDmaRows = PA_EXT_ROWS;  // query rows per workgroup: NW waves of 16 * NT rows

// waves per workgroup of the ring kernel (16-row query tiles per wave = 128 / (16 NW));
// head_dim 64 keeps four waves so that every thread issues a whole copy per tile
#ifndef PA_EXT_WAVES
#define PA_EXT_WAVES 8
#endif
template <int D> constexpr int dma_waves() { return D == 128 ? PA_EXT_WAVES : 4; }

template <int D, int NW>
struct DmaGeo {
  static constexpr int PPR = D * 2 / 16;                    // 16-byte pieces per row
  static constexpr int ROW_B = D * 2;
  static constexpr int TILE_B = kExtChunk * ROW_B;          // K (or V) of one chunk
  static constexpr int STAGE_B = 2 * TILE_B;
  static constexpr int PPT = kExtChunk * PPR / (NW * 64);   // copies per thread per tile
  static constexpr int NKS = D / 32;
  static constexpr int NDT = D / 16;
  static_assert(PPT >= 1 && kExtChunk * PPR % (NW * 64) == 0, "whole copies");
  static __device__ __forceinline__ int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  static __device__ __forceinline__ int swz_v(int r) { return D == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3); }
};

__device__ __forceinline__ void lds_copy16(const void* src, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %1, off" ::"{m0}"(lds_base), "v"(src) : "memory");
}

// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt");
  __builtin_amdgcn_s_waitcnt(N | (0x7 << 4) | (0xF << 8));
}

template <int IO, int D, int G, int NW>
__global__ void __launch_bounds__(NW * 64) extend_dma_kernel(const ExtendArgs a) {
  using Geo = DmaGeo<D, NW>;
  using vec = typename Mma<IO>::vec;
  using M16 = Mma16<IO>;
  constexpr int QT = kDmaRows / G;  // new tokens per workgroup
  constexpr int NT = kDmaRows / (16 * NW);  // query tiles per wave
  constexpr int RW = 16 * NT;               // query rows per wave
  constexpr int NTH = NW * 64;
  constexpr int CPS = 2 * Geo::PPT; // copies per thread per stage
  // probabilities as f16 keep 11 significant bits (error <= 2^-12 relative, about 1e-3 of
  // the largest |V| at most); bf16 keeps 8, so there they go as high + low halves
  constexpr bool SPLIT = IO == kBF16;

  __shared__ __attribute__((aligned(1024))) char lds[kDmaStages * Geo::STAGE_B];

  const int unit = xcd_unit((int)blockIdx.x, (int)gridDim.x);
  const int qt = a.q_tiles - 1 - unit % a.q_tiles;
  const int sg = unit / a.q_tiles;
  // KV-head-major: each XCD's contiguous range of units holds a few KV heads of every
  // sequence (balanced however the context lengths differ); the query tiles of one
  // (sequence, KV head) stay together and share the chunks through that XCD's L2
  const int s = sg % a.num_seqs;
  const int g = sg / a.num_seqs;
  if (g >= a.num_kv_heads) return;

  const int q0 = a.query_start_loc[s];
  const int Q = a.query_start_loc[s + 1] - q0;
  const int i0 = qt * QT;
  // whole workgroup: no query rows here, or a short query the grouped decode kernel takes
  if (Q <= 0 || i0 >= Q || Q <= a.skip_q) return;
  const int cap = a.max_blocks_per_seq << a.bs_shift;
  const int L = min(max(a.context_lens[s], 0), cap);
  const int i_end = min(Q, i0 + QT);
  const int p0 = L - Q;
  const int p_last = p0 + i_end - 1;
  const int nch = p_last >= 0 ? p_last / kExtChunk + 1 : 0;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 15;
  const int lq = lane >> 4;

  // query rows of this lane: tile tq holds row RW * wave + 16 * tq + n
  int ti[NT], hh[NT], pos[NT];
  bool row_ok[NT];
#pragma unroll
  for (int tq = 0; tq < NT; ++tq) {
    const int row = RW * wave + 16 * tq + n;
    ti[tq] = i0 + row / G;
    hh[tq] = g * G + row % G;
    row_ok[tq] = ti[tq] < i_end;
    pos[tq] = p0 + ti[tq];
  }
  const int w_first = i0 + (RW * wave) / G;
  const int w_last = min(i_end, i0 + (RW * wave + RW - 1) / G + 1) - 1;
  const bool wave_live = w_first < i_end;
  const int wp_min = p0 + w_first;
  const int wp_max = p0 + w_last;

  vec qv[NT][Geo::NKS];
#pragma unroll
  for (int tq = 0; tq < NT; ++tq) {
    const int64_t base = ((int64_t)(q0 + (row_ok[tq] ? ti[tq] : 0)) * a.num_heads + hh[tq]) * D;
#pragma unroll
    for (int ks = 0; ks < Geo::NKS; ++ks) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (row_ok[tq]) w = *(const uint4*)((const char*)a.q + (base + 32 * ks + 8 * lq) * 2);
      qv[tq][ks] = __builtin_bit_cast(vec, w);
    }
  }
  // the query loads complete here: afterwards the only outstanding vector-memory
  // operations are the chunk copies, which the loop counts itself
  asm volatile("" ::: "memory");
  wait_vm<0>();

  // copy geometry: thread piece u sits at physical slot P = NTH u + 64 wave + lane of a tile
  const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  const int bs_mask = (1 << a.bs_shift) - 1;
  const int64_t tile_bytes = (int64_t)Geo::ROW_B << a.bs_shift;
  const int64_t blk_stride = tile_bytes * a.num_kv_heads;
  const char* kb = (const char*)a.k_pool + (int64_t)g * tile_bytes;
  const char* vb = (const char*)a.v_pool + (int64_t)g * tile_bytes;
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
  int crow[Geo::PPT], ck[Geo::PPT], cv[Geo::PPT];
#pragma unroll
  for (int u = 0; u < Geo::PPT; ++u) {
    const int P = NTH * u + 64 * wave + lane;
    crow[u] = P / Geo::PPR;
    const int pc = P % Geo::PPR;
    ck[u] = pc ^ Geo::swz_k(crow[u]);
    cv[u] = pc ^ Geo::swz_v(crow[u]);
  }
  // Block ids of the copies, 64 chunks at a time: lane l of win[u] holds the block of
  // copy u of chunk 64 * wb + l (the rows of one copy instruction lie in one block). A
  // window is loaded when the copies first need it and waited for at once (one drain of
  // the copies in flight per 64 chunks), so no table load sits on the per-chunk path.
  int win[Geo::PPT];
  int wb = -1;
  auto load_window = [&](int w) {
#pragma unroll
    for (int u = 0; u < Geo::PPT; ++u) {
      const int cc = 64 * w + lane;
      int b = 0;
      if (cc < nch) b = bt[min(cc * kExtChunk + (NTH * u + 64 * wave) / Geo::PPR, L - 1) >> a.bs_shift];
      // contract: 0 <= b < num_blocks; clamp so that a bad table never reads outside
      win[u] = min(max(b, 0), a.num_blocks - 1);
    }
    asm volatile("" ::: "memory");
    wait_vm<0>();
  };
  auto issue = [&](int c) {
    const int buf = c % kDmaStages;
    if ((c >> 6) != wb) {  // uniform
      wb = c >> 6;
      load_window(wb);
    }
#pragma unroll
    for (int u = 0; u < Geo::PPT; ++u) {
      const int b = __builtin_amdgcn_readlane(win[u], c & 63);
      const int ts = min(c * kExtChunk + crow[u], L - 1);
      const int64_t roff = (int64_t)b * blk_stride + (int64_t)(ts & bs_mask) * Geo::ROW_B;
      const uint32_t dst = lds0 + buf * Geo::STAGE_B + (NTH * u + 64 * wave) * 16;
      lds_copy16(kb + roff + 16 * ck[u], dst);
      lds_copy16(vb + roff + 16 * cv[u], dst + Geo::TILE_B);
    }
  };

  float m[NT];
  f32x4_t lacc[NT];  // softmax denominator (the four entries are equal)
  f32x4_t o[NT][Geo::NDT];
#pragma unroll
  for (int tq = 0; tq < NT; ++tq) {
    m[tq] = -3.0e38f;
    lacc[tq] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < Geo::NDT; ++dt) o[tq][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  constexpr uint32_t kOne2 = IO == kF16 ? 0x3C003C00u : 0x3F803F80u;  // two 16-bit 1.0
  const vec ones = __builtin_bit_cast(vec, make_uint4(kOne2, kOne2, kOne2, kOne2));

  // Per-lane LDS byte offsets inside a ring stage; the stage base is a compile-time
  // immediate of each read (the chunk loop is unrolled over the ring's stages).
  uint32_t koff[2][Geo::NKS];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int ks = 0; ks < Geo::NKS; ++ks) {
      const int r = 16 * hf + n;
      koff[hf][ks] = r * Geo::ROW_B + 16 * ((4 * ks + lq) ^ Geo::swz_k(r));
    }
  // V^T operand of tile dt: rows 4lq .. 4lq+3 (and the same 16 rows further), 8 bytes
  uint32_t voff[Geo::NDT];
  {
    const int r0 = 4 * lq + (n >> 2);
#pragma unroll
    for (int dt = 0; dt < Geo::NDT; ++dt) {
      const int cc = 2 * dt + ((n & 3) >> 1);
      voff[dt] = Geo::TILE_B + r0 * Geo::ROW_B + 16 * (cc ^ Geo::swz_v(r0)) + (n & 1) * 8;
    }
  }

  // S^T of one chunk for the wave's query tiles: acc[tq][hf] = K rows 16hf .. 16hf+15
  auto qk = [&](const char* kt, f32x4_t (&acc)[NT][2]) {
#pragma unroll
    for (int tq = 0; tq < NT; ++tq)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) acc[tq][hf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < Geo::NKS; ++ks)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const vec kop = *(const vec*)(kt + koff[hf][ks]);
#pragma unroll
        for (int tq = 0; tq < NT; ++tq) acc[tq][hf] = Mma<IO>::mma(kop, qv[tq][ks], acc[tq][hf]);
      }
  };

  // online softmax of one chunk's scores (raw dot products; scale folded into the
  // exponent) into 16-bit probability operands, rescaling o and l when the max rises
  auto softmax = [&](f32x4_t (&acc)[NT][2], int t0, vec (&bhi)[NT], vec (&blo)[NT]) {
    const bool need_mask = t0 + kExtChunk - 1 > wp_min;  // uniform
#pragma unroll
    for (int tq = 0; tq < NT; ++tq) {
      float z[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) z[j] = acc[tq][j >> 2][j & 3];
      if (need_mask) {
        asm volatile("" ::: "memory");  // a real branch: most chunks need no mask
        const int lim = pos[tq] - t0 - 4 * lq;
#pragma unroll
        for (int j = 0; j < 8; ++j) z[j] = 16 * (j >> 2) + (j & 3) <= lim ? z[j] : -INFINITY;
      }
      // The row max is needed only when it may rise past the lazy threshold: test the
      // lane's own max first (a row's max exceeds it only if one of its four lanes' does)
      // and exchange across the row's lanes only then.
      float mx = max3(max3(z[0], z[1], z[2]), max3(z[3], z[4], z[5]), fmaxf(z[6], z[7]));
      mx *= a.q_mul;  // q_mul > 0
      if (__builtin_amdgcn_ballot_w64(mx > m[tq] + kLazyRescale) != 0) {
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const bool raise = mx > m[tq] + kLazyRescale;
        const float mn = raise ? mx : m[tq];
        const float alpha = __builtin_amdgcn_exp2f(m[tq] - mn);
        m[tq] = mn;
#pragma unroll
        for (int r = 0; r < 4; ++r) lacc[tq][r] *= alpha;
#pragma unroll
        for (int dt = 0; dt < Geo::NDT; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[tq][dt][r] *= alpha;
      }
      const float nm = -m[tq];
      float p[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) p[j] = __builtin_amdgcn_exp2f(fmaf(z[j], a.q_mul, nm));
      if constexpr (SPLIT) {
        uint16_t phi[8], plo[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) M16::split(p[j], phi[j], plo[j]);
        uint4 bh, bl;
        bh.x = phi[0] | ((uint32_t)phi[1] << 16);
        bh.y = phi[2] | ((uint32_t)phi[3] << 16);
        bh.z = phi[4] | ((uint32_t)phi[5] << 16);
        bh.w = phi[6] | ((uint32_t)phi[7] << 16);
        bl.x = plo[0] | ((uint32_t)plo[1] << 16);
        bl.y = plo[2] | ((uint32_t)plo[3] << 16);
        bl.z = plo[4] | ((uint32_t)plo[5] << 16);
        bl.w = plo[6] | ((uint32_t)plo[7] << 16);
        bhi[tq] = __builtin_bit_cast(vec, bh);
        blo[tq] = __builtin_bit_cast(vec, bl);
      } else {
        vec v;
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = (_Float16)p[j];
        bhi[tq] = v;
      }
    }
  };

  // O^T += V^T P^T over the chunk
  auto pv = [&](const char* st_base, const vec (&bhi)[NT], const vec (&blo)[NT]) {
#pragma unroll
    for (int dt = 0; dt < Geo::NDT; ++dt) {
      const i16x4_t x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4_t*)(st_base + voff[dt]));
      const i16x4_t x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4_t*)(st_base + voff[dt] + 16 * Geo::ROW_B));
      const uint2 w0 = __builtin_bit_cast(uint2, x0);
      const uint2 w1 = __builtin_bit_cast(uint2, x1);
      const vec av = __builtin_bit_cast(vec, make_uint4(w0.x, w0.y, w1.x, w1.y));
#pragma unroll
      for (int tq = 0; tq < NT; ++tq) {
        o[tq][dt] = Mma<IO>::mma(av, bhi[tq], o[tq][dt]);
        if constexpr (SPLIT) o[tq][dt] = Mma<IO>::mma(av, blo[tq], o[tq][dt]);
      }
    }
    // the softmax denominator as one more tile with V^T = 1: every lane receives its
    // query row's sum over the chunk's tokens, of the same 16-bit probabilities
#pragma unroll
    for (int tq = 0; tq < NT; ++tq) {
      lacc[tq] = Mma<IO>::mma(ones, bhi[tq], lacc[tq]);
      if constexpr (SPLIT) lacc[tq] = Mma<IO>::mma(ones, blo[tq], lacc[tq]);
    }
  };

  // wait until at most `newer` chunks' copies of this thread are outstanding
  auto wait_chunks = [&](int newer) {
    static_assert(kDmaStages >= 2 && kDmaStages <= 6, "ring depth");
    if (kDmaStages >= 6 && newer >= 4) wait_vm<(kDmaStages >= 6 ? 4 : 0) * CPS>();
    else if (kDmaStages >= 5 && newer >= 3) wait_vm<(kDmaStages >= 5 ? 3 : 0) * CPS>();
    else if (kDmaStages >= 4 && newer >= 2) wait_vm<(kDmaStages >= 4 ? 2 : 0) * CPS>();
    else if (newer >= 1) wait_vm<CPS>();
    else wait_vm<0>();
  };

#pragma unroll
  for (int j = 0; j < kDmaStages - 1; ++j)
    if (j < nch) issue(j);

  // Software pipeline: iteration c computes the scores of chunk c + 1 (its K is in the
  // ring by then) before the softmax and V product of chunk c, so the matrix cores work
  // while the vector unit runs the softmax. The scores alternate between two register
  // sets by chunk parity (the ring depth is even, so the parity of the unrolled stage
  // is the parity of the chunk).
  static_assert(kDmaStages % 2 == 0 && kDmaStages >= 4,
                "score buffers alternate by stage parity; two chunks in flight ahead of c + 1");
  f32x4_t sc[2][NT][2];
  if (nch > 0) {
    wait_chunks(min(kDmaStages - 2, nch - 1));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (wave_live && 0 <= wp_max) qk(lds, sc[0]);
  }
  for (int c0 = 0; c0 < nch; c0 += kDmaStages) {
#pragma unroll
    for (int st = 0; st < kDmaStages; ++st) {
      const int c = c0 + st;
      if (c >= nch) break;
      if (c + 1 < nch) {
        // chunk c + 1 has landed once at most the copies of the chunks after it remain;
        // the barrier also frees the stage of chunk c - 1 for the copy issued next
        wait_chunks(min(kDmaStages - 3, nch - 2 - c));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (c + kDmaStages - 1 < nch) issue(c + kDmaStages - 1);
      }
      const int t0 = c * kExtChunk;
      if (wave_live && t0 <= wp_max) {
        vec bhi[NT], blo[NT];
        softmax(sc[st & 1], t0, bhi, blo);
        // the next chunk's scores go with this chunk's V product, so the two interleave on
        // the matrix cores; past the wave's last chunk they are computed and never used
        // (the stage holds an older chunk then, never one being copied)
        qk(lds + ((st + 1) % kDmaStages) * Geo::STAGE_B, sc[(st + 1) & 1]);
        pv(lds + st * Geo::STAGE_B, bhi, blo);
      }
    }
  }

#pragma unroll
  for (int tq = 0; tq < NT; ++tq) {
    const float lt = lacc[tq][0];
    if (!row_ok[tq]) continue;
    const float inv = pos[tq] >= 0 && lt > 0.f ? a.v_scale / lt : 0.f;
    const int64_t obase = ((int64_t)(q0 + ti[tq]) * a.num_heads + hh[tq]) * D;
#pragma unroll
    for (int dt = 0; dt < Geo::NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) store_io<IO>(a.out, obase + 16 * dt + 4 * lq + r, o[tq][dt][r] * inv);
  }
}

template <int IO, int KV, int D>
int launch_ext_g(const ExtendArgs& a, int G, int grid, hipStream_t st) {
  if constexpr (KV == IO) {
    constexpr int NW = dma_waves<D>();
    switch (G) {
      case 1: hipLaunchKernelGGL((extend_dma_kernel<IO, D, 1, NW>), dim3(grid), dim3(NW * 64), 0, st, a); break;
      case 2: hipLaunchKernelGGL((extend_dma_kernel<IO, D, 2, NW>), dim3(grid), dim3(NW * 64), 0, st, a); break;
      case 4: hipLaunchKernelGGL((extend_dma_kernel<IO, D, 4, NW>), dim3(grid), dim3(NW * 64), 0, st, a); break;
      case 8: hipLaunchKernelGGL((extend_dma_kernel<IO, D, 8, NW>), dim3(grid), dim3(NW * 64), 0, st, a); break;
      default: return PA_ERR_UNSUPPORTED;
    }
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
  }
  switch (G) {
    case 1: hipLaunchKernelGGL((extend_kernel<IO, KV, D, 1>), dim3(grid), dim3(kExtWaves * 64), 0, st, a); break;
    case 2: hipLaunchKernelGGL((extend_kernel<IO, KV, D, 2>), dim3(grid), dim3(kExtWaves * 64), 0, st, a); break;
    case 4: hipLaunchKernelGGL((extend_kernel<IO, KV, D, 4>), dim3(grid), dim3(kExtWaves * 64), 0, st, a); break;
    case 8: hipLaunchKernelGGL((extend_kernel<IO, KV, D, 8>), dim3(grid), dim3(kExtWaves * 64), 0, st, a); break;
    default: return PA_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

template <int IO, int KV>
int launch_ext_d(const ExtendArgs& a, int D, int G, int grid, hipStream_t st) {
  switch (D) {
    case 64: return launch_ext_g<IO, KV, 64>(a, G, grid, st);
    case 128: return launch_ext_g<IO, KV, 128>(a, G, grid, st);
    default: return PA_ERR_UNSUPPORTED;
  }
}

bool ext_pos_finite(float x) { return std::isfinite(x) && x > 0.f; }

}  // namespace
}  // namespace pa

extern "C" int pa_extend(const void* q, const void* k_pool, const void* v_pool,
                         const int32_t* block_tables, const int32_t* context_lens,
                         const int32_t* query_start_loc, int num_seqs, int max_blocks_per_seq,
                         int num_blocks, int max_query_len, int num_heads, int num_kv_heads,
                         int head_dim, int block_size, float scale, int io_dtype, int kv_dtype,
                         float k_scale, float v_scale, void* out, void* stream) {
  using namespace pa;
  try {
    if (!q || !k_pool || !v_pool || !block_tables || !context_lens || !query_start_loc || !out)
      return PA_ERR_INVALID;
    if (num_seqs <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 || max_query_len < 0 ||
        num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0)
      return PA_ERR_INVALID;
    if (io_dtype != PA_F32 && io_dtype != PA_F16 && io_dtype != PA_BF16) return PA_ERR_INVALID;
    if (kv_dtype != PA_F32 && kv_dtype != PA_F16 && kv_dtype != PA_BF16 && kv_dtype != PA_FP8_E4M3)
      return PA_ERR_INVALID;
    if (num_heads % num_kv_heads != 0) return PA_ERR_INVALID;
    if (!ext_pos_finite(scale)) return PA_ERR_INVALID;
    if (kv_dtype == PA_FP8_E4M3 && (!ext_pos_finite(k_scale) || !ext_pos_finite(v_scale)))
      return PA_ERR_INVALID;
    if (((uintptr_t)q | (uintptr_t)k_pool | (uintptr_t)v_pool | (uintptr_t)out) & 15u) return PA_ERR_INVALID;
    if ((int64_t)max_blocks_per_seq * block_size > INT_MAX / 2) return PA_ERR_INVALID;
    if (io_dtype == PA_F32) return PA_ERR_UNSUPPORTED;  // matrix-core path: 16-bit queries
    if (kv_dtype != io_dtype && kv_dtype != PA_FP8_E4M3) return PA_ERR_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (block_size < 8 || block_size > 512 || (block_size & (block_size - 1)) != 0) return PA_ERR_UNSUPPORTED;
    const int G = num_heads / num_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8) return PA_ERR_UNSUPPORTED;
    if (max_query_len == 0) return PA_OK;
    ExtendArgs a{};
    a.q = q;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.query_start_loc = query_start_loc;
    a.out = out;
    a.num_seqs = num_seqs;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.num_blocks = num_blocks;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.bs_shift = __builtin_ctz((unsigned)block_size);
    const int QT = (kv_dtype == io_dtype ? kDmaRows : kExtRows) / G;  // new tokens per workgroup
    a.q_tiles = (max_query_len + QT - 1) / QT;
    a.q_mul = scale * kLog2e * (kv_dtype == PA_FP8_E4M3 ? k_scale : 1.f);
    a.v_scale = kv_dtype == PA_FP8_E4M3 ? v_scale : 1.f;
    const int64_t grid = (int64_t)num_seqs * num_kv_heads * a.q_tiles;
    if (grid > INT_MAX) return PA_ERR_INVALID;
    hipStream_t st = (hipStream_t)stream;
    const int D = head_dim;
    // Short queries (at most 16 / G new tokens, e.g. a few tokens checked at once): their
    // G x Q query rows fill the 16 columns of the grouped decode kernel, which walks the
    // sequence's blocks once for all of them with the context split over its waves (a
    // causal end per row) instead of one wave walking it alone.
    const int row_bytes = D * (kv_dtype == PA_FP8_E4M3 ? 1 : 2);
    if ((G == 2 || G == 4 || G == 8) && block_size >= 16 && row_bytes >= 128 && row_bytes % 128 == 0) {
      DecodeArgs d{};
      d.q = q;
      d.k_pool = k_pool;
      d.v_pool = v_pool;
      d.block_tables = block_tables;
      d.context_lens = context_lens;
      d.out = out;
      d.num_seqs = num_seqs;
      d.max_blocks_per_seq = max_blocks_per_seq;
      d.num_blocks = num_blocks;
      d.num_heads = num_heads;
      d.num_kv_heads = num_kv_heads;
      d.max_ctx = max_blocks_per_seq * block_size;
      d.part_tokens = d.max_ctx;
      d.num_parts = 1;
      d.q_mul = a.q_mul;
      d.out_mul = a.v_scale;
      d.query_start_loc = query_start_loc;
      LaunchSpec ls{};
      ls.args = d;
      ls.head_dim = D;
      ls.block_size = block_size;
      ls.group = G;
      ls.grouped = true;
      ls.grid = num_seqs * num_kv_heads;
      ls.stream = st;
      const bool large = block_size > 32;
      int rc;
      if (io_dtype == PA_F16)
        rc = kv_dtype == PA_FP8_E4M3 ? (large ? launch_f16_fp8_large(ls) : launch_f16_fp8(ls))
                                     : (large ? launch_f16_f16_large(ls) : launch_f16_f16(ls));
      else
        rc = kv_dtype == PA_FP8_E4M3 ? (large ? launch_bf16_fp8_large(ls) : launch_bf16_fp8(ls))
                                     : (large ? launch_bf16_bf16_large(ls) : launch_bf16_bf16(ls));
      if (rc != PA_OK) return rc;
      a.skip_q = 16 / G;
    }
    if (io_dtype == PA_F16)
      return kv_dtype == PA_FP8_E4M3 ? launch_ext_d<kF16, kFP8>(a, D, G, (int)grid, st)
                                     : launch_ext_d<kF16, kF16>(a, D, G, (int)grid, st);
    return kv_dtype == PA_FP8_E4M3 ? launch_ext_d<kBF16, kFP8>(a, D, G, (int)grid, st)
                                   : launch_ext_d<kBF16, kBF16>(a, D, G, (int)grid, st);
  } catch (...) {
    return PA_ERR_LAUNCH;
  }
}
