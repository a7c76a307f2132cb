// Appending new tokens' keys and values to the paged cache (the write that precedes every
// decode step).
//
// Pages cited by title and section:
//   [P1] "突破GPU内存瓶颈：vLLM与PagedAttention技术深度解析" §2 — fixed-size blocks, block
//        table from logical to physical blocks; only the last block is partly filled.
//   [P3] "内存优化：KV Cache管理、PagedAttention原理与内存池配置", paged-pool section — a
//        growing request gets new blocks appended; blocks live in one global pool.
//   [P2] vLLM architecture deep-dive §2.1 (decode mode: one new token per step) and §4.2
//        (FP8 KV cache).
//
// Token t of sequence s at logical position p goes to physical block bt[s][p / BS], slot
// p % BS, of every KV head. One thread writes one 16-byte piece of one output row (K and
// V), so a wave stores whole 1 KiB runs of a (block, head) tile.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>

#include "pa.h"
#include "pa_decode_impl.h"

namespace pa {
namespace {

struct AppendArgs {
  const void* k_new;
  const void* v_new;
  const int32_t* seq_ids;
  const int32_t* positions;
  const int32_t* block_tables;
  void* k_pool;
  void* v_pool;
  int num_tokens;
  int num_seqs;
  int max_blocks_per_seq;
  int num_blocks;
  int num_kv_heads;
  float k_scale;  // fp8 pools only
  float v_scale;
};

// two fp32 values -> two e4m3 codes: y = x / scale rounded to fp32, magnitudes above 448
// saturated to +-448, then the hardware conversion (round to nearest even); NaN -> 0x7F
__device__ __forceinline__ uint32_t to_fp8_pair(float a, float b, float scale) {
  const float ya = a / scale;
  const float yb = b / scale;
  const bool na = ya != ya, nb = yb != yb;
  const uint32_t c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
      na ? 0.f : fminf(fmaxf(ya, -448.f), 448.f), nb ? 0.f : fminf(fmaxf(yb, -448.f), 448.f), 0, false);
  return (na ? 0x7Fu : (c & 0xffu)) | ((nb ? 0x7Fu : ((c >> 8) & 0xffu)) << 8);
}

// VEC output values from the new row starting at element e0, stored as 16 bytes of KV type
template <int SRC, int KV>
__device__ __forceinline__ uint4 encode16(const void* src, int64_t e0, float scale) {
  if constexpr (KV == kFP8) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = to_fp8_pair(load_io<SRC>(src, e0 + 4 * i), load_io<SRC>(src, e0 + 4 * i + 1), scale);
      const uint32_t hi = to_fp8_pair(load_io<SRC>(src, e0 + 4 * i + 2), load_io<SRC>(src, e0 + 4 * i + 3), scale);
      w[i] = lo | (hi << 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    // same type: copy the stored bits
    return *(const uint4*)((const char*)src + e0 * ElemBytes<SRC>::value);
  }
}

template <int SRC, int KV, int D, int BS>
__global__ void __launch_bounds__(256) append_kernel(const AppendArgs a) {
  constexpr int E = ElemBytes<KV>::value;
  constexpr int VEC = 16 / E;           // output values per thread
  constexpr int PIECES = D / VEC;       // threads per (token, head) row
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t rows = (int64_t)a.num_tokens * a.num_kv_heads;
  if (gid >= rows * PIECES) return;
  const int piece = (int)(gid % PIECES);
  const int64_t row = gid / PIECES;
  const int g = (int)(row % a.num_kv_heads);
  const int t = (int)(row / a.num_kv_heads);
  const int s = a.seq_ids[t];
  const int p = a.positions[t];
  // contract violations write nothing (pa_check_tables and the host checks report them)
  if (s < 0 || s >= a.num_seqs || p < 0 || p / BS >= a.max_blocks_per_seq) return;
  const int b = a.block_tables[(int64_t)s * a.max_blocks_per_seq + p / BS];
  if (b < 0 || b >= a.num_blocks) return;
  const int64_t dst = ((((int64_t)b * a.num_kv_heads + g) * BS + p % BS) * D + (int64_t)piece * VEC) * E;
  const int64_t e0 = row * D + (int64_t)piece * VEC;
  *(uint4*)((char*)a.k_pool + dst) = encode16<SRC, KV>(a.k_new, e0, a.k_scale);
  *(uint4*)((char*)a.v_pool + dst) = encode16<SRC, KV>(a.v_new, e0, a.v_scale);
}

template <int SRC, int KV, int D>
int launch_append_bs(const AppendArgs& a, int BS, hipStream_t st) {
  constexpr int VEC = 16 / ElemBytes<KV>::value;
  const int64_t threads = (int64_t)a.num_tokens * a.num_kv_heads * (D / VEC);
  const int64_t grid = (threads + 255) / 256;
  if (grid > INT_MAX) return PA_ERR_INVALID;
  switch (BS) {
    case 8: hipLaunchKernelGGL((append_kernel<SRC, KV, D, 8>), dim3(grid), dim3(256), 0, st, a); break;
    case 16: hipLaunchKernelGGL((append_kernel<SRC, KV, D, 16>), dim3(grid), dim3(256), 0, st, a); break;
    case 32: hipLaunchKernelGGL((append_kernel<SRC, KV, D, 32>), dim3(grid), dim3(256), 0, st, a); break;
    case 64: hipLaunchKernelGGL((append_kernel<SRC, KV, D, 64>), dim3(grid), dim3(256), 0, st, a); break;
    case 128: hipLaunchKernelGGL((append_kernel<SRC, KV, D, 128>), dim3(grid), dim3(256), 0, st, a); break;
    case 256: hipLaunchKernelGGL((append_kernel<SRC, KV, D, 256>), dim3(grid), dim3(256), 0, st, a); break;
    case 512: hipLaunchKernelGGL((append_kernel<SRC, KV, D, 512>), dim3(grid), dim3(256), 0, st, a); break;
    default: return PA_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

template <int SRC, int KV>
int launch_append_d(const AppendArgs& a, int D, int BS, hipStream_t st) {
  if constexpr (KV == kFP8 || ElemBytes<SRC>::value == ElemBytes<KV>::value) {
    switch (D) {
      case 64: return launch_append_bs<SRC, KV, 64>(a, BS, st);
      case 128: return launch_append_bs<SRC, KV, 128>(a, BS, st);
      case 256: return launch_append_bs<SRC, KV, 256>(a, BS, st);
      default: return PA_ERR_UNSUPPORTED;
    }
  }
  return PA_ERR_UNSUPPORTED;
}

// Copies whole physical blocks (all KV heads, K and V) for copy-on-write: pair i copies
// block pairs[i][0] to block pairs[i][1]. One thread moves one 16-byte piece; pairs with
// an id outside the pool, or with src == dst, are skipped.
__global__ void __launch_bounds__(256) copy_blocks_kernel(char* k_pool, char* v_pool, const int32_t* pairs,
                                                          int num_pairs, int num_blocks, int64_t pieces_per_block) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)num_pairs * pieces_per_block) return;
  const int i = (int)(gid / pieces_per_block);
  const int64_t piece = gid % pieces_per_block;
  const int src = pairs[2 * i], dst = pairs[2 * i + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst) return;
  const int64_t from = ((int64_t)src * pieces_per_block + piece) * 16;
  const int64_t to = ((int64_t)dst * pieces_per_block + piece) * 16;
  *(uint4*)(k_pool + to) = *(const uint4*)(k_pool + from);
  *(uint4*)(v_pool + to) = *(const uint4*)(v_pool + from);
}

}  // namespace
}  // namespace pa

extern "C" int pa_append_kv(const void* k_new, const void* v_new, const int32_t* seq_ids,
                            const int32_t* positions, int num_tokens, const int32_t* block_tables,
                            int num_seqs, int max_blocks_per_seq, void* k_pool, void* v_pool,
                            int num_blocks, int num_kv_heads, int head_dim, int block_size,
                            int src_dtype, int kv_dtype, float k_scale, float v_scale, void* stream) {
  using namespace pa;
  try {
    if (!k_new || !v_new || !seq_ids || !positions || !block_tables || !k_pool || !v_pool)
      return PA_ERR_INVALID;
    if (num_tokens < 0 || num_seqs <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 ||
        num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0)
      return PA_ERR_INVALID;
    if (src_dtype != PA_F32 && src_dtype != PA_F16 && src_dtype != PA_BF16) return PA_ERR_INVALID;
    if (kv_dtype != PA_F32 && kv_dtype != PA_F16 && kv_dtype != PA_BF16 && kv_dtype != PA_FP8_E4M3)
      return PA_ERR_INVALID;
    if (kv_dtype != src_dtype && kv_dtype != PA_FP8_E4M3) return PA_ERR_UNSUPPORTED;
    if (kv_dtype == PA_FP8_E4M3 && (!std::isfinite(k_scale) || !(k_scale > 0.f) ||
                                    !std::isfinite(v_scale) || !(v_scale > 0.f)))
      return PA_ERR_INVALID;
    if (((uintptr_t)k_new | (uintptr_t)v_new | (uintptr_t)k_pool | (uintptr_t)v_pool) & 15u)
      return PA_ERR_INVALID;
    if (head_dim != 64 && head_dim != 128 && head_dim != 256) return PA_ERR_UNSUPPORTED;
    if (block_size != 8 && block_size != 16 && block_size != 32 && block_size != 64 && block_size != 128 &&
        block_size != 256 && block_size != 512)
      return PA_ERR_UNSUPPORTED;
    if (num_tokens == 0) return PA_OK;
    AppendArgs a{k_new, v_new, seq_ids, positions, block_tables, k_pool, v_pool, num_tokens,
                 num_seqs, max_blocks_per_seq, num_blocks, num_kv_heads, k_scale, v_scale};
    hipStream_t st = (hipStream_t)stream;
    const int D = head_dim, BS = block_size;
    switch (src_dtype * 4 + kv_dtype) {
      case PA_F32 * 4 + PA_F32: return launch_append_d<kF32, kF32>(a, D, BS, st);
      case PA_F16 * 4 + PA_F16: return launch_append_d<kF16, kF16>(a, D, BS, st);
      case PA_BF16 * 4 + PA_BF16: return launch_append_d<kBF16, kBF16>(a, D, BS, st);
      case PA_F32 * 4 + PA_FP8_E4M3: return launch_append_d<kF32, kFP8>(a, D, BS, st);
      case PA_F16 * 4 + PA_FP8_E4M3: return launch_append_d<kF16, kFP8>(a, D, BS, st);
      case PA_BF16 * 4 + PA_FP8_E4M3: return launch_append_d<kBF16, kFP8>(a, D, BS, st);
      default: return PA_ERR_UNSUPPORTED;
    }
  } catch (...) {
    return PA_ERR_LAUNCH;
  }
}

extern "C" int pa_copy_blocks(void* k_pool, void* v_pool, const int32_t* block_pairs, int num_pairs,
                              int num_blocks, int num_kv_heads, int head_dim, int block_size,
                              int kv_dtype, void* stream) {
  using namespace pa;
  try {
    if (!k_pool || !v_pool || (num_pairs > 0 && !block_pairs)) return PA_ERR_INVALID;
    if (num_pairs < 0 || num_blocks <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0)
      return PA_ERR_INVALID;
    int e = 0;
    switch (kv_dtype) {
      case PA_F32: e = 4; break;
      case PA_F16: case PA_BF16: e = 2; break;
      case PA_FP8_E4M3: e = 1; break;
      default: return PA_ERR_INVALID;
    }
    const int64_t block_bytes = (int64_t)num_kv_heads * block_size * head_dim * e;
    if (block_bytes % 16 != 0) return PA_ERR_UNSUPPORTED;
    if (((uintptr_t)k_pool | (uintptr_t)v_pool) & 15u) return PA_ERR_INVALID;
    if (num_pairs == 0) return PA_OK;
    const int64_t pieces = block_bytes / 16;
    const int64_t grid = ((int64_t)num_pairs * pieces + 255) / 256;
    if (grid > INT_MAX) return PA_ERR_INVALID;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (char*)k_pool,
                       (char*)v_pool, block_pairs, num_pairs, num_blocks, pieces);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
  } catch (...) {
    return PA_ERR_LAUNCH;
  }
}
