// C interface of the paged-attention decode library: argument checks, kernel choice,
// the split-context log-sum-exp merge, the block-table checker and the fp8 probe.
//
// Pages cited by title and section:
//   [P1] "突破GPU内存瓶颈：vLLM与PagedAttention技术深度解析" §2 (block table, shared blocks)
//   [P2] vLLM architecture deep-dive §1.1 (paged-attention call), §2.2 (metadata),
//        §3.3 / §4.1 (second, split-context kernel for long text), §4.2 (FP8 KV cache)
//   [P3] "内存优化：KV Cache管理、PagedAttention原理与内存池配置" (decode over all cached K/V)
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "pa.h"
#include "pa_decode_impl.h"

// Partition states of pa_decode_partitioned_noalloc: one copy per GPU, held by the loaded
// code object until the process ends. Host code never passes this name to a kernel (on
// the host it is only a stand-in); it uses the device address from hipGetSymbolAddress.
static __device__ __align__(256) char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace pa {
namespace {

constexpr int kDefaultPartition = 512;

struct MergeArgs {
  const float* ws;
  const int32_t* context_lens;
  void* out;
  int num_seqs;
  int num_heads;
  int num_parts;
  int part_tokens;
  int max_ctx;
  int fixed_parts;  // > 0: every sequence has this many partial states (grouped splits)
};

// Log-sum-exp merge of the partitions of one (sequence, head) per workgroup ([P2] §3.3 /
// §4.1 split-context kernel; the merge rule is the exact recombination of softmax
// partial sums): M = max_p m_p, w_p = exp2(m_p - M), out = sum_p w_p o_p / sum_p w_p l_p.
// Scores are in log2 units, as the decode kernel wrote them. Thread t reads the 16-byte
// column group t % (D/4) of the partitions t / (D/4) + k * SL (SL = 1024 / D slices),
// eight partitions in flight, all issued before the maximum M is known; the slices are
// summed through LDS at the end.
constexpr int kMergeThreads = 256;
constexpr int kMergeDepth = 8;

template <int IO, int D>
__global__ void __launch_bounds__(kMergeThreads) merge_kernel(const MergeArgs a) {
  constexpr int TPR = D / 4;                 // threads per partition row
  constexpr int SL = kMergeThreads / TPR;    // partitions read side by side
  __shared__ float sm_max[kMergeThreads / 64];
  __shared__ float4 sm_acc[SL][TPR];
  __shared__ float sm_den[SL][TPR];
  const int pair = blockIdx.x;
  const int s = pair / a.num_heads;
  int L = a.context_lens[s];
  L = min(max(L, 0), a.max_ctx);
  const int n = a.fixed_parts > 0 ? a.fixed_parts : (L + a.part_tokens - 1) / a.part_tokens;
  if (a.fixed_parts == 0 && n <= 1) return;  // written directly by the decode kernel (whole workgroup)
  const int64_t NPH = (int64_t)a.num_seqs * a.num_heads * a.num_parts;
  const float* m = a.ws + (int64_t)pair * a.num_parts;
  const float* l = a.ws + NPH + (int64_t)pair * a.num_parts;
  const float4* o = (const float4*)(a.ws + 2 * NPH + (int64_t)pair * a.num_parts * D);
  const int t = threadIdx.x;
  const int col = t % TPR;
  const int slice = t / TPR;

  // first group of partitions: loads issued before the maximum is formed
  float4 ov[kMergeDepth];
  float mv[kMergeDepth], lv[kMergeDepth];
#pragma unroll
  for (int k = 0; k < kMergeDepth; ++k) {
    const int p = min(slice + k * SL, n - 1);  // past the end: a valid partition, weight 0 below
    ov[k] = o[(int64_t)p * TPR + col];
    mv[k] = m[p];
    lv[k] = l[p];
  }
  float M = -3.0e38f;
  for (int p = t; p < n; p += kMergeThreads) M = fmaxf(M, m[p]);
  M = rows_max<1>(M);
  if ((t & 63) == 0) sm_max[t >> 6] = M;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kMergeThreads / 64; ++w) M = fmaxf(M, sm_max[w]);

  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float den = 0.f;
  for (int p0 = slice;; p0 += kMergeDepth * SL) {
#pragma unroll
    for (int k = 0; k < kMergeDepth; ++k) {
      const float w = p0 + k * SL < n ? __builtin_amdgcn_exp2f(mv[k] - M) : 0.f;
      den = fmaf(w, lv[k], den);
      acc.x = fmaf(w, ov[k].x, acc.x);
      acc.y = fmaf(w, ov[k].y, acc.y);
      acc.z = fmaf(w, ov[k].z, acc.z);
      acc.w = fmaf(w, ov[k].w, acc.w);
    }
    if (p0 + kMergeDepth * SL >= n) break;
#pragma unroll
    for (int k = 0; k < kMergeDepth; ++k) {
      const int p = min(p0 + (kMergeDepth + k) * SL, n - 1);
      ov[k] = o[(int64_t)p * TPR + col];
      mv[k] = m[p];
      lv[k] = l[p];
    }
  }
  sm_acc[slice][col] = acc;
  sm_den[slice][col] = den;
  __syncthreads();
  if (t < TPR) {
    float4 x = sm_acc[0][t];
    float dsum = sm_den[0][t];
#pragma unroll
    for (int k = 1; k < SL; ++k) {
      const float4 y = sm_acc[k][t];
      x.x += y.x;
      x.y += y.y;
      x.z += y.z;
      x.w += y.w;
      dsum += sm_den[k][t];
    }
    // dsum is 0 only when every state is empty (a context of length 0); x is 0 then too
    const float d = dsum > 0.f ? dsum : 1.f;
    const int64_t base = (int64_t)pair * D + 4 * t;
    store_io<IO>(a.out, base + 0, x.x / d);
    store_io<IO>(a.out, base + 1, x.y / d);
    store_io<IO>(a.out, base + 2, x.z / d);
    store_io<IO>(a.out, base + 3, x.w / d);
  }
}

// One thread per sequence checks its used block-table entries.
__global__ void check_tables_kernel(const int32_t* bt, const int32_t* cl, int S, int MB, int NB,
                                    int BS, int max_ctx, int32_t* err) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= S) return;
  const int L = cl[s];
  int e = 0;
  if (L < 0) e |= 1;
  if ((int64_t)L > (int64_t)MB * BS) e |= 2;
  if (max_ctx > 0 && L > max_ctx) e |= 8;
  const int64_t nb = L > 0 ? min(((int64_t)L + BS - 1) / BS, (int64_t)MB) : 0;
  for (int64_t j = 0; j < nb; ++j) {
    const int b = bt[(int64_t)s * MB + j];
    if (b < 0 || b >= NB) {
      e |= 4;
      break;
    }
  }
  err[s] = e;
}

__global__ void fp8_probe_kernel(const uint8_t* codes, float* out, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int base = i * 16;
  if (base >= n) return;
  uint8_t b[16];
  for (int k = 0; k < 16; ++k) b[k] = base + k < n ? codes[base + k] : 0;
  uint4 r;
  r.x = b[0] | (b[1] << 8) | (b[2] << 16) | ((uint32_t)b[3] << 24);
  r.y = b[4] | (b[5] << 8) | (b[6] << 16) | ((uint32_t)b[7] << 24);
  r.z = b[8] | (b[9] << 8) | (b[10] << 16) | ((uint32_t)b[11] << 24);
  r.w = b[12] | (b[13] << 8) | (b[14] << 16) | ((uint32_t)b[15] << 24);
  float f[16];
  widen16<kFP8>(r, f);
  for (int k = 0; k < 16; ++k)
    if (base + k < n) out[base + k] = f[k];
}

// The matrix-core operand conversion (fp8x8_operand, also used for the V tile): lane i
// converts the 16 codes base .. base + 15 as two operands of eight 16-bit values.
template <int MT>
__global__ void fp8_mt_probe_kernel(const uint8_t* codes, uint16_t* out, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int base = i * 16;
  if (base >= n) return;
  uint32_t w[4];
  for (int k = 0; k < 4; ++k) {
    uint32_t x = 0;
    for (int j = 0; j < 4; ++j) {
      const int idx = base + 4 * k + j;
      x |= (uint32_t)(idx < n ? codes[idx] : 0) << (8 * j);
    }
    w[k] = x;
  }
  const uint4 lo = __builtin_bit_cast(uint4, fp8x8_operand<MT>(w[0], w[1]));
  const uint4 hi = __builtin_bit_cast(uint4, fp8x8_operand<MT>(w[2], w[3]));
  const uint32_t r[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  for (int k = 0; k < 16; ++k)
    if (base + k < n) out[base + k] = (uint16_t)(r[k / 2] >> (16 * (k % 2)));
}

bool is_pow_group(int g) { return g == 1 || g == 2 || g == 4 || g == 8; }

int elem_bytes(int dt) {
  switch (dt) {
    case PA_F32: return 4;
    case PA_F16: return 2;
    case PA_BF16: return 2;
    case PA_FP8_E4M3: return 1;
    default: return 0;
  }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool pos_finite(float x) { return std::isfinite(x) && x > 0.f; }

struct Common {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* bt;
  const int32_t* cl;
  int S, MB, NB, H, Hkv, D, BS;
  float scale;
  int io, kv;
  float ks, vs;
  void* out;
};

int validate(const Common& c) {
  if (!c.q || !c.k_pool || !c.v_pool || !c.bt || !c.cl || !c.out) return PA_ERR_INVALID;
  if (c.S <= 0 || c.MB <= 0 || c.NB <= 0 || c.H <= 0 || c.Hkv <= 0 || c.D <= 0 || c.BS <= 0)
    return PA_ERR_INVALID;
  if (c.io != PA_F32 && c.io != PA_F16 && c.io != PA_BF16) return PA_ERR_INVALID;
  if (elem_bytes(c.kv) == 0) return PA_ERR_INVALID;
  if (c.H % c.Hkv != 0) return PA_ERR_INVALID;
  if (!pos_finite(c.scale)) return PA_ERR_INVALID;
  if (c.kv == PA_FP8_E4M3 && (!pos_finite(c.ks) || !pos_finite(c.vs))) return PA_ERR_INVALID;
  if (!aligned16(c.q) || !aligned16(c.k_pool) || !aligned16(c.v_pool) || !aligned16(c.out))
    return PA_ERR_INVALID;
  if ((int64_t)c.MB * c.BS > INT_MAX / 2) return PA_ERR_INVALID;
  if (c.kv != c.io && c.kv != PA_FP8_E4M3) return PA_ERR_UNSUPPORTED;
  if (c.D != 64 && c.D != 128 && c.D != 256) return PA_ERR_UNSUPPORTED;
  if (c.BS != 8 && c.BS != 16 && c.BS != 32 && c.BS != 64 && c.BS != 128 && c.BS != 256 && c.BS != 512)
    return PA_ERR_UNSUPPORTED;
  if (!is_pow_group(c.H / c.Hkv)) return PA_ERR_UNSUPPORTED;
  const int lpt = c.D * elem_bytes(c.kv) / 16;
  const int tpl = 64 / lpt;
  if ((c.BS < 32 ? c.BS : 32) % tpl != 0) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

int launch_pair(int io, int kv, const LaunchSpec& ls) {
  const bool large = ls.block_size > 32;
  if (kv == PA_FP8_E4M3) {
    switch (io) {
      case PA_F32: return large ? launch_f32_fp8_large(ls) : launch_f32_fp8(ls);
      case PA_F16: return large ? launch_f16_fp8_large(ls) : launch_f16_fp8(ls);
      case PA_BF16: return large ? launch_bf16_fp8_large(ls) : launch_bf16_fp8(ls);
    }
  } else {
    switch (io) {
      case PA_F32: return large ? launch_f32_f32_large(ls) : launch_f32_f32(ls);
      case PA_F16: return large ? launch_f16_f16_large(ls) : launch_f16_f16(ls);
      case PA_BF16: return large ? launch_bf16_bf16_large(ls) : launch_bf16_bf16(ls);
    }
  }
  return PA_ERR_UNSUPPORTED;
}

template <int IO>
int launch_merge_io(int D, const MergeArgs& m, int grid, hipStream_t st) {
  if (D == 64) {
    hipLaunchKernelGGL((merge_kernel<IO, 64>), dim3(grid), dim3(kMergeThreads), 0, st, m);
  } else if (D == 128) {
    hipLaunchKernelGGL((merge_kernel<IO, 128>), dim3(grid), dim3(kMergeThreads), 0, st, m);
  } else {
    hipLaunchKernelGGL((merge_kernel<IO, 256>), dim3(grid), dim3(kMergeThreads), 0, st, m);
  }
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int launch_merge(int io, int D, const MergeArgs& m, int grid, hipStream_t st) {
  switch (io) {
    case PA_F32: return launch_merge_io<kF32>(D, m, grid, st);
    case PA_F16: return launch_merge_io<kF16>(D, m, grid, st);
    case PA_BF16: return launch_merge_io<kBF16>(D, m, grid, st);
  }
  return PA_ERR_UNSUPPORTED;
}

DecodeArgs base_args(const Common& c) {
  DecodeArgs a{};
  a.q = c.q;
  a.k_pool = c.k_pool;
  a.v_pool = c.v_pool;
  a.block_tables = c.bt;
  a.context_lens = c.cl;
  a.out = c.out;
  a.num_seqs = c.S;
  a.max_blocks_per_seq = c.MB;
  a.num_blocks = c.NB;
  a.num_heads = c.H;
  a.num_kv_heads = c.Hkv;
  const bool fp8 = c.kv == PA_FP8_E4M3;
  a.q_mul = c.scale * kLog2e * (fp8 ? c.ks : 1.f);
  a.out_mul = fp8 ? c.vs : 1.f;
  return a;
}


// Device address of the current device's copy of `scratch`, looked up once per device
// (with that device current) and kept.
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];

int scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_LAUNCH;
  if (dev < 0 || dev >= kMaxScratchDevices) return PA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return PA_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

int64_t num_parts_for(int max_context_len, int P) {
  const int64_t n = ((int64_t)max_context_len + P - 1) / P;
  return n < 1 ? 1 : n;
}

// Compute units of the current device (queried once per device, thread-safe through the
// static local).
int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];  // zero-initialised; 0 = not yet queried
  if (dev >= 0 && dev < kMaxDev) {
    const int known = cache[dev].load(std::memory_order_relaxed);
    if (known > 0) return known;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (dev >= 0 && dev < kMaxDev) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Workgroups the balanced scheduler uses by default: two per compute unit.
int default_balanced_workgroups() { return 2 * device_cus(); }

// Waves per compute unit the split-context streaming kernel aims for: each wave takes
// as many consecutive partitions as keeps the grid at about this many waves per CU.
#ifndef PA_STREAM_WAVES_PER_CU
#define PA_STREAM_WAVES_PER_CU 4
#endif

// Runs of the streaming kernel: every cps-th partition (1) or consecutive partitions (0).
#ifndef PA_STREAM_INTERLEAVE
#define PA_STREAM_INTERLEAVE 0
#endif

// Tokens per wave step of the vector kernel (its SB_MAX): 32, fewer for long rows.
int vector_step_tokens(int D, int kv) {
  const int t = 8192 / (D * elem_bytes(kv));
  return t < 32 ? t : 32;
}

// Shapes that take the vector kernel rather than the matrix-core one (the per-unit kernels'
// choice in launch_one: matrix cores for 2 to 8 query heads per KV head with 16-bit io, KV
// of the io type or fp8, head_dim <= 128 and token rows of a multiple of 128 bytes).
bool vector_shape(const Common& c) {
  const int g = c.H / c.Hkv;
  const int row = c.D * elem_bytes(c.kv);
  const bool mfma = g >= 2 && (c.io == PA_F16 || c.io == PA_BF16) && (c.kv == c.io || c.kv == PA_FP8_E4M3) &&
                    c.D <= 128 && row >= 128 && row % 128 == 0;
  return !mfma;
}

// The balanced scheduler covers 1, 2, 4 or 8 query heads per KV head, io f16 / bf16, KV
// = io or fp8, 128 or 256 bytes per token row, at most kMaxBalancedSeqs sequences.
bool balanced_shape(const Common& c) {
  const int g = c.H / c.Hkv;
  if (g != 1 && g != 2 && g != 4 && g != 8) return false;
  if (c.io != PA_F16 && c.io != PA_BF16) return false;
  if (c.kv != c.io && c.kv != PA_FP8_E4M3) return false;
  const int row = c.D * elem_bytes(c.kv);
  if (c.D > 128 || (row != 128 && row != 256)) return false;
  return c.S <= kMaxBalancedSeqs;
}

struct BalancedLayout {
  size_t counter_bytes;  // int32 per (KV head, sequence), padded to 256 bytes
  size_t slot_bytes;     // fp32 m[G], l[G], o[G][D], two slots per workgroup
  size_t total;
};

BalancedLayout balanced_layout(int S, int H, int Hkv, int D, int nwg) {
  BalancedLayout b{};
  const int64_t G = H / Hkv;
  b.counter_bytes = (size_t)((((int64_t)Hkv * S * 4) + 255) / 256 * 256);
  b.slot_bytes = (size_t)((int64_t)nwg * 2 * G * (D + 2) * 4);
  b.total = b.counter_bytes + b.slot_bytes;
  return b;
}

// Shapes of the grouped (shared-prefix) kernel: 2, 4 or 8 query heads per KV head on the
// matrix cores (16-bit io, KV of the io type or fp8, head_dim <= 128, token rows of a
// multiple of 128 bytes) and blocks of at least 16 tokens.
bool grouped_shape(const Common& c) {
  const int g = c.H / c.Hkv;
  const int row = c.D * elem_bytes(c.kv);
  return (g == 2 || g == 4 || g == 8) && (c.io == PA_F16 || c.io == PA_BF16) &&
         (c.kv == c.io || c.kv == PA_FP8_E4M3) && c.D <= 128 && row >= 128 && row % 128 == 0 && c.BS >= 16;
}

// Splits of each (KV head, group) for the grouped kernel: num_splits, or for 0 as many as
// give about two workgroups per compute unit (at most 16).
int grouped_splits(int S, int H, int Hkv, int num_splits) {
  if (num_splits > 0) return num_splits;
  const int64_t ng = 16 / (H / Hkv);
  const int64_t units = (int64_t)Hkv * ((S + ng - 1) / ng);
  const int64_t want = (2 * (int64_t)device_cus() + units - 1) / units;
  return (int)(want < 1 ? 1 : (want > 16 ? 16 : want));
}

size_t grouped_workspace_bytes(int S, int H, int D, int nsplit) {
  return nsplit <= 1 ? 0 : (size_t)((int64_t)S * H * nsplit * (D + 2) * 4);
}

enum class Mode { kSingle, kPartitioned, kBalanced, kOrdered, kGrouped };

// Shared body of every entry point. P is the partition size (partitioned mode), nwg the
// workgroup count (balanced mode).
int run(const Common& c, Mode mode, int max_context_len, int P, int nwg, void* workspace,
        size_t ws_bytes, void* dk, void* dv, int32_t* dcounts, bool debug, hipStream_t st,
        int32_t* dblock_reads = nullptr) {
  int rc = validate(c);
  if (rc != PA_OK) return rc;
  LaunchSpec ls{};
  ls.args = base_args(c);
  ls.head_dim = c.D;
  ls.block_size = c.BS;
  ls.group = c.H / c.Hkv;
  ls.debug = debug;
  ls.stream = st;
  const int cap = c.MB * c.BS;  // a table row covers at most this many tokens
  if (mode == Mode::kBalanced && !balanced_shape(c)) mode = Mode::kSingle;  // same result
  if (mode == Mode::kGrouped && !grouped_shape(c)) mode = Mode::kSingle;    // same result
  int64_t NP = 1;
  if (mode == Mode::kPartitioned) {
    if (max_context_len < 0) return PA_ERR_INVALID;
    if (P % c.BS != 0) return PA_ERR_INVALID;
    NP = num_parts_for(max_context_len, P);
    const size_t need = pa_partitioned_workspace_bytes(c.S, c.H, c.D, max_context_len, P);
    if (need == 0) return PA_ERR_INVALID;
    if (NP > 1 && (!workspace || ws_bytes < need)) return PA_ERR_WORKSPACE;
    if (NP > 1 && !aligned16(workspace)) return PA_ERR_INVALID;
    ls.args.part_tokens = P;
    ls.args.max_ctx = max_context_len < cap ? max_context_len : cap;
  } else {
    ls.args.max_ctx = cap;
    if (max_context_len >= 0 && max_context_len < cap) ls.args.max_ctx = max_context_len;
    ls.args.part_tokens = ls.args.max_ctx > 0 ? ls.args.max_ctx : 1;
  }
  ls.args.num_parts = (int)NP;
  ls.args.ws = (float*)workspace;
  if (debug) {
    if (!dk || !dv || !dcounts || max_context_len <= 0) return PA_ERR_INVALID;
    if (!aligned16(dk) || !aligned16(dv)) return PA_ERR_INVALID;
    ls.args.dbg_k = dk;
    ls.args.dbg_v = dv;
    ls.args.dbg_counts = dcounts;
    ls.args.dbg_block_reads = dblock_reads;
    ls.args.dbg_max_ctx = max_context_len;
    if (ls.args.max_ctx > max_context_len) ls.args.max_ctx = max_context_len;
  }
  if (mode == Mode::kBalanced) {
    if (nwg < 0) return PA_ERR_INVALID;
    if (nwg == 0) nwg = default_balanced_workgroups();
    const BalancedLayout lay = balanced_layout(c.S, c.H, c.Hkv, c.D, nwg);
    if (!workspace || ws_bytes < lay.total) return PA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return PA_ERR_INVALID;
    ls.args.counters = (int32_t*)workspace;
    ls.args.ws = (float*)((char*)workspace + lay.counter_bytes);
    ls.args.nwg = nwg;
    ls.balanced = true;
    ls.grid = nwg;
    return launch_pair(c.io, c.kv, ls);
  }
  if (mode == Mode::kGrouped) {
    const int nsplit = grouped_splits(c.S, c.H, c.Hkv, nwg);
    const int64_t ng = 16 / (c.H / c.Hkv);
    const int64_t grid = (int64_t)c.Hkv * ((c.S + ng - 1) / ng) * nsplit;
    if (grid > INT_MAX) return PA_ERR_INVALID;
    if (nsplit > 1) {
      if (!workspace || ws_bytes < grouped_workspace_bytes(c.S, c.H, c.D, nsplit)) return PA_ERR_WORKSPACE;
      if (!aligned16(workspace)) return PA_ERR_INVALID;
    }
    ls.args.ws = (float*)workspace;
    ls.args.num_parts = nsplit;
    ls.grouped = true;
    ls.grid = (int)grid;
    rc = launch_pair(c.io, c.kv, ls);
    if (rc != PA_OK || nsplit <= 1) return rc;
    MergeArgs m{};
    m.ws = (const float*)workspace;
    m.context_lens = c.cl;
    m.out = c.out;
    m.num_seqs = c.S;
    m.num_heads = c.H;
    m.num_parts = nsplit;
    m.part_tokens = 1;
    m.max_ctx = ls.args.max_ctx;
    m.fixed_parts = nsplit;
    return launch_merge(c.io, c.D, m, c.S * c.H, st);
  }
  if (mode == Mode::kOrdered && c.S <= kOrderLdsSeqs) {
    // the decode launch derives the longest-first order itself (no workspace); larger
    // batches keep the index order (same result)
    ls.args.ordered = 1;
    ls.args.order_hpx = c.Hkv % 8 == 0 ? c.Hkv / 8 : 0;
  }
  const int64_t grid = (int64_t)c.Hkv * c.S * NP;
  if (grid > INT_MAX) return PA_ERR_INVALID;
  ls.grid = (int)grid;
  if (mode == Mode::kPartitioned && NP > 1 && vector_shape(c) && P % vector_step_tokens(c.D, c.kv) == 0) {
    // streaming kernel: runs of k consecutive partitions per wave, about
    // PA_STREAM_WAVES_PER_CU waves per compute unit; runs of one (sequence, KV head) as
    // even as the partition count allows
    const int64_t units = (int64_t)c.Hkv * c.S;
    const int64_t target = (int64_t)PA_STREAM_WAVES_PER_CU * device_cus();
    int64_t runs = target / units;
    runs = runs < 1 ? 1 : (runs > NP ? NP : runs);
    const int64_t k = (NP + runs - 1) / runs;
    const int64_t chunks = (NP + k - 1) / k;
    ls.stream_kernel = true;
    ls.args.wave_parts = (int)k;
    ls.args.wave_chunks = (int)chunks;
    ls.args.wave_interleave = PA_STREAM_INTERLEAVE;
    // the runs of each unit fill whole workgroups and every run's states fit its wave's
    // buffer: the workgroups merge the partitions themselves (no merge launch)
    const int G = c.H / c.Hkv;
    ls.args.wave_merge = (PA_WAVES % chunks == 0 && k <= stream_states(G, c.D)) ? 1 : 0;
    ls.stream_waves = (int)((int64_t)c.Hkv * c.S * chunks);
  }
  rc = launch_pair(c.io, c.kv, ls);
  if (rc != PA_OK || NP <= 1 || ls.args.wave_merge) return rc;
  MergeArgs m{};
  m.ws = (const float*)workspace;
  m.context_lens = c.cl;
  m.out = c.out;
  m.num_seqs = c.S;
  m.num_heads = c.H;
  m.num_parts = (int)NP;
  m.part_tokens = P;
  m.max_ctx = ls.args.max_ctx;
  const int64_t pairs = (int64_t)c.S * c.H;
  return launch_merge(c.io, c.D, m, (int)pairs, st);
}

}  // namespace
}  // namespace pa

extern "C" {

int pa_decode(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_tables,
              const int32_t* context_lens, int num_seqs, int max_blocks_per_seq, int num_blocks,
              int num_heads, int num_kv_heads, int head_dim, int block_size, float scale,
              int io_dtype, int kv_dtype, float k_scale, float v_scale, void* out, void* stream) {
  try {
    pa::Common c{q, k_pool, v_pool, block_tables, context_lens, num_seqs, max_blocks_per_seq,
                 num_blocks, num_heads, num_kv_heads, head_dim, block_size, scale, io_dtype,
                 kv_dtype, k_scale, v_scale, out};
    return pa::run(c, pa::Mode::kSingle, -1, 0, 0, nullptr, 0, nullptr, nullptr, nullptr, false,
                   (hipStream_t)stream);
  } catch (...) {
    return PA_ERR_LAUNCH;
  }
}

size_t pa_partitioned_workspace_bytes(int num_seqs, int num_heads, int head_dim,
                                      int max_context_len, int partition_size) {
  if (num_seqs <= 0 || num_heads <= 0 || head_dim <= 0 || max_context_len < 0 || partition_size < 0)
    return 0;
  const int P = partition_size == 0 ? pa::kDefaultPartition : partition_size;
  const int64_t NP = pa::num_parts_for(max_context_len, P);
  const int64_t floats = (int64_t)num_seqs * num_heads * NP * (head_dim + 2);
  return (size_t)(floats * 4);
}

int pa_decode_partitioned(const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                          int max_blocks_per_seq, int num_blocks, int num_heads, int num_kv_heads,
                          int head_dim, int block_size, float scale, int io_dtype, int kv_dtype,
                          float k_scale, float v_scale, int max_context_len, int partition_size,
                          void* workspace, size_t workspace_bytes, void* out, void* stream) {
  try {
    if (partition_size < 0) return PA_ERR_INVALID;
    const int P = partition_size == 0 ? pa::kDefaultPartition : partition_size;
    pa::Common c{q, k_pool, v_pool, block_tables, context_lens, num_seqs, max_blocks_per_seq,
                 num_blocks, num_heads, num_kv_heads, head_dim, block_size, scale, io_dtype,
                 kv_dtype, k_scale, v_scale, out};
    return pa::run(c, pa::Mode::kPartitioned, max_context_len, P, 0, workspace, workspace_bytes,
                   nullptr, nullptr, nullptr, false, (hipStream_t)stream);
  } catch (...) {
    return PA_ERR_LAUNCH;
  }
}

int pa_decode_partitioned_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                  const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                                  int max_blocks_per_seq, int num_blocks, int num_heads, int num_kv_heads,
                                  int head_dim, int block_size, float scale, int io_dtype, int kv_dtype,
                                  float k_scale, float v_scale, int max_context_len, int partition_size,
                                  void* out, void* stream) {
  try {
    if (partition_size < 0 || max_context_len < 0) return PA_ERR_INVALID;
    const int P = partition_size == 0 ? pa::kDefaultPartition : partition_size;
    pa::Common c{q, k_pool, v_pool, block_tables, context_lens, num_seqs, max_blocks_per_seq,
                 num_blocks, num_heads, num_kv_heads, head_dim, block_size, scale, io_dtype,
                 kv_dtype, k_scale, v_scale, out};
    // every host check before the first HIP call
    int rc = pa::validate(c);
    if (rc != PA_OK) return rc;
    if (P % block_size != 0) return PA_ERR_INVALID;
    const size_t need = pa_partitioned_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len, P);
    if (need == 0) return PA_ERR_INVALID;
    if (need > PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_SCRATCH;
    void* ws = nullptr;
    rc = pa::scratch_ptr(&ws);
    if (rc != PA_OK) return rc;
    return pa::run(c, pa::Mode::kPartitioned, max_context_len, P, 0, ws, PA_NOALLOC_SCRATCH_BYTES, nullptr,
                   nullptr, nullptr, false, (hipStream_t)stream);
  } catch (...) {
    return PA_ERR_LAUNCH;
  }
}

size_t pa_balanced_workspace_bytes(int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                                   int num_workgroups) {
  if (num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || num_workgroups < 0 ||
      num_heads % num_kv_heads != 0)
    return 0;
  try {
    const int nwg = num_workgroups == 0 ? pa::default_balanced_workgroups() : num_workgroups;
    return pa::balanced_layout(num_seqs, num_heads, num_kv_heads, head_dim, nwg).total;
  } catch (...) {
    return 0;
  }
}

int pa_decode_balanced(const void* q, const void* k_pool, const void* v_pool,
                       const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                       int max_blocks_per_seq, int num_blocks, int num_heads, int num_kv_heads,
                       int head_dim, int block_size, float scale, int io_dtype, int kv_dtype,
                       float k_scale, float v_scale, int num_workgroups, void* workspace,
                       size_t workspace_bytes, void* out, void* stream) {
  try {
    if (num_workgroups < 0) return PA_ERR_INVALID;
    pa::Common c{q, k_pool, v_pool, block_tables, context_lens, num_seqs, max_blocks_per_seq,
                 num_blocks, num_heads, num_kv_heads, head_dim, block_size, scale, io_dtype,
                 kv_dtype, k_scale, v_scale, out};
    return pa::run(c, pa::Mode::kBalanced, -1, 0, num_workgroups, workspace, workspace_bytes,
                   nullptr, nullptr, nullptr, false, (hipStream_t)stream);
  } catch (...) {
    return PA_ERR_LAUNCH;
  }
}

size_t pa_grouped_workspace_bytes(int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                                  int num_splits) {
  if (num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || num_splits < 0 ||
      num_heads % num_kv_heads != 0)
    return 0;
  try {
    const int G = num_heads / num_kv_heads;
    if (G != 2 && G != 4 && G != 8) return 0;
    const int nsplit = pa::grouped_splits(num_seqs, num_heads, num_kv_heads, num_splits);
    return pa::grouped_workspace_bytes(num_seqs, num_heads, head_dim, nsplit);
  } catch (...) {
    return 0;
  }
}

int pa_decode_grouped(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_tables,
                      const int32_t* context_lens, int num_seqs, int max_blocks_per_seq, int num_blocks,
                      int num_heads, int num_kv_heads, int head_dim, int block_size, float scale, int io_dtype,
                      int kv_dtype, float k_scale, float v_scale, int num_splits, void* workspace,
                      size_t workspace_bytes, void* out, void* stream) {
  try {
    if (num_splits < 0) return PA_ERR_INVALID;
    pa::Common c{q, k_pool, v_pool, block_tables, context_lens, num_seqs, max_blocks_per_seq,
                 num_blocks, num_heads, num_kv_heads, head_dim, block_size, scale, io_dtype,
                 kv_dtype, k_scale, v_scale, out};
    return pa::run(c, pa::Mode::kGrouped, -1, 0, num_splits, workspace, workspace_bytes, nullptr, nullptr,
                   nullptr, false, (hipStream_t)stream);
  } catch (...) {
    return PA_ERR_LAUNCH;
  }
}

int pa_debug_trace_grouped(const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                           int max_blocks_per_seq, int num_blocks, int num_heads, int num_kv_heads,
                           int head_dim, int block_size, float scale, int io_dtype, int kv_dtype,
                           float k_scale, float v_scale, int max_context_len, int num_splits,
                           void* workspace, size_t workspace_bytes, void* out, void* k_rows,
                           void* v_rows, int32_t* read_counts, int32_t* block_reads, void* stream) {
  try {
    if (num_splits < 0) return PA_ERR_INVALID;
    pa::Common c{q, k_pool, v_pool, block_tables, context_lens, num_seqs, max_blocks_per_seq,
                 num_blocks, num_heads, num_kv_heads, head_dim, block_size, scale, io_dtype,
                 kv_dtype, k_scale, v_scale, out};
    const int rc = pa::validate(c);
    if (rc != PA_OK) return rc;
    if (!pa::grouped_shape(c)) return PA_ERR_UNSUPPORTED;
    if (!block_reads) return PA_ERR_INVALID;
    return pa::run(c, pa::Mode::kGrouped, max_context_len, 0, num_splits, workspace, workspace_bytes,
                   k_rows, v_rows, read_counts, true, (hipStream_t)stream, block_reads);
  } catch (...) {
    return PA_ERR_LAUNCH;
  }
}

size_t pa_ordered_workspace_bytes(int num_seqs) {
  (void)num_seqs;
  return 0;
}

int pa_decode_ordered(const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                      int max_blocks_per_seq, int num_blocks, int num_heads, int num_kv_heads,
                      int head_dim, int block_size, float scale, int io_dtype, int kv_dtype,
                      float k_scale, float v_scale, void* workspace, size_t workspace_bytes,
                      void* out, void* stream) {
  try {
    pa::Common c{q, k_pool, v_pool, block_tables, context_lens, num_seqs, max_blocks_per_seq,
                 num_blocks, num_heads, num_kv_heads, head_dim, block_size, scale, io_dtype,
                 kv_dtype, k_scale, v_scale, out};
    return pa::run(c, pa::Mode::kOrdered, -1, 0, 0, workspace, workspace_bytes, nullptr, nullptr,
                   nullptr, false, (hipStream_t)stream);
  } catch (...) {
    return PA_ERR_LAUNCH;
  }
}

int pa_debug_trace(const void* q, const void* k_pool, const void* v_pool,
                   const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                   int max_blocks_per_seq, int num_blocks, int num_heads, int num_kv_heads,
                   int head_dim, int block_size, float scale, int io_dtype, int kv_dtype,
                   float k_scale, float v_scale, int max_context_len, int partition_size,
                   int num_workgroups, void* workspace, size_t workspace_bytes, void* out,
                   void* k_rows, void* v_rows, int32_t* read_counts, void* stream) {
  try {
    if (partition_size < 0 || num_workgroups < 0) return PA_ERR_INVALID;
    if (partition_size > 0 && num_workgroups > 0) return PA_ERR_INVALID;
    pa::Common c{q, k_pool, v_pool, block_tables, context_lens, num_seqs, max_blocks_per_seq,
                 num_blocks, num_heads, num_kv_heads, head_dim, block_size, scale, io_dtype,
                 kv_dtype, k_scale, v_scale, out};
    const pa::Mode mode = num_workgroups > 0 ? pa::Mode::kBalanced
                          : partition_size > 0 ? pa::Mode::kPartitioned
                                               : pa::Mode::kSingle;
    return pa::run(c, mode, max_context_len, partition_size, num_workgroups, workspace,
                   workspace_bytes, k_rows, v_rows, read_counts, true, (hipStream_t)stream);
  } catch (...) {
    return PA_ERR_LAUNCH;
  }
}

int pa_check_tables(const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                    int max_blocks_per_seq, int num_blocks, int block_size, int max_context_len,
                    int32_t* errors, void* stream) {
  if (!block_tables || !context_lens || !errors) return PA_ERR_INVALID;
  if (num_seqs <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 || block_size <= 0)
    return PA_ERR_INVALID;
  const int threads = 256;
  const int grid = (num_seqs + threads - 1) / threads;
  hipLaunchKernelGGL(pa::check_tables_kernel, dim3(grid), dim3(threads), 0, (hipStream_t)stream,
                     block_tables, context_lens, num_seqs, max_blocks_per_seq, num_blocks,
                     block_size, max_context_len, errors);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int pa_debug_fp8_to_f32(const uint8_t* codes, float* out, int n, void* stream) {
  if (!codes || !out || n <= 0) return PA_ERR_INVALID;
  const int lanes = (n + 15) / 16;
  const int grid = (lanes + 255) / 256;
  hipLaunchKernelGGL(pa::fp8_probe_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, codes, out, n);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int pa_debug_fp8_to_16bit(const uint8_t* codes, uint16_t* out, int n, int out_dtype, void* stream) {
  if (!codes || !out || n <= 0) return PA_ERR_INVALID;
  if (out_dtype != PA_F16 && out_dtype != PA_BF16) return PA_ERR_INVALID;
  const int lanes = (n + 15) / 16;
  const int grid = (lanes + 255) / 256;
  if (out_dtype == PA_F16) {
    hipLaunchKernelGGL(pa::fp8_mt_probe_kernel<pa::kF16>, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       codes, out, n);
  } else {
    hipLaunchKernelGGL(pa::fp8_mt_probe_kernel<pa::kBF16>, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       codes, out, n);
  }
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

const char* pa_status_str(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported shape or dtype combination";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_LAUNCH: return "kernel launch failed";
    case PA_ERR_SCRATCH: return "request exceeds the library's static scratch (PA_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int pa_version(void) { return 200; }

}  // extern "C"
