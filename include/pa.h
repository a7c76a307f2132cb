/*
 * pa.h — paged-attention decode over a block table, for AMD Instinct MI355X (gfx950).
 *
 * One query token per sequence attends over that sequence's cached keys and values.
 * The cache lives in fixed-size physical blocks of a shared pool; a per-sequence
 * block table maps logical block j (tokens j*block_size ... j*block_size +
 * block_size - 1) to a physical block, and several sequences may name the same
 * physical block (shared prefixes).
 *
 * Pages this interface follows (cited by title and section):
 *   [P1] "突破GPU内存瓶颈：vLLM与PagedAttention技术深度解析" (ocdem.com), §2: fixed-size
 *        KV blocks, block table from logical to physical blocks, shared blocks, only
 *        the last block of a sequence partly filled.
 *   [P2] vLLM architecture deep-dive (lshu.cn), §1.1: the paged-attention call takes
 *        queries, blocked key cache, blocked value cache and block tables, and scores
 *        are q.K^T / sqrt(head_dim); §2.2: attention metadata = block tables, context
 *        lengths, head count, head size; §3.3 and §4.1: a second, split-context kernel
 *        for long text; §4.2: FP8 KV cache.
 *   [P3] "内存优化：KV Cache管理、PagedAttention原理与内存池配置" (5688vip.com): the
 *        decode step scores the current token's query against all cached K/V; block
 *        pool figure; KV-size formula.
 *
 * What every entry point computes, for sequence s of context length L = context_lens[s]
 * and query head h (G = num_heads / num_kv_heads, KV head g = h / G):
 *     z_t = scale * sum_d q[s][h][d] * K(s, g, t)[d]            t = 0 .. L-1
 *     out[s][h][:] = sum_t softmax(z)_t * V(s, g, t)[:]          (L = 0: zeros)
 *     K(s, g, t) = k_pool[ block_tables[s][t / block_size] ][g][t % block_size][:]
 * with fp8 keys/values dequantized as code_value * k_scale (resp. v_scale).
 * Accumulation is fp32; out is rounded to the io dtype (round to nearest even).
 *
 * Layouts (all row-major, all DEVICE memory, all owned by the caller):
 *   q            [num_seqs][num_heads][head_dim]                 io_dtype
 *   k_pool       [num_blocks][num_kv_heads][block_size][head_dim] kv_dtype
 *   v_pool       [num_blocks][num_kv_heads][block_size][head_dim] kv_dtype
 *   block_tables [num_seqs][max_blocks_per_seq] int32; entries at or past
 *                ceil(L / block_size) are never read (pad them with anything)
 *   context_lens [num_seqs] int32
 *   out          [num_seqs][num_heads][head_dim]                 io_dtype
 * Pointers to q, the pools and out must be 16-byte aligned.
 *
 * Ownership and ordering: the library allocates nothing, frees nothing, keeps no
 * per-call state and never synchronizes. Each call enqueues its kernels on `stream`
 * (a hipStream_t; NULL = the default stream) and returns. Inputs must stay unchanged,
 * and out / workspace untouched, until the stream has passed the call; out must not
 * alias any input. Calls that share one workspace must be ordered on one stream.
 *
 * Errors: the return value is a pa_status. Every argument check runs on the host
 * before any HIP call; on an error nothing is enqueued. A failed launch returns
 * PA_ERR_LAUNCH. No C++ exception crosses this interface. Device-side contract
 * violations (a used block-table entry outside [0, num_blocks), a context length
 * above max_blocks_per_seq * block_size or above max_context_len) never make the
 * kernels read outside the buffers: ids are clamped into the pool and lengths into
 * the bound, and the result for that sequence is unspecified. pa_check_tables reports
 * such violations.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage types. PA_FP8_E4M3 is the OCP 8-bit e4m3 format (bias 7, max 448, NaN =
 * S.1111.111, no infinities), valid only as kv_dtype. */
typedef enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2, PA_FP8_E4M3 = 3 } pa_dtype;

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID = -1,     /* null pointer, non-positive size, bad dtype code, ... */
  PA_ERR_UNSUPPORTED = -2, /* valid but not compiled: head_dim, block_size, group, dtype pair */
  PA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than pa_partitioned_workspace_bytes */
  PA_ERR_LAUNCH = -4,      /* the HIP launch itself failed */
  PA_ERR_SCRATCH = -5      /* the request needs more than the library's static scratch */
} pa_status;

/* Supported shapes: head_dim in {64, 128, 256} (256 on the vector kernel only, single
 * pass or partitioned); block_size in {8, 16, 32, 64, 128, 256, 512}
 * ([P1] §2 and [P3] use 16; [P2] §3.1 uses 256 by default, 128 for short and 512 for
 * long texts; with fp8 and head_dim 64, block_size >= 16); num_heads / num_kv_heads in
 * {1, 2, 4, 8};
 * io_dtype in {F32, F16, BF16}; kv_dtype == io_dtype or PA_FP8_E4M3.
 * scale, k_scale, v_scale must be finite and > 0 (k_scale / v_scale are ignored unless
 * kv_dtype is PA_FP8_E4M3). */

/* Single-pass decode ([P2] §1.1 paged-attention call; [P3] decode step): one
 * workgroup per (sequence, KV head) reads every cached token of that head once,
 * shares it across the G query heads of the group, and writes out directly. Best for
 * short and medium contexts; needs no workspace. num_blocks is the pool size. */
int pa_decode(const void* q, const void* k_pool, const void* v_pool,
              const int32_t* block_tables, const int32_t* context_lens,
              int num_seqs, int max_blocks_per_seq, int num_blocks,
              int num_heads, int num_kv_heads, int head_dim, int block_size,
              float scale, int io_dtype, int kv_dtype, float k_scale, float v_scale,
              void* out, void* stream);

/* Workspace for pa_decode_partitioned, in bytes (0 on invalid sizes). Holds, per
 * (sequence, query head, partition), the running max, the exp-sum and the fp32
 * partial output. partition_size 0 means the library's default (512 tokens). */
size_t pa_partitioned_workspace_bytes(int num_seqs, int num_heads, int head_dim,
                                      int max_context_len, int partition_size);

/* Split-context decode for long contexts ([P2] §3.3 and §4.1 second-version kernel).
 * The context of every sequence is cut into partitions of partition_size tokens (a
 * multiple of block_size; 0 = default 512); each partition's max, exp-sum and
 * unnormalized output are combined per (sequence, head) by log-sum-exp weighting.
 * Sequences with one partition are written directly. How the partitions are scheduled
 * depends on the shape: with the matrix-core kernels one workgroup per (sequence, KV
 * head, partition) writes its state into the workspace and a second kernel on the same
 * stream merges; with the vector kernel (one query head per KV head, fp32, head_dim 256,
 * fp8 with head_dim 64) each wave streams a run of consecutive partitions, and when the
 * runs of a (sequence, KV head) are the waves of one workgroup the workgroup merges them
 * itself (one launch, the workspace untouched), else the states go to the workspace for
 * the merge kernel.
 * The workspace is required whenever there is more than one partition. max_context_len
 * is a host-known bound >= every context_lens[s]; it sizes the grid and the workspace. */
int pa_decode_partitioned(const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* block_tables, const int32_t* context_lens,
                          int num_seqs, int max_blocks_per_seq, int num_blocks,
                          int num_heads, int num_kv_heads, int head_dim, int block_size,
                          float scale, int io_dtype, int kv_dtype, float k_scale,
                          float v_scale, int max_context_len, int partition_size,
                          void* workspace, size_t workspace_bytes,
                          void* out, void* stream);

/* Bytes of the device scratch of pa_decode_partitioned_noalloc (per GPU). */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/* pa_decode_partitioned without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). Same kernels and the same result, bit for bit, as pa_decode_partitioned
 * with the same arguments; the partition states live instead in a device array that the
 * library holds, PA_NOALLOC_SCRATCH_BYTES (16 MiB) on each GPU it runs on, until the
 * process ends. Calls whose pa_partitioned_workspace_bytes(num_seqs, num_heads, head_dim,
 * max_context_len, partition_size) exceeds that return PA_ERR_SCRATCH before anything is
 * enqueued (16 MiB holds e.g. 8 sequences x 32 heads x head_dim 128 up to 32768 tokens in
 * 512-token partitions). The call allocates nothing; its first call on a device looks up
 * that device's copy of the array (no allocation). Every call on one GPU uses that GPU's
 * one array, so calls that overlap on a GPU (two streams, two threads) race and give
 * undefined results: order them on one stream. Nothing needs to be cleared between calls
 * (each call writes every partition state it reads). Errors as pa_decode_partitioned,
 * plus PA_ERR_SCRATCH. */
int pa_decode_partitioned_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  int num_seqs, int max_blocks_per_seq, int num_blocks,
                                  int num_heads, int num_kv_heads, int head_dim, int block_size,
                                  float scale, int io_dtype, int kv_dtype, float k_scale,
                                  float v_scale, int max_context_len, int partition_size,
                                  void* out, void* stream);

/* Workspace for pa_decode_balanced, in bytes (0 on invalid sizes): one int32 arrival
 * counter per (KV head, sequence), padded to 256 bytes, then two fp32 partial-state slots
 * (G running maxima, G exp-sums, G x head_dim partial outputs; G = num_heads /
 * num_kv_heads) per workgroup. num_workgroups 0 means the library's default (two per
 * compute unit of the current device). */
size_t pa_balanced_workspace_bytes(int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                                   int num_workgroups);

/* Work-balanced decode. Same result as pa_decode up to rounding order; the schedule
 * differs: the cached tokens of every (KV head, sequence) are cut into chunks of 16 or 32
 * tokens (by kernel shape), and a fixed grid of num_workgroups workgroups (0 = library
 * default) takes equal shares of the batch's work (its chunks plus a fixed cost for each
 * sequence piece a workgroup handles), whatever the mix of context lengths. A (KV head, sequence) whose chunks are
 * shared by several workgroups is finished by the last of them to arrive, which merges
 * the others' partial states by log-sum-exp weighting (the rule of the split-context
 * kernel, [P2] §3.3 / §4.1). Everything happens in one kernel launch.
 * Workspace: pa_balanced_workspace_bytes(...) bytes, 16-byte aligned. Its counter area
 * must be zero before the first call (e.g. hipMemset once after allocating); every
 * completed call leaves it zero again. Calls sharing a workspace must be ordered on one
 * stream. Shapes the balanced kernel does not take run the single-pass kernel of
 * pa_decode instead and leave the workspace untouched: fp32 io or KV, head_dim 256, token
 * rows (head_dim times the KV element size) other than 128 or 256 bytes (e.g. fp8 with
 * head_dim 64), and batches of more than 4096 sequences. */
int pa_decode_balanced(const void* q, const void* k_pool, const void* v_pool,
                       const int32_t* block_tables, const int32_t* context_lens,
                       int num_seqs, int max_blocks_per_seq, int num_blocks,
                       int num_heads, int num_kv_heads, int head_dim, int block_size,
                       float scale, int io_dtype, int kv_dtype, float k_scale, float v_scale,
                       int num_workgroups, void* workspace, size_t workspace_bytes,
                       void* out, void* stream);

/* Workspace for pa_decode_ordered, in bytes: 0, it needs none (the decode launch derives
 * the order itself). Kept so that callers sizing a workspace for it need no change. */
size_t pa_ordered_workspace_bytes(int num_seqs);

/* Longest-first decode. Same result as pa_decode, bit for bit (the same kernels compute
 * every (KV head, sequence)); only the dispatch order differs. Every workgroup of the one
 * decode launch finds its sequence by rank in the order "context-length class descending
 * (four classes per doubling of the length), then sequence index ascending", from the
 * context lengths alone (a class histogram and a prefix sum in LDS), and each XCD's share
 * of the (KV head, sequence) units is handed out longest sequence first, so that batches
 * mixing short and long contexts ([P2] §5.3's length mix) do not end with a few long
 * sequences running alone. Batches of more than 2048 sequences are dispatched in index
 * order, as by pa_decode: every workgroup reads all the lengths to find its rank, which
 * costs more there than the tail it removes. workspace and workspace_bytes are not used
 * (NULL and 0 are fine). Errors as pa_decode. */
int pa_decode_ordered(const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_tables, const int32_t* context_lens,
                      int num_seqs, int max_blocks_per_seq, int num_blocks,
                      int num_heads, int num_kv_heads, int head_dim, int block_size,
                      float scale, int io_dtype, int kv_dtype, float k_scale, float v_scale,
                      void* workspace, size_t workspace_bytes, void* out, void* stream);

/* Workspace for pa_decode_grouped, in bytes (0 when none is needed or on invalid sizes):
 * fp32 partial states (running maximum, exp-sum, head_dim partial outputs) for every
 * (sequence, query head) and split, when the call runs more than one split. num_splits 0
 * means the library's choice (about two workgroups per compute unit of the current device,
 * at most 16). */
size_t pa_grouped_workspace_bytes(int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                                  int num_splits);

/* Shared-prefix decode. Same result as pa_decode up to rounding order. Sequences whose
 * block tables name the same physical blocks (a shared prompt, [P1] §2 and §5: shared
 * blocks with reference counts; parallel samples of one prompt) read each shared block
 * once per KV head: a workgroup takes one KV head and a group of 16 / G consecutive
 * sequences (G = num_heads / num_kv_heads, 2, 4 or 8), walks their block tables side by
 * side, and runs the scores and the value products of one physical block for all group
 * members that name it at the same logical position together, on the matrix cores
 * (16 query rows = the members' query heads). Blocks a member does not share are read
 * for it alone. A group's logical blocks are cut in num_splits interleaved parts (0 =
 * library choice) run by separate workgroups; with more than one split a second launch
 * merges the parts by log-sum-exp weighting ([P2] §3.3 / §4.1), using the workspace
 * (pa_grouped_workspace_bytes(...) bytes, 16-byte aligned; NULL allowed when that is 0).
 * Sharing is found only between sequences of one group (consecutive indices) at equal
 * logical block positions: order a batch so that sequences with a common prefix are
 * adjacent. Shapes the grouped kernel does not take run the single-pass kernel of
 * pa_decode instead (same result; workspace unused): G not in {2, 4, 8}, fp32 io or KV,
 * head_dim above 128, token rows (head_dim times the KV element size) that are not a
 * multiple of 128 bytes, block_size below 16. */
int pa_decode_grouped(const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_tables, const int32_t* context_lens,
                      int num_seqs, int max_blocks_per_seq, int num_blocks,
                      int num_heads, int num_kv_heads, int head_dim, int block_size,
                      float scale, int io_dtype, int kv_dtype, float k_scale, float v_scale,
                      int num_splits, void* workspace, size_t workspace_bytes,
                      void* out, void* stream);

/* Instrumented decode for tests ([P1] §2 block-table reading; every cached position
 * is read exactly once). Runs the same kernels as pa_decode (partition_size == 0 and
 * num_workgroups == 0), pa_decode_partitioned (partition_size > 0, workspace required) or
 * pa_decode_balanced (num_workgroups > 0, workspace required, counters zero) and, as the
 * kernel consumes each valid cached row of (sequence s, KV head g, token t), also
 *   copies the raw K row to k_rows[((s * num_kv_heads + g) * max_context_len + t) * head_dim]
 *   copies the raw V row to v_rows[ same ]                      (kv_dtype elements)
 *   adds 1 to read_counts[(s * num_kv_heads + g) * max_context_len + t]
 * read_counts must be zeroed by the caller; rows never consumed are left untouched.
 * max_context_len must be >= every context length. */
int pa_debug_trace(const void* q, const void* k_pool, const void* v_pool,
                   const int32_t* block_tables, const int32_t* context_lens,
                   int num_seqs, int max_blocks_per_seq, int num_blocks,
                   int num_heads, int num_kv_heads, int head_dim, int block_size,
                   float scale, int io_dtype, int kv_dtype, float k_scale, float v_scale,
                   int max_context_len, int partition_size, int num_workgroups,
                   void* workspace, size_t workspace_bytes, void* out,
                   void* k_rows, void* v_rows, int32_t* read_counts, void* stream);

/* Instrumented pa_decode_grouped for tests: the trace of pa_debug_trace (k_rows, v_rows,
 * read_counts, per (sequence, KV head, token) consumed), and in addition
 *   adds 1 to block_reads[b * num_kv_heads + g]
 * for every load of 16 cached rows of physical block b for KV head g, however many
 * sequences of the group use that load. block_reads [num_blocks][num_kv_heads] int32 must
 * be zeroed by the caller. PA_ERR_UNSUPPORTED for shapes the grouped kernel does not take. */
int pa_debug_trace_grouped(const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* block_tables, const int32_t* context_lens,
                           int num_seqs, int max_blocks_per_seq, int num_blocks,
                           int num_heads, int num_kv_heads, int head_dim, int block_size,
                           float scale, int io_dtype, int kv_dtype, float k_scale, float v_scale,
                           int max_context_len, int num_splits, void* workspace,
                           size_t workspace_bytes, void* out, void* k_rows, void* v_rows,
                           int32_t* read_counts, int32_t* block_reads, void* stream);

/* Appends new tokens' keys and values to the paged cache ([P1] §2 block table; [P3]
 * paged pool: a growing request writes into its last block and gets blocks appended;
 * [P2] §2.1 decode mode). Token t (of num_tokens) belongs to sequence seq_ids[t] at
 * logical position positions[t]; its rows
 *   k_new[t][g][:], v_new[t][g][:]   (layout [num_tokens][num_kv_heads][head_dim], src_dtype)
 * are stored, for every KV head g, at
 *   k_pool[ block_tables[s][p / block_size] ][g][p % block_size][:]   (and v_pool)
 * src_dtype is F32, F16 or BF16; kv_dtype equals it (the bits are copied) or is
 * PA_FP8_E4M3, which stores e4m3(x / k_scale) (v_scale for V): the quotient rounded to
 * fp32, then to the nearest e4m3 value (ties to even), magnitudes above 448 saturated to
 * +-448, NaN kept as NaN. The caller allocates the blocks (the table entries must exist);
 * a token whose sequence, position or block lies outside the tables or the pool is
 * skipped. Pointers to k_new, v_new and the pools must be 16-byte aligned; head_dim in
 * {64, 128, 256}, block_size in {8, 16, ..., 512} (powers of two). Asynchronous on `stream`;
 * allocates nothing. */
int pa_append_kv(const void* k_new, const void* v_new, const int32_t* seq_ids,
                 const int32_t* positions, int num_tokens, const int32_t* block_tables,
                 int num_seqs, int max_blocks_per_seq, void* k_pool, void* v_pool,
                 int num_blocks, int num_kv_heads, int head_dim, int block_size,
                 int src_dtype, int kv_dtype, float k_scale, float v_scale, void* stream);

/* Copies whole physical blocks for copy-on-write ([P3] paged pool: sequences of a parallel
 * sample or a beam share physical blocks by reference count; [P1] §5 beam search). The
 * pages share blocks but do not say what happens when one sharer writes into a shared,
 * partly filled block; the plainest reading, and what pa_bm_append_token reports, is
 * that the writer first gets a private copy. For each i < num_pairs, with
 * src = block_pairs[2i] and dst = block_pairs[2i + 1] (device int32 array):
 *   k_pool[dst][:][:][:] = k_pool[src][:][:][:]   and the same for v_pool
 * (layout [num_blocks][num_kv_heads][block_size][head_dim], kv_dtype elements; every byte
 * of the block is copied, whatever its fill). Pairs run in parallel: no dst may be the src
 * or the dst of another pair. Pairs with an id outside [0, num_blocks) or src == dst are
 * skipped. Pools must be 16-byte aligned and a block's bytes a multiple of 16.
 * num_pairs == 0 is a no-op. Asynchronous on `stream`; allocates nothing. */
int pa_copy_blocks(void* k_pool, void* v_pool, const int32_t* block_pairs, int num_pairs,
                   int num_blocks, int num_kv_heads, int head_dim, int block_size,
                   int kv_dtype, void* stream);

/* Paged attention for several new tokens per sequence: prefill and extend ([P2] §2.1
 * names both modes next to decode; §2.2's metadata holds block tables, context lengths
 * and query lengths; [P1] §2 block tables). Sequence s has L = context_lens[s] cached
 * tokens, counting its new ones, whose K/V are already in the pools (pa_append_kv);
 * the new ones are its last Q = query_start_loc[s+1] - query_start_loc[s] positions
 * (the metadata's query lengths are these differences). New token i < Q sits at
 * position p = L - Q + i; for every query head h (KV head g = h / (H / Hkv)):
 *   out[query_start_loc[s] + i][h][:] = softmax(scale * K_s[0..p] q) V_s[0..p]
 *   with q = q[query_start_loc[s] + i][h][:] and K_s / V_s read through the table
 * i.e. causal among the new tokens (the plainest reading: the pages do not spell it
 * out). q and out are [T][H][D] in io_dtype with T = query_start_loc[num_seqs];
 * query_start_loc is a device int32 array [num_seqs + 1], non-decreasing, starting at 0;
 * max_query_len (host) is >= every Q and sizes the grid. Rows with p < 0 (Q > L,
 * outside the contract) are written as zeros. fp32 accumulation on the matrix cores:
 * io_dtype F16 or BF16 (F32 is PA_ERR_UNSUPPORTED), kv_dtype == io_dtype or
 * PA_FP8_E4M3, head_dim in {64, 128}, block_size a power of two in [8, 512],
 * num_heads / num_kv_heads in {1, 2, 4, 8}. max_query_len == 0 is a no-op. With 2, 4 or
 * 8 query heads per KV head, block_size >= 16 and token rows of at least 128 bytes, the
 * sequences with at most 16 / G new tokens are computed by a decode-style kernel (all
 * their query rows walk the blocks together) enqueued before the prefill kernel, which
 * then skips them. Asynchronous on `stream`; allocates nothing. */
int pa_extend(const void* q, const void* k_pool, const void* v_pool,
              const int32_t* block_tables, const int32_t* context_lens,
              const int32_t* query_start_loc, int num_seqs, int max_blocks_per_seq,
              int num_blocks, int max_query_len, int num_heads, int num_kv_heads,
              int head_dim, int block_size, float scale, int io_dtype, int kv_dtype,
              float k_scale, float v_scale, void* out, void* stream);

/* Device-side check of the block-table contract. For each sequence s writes
 * errors[s] = 0 if fine, else a bit set: 1 = context length < 0, 2 = context length
 * above max_blocks_per_seq * block_size, 4 = some used entry outside [0, num_blocks),
 * 8 = context length above max_context_len (if max_context_len > 0). */
int pa_check_tables(const int32_t* block_tables, const int32_t* context_lens,
                    int num_seqs, int max_blocks_per_seq, int num_blocks, int block_size,
                    int max_context_len, int32_t* errors, void* stream);

/* Converts n OCP e4m3 codes to fp32 with the same in-register conversion the decode
 * kernels use (for tests of the fp8 path). */
int pa_debug_fp8_to_f32(const uint8_t* codes, float* out, int n, void* stream);

/* Converts n OCP e4m3 codes to 16-bit values with the conversion that feeds the matrix
 * cores (the K operand of the score product for fp8 KV, and the V tile of the matrix-core
 * V product): out_dtype PA_F16 or PA_BF16 selects the type, out receives n 16-bit codes
 * in the order of the input (for tests of the fp8 path; every e4m3 value is exact in
 * both types). PA_ERR_INVALID on null pointers, n <= 0 or another out_dtype. */
int pa_debug_fp8_to_16bit(const uint8_t* codes, uint16_t* out, int n, int out_dtype, void* stream);

/* Measurement aid: reads bytes of device memory at buf once with the decode kernels'
 * load shape (16-byte loads, each wave instruction one contiguous 1 KiB run) and nothing
 * else, so that the time of this launch is the device's streaming-read rate for that shape
 * (the ceiling the decode kernels' K/V streams are compared with). unroll in {4, 8, 16} is
 * the loads each thread issues before using any; bytes must be a positive multiple of
 * 4096 * unroll and buf 16-byte aligned. num_workgroups 0 gives every workgroup one
 * iteration (bytes / (4096 * unroll) workgroups), else the workgroups stride over the
 * buffer. nontemporal 1 marks the loads non-temporal (as the split-context stream does),
 * 0 leaves them plain. sink: 256 uint32 of device memory, almost never written (only when
 * the folded words hit a fixed pattern). PA_ERR_INVALID on other arguments. Asynchronous on
 * `stream`. */
int pa_debug_stream_read(const void* buf, size_t bytes, int unroll, int num_workgroups, int nontemporal,
                         uint32_t* sink, void* stream);

/* ---------------------------------------------------------------------------------
 * Host block manager ([P1] §2 and §5; [P3] paged-pool and prefix-caching sections): owns
 * the physical block pool of one paged KV cache on the host and produces the block tables
 * and slots that the kernels above consume. Host memory only, no HIP calls; one manager
 * must not be used from several threads at once.
 *   - Free blocks form a stack (allocation and release are O(1)); a sequence holds only
 *     the blocks its tokens use and gets a new block when its last one is full.
 *   - Blocks are shared by reference count (forked sequences, prefix cache hits).
 *   - With prefix caching, every full block is indexed under (parent block, parent's
 *     generation, its token ids); a new sequence reuses the longest chain of indexed
 *     blocks that matches its prompt exactly. Indexed blocks whose count drops to zero
 *     stay reusable until the free stack runs out; then one is evicted by LRU-K ([P2]
 *     §2.3): a logical clock advances once per add, append or fork; a block is accessed
 *     when a sequence gains a reference to it or writes into it (once per operation); the
 *     victim is the block whose K-th most recent access is oldest (fewer than K accesses
 *     count as oldest), ties to the older last access, then to the block deeper in its
 *     prefix chain, then to the lower id.
 *   - Appending to a partly filled block that is shared copies it first: the manager
 *     allocates the new block and reports (copy_src, copy_dst); the caller copies the
 *     block's K/V on the device before writing the new token.
 * Status codes as above; PA_ERR_WORKSPACE means the pool has no block to give (the
 * manager is then unchanged). Sequence handles are small integers that are never reused.
 * --------------------------------------------------------------------------------- */
typedef struct pa_block_manager pa_block_manager;

/* New manager over num_blocks blocks of block_size tokens; lru_k in 1..4 is K of the
 * eviction policy (0 means 2, LRU-2). NULL on invalid arguments. */
pa_block_manager* pa_bm_create(int num_blocks, int block_size, int enable_prefix_caching, int lru_k);
void pa_bm_destroy(pa_block_manager* bm);
/* Blocks that can still be allocated (free plus evictable cached blocks). */
int pa_bm_num_free(const pa_block_manager* bm);
/* Adds a sequence holding the num_tokens prompt tokens; returns its handle (>= 0).
 * *num_cached_tokens (may be NULL) receives how many leading tokens were found in the
 * prefix cache (their K/V need not be computed again). */
int pa_bm_add_sequence(pa_block_manager* bm, const int32_t* token_ids, int num_tokens,
                       int* num_cached_tokens);
/* Appends one token; *slot = block * block_size + offset of its K/V. *copy_src and
 * *copy_dst are -1, or the blocks to copy before writing (copy on write). */
int pa_bm_append_token(pa_block_manager* bm, int seq, int32_t token_id, int32_t* slot,
                       int32_t* copy_src, int32_t* copy_dst);
/* A new sequence sharing every block of `parent` (beam search, parallel sampling). */
int pa_bm_fork(pa_block_manager* bm, int parent);
/* Releases a sequence's blocks. */
int pa_bm_free_sequence(pa_block_manager* bm, int seq);
int pa_bm_context_len(const pa_block_manager* bm, int seq);
/* Writes the sequence's table into out[0 .. max_blocks) padded with -1; returns the number
 * of blocks (PA_ERR_WORKSPACE if more than max_blocks). */
int pa_bm_block_table(const pa_block_manager* bm, int seq, int32_t* out, int max_blocks);
int pa_bm_ref_count(const pa_block_manager* bm, int block);
/* Block tables [n][max_blocks] (-1 padded) and context lengths of n sequences, in host
 * arrays ready to copy to the device. */
int pa_bm_export(const pa_block_manager* bm, const int32_t* seqs, int n, int max_blocks,
                 int32_t* block_tables, int32_t* context_lens);

/* Static text for a status code. */
const char* pa_status_str(int status);

/* Library version: major * 10000 + minor * 100 + patch. */
int pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
