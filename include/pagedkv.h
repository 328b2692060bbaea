/*
 * pagedkv.h -- C ABI of libpagedkv, paged decode attention and the paged KV
 * cache append for AMD Instinct MI355X (gfx950).
 *
 * The operations are the two fused kernels the PagedAttention pages describe:
 *
 *   - the cache append ("fused reshape and block write"): new tokens' K and V
 *     rows are written into their pool slots through the block table
 *     ("PagedAttention 完全拆解：操作系统分页思想如何拯救 LLM 推理的内存利用率",
 *     section 原理详解（三）：kernel 实现, item 1);
 *   - single-query decode attention that reads K and V block by block through
 *     the block table ("fused block read and attention", same section, item 2;
 *     the attention itself is the equation of section 背景 / 自回归生成与两阶段
 *     推理, computed in the blockwise form of section 原理详解（二）).
 *
 * Long contexts are split into partitions whose partial results are merged
 * by the log-sum-exp rule (the iaim.asia block-table article, section
 * "vLLM 内核里的缓解写法": segments processed in parallel, then reduced).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every data pointer is a DEVICE pointer unless stated otherwise; every
 *    struct pointer (pkv_pool) is a HOST pointer read during the call only.
 *  - The caller owns all memory, including the decode workspace.  The library
 *    allocates no device memory and keeps no pointer after a call returns.
 *    Its only state is a cache of each device's compute-unit count and of the
 *    decode kernels' occupancy, filled on first use under a lock.  It never
 *    synchronises: each call only enqueues kernels on `stream` (a
 *    hipStream_t; NULL means the default stream) of the current device and
 *    returns.  Calls are thread-safe.  Kernels are all a call enqueues (no
 *    memory sets, copies or allocations), so a call can be captured in a HIP
 *    graph and replayed; the one-time set-up above runs on the first call,
 *    which should be made before a capture.
 *  - Host-side validation runs before anything is enqueued; a call that
 *    returns an error status has enqueued nothing.  PKV_ERR_HIP means the
 *    runtime rejected a launch or a device query.
 *  - Element types: 16-bit IEEE binary16 (PKV_F16) or bfloat16 (PKV_BF16).
 *    Arithmetic is float32 with exact products; outputs are rounded to the
 *    element type, nearest-even.
 *
 * Pool layout (both pools identical)
 * ----------------------------------
 *  k_pool, v_pool: [num_blocks][num_kv_heads][block_size][head_dim], C order,
 *  so one (block, head) tile of block_size x head_dim elements is contiguous
 *  and a wavefront reading a tile touches adjacent bytes wherever the block
 *  sits in the pool.  pkv_pool_index() is the formula.
 *
 *  A token at logical position pos of sequence s lives in pool block
 *  block_tables[s][pos / block_size], at offset pos % block_size inside it
 *  (iaim.asia block-table article, section "KV Cache 如何按块分配", BLOCK_SIZE=16
 *  table; "PagedAttention 完全拆解", 原理详解（一）, Figure 6).  The flat "slot" of
 *  that token is block * block_size + offset.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_VERSION 2

typedef enum {
  PKV_OK = 0,
  PKV_ERR_NULL = 1,        /* a required pointer is NULL                          */
  PKV_ERR_SHAPE = 2,       /* a size is out of range or sizes are inconsistent    */
  PKV_ERR_UNSUPPORTED = 3, /* head_dim, block_size, dtype, GQA ratio or partition */
  PKV_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than required             */
  PKV_ERR_HIP = 5,         /* the HIP runtime rejected a launch                   */
  PKV_ERR_SCRATCH = 6      /* pkv_paged_attention_decode_noalloc: the call needs
                              more than the library's static scratch holds        */
} pkv_status;

typedef enum { PKV_F16 = 0, PKV_BF16 = 1 } pkv_dtype;

/*
 * Pool flags (pkv_pool.flags), a hint for the decode calls' K/V reads:
 *   0               every pool block is read once per call (the usual decode
 *                   batch): K/V rows are read with non-temporal loads, which
 *                   stream past the caches;
 *   PKV_POOL_REUSE  blocks are read by several sequences in one call (shared
 *                   prompt prefixes, parallel samples): ordinary cached
 *                   loads, so later readers can hit the last-level cache.
 * The flag changes speed only, never results.  Other bits: PKV_ERR_UNSUPPORTED.
 */
#define PKV_POOL_REUSE 1

/* Shape of one K pool (the V pool has the same shape). */
typedef struct {
  int64_t num_blocks;   /* N >= 1                                   */
  int32_t block_size;   /* B: 8, 16, 32 or 64 tokens                */
  int32_t num_kv_heads; /* Hkv >= 1                                 */
  int32_t head_dim;     /* D: 64 or 128                             */
  int32_t dtype;        /* pkv_dtype                                */
  int32_t flags;        /* 0 or PKV_POOL_REUSE                      */
} pkv_pool;

/* Library ABI version (PKV_VERSION). */
int pkv_version(void);

/* Static English text for a status code; never NULL. */
const char *pkv_status_string(int status);

/* Bytes of ONE pool (K or V): N * Hkv * B * D * 2.  0 if the shape is invalid. */
size_t pkv_pool_bytes(const pkv_pool *p);

/* Element index of (block, head, offset, dim) in a pool; -1 if out of range. */
int64_t pkv_pool_index(const pkv_pool *p, int64_t block, int32_t head, int32_t offset, int32_t dim);

/*
 * pkv_slot_mapping -- translate (sequence, position) pairs into pool slots.
 *
 * For token t: s = token_seq[t], pos = token_pos[t];
 *   slot_mapping[t] = block_tables[s][pos / B] * B + pos % B.
 * The translation rule is the one stated above (Figure 6 walk-through and the
 * BLOCK_SIZE=16 table).  A token gets -1 (padding, skipped by the append) when
 * s or pos is negative, s >= num_seqs, pos >= max_blocks_per_seq * B, or the
 * table entry is outside [0, N).
 *
 *   slot_mapping  int64 [num_tokens]                       (written)
 *   block_tables  int32 [num_seqs][max_blocks_per_seq], row-major
 *   token_seq     int32 [num_tokens]
 *   token_pos     int32 [num_tokens]
 * num_tokens == 0 is a no-op.
 */
pkv_status pkv_slot_mapping(int64_t *slot_mapping, const int32_t *block_tables, int32_t num_seqs,
                            int32_t max_blocks_per_seq, const int32_t *token_seq,
                            const int32_t *token_pos, int32_t num_tokens, const pkv_pool *p,
                            void *stream);

/*
 * pkv_reshape_and_cache -- append new tokens' K and V rows to the pools.
 *
 * For every token t with 0 <= slot_mapping[t] < N * B and every head h:
 *   k_pool[slot / B][h][slot % B][:] = k[t][h][:],  v_pool likewise.
 * ("PagedAttention 完全拆解", 原理详解（三）, item 1: rearrange into the block
 * layout and write through the table in one kernel.)  The copy is bit-exact.
 * Tokens with a negative or out-of-range slot are skipped.  Slots must be
 * unique within one call (duplicates race; the winner is unspecified).
 *
 *   k, v            [num_tokens][Hkv][D] with heads and dims contiguous; the
 *                   distance between consecutive tokens is k_token_stride /
 *                   v_token_stride ELEMENTS (0 means Hkv * D), so k and v may
 *                   be views into a fused QKV projection output.  Rows must be
 *                   16-byte aligned.
 *   slot_mapping    int64 [num_tokens]
 * num_tokens == 0 is a no-op.
 */
pkv_status pkv_reshape_and_cache(void *k_pool, void *v_pool, const void *k, const void *v,
                                 int64_t k_token_stride, int64_t v_token_stride,
                                 const int64_t *slot_mapping, int32_t num_tokens,
                                 const pkv_pool *p, void *stream);

/*
 * pkv_copy_blocks -- copy whole pool blocks (every head, every slot) of both
 * pools in one launch: for each pair i, with (src, dst) = block_pairs[i],
 *   k_pool[dst][:][:][:] = k_pool[src][:][:][:],  v_pool likewise.
 * This is the copy of copy-on-write: a sequence about to append into a
 * partly filled block it shares with other sequences first gets a private
 * copy ("PagedAttention 完全拆解", 内存共享 / Figure 8 and the fork / append
 * primitives).  The copy is bit-exact.
 *
 *   block_pairs  int64 [num_pairs][2] (src, dst), device memory, 8-byte aligned
 * Pairs with src or dst outside [0, N) are skipped.  The copies run
 * concurrently: a dst must appear once, and no dst may be the src of another
 * pair in the same call.  num_pairs == 0 is a no-op.  PKV_ERR_SHAPE when
 * num_pairs * ceil(Hkv * B * D / 8192) exceeds 2^31 - 1 (the launch's
 * workgroups: 16 KiB of each pool per workgroup).
 */
pkv_status pkv_copy_blocks(void *k_pool, void *v_pool, const int64_t *block_pairs, int32_t num_pairs,
                           const pkv_pool *p, void *stream);

/*
 * How the context is split, and the workspace.
 *
 * partition_size selects how each sequence's context is cut into pieces that
 * run in parallel before the log-sum-exp merge:
 *
 *  - partition_size > 0: fixed partitions of P tokens, partition p holding
 *    tokens [p*P, min((p+1)*P, L)).  P must be a multiple of B and of the 16
 *    (D = 128) or 32 (D = 64) tokens one wavefront step covers, with P / B <= 512.
 *  - partition_size == 0: a work-balanced split.  All the batch's chunks of
 *    16 (D = 128) or 32 (D = 64) tokens of one (sequence, head) are cut into
 *    equal slices, one per wavefront, with as many wavefronts as the device
 *    holds at once, so batches with very different context lengths keep
 *    every compute unit busy.  The cut points depend on the context lengths
 *    and on the device (compute units and occupancy), so results are
 *    identical run to run on one device and build.  Batches of more than
 *    4096 sequences fall back to fixed partitions (partition_size 0 then
 *    means: one partition when max_blocks_per_seq * B <= 512, else 512).
 *
 * pkv_decode_partition_size() returns the P a call uses: P > 0 for fixed
 * partitions, 0 for the balanced split, -1 if the arguments are invalid.
 * pkv_decode_workspace_bytes() returns the workspace a call needs (0 when none
 * is needed or the arguments are invalid; the balanced split always needs
 * one).
 *
 * Workspace layout of fixed partitions (float32), with
 * MP = ceil(max_blocks_per_seq * B / P) and U = num_seqs * num_heads * MP,
 * unit u = (s * num_heads + h) * MP + p:
 *   [ m: U floats ][ l: U floats ][ o: U * D floats ], each section starting on
 *   a 256-byte boundary.  m is the partition's largest score z = scale * q.k
 *   (natural-log units), l = sum exp(z - m), o = sum exp(z - m) * v.
 * The balanced split's workspace holds a chunk prefix over sequences and
 * per-piece partial results in the same (m, l, o) form; its layout is
 * internal.  One call at a
 * time may use a workspace.
 */
int32_t pkv_decode_partition_size(int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                  const pkv_pool *p, int32_t partition_size);

size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                  const pkv_pool *p, int32_t partition_size);

/*
 * pkv_decode_launch_info -- what the split pass of a decode call with these
 * arguments launches, read from the library's own code objects (no kernel
 * runs, nothing is allocated).  num_queries, fp8 and append select the path
 * as the corresponding entry points do: num_queries > 1 or grouped heads the
 * matrix-core kernel, fp8 != 0 the e4m3 kernels, append != 0 the kernels
 * of the decode step with the fused append (16-bit, and e4m3 with one row
 * per KV head).  On the current device it fills:
 *   workgroups, waves_per_workgroup  the split pass's grid;
 *   waves_per_simd      wavefronts of that kernel that fit on a SIMD
 *                       (hipOccupancyMaxActiveBlocksPerMultiprocessor); the
 *                       balanced split sizes its grid for the smallest value
 *                       among the kernels a call may use (with or without
 *                       the fused append, streamed or cached loads), so the
 *                       grid can hold fewer;
 *   compute_units       of the device;
 *   registers           per lane (hipFuncGetAttributes numRegs);
 *   lds_static_bytes, lds_dynamic_bytes  per workgroup;
 *   scratch_bytes       per lane (register spills; 0 for every kernel here);
 *   balanced, partition_size  the split the call uses.
 * Returns PKV_ERR_NULL for a NULL info, the argument errors of the decode
 * calls, PKV_ERR_HIP if the device cannot be queried.  Used for the
 * occupancy and resource figures of the benchmark.
 */
typedef struct {
  int32_t workgroups, waves_per_workgroup, waves_per_simd, compute_units;
  int32_t registers, lds_static_bytes, lds_dynamic_bytes, scratch_bytes;
  int32_t balanced, partition_size;
} pkv_launch_info;

pkv_status pkv_decode_launch_info(int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                  const pkv_pool *p, int32_t partition_size, int32_t num_queries,
                                  int32_t fp8, int32_t append, pkv_launch_info *info);

/*
 * pkv_paged_attention_decode -- one query token per sequence over paged K/V.
 *
 * For every sequence s and head h, with L = context_lens[s]:
 *   z_j = scale * q[s][h] . k_j          for logical tokens j = 0 .. L-1,
 *   o[s][h] = sum_j exp(z_j - m) v_j / sum_j exp(z_j - m),  m = max_j z_j,
 * where k_j, v_j are read through block_tables ("PagedAttention 完全拆解",
 * 背景 attention equation and 原理详解（二） blockwise form; the max is
 * subtracted for numerical stability).  context_lens counts the token appended
 * this step, so append first (pkv_reshape_and_cache), then decode.
 *
 *   out           [num_seqs][num_heads][D]        element type of the pool (written)
 *   q             [num_seqs][num_heads][D]
 *   block_tables  int32 [num_seqs][max_blocks_per_seq]; only the first
 *                 ceil(L / B) entries of a row are read
 *   context_lens  int32 [num_seqs]
 *   scale         float32, normally 1 / sqrt(D)
 *   num_heads     query heads, a multiple of Hkv; query head h reads KV head
 *                 h / (num_heads / Hkv) (grouped-query attention, the
 *                 Llama-2-70B shape of the iaim.asia block-table article,
 *                 "末尾块的内部碎片").  With more than one query head per KV
 *                 head the matrix-core kernel runs: head_dim 64 or 128,
 *                 partition_size 0, at most 16 query heads per KV head and
 *                 num_seqs <= 4096, else PKV_ERR_UNSUPPORTED.  The
 *                 fused-append entry points then run the append as its own
 *                 launch (slots from the table) before the split pass.
 *   out           must be 16-byte aligned
 *   workspace     >= pkv_decode_workspace_bytes(...) bytes, 256-byte aligned;
 *                 may be NULL only when that size is 0
 *
 * Runs the split pass, then (when some row may be split) the merge pass, both
 * on `stream`.  Deterministic: on a given device the result depends only on
 * logical positions, not on where blocks sit in the pool or whether they are
 * shared.
 *
 * Device-side data rules: L == 0 gives a zero row; L < 0 or
 * L > max_blocks_per_seq * B gives a NaN row; a needed table entry outside
 * [0, N) gives a NaN row for that sequence; the pools are never read outside
 * [0, N).  Unused slots of a last block may hold anything (NaN included) and
 * never reach the output.
 */
pkv_status pkv_paged_attention_decode(void *out, const void *q, const void *k_pool,
                                      const void *v_pool, const int32_t *block_tables,
                                      const int32_t *context_lens, float scale, int32_t num_seqs,
                                      int32_t num_heads, int32_t max_blocks_per_seq,
                                      const pkv_pool *p, int32_t partition_size, void *workspace,
                                      size_t workspace_bytes, void *stream);

/*
 * pkv_paged_attention_decode_shared -- decode for batches whose sequences
 * come in groups that share a prompt prefix (parallel samples of one prompt,
 * the beams of one request, a common system prompt: "PagedAttention 完全拆解",
 * 内存共享：并行采样、Beam Search 与共享前缀 and 共享前缀与系统提示词, where the
 * prefix blocks are referenced by every sequence of the group).
 *
 * Computes exactly what pkv_paged_attention_decode computes (every
 * sequence's attention over all its L tokens), but reads each group's prefix
 * once for all its sequences instead of once per sequence.  The sum over a
 * context splits into a prefix part and a suffix part merged by the
 * log-sum-exp rule (the blockwise form of 原理详解（二）; the segment
 * reduction of the iaim.asia block-table article, "vLLM 内核里的缓解写法"):
 *   1. prefix pass (matrix-core kernel): per group and head, the prefix K/V
 *      rows are streamed once and scored against the group_size query rows of
 *      its sequences (a real contraction: group_size rows per K/V row); each
 *      row's softmax state (max, sum, unnormalised V sum) goes to the
 *      workspace;
 *   2. suffix pass: each sequence's tokens prefix_len .. L - 1, starting from
 *      its prefix state, then the merge of rows the split cut.
 * Four launches on `stream`.
 *
 *   group_size    sequences per group (2 .. 16): sequences g * group_size ..
 *                 (g + 1) * group_size - 1 form group g; num_seqs must be a
 *                 multiple of it (else PKV_ERR_SHAPE)
 *   prefix_lens   int32 [num_seqs / group_size], device: the leading tokens
 *                 every sequence of group g shares.  Tokens 0 .. prefix_lens[g] - 1
 *                 must hold the same K and V in every sequence of the group
 *                 (shared blocks, or copies with the same contents); the
 *                 prefix pass reads them through the group's first sequence's
 *                 table row.  0 means no shared prefix.
 *   workspace     >= pkv_shared_prefix_workspace_bytes(...) bytes, 256-byte
 *                 aligned; needs no initialisation.
 * Other arguments, layouts and device-side rules as in
 * pkv_paged_attention_decode; a sequence shorter than its group's prefix
 * gets a NaN row.  Restrictions (else PKV_ERR_UNSUPPORTED): 16-bit pools,
 * num_heads == num_kv_heads, num_seqs <= 4096.  The result depends only on
 * the prefix contents: shared blocks and per-sequence copies give the same
 * bits.  Differs from pkv_paged_attention_decode only by rounding.
 */
size_t pkv_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                         const pkv_pool *p, int32_t group_size);
pkv_status pkv_paged_attention_decode_shared(void *out, const void *q, const void *k_pool, const void *v_pool,
                                             const int32_t *block_tables, const int32_t *context_lens, float scale,
                                             int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                             const pkv_pool *p, int32_t group_size, const int32_t *prefix_lens,
                                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * pkv_paged_attention_decode_noalloc -- pkv_paged_attention_decode with no
 * workspace argument and no allocation, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc.  The caller still owns q, the pools, the tables,
 * context_lens and out.
 *
 * It computes exactly what pkv_paged_attention_decode computes with
 * partition_size 0 (the balanced split), with the same kernels and the same
 * split, so its output is bit for bit that call's on the same device.  The
 * partial results and the chunk prefix go to a static device array of
 * 16 MiB (256-byte aligned) inside the library instead of a workspace.  Each
 * GPU the library runs on holds its own copy of that array until the process
 * ends; its device address is taken on the first call on each device (with
 * that device current).  The array needs no clearing: every call writes what
 * it later reads.
 *
 * Need: (S + 1) * 8 bytes of chunk prefix, then (m, l, o) of float32, i.e.
 * (D + 2) * 4 bytes, for each of (min(G, workers) + S * Hkv) * (H / Hkv)
 * partial rows, each section rounded up to 256 bytes (G = worker wavefronts
 * launched: compute units x resident workgroups x 4).  A call that needs more
 * than 16 MiB returns PKV_ERR_SCRATCH and enqueues nothing.  On MI355X
 * (G = 3072 at one query row per KV head) that admits, at D = 128, about
 * 29,000 (sequence, head) rows: the 64 x 40 and 256 x 40 batches fit.
 *
 * Calls on one GPU share that GPU's array: two calls whose kernels may
 * overlap on the same device (different streams, or different host threads
 * without ordering) race and give wrong results.  Calls on one stream are
 * ordered and safe.  partition_size is always 0; more than 4096 sequences
 * (which need fixed partitions) return PKV_ERR_UNSUPPORTED.  Other
 * arguments, layouts, restrictions and device-side rules as in
 * pkv_paged_attention_decode.  Calls no hipMalloc, hipFree or other
 * allocating routine.
 */
pkv_status pkv_paged_attention_decode_noalloc(void *out, const void *q, const void *k_pool,
                                              const void *v_pool, const int32_t *block_tables,
                                              const int32_t *context_lens, float scale, int32_t num_seqs,
                                              int32_t num_heads, int32_t max_blocks_per_seq,
                                              const pkv_pool *p, void *stream);

/*
 * pkv_paged_attention_decode_append -- one decode step with the append fused
 * in: equivalent to appending row s of k_new / v_new as token L_s - 1 of
 * every sequence with 1 <= L_s <= max_blocks_per_seq * B (pkv_slot_mapping
 * with pos = L_s - 1, then pkv_reshape_and_cache), followed by
 * pkv_paged_attention_decode -- in two launches instead of four (with more
 * than one query head per KV head: three, the append as its own launch with
 * slots from the table).  The pool slot of token L_s - 1 receives the new row
 * bit for bit, and attention uses the new row for that token ("PagedAttention
 * 完全拆解", 原理详解（一）, Figure 6 walk-through: the new token's K/V goes into
 * its block, then attention runs over the blocks).  With the balanced split
 * and one query head per KV head the split pass takes the new row from
 * k_new / v_new and the merge launch writes it to the pool.
 *
 *   k_new, v_new  [num_seqs][Hkv][D], consecutive sequences new_token_stride
 *                 ELEMENTS apart (0 means Hkv * D); rows 16-byte aligned
 *   k_pool, v_pool  written (one row per sequence and head), otherwise read
 * Other arguments and rules as in pkv_paged_attention_decode.  Rows whose
 * table entry for token L_s - 1 lies outside [0, N) are not written and their
 * output row is NaN.
 */
pkv_status pkv_paged_attention_decode_append(void *out, const void *q, const void *k_new,
                                             const void *v_new, int64_t new_token_stride,
                                             void *k_pool, void *v_pool,
                                             const int32_t *block_tables,
                                             const int32_t *context_lens, float scale,
                                             int32_t num_seqs, int32_t num_heads,
                                             int32_t max_blocks_per_seq, const pkv_pool *p,
                                             int32_t partition_size, void *workspace,
                                             size_t workspace_bytes, void *stream);

/*
 * pkv_decode_partitions_append -- the split pass of
 * pkv_paged_attention_decode_append on its own (the pool writes of the append
 * happen here); pkv_decode_merge completes it.  Arguments as in
 * pkv_paged_attention_decode_append.
 */
pkv_status pkv_decode_partitions_append(void *out, const void *q, const void *k_new,
                                        const void *v_new, int64_t new_token_stride, void *k_pool,
                                        void *v_pool, const int32_t *block_tables,
                                        const int32_t *context_lens, float scale, int32_t num_seqs,
                                        int32_t num_heads, int32_t max_blocks_per_seq,
                                        const pkv_pool *p, int32_t partition_size, void *workspace,
                                        size_t workspace_bytes, void *stream);

/*
 * pkv_decode_partitions -- the split pass of pkv_paged_attention_decode on its
 * own.  With fixed partitions (P > 0): sequences with ceil(L / P) <= 1 get
 * their final output row in `out`, rows of empty (L == 0) or invalid contexts
 * are written as described above, and for every other sequence each partition
 * p < ceil(L / P) writes its partial (m, l, o) into the workspace (layout
 * above) while its `out` row is untouched.  With the balanced split (P == 0):
 * every (sequence, head) handled in one piece gets its output row, the others
 * leave partials; the merge pass completes the output.  Same arguments and
 * rules as pkv_paged_attention_decode.
 */
pkv_status pkv_decode_partitions(void *out, const void *q, const void *k_pool, const void *v_pool,
                                 const int32_t *block_tables, const int32_t *context_lens,
                                 float scale, int32_t num_seqs, int32_t num_heads,
                                 int32_t max_blocks_per_seq, const pkv_pool *p,
                                 int32_t partition_size, void *workspace, size_t workspace_bytes,
                                 void *stream);

/*
 * pkv_decode_merge -- the merge pass on its own.  With fixed partitions, for
 * every sequence with n = ceil(L / P) >= 2 partitions and
 * 0 <= L <= max_blocks_per_seq * B:
 *   M = max_p m_p,  out[s][h] = sum_p exp(m_p - M) o_p / sum_p exp(m_p - M) l_p,
 * reading partials p < n from the workspace; other rows of `out` are not
 * touched.  With the balanced split it merges the (sequence, head) rows that
 * were cut into several pieces and writes the rows of empty or invalid
 * contexts.  Arguments as in pkv_paged_attention_decode.
 */
pkv_status pkv_decode_merge(void *out, const int32_t *context_lens, int32_t num_seqs,
                            int32_t num_heads, int32_t max_blocks_per_seq, const pkv_pool *p,
                            int32_t partition_size, const void *workspace, size_t workspace_bytes,
                            void *stream);

/*
 * pkv_paged_attention_multi -- several query tokens per sequence over paged
 * K/V, causal: query i (0 <= i < num_queries) of sequence s sits at position
 * L - num_queries + i (the last num_queries tokens of the context, already
 * appended) and attends over tokens 0 .. L - num_queries + i, with the same
 * attention equation and rules as pkv_paged_attention_decode (the per-token
 * equation of "PagedAttention 完全拆解", 背景, for each query row; a query
 * attends to itself).  This serves chunked prefill and the verification of
 * several candidate tokens in one step.
 *
 *   out, q        [num_seqs][num_queries][num_heads][head_dim], element type of
 *                 the pool; out 16-byte aligned
 *   num_heads     a multiple of Hkv (as above); (num_heads / Hkv) *
 *                 num_queries <= 16 query rows per KV head, head_dim 64 or
 *                 128 (e4m3 pools: 128), num_seqs <= 4096, else
 *                 PKV_ERR_UNSUPPORTED
 *   workspace     >= pkv_multi_workspace_bytes(...) bytes, 256-byte aligned
 * Rows of a sequence with 0 < L < num_queries (or an invalid L) are NaN (the
 * queries must be part of the context); L == 0 gives zero rows.  Runs a split
 * pass and a merge pass (balanced split) on `stream`.
 * pkv_multi_workspace_bytes returns 0 for invalid or unsupported arguments.
 */
size_t pkv_multi_workspace_bytes(int32_t num_seqs, int32_t num_queries, int32_t num_heads,
                                 int32_t max_blocks_per_seq, const pkv_pool *p);
pkv_status pkv_paged_attention_multi(void *out, const void *q, const void *k_pool, const void *v_pool,
                                     const int32_t *block_tables, const int32_t *context_lens, float scale,
                                     int32_t num_seqs, int32_t num_queries, int32_t num_heads,
                                     int32_t max_blocks_per_seq, const pkv_pool *p, void *workspace,
                                     size_t workspace_bytes, void *stream);

/*
 * FP8 KV cache
 * ------------
 * "PagedAttention 完全拆解", 总结 item 6, names an FP8-quantised KV cache as a
 * later layer on top of the paged cache; the pages fix no format.  The one
 * served here: pools of OCP e4m3 codes (1 sign bit, 4 exponent bits with bias
 * 7, 3 mantissa bits; largest finite magnitude 448; no infinities; 0x7F and
 * 0xFF are NaN) in the pool layout above, ONE BYTE per element.  Each pool
 * has one float32 scale: code c stands for e4m3(c) * scale.  The pkv_pool
 * descriptor is unchanged; its dtype names the 16-bit type of q, out and the
 * new K / V rows.  Half the bytes of a 16-bit cache per token.
 */

/* Bytes of ONE fp8 pool: N * Hkv * B * D.  0 if the shape is invalid. */
size_t pkv_fp8_pool_bytes(const pkv_pool *p);

/*
 * pkv_reshape_and_cache_fp8 -- pkv_reshape_and_cache into e4m3 pools, with
 * the same slot rules, strides and alignment.  Each element is quantised:
 *   code = e4m3(x * r),  r = 1 / scale rounded to float32 (on the host),
 * the product rounded to float32, then to the nearest e4m3 value, ties to
 * the even code; magnitudes past 448 (infinities too) saturate to +-448, NaN
 * stays NaN, the sign of a zero is kept.
 *   k_scale, v_scale  positive, finite, with a finite reciprocal, else
 *                     PKV_ERR_SHAPE
 */
pkv_status pkv_reshape_and_cache_fp8(void *k_pool, void *v_pool, const void *k, const void *v,
                                     int64_t k_token_stride, int64_t v_token_stride,
                                     const int64_t *slot_mapping, int32_t num_tokens, float k_scale,
                                     float v_scale, const pkv_pool *p, void *stream);

/*
 * pkv_paged_attention_decode_fp8 -- pkv_paged_attention_decode over e4m3
 * pools: every K element is e4m3(code) * k_scale and every V element
 * e4m3(code) * v_scale; the attention equation, the rules for empty, invalid
 * and out-of-pool contexts and the output rounding are those of
 * pkv_paged_attention_decode (balanced split, then the merge pass).
 *   out, q        [num_seqs][num_heads][head_dim] 16-bit (p->dtype)
 *   num_heads     a multiple of Hkv, at most 16 query heads per KV head
 *                 (grouped-query heads run on the matrix-core kernel, with
 *                 the codes widened to the 16-bit type in registers, and
 *                 need head_dim 128); one query head per KV head: head_dim
 *                 64 or 128; num_seqs <= 4096; else PKV_ERR_UNSUPPORTED
 *   k_scale, v_scale  as for pkv_reshape_and_cache_fp8
 *   workspace     >= pkv_fp8_decode_workspace_bytes(...) bytes, 256-byte aligned
 * pkv_fp8_decode_workspace_bytes returns 0 for invalid or unsupported
 * arguments.
 */
size_t pkv_fp8_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                      const pkv_pool *p);
pkv_status pkv_paged_attention_decode_fp8(void *out, const void *q, const void *k_pool, const void *v_pool,
                                          const int32_t *block_tables, const int32_t *context_lens, float scale,
                                          float k_scale, float v_scale, int32_t num_seqs, int32_t num_heads,
                                          int32_t max_blocks_per_seq, const pkv_pool *p, void *workspace,
                                          size_t workspace_bytes, void *stream);

/*
 * pkv_paged_attention_decode_append_fp8 -- one decode step over e4m3 pools
 * with the append fused in: for every sequence s with a valid context
 * (0 < L <= max_blocks_per_seq * B), row s of k_new / v_new ([S][Hkv][D],
 * 16-bit, token stride new_token_stride elements, 0 = Hkv * D, a multiple of
 * 8; 16-byte aligned) is quantised exactly as pkv_reshape_and_cache_fp8 does
 * and written to the slot of token L - 1; the attention of
 * pkv_paged_attention_decode_fp8 runs over the context with that token's
 * codes (append first, then attend: "PagedAttention 完全拆解", 原理详解（一）,
 * Figure 6 walk-through).  A needed table entry outside the pool writes
 * nothing and gives a NaN row.  Same restrictions, scales and workspace as
 * pkv_paged_attention_decode_fp8.  One row per KV head: two launches, the
 * split pass (which quantises each new token itself and uses those codes in
 * place of the pool's) and the merge pass (which also writes the codes to
 * the pool).  Grouped heads: three, a separate append (slots from the table,
 * no slot list) before the two passes.  The output and the pool bytes are
 * the same either way, and bit for bit those of pkv_reshape_and_cache_fp8
 * followed by pkv_paged_attention_decode_fp8.
 */
pkv_status pkv_paged_attention_decode_append_fp8(void *out, const void *q, const void *k_new, const void *v_new,
                                                 int64_t new_token_stride, void *k_pool, void *v_pool,
                                                 const int32_t *block_tables, const int32_t *context_lens,
                                                 float scale, float k_scale, float v_scale, int32_t num_seqs,
                                                 int32_t num_heads, int32_t max_blocks_per_seq, const pkv_pool *p,
                                                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * pkv_paged_attention_multi_fp8 -- pkv_paged_attention_multi over e4m3 pools
 * (several query tokens per sequence, causal, grouped-query heads allowed),
 * with the scales of pkv_paged_attention_decode_fp8.  Same layouts, rules and
 * restrictions as pkv_paged_attention_multi; workspace >=
 * pkv_fp8_multi_workspace_bytes(...) bytes (0 for invalid or unsupported
 * arguments).
 */
size_t pkv_fp8_multi_workspace_bytes(int32_t num_seqs, int32_t num_queries, int32_t num_heads,
                                     int32_t max_blocks_per_seq, const pkv_pool *p);
pkv_status pkv_paged_attention_multi_fp8(void *out, const void *q, const void *k_pool, const void *v_pool,
                                         const int32_t *block_tables, const int32_t *context_lens, float scale,
                                         float k_scale, float v_scale, int32_t num_seqs, int32_t num_queries,
                                         int32_t num_heads, int32_t max_blocks_per_seq, const pkv_pool *p,
                                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * pkv_decode_partitions_fp8, pkv_decode_merge_fp8 -- the two passes of
 * pkv_paged_attention_multi_fp8 (and, with num_queries == 1, of
 * pkv_paged_attention_decode_fp8) as separate calls, as pkv_decode_partitions
 * and pkv_decode_merge are for 16-bit pools (attention over a context cut
 * into pieces, each piece's (m, l, o) combined by the log-sum-exp merge:
 * "PagedAttention 完全拆解", 原理详解（二）): the split pass leaves the output
 * rows of the (sequence, head) rows it handled in one piece and partial
 * results for the rest in the workspace; the merge pass completes them and
 * writes the rows of empty or invalid contexts.  The V scale is applied by
 * the split pass, so the merge takes no scales.  Both calls must get the same
 * shape arguments, pool and workspace; in between the workspace must not be
 * touched.  Arguments, rules and errors as in pkv_paged_attention_multi_fp8;
 * the output and the workspace are the caller's, the calls only enqueue
 * kernels on `stream`.  The two calls give the one call's output bit for bit.
 */
pkv_status pkv_decode_partitions_fp8(void *out, const void *q, const void *k_pool, const void *v_pool,
                                     const int32_t *block_tables, const int32_t *context_lens, float scale,
                                     float k_scale, float v_scale, int32_t num_seqs, int32_t num_queries,
                                     int32_t num_heads, int32_t max_blocks_per_seq, const pkv_pool *p,
                                     void *workspace, size_t workspace_bytes, void *stream);
pkv_status pkv_decode_merge_fp8(void *out, const int32_t *context_lens, int32_t num_seqs, int32_t num_queries,
                                int32_t num_heads, int32_t max_blocks_per_seq, const pkv_pool *p,
                                const void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* PAGEDKV_H */
