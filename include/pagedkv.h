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
 *    allocates nothing, keeps no pointer after a call returns, holds no global
 *    mutable state and never synchronises: each call only enqueues kernels on
 *    `stream` (a hipStream_t; NULL means the default stream) and returns.
 *    Calls are thread-safe.
 *  - Host-side validation runs before anything is enqueued; a call that
 *    returns an error status has enqueued nothing.  PKV_ERR_HIP means a launch
 *    was rejected by the runtime.
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

#define PKV_VERSION 1

typedef enum {
  PKV_OK = 0,
  PKV_ERR_NULL = 1,        /* a required pointer is NULL                          */
  PKV_ERR_SHAPE = 2,       /* a size is out of range or sizes are inconsistent    */
  PKV_ERR_UNSUPPORTED = 3, /* head_dim, block_size, dtype, GQA ratio or partition */
  PKV_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than required             */
  PKV_ERR_HIP = 5          /* the HIP runtime rejected a launch                   */
} pkv_status;

typedef enum { PKV_F16 = 0, PKV_BF16 = 1 } pkv_dtype;

/* Shape of one K pool (the V pool has the same shape). */
typedef struct {
  int64_t num_blocks;   /* N >= 1                                   */
  int32_t block_size;   /* B: 8, 16, 32 or 64 tokens                */
  int32_t num_kv_heads; /* Hkv >= 1                                 */
  int32_t head_dim;     /* D: 64 or 128                             */
  int32_t dtype;        /* pkv_dtype                                */
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
 * Partition size and workspace.
 *
 * partition_size P (tokens) splits each sequence's context into chunks of P
 * tokens processed by separate workgroups.  P must be a multiple of B and of
 * the 16 (D = 128) or 32 (D = 64) tokens one wavefront step covers, with
 * P / B <= 512.  0 selects a size from (num_seqs, num_heads, max_blocks, B, D).
 * pkv_decode_partition_size() returns the size a call would use (0 if the
 * arguments are invalid).
 *
 * Workspace layout (float32), with MP = ceil(max_blocks_per_seq * B / P) and
 * U = num_seqs * num_heads * MP, unit u = (s * num_heads + h) * MP + p:
 *   [ m: U floats ][ l: U floats ][ o: U * D floats ], each section starting on
 *   a 256-byte boundary.  m is the partition's largest score z = scale * q.k
 *   (natural-log units), l = sum exp(z - m), o = sum exp(z - m) * v.
 */
int32_t pkv_decode_partition_size(int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                  const pkv_pool *p, int32_t partition_size);

size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                  const pkv_pool *p, int32_t partition_size);

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
 *   num_heads     query heads; must equal Hkv in this version
 *   workspace     >= pkv_decode_workspace_bytes(...) bytes, 256-byte aligned;
 *                 may be NULL only when that size is 0
 *
 * Runs the partition pass, then (only if some sequence may span several
 * partitions) the merge pass, both on `stream`.  Deterministic: the result
 * depends only on logical positions, not on where blocks sit in the pool or
 * whether they are shared.
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
 * pkv_decode_partitions -- the partition pass of pkv_paged_attention_decode on
 * its own.  Sequences with ceil(L / P) <= 1 get their final output row in
 * `out`; for every other sequence each partition p < ceil(L / P) writes its
 * partial (m, l, o) into the workspace (layout above) and `out` is untouched.
 * Same arguments and rules as pkv_paged_attention_decode.
 */
pkv_status pkv_decode_partitions(void *out, const void *q, const void *k_pool, const void *v_pool,
                                 const int32_t *block_tables, const int32_t *context_lens,
                                 float scale, int32_t num_seqs, int32_t num_heads,
                                 int32_t max_blocks_per_seq, const pkv_pool *p,
                                 int32_t partition_size, void *workspace, size_t workspace_bytes,
                                 void *stream);

/*
 * pkv_decode_merge -- the merge pass on its own.  For every sequence with
 * n = ceil(L / P) >= 2 partitions and 0 <= L <= max_blocks_per_seq * B:
 *   M = max_p m_p,  out[s][h] = sum_p exp(m_p - M) o_p / sum_p exp(m_p - M) l_p,
 * reading partials p < n from the workspace.  Other rows of `out` are not
 * touched.  Arguments as in pkv_paged_attention_decode.
 */
pkv_status pkv_decode_merge(void *out, const int32_t *context_lens, int32_t num_seqs,
                            int32_t num_heads, int32_t max_blocks_per_seq, const pkv_pool *p,
                            int32_t partition_size, const void *workspace, size_t workspace_bytes,
                            void *stream);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* PAGEDKV_H */
