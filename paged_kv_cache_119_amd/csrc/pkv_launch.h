// Internal launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

// Wavefronts per workgroup of the decode kernels (build-time setting).
#ifndef PKV_DECODE_WAVES
#define PKV_DECODE_WAVES 4
#endif
// 16-byte loads per lane per tensor in one wavefront step (build-time setting).
#ifndef PKV_DECODE_LOADS
#define PKV_DECODE_LOADS 4
#endif

namespace pkv {

constexpr int kDecodeLoads = PKV_DECODE_LOADS;
// Largest number of table entries one fixed partition stages in LDS.
constexpr int kTabMax = 512;
// Balanced split: smallest slice a worker gets, in chunks (this also bounds
// the number of workers, hence of partial results, independently of the GPU).
constexpr int kMinWorkerChunks = 8;
// Balanced split: most sequences (the per-workgroup cost prefix lives in LDS).
constexpr int kBalancedMaxSeqs = 4096;
// Balanced split: most wavefronts launched.
constexpr int kMaxWorkers = 16384;
// Consecutive logical work items kept on one XCD (fixed partitions).
constexpr int kXcdGroup = 16;

struct DecodeParams {
  void *out;               // [S][H][D] 16-bit
  const void *q;           // [S][H][D] 16-bit
  const void *k_pool;      // [N][Hkv][B][D]
  const void *v_pool;
  const int32_t *tables;   // [S][maxb]
  const int32_t *lens;     // [S]
  float *ws_m;             // partial maxima
  float *ws_l;             // partial sums
  float *ws_o;             // partial weighted V sums, D per partial
  int64_t *ws_cum;         // balanced split: chunk prefix over sequences [S + 1]
  float scale_log2;        // scale * log2(e)
  int64_t num_blocks;      // N
  int32_t S, H, Hkv, maxb, B, D, P, MP;
  int32_t items;           // fixed partitions: S * H * MP
  int32_t G;               // balanced split: workers (wavefronts) launched, a multiple of the waves per workgroup
  int32_t balanced;        // 1: work-balanced split, 0: fixed partitions of P tokens
  int32_t dtype;
  // Fused append (append != 0): the row of token L - 1 of every (sequence,
  // head) is taken from k_new / v_new ([S][Hkv][D], token stride new_stride
  // elements) and also written to its pool slot.
  int32_t append;
  // Balanced 16-bit split with the append: the split pass only substitutes
  // the new rows, and extra workgroups of the merge launch write them.
  int32_t append_in_merge;
  const void *k_new;
  const void *v_new;
  int64_t new_stride;
  // Query rows per KV head: H / Hkv query heads times nq query tokens per
  // sequence (q and out are [S][nq][H][D]); group != 0 selects the
  // matrix-core kernel for more than one row.
  int32_t nq;
  int32_t group;
  // FP8 pools (fp8 != 0): k_pool / v_pool hold OCP e4m3 codes, one byte per
  // element; the K scale is folded into scale_log2 and every V sum is
  // multiplied by v_scale.
  int32_t fp8;
  float v_scale;
  // FP8 decode step with the append (fp8 and append != 0): 1 / k_scale and
  // 1 / v_scale, the factors the new rows are quantised with
  float k_inv, v_inv;
  // 1: K/V loads of the stream kernels are non-temporal (blocks read once
  // per call); 0: ordinary cached loads (blocks shared between sequences).
  int32_t stream_kv;
  // Shared prompt prefixes (groups of pfx_group consecutive sequences whose
  // first pfx_lens[group] tokens hold the same K/V).
  //  pfx_pass 1, the prefix pass (matrix-core kernel): the sequences of this
  //   launch are the groups (lens = pfx_lens, table row of group i = the row
  //   of its first sequence), the query rows of a group are its sequences,
  //   every row sees every prefix token, and each row's softmax state goes to
  //   pfx_m (log2 units) / pfx_l / pfx_o (unnormalised) instead of out;
  //  pfx_pass 2, the suffix pass (balanced kernel): sequence s attends over
  //   tokens pfx_lens[s / pfx_group] .. L - 1, starting from that state.
  int32_t pfx_pass;
  int32_t pfx_group;
  const int32_t *pfx_lens;
  float *pfx_m;   // [S * H]
  float *pfx_l;   // [S * H]
  float *pfx_o;   // [S * H][D]
};

int decode_waves();
// The suffix pass of the shared-prefix decode (16-bit pools): its kernel
// instance, dynamic LDS and launch (the merge is launch_decode_merge).
const void *suffix_kernel(int dtype, int head_dim, int block_size, int nt);
size_t suffix_lds_bytes(int num_seqs);
hipError_t launch_suffix(const DecodeParams &a, hipStream_t stream);
// Tokens one wavefront step covers (partition sizes are multiples of it).
int decode_chunk_tokens(int head_dim);
// Dynamic LDS of the balanced kernel for num_seqs sequences.
size_t balanced_lds_bytes(int num_seqs);
// The balanced kernel instance for (dtype, D, B, append, non-temporal K/V
// loads), for occupancy queries.
const void *balanced_kernel(int dtype, int head_dim, int block_size, int append, int nt);
// The fixed-partition kernel instance and the number of workgroups it is
// launched with for `items` (sequence, head, partition) items.
const void *partition_kernel(int dtype, int head_dim, int block_size, int nt);
int64_t partition_grid(int64_t items);

hipError_t launch_decode_partitions(const DecodeParams &a, hipStream_t stream);
// Several query rows per KV head (grouped-query heads, multi-token queries).
size_t group_lds_bytes(int num_seqs);
const void *group_kernel(int dtype, int head_dim, int block_size, int nt, int fp8);
hipError_t launch_group_decode(const DecodeParams &a, hipStream_t stream);
hipError_t launch_group_merge(const DecodeParams &a, hipStream_t stream);
hipError_t launch_decode_merge(const DecodeParams &a, hipStream_t stream);
// FP8 (e4m3) pools, head_dim 64 or 128, one query row per KV head.
int fp8_chunk_tokens(int head_dim);
size_t fp8_lds_bytes(int num_seqs);
const void *fp8_kernel(int dtype, int head_dim, int block_size, int nt, int append);
// The decode step's append into e4m3 pools: token L - 1 of every sequence
// from k_new / v_new (a.append fields), slots from the block table.
hipError_t launch_append_last_fp8(const DecodeParams &a, float k_inv, float v_inv, hipStream_t stream);
hipError_t launch_fp8_decode(const DecodeParams &a, hipStream_t stream);
hipError_t launch_reshape_and_cache_fp8(void *k_pool, void *v_pool, const void *k, const void *v,
                                        int64_t k_stride, int64_t v_stride, const int64_t *slots,
                                        int32_t T, int32_t Hkv, int32_t B, int32_t D, int64_t num_blocks,
                                        int dtype, float k_inv, float v_inv, hipStream_t stream);

hipError_t launch_reshape_and_cache(void *k_pool, void *v_pool, const void *k, const void *v,
                                    int64_t k_stride, int64_t v_stride, const int64_t *slots,
                                    int32_t T, int32_t Hkv, int32_t B, int32_t D,
                                    int64_t num_blocks, hipStream_t stream);

// The decode step's append of 16-bit rows, slots from the block table (the
// append fields of `a`).
hipError_t launch_append_last(const DecodeParams &a, hipStream_t stream);

// Block copy: each workgroup of kCopyThreads threads copies kCopyUnroll
// 16-byte pieces per thread of one block of each pool; the launch has
// copy_blocks_workgroups(...) workgroups (at most 2^31 - 1 are launched).
constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;
int64_t copy_blocks_workgroups(int64_t num_pairs, int32_t Hkv, int32_t B, int32_t D);
hipError_t launch_copy_blocks(void *k_pool, void *v_pool, const int64_t *pairs, int32_t n,
                              int32_t Hkv, int32_t B, int32_t D, int64_t num_blocks,
                              hipStream_t stream);

hipError_t launch_slot_mapping(int64_t *slots, const int32_t *tables, int32_t S, int32_t maxb,
                               const int32_t *seq, const int32_t *pos, int32_t T, int32_t B,
                               int64_t num_blocks, hipStream_t stream);

}  // namespace pkv
