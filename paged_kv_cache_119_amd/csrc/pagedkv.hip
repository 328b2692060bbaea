// C ABI of libpagedkv: argument validation, partition sizing, workspace
// layout and dispatch to the kernels.  Declarations and the contract of every
// entry point are in include/pagedkv.h.

#include "pagedkv.h"

#include <hip/hip_runtime.h>

#include "pkv_launch.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool pool_ok(const pkv_pool *p) {
  if (!p) return false;
  if (p->num_blocks < 1) return false;
  if (p->block_size != 8 && p->block_size != 16 && p->block_size != 32 && p->block_size != 64)
    return false;
  if (p->num_kv_heads < 1) return false;
  if (p->head_dim != 64 && p->head_dim != 128) return false;
  if (p->dtype != PKV_F16 && p->dtype != PKV_BF16) return false;
  // every element index must fit in int64 (and slot numbers N * B as well)
  const double elems = (double)p->num_blocks * p->num_kv_heads * p->block_size * p->head_dim;
  return elems < 9.0e18;
}

// Tokens one wavefront step of the partition kernel covers.
#ifndef PKV_DECODE_LOADS
#define PKV_DECODE_LOADS 4
#endif
int chunk_tokens(int head_dim) { return PKV_DECODE_LOADS * (64 / (head_dim / 8)); }

int partition_unit(const pkv_pool *p) {
  const int tc = chunk_tokens(p->head_dim);
  return p->block_size > tc ? p->block_size : tc;
}

// Resolve the partition size; returns 0 if invalid.
int32_t resolve_partition(int32_t max_blocks, const pkv_pool *p, int32_t requested) {
  const int unit = partition_unit(p);
  const int64_t ctx = (int64_t)max_blocks * p->block_size;
  int64_t P = requested;
  if (P == 0) {
    P = ctx <= 512 ? (ctx + unit - 1) / unit * unit : 512;
  }
  if (P <= 0 || P % unit != 0 || P / p->block_size > pkv::kTabMax) return 0;
  return (int32_t)P;
}

bool aligned(const void *ptr, size_t a) { return ((uintptr_t)ptr & (a - 1)) == 0; }

struct Layout {
  int32_t P, MP;
  int64_t units;
  size_t off_l, off_o, bytes;
};

pkv_status decode_layout(int32_t num_seqs, int32_t num_heads, int32_t max_blocks,
                         const pkv_pool *p, int32_t partition_size, Layout *lay) {
  if (!pool_ok(p)) return p ? PKV_ERR_UNSUPPORTED : PKV_ERR_NULL;
  if (num_seqs < 0 || num_heads < 1 || max_blocks < 1) return PKV_ERR_SHAPE;
  if ((int64_t)max_blocks * p->block_size > (1 << 30)) return PKV_ERR_SHAPE;
  if (num_heads != p->num_kv_heads) return PKV_ERR_UNSUPPORTED;
  const int32_t P = resolve_partition(max_blocks, p, partition_size);
  if (P == 0) return PKV_ERR_UNSUPPORTED;
  const int64_t ctx = (int64_t)max_blocks * p->block_size;
  const int32_t MP = (int32_t)((ctx + P - 1) / P);
  const int64_t units = (int64_t)num_seqs * num_heads * MP;
  if (units > (int64_t)0x7FFFFF00) return PKV_ERR_SHAPE;  // 1-D grid limit
  lay->P = P;
  lay->MP = MP;
  lay->units = units;
  if (MP < 2 || units == 0) {
    lay->off_l = lay->off_o = lay->bytes = 0;
  } else {
    const size_t sec = align_up((size_t)units * sizeof(float), kAlign);
    lay->off_l = sec;
    lay->off_o = 2 * sec;
    lay->bytes = 2 * sec + align_up((size_t)units * p->head_dim * sizeof(float), kAlign);
  }
  return PKV_OK;
}

pkv_status fill_params(void *out, const void *q, const void *k_pool, const void *v_pool,
                       const int32_t *block_tables, const int32_t *context_lens, float scale,
                       int32_t num_seqs, int32_t num_heads, int32_t max_blocks, const pkv_pool *p,
                       int32_t partition_size, const void *workspace, size_t workspace_bytes,
                       bool need_inputs, pkv::DecodeParams *a) {
  Layout lay;
  const pkv_status st = decode_layout(num_seqs, num_heads, max_blocks, p, partition_size, &lay);
  if (st != PKV_OK) return st;
  if (num_seqs > 0) {
    if (!out || !context_lens) return PKV_ERR_NULL;
    if (need_inputs && (!q || !k_pool || !v_pool || !block_tables)) return PKV_ERR_NULL;
    if (need_inputs && (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16)))
      return PKV_ERR_SHAPE;
    if (!aligned(out, 2)) return PKV_ERR_SHAPE;
  }
  if (lay.bytes > 0) {
    if (!workspace || workspace_bytes < lay.bytes || !aligned(workspace, kAlign))
      return PKV_ERR_WORKSPACE;
  }
  char *ws = (char *)workspace;
  a->out = out;
  a->q = q;
  a->k_pool = k_pool;
  a->v_pool = v_pool;
  a->tables = block_tables;
  a->lens = context_lens;
  a->ws_m = lay.bytes ? (float *)ws : nullptr;
  a->ws_l = lay.bytes ? (float *)(ws + lay.off_l) : nullptr;
  a->ws_o = lay.bytes ? (float *)(ws + lay.off_o) : nullptr;
  a->scale_log2 = scale * 1.4426950408889634f;
  a->num_blocks = p->num_blocks;
  a->S = num_seqs;
  a->H = num_heads;
  a->Hkv = p->num_kv_heads;
  a->maxb = max_blocks;
  a->B = p->block_size;
  a->D = p->head_dim;
  a->P = lay.P;
  a->MP = lay.MP;
  a->items = (int32_t)lay.units;
  a->dtype = p->dtype;
  return PKV_OK;
}

pkv_status hip_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_HIP; }

}  // namespace

extern "C" {

int pkv_version(void) { return PKV_VERSION; }

const char *pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "a required pointer is NULL";
    case PKV_ERR_SHAPE: return "a size is out of range, sizes are inconsistent or a pointer is misaligned";
    case PKV_ERR_UNSUPPORTED: return "unsupported head_dim, block_size, dtype, head ratio or partition size";
    case PKV_ERR_WORKSPACE: return "workspace is NULL, too small or not 256-byte aligned";
    case PKV_ERR_HIP: return "the HIP runtime rejected a kernel launch";
    default: return "unknown status";
  }
}

size_t pkv_pool_bytes(const pkv_pool *p) {
  if (!pool_ok(p)) return 0;
  return (size_t)p->num_blocks * p->num_kv_heads * p->block_size * p->head_dim * 2;
}

int64_t pkv_pool_index(const pkv_pool *p, int64_t block, int32_t head, int32_t offset,
                       int32_t dim) {
  if (!pool_ok(p)) return -1;
  if (block < 0 || block >= p->num_blocks || head < 0 || head >= p->num_kv_heads || offset < 0 ||
      offset >= p->block_size || dim < 0 || dim >= p->head_dim)
    return -1;
  return ((block * p->num_kv_heads + head) * p->block_size + offset) * p->head_dim + dim;
}

pkv_status pkv_slot_mapping(int64_t *slot_mapping, const int32_t *block_tables, int32_t num_seqs,
                            int32_t max_blocks_per_seq, const int32_t *token_seq,
                            const int32_t *token_pos, int32_t num_tokens, const pkv_pool *p,
                            void *stream) {
  if (!p) return PKV_ERR_NULL;
  if (!pool_ok(p)) return PKV_ERR_UNSUPPORTED;
  if (num_tokens < 0 || num_seqs < 0 || max_blocks_per_seq < 1) return PKV_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * p->block_size > (1 << 30)) return PKV_ERR_SHAPE;
  if (num_tokens == 0) return PKV_OK;
  if (!slot_mapping || !token_seq || !token_pos || (num_seqs > 0 && !block_tables))
    return PKV_ERR_NULL;
  return hip_status(pkv::launch_slot_mapping(slot_mapping, block_tables, num_seqs,
                                             max_blocks_per_seq, token_seq, token_pos, num_tokens,
                                             p->block_size, p->num_blocks, (hipStream_t)stream));
}

pkv_status pkv_reshape_and_cache(void *k_pool, void *v_pool, const void *k, const void *v,
                                 int64_t k_token_stride, int64_t v_token_stride,
                                 const int64_t *slot_mapping, int32_t num_tokens,
                                 const pkv_pool *p, void *stream) {
  if (!p) return PKV_ERR_NULL;
  if (!pool_ok(p)) return PKV_ERR_UNSUPPORTED;
  if (num_tokens < 0) return PKV_ERR_SHAPE;
  if (num_tokens == 0) return PKV_OK;
  if (!k_pool || !v_pool || !k || !v || !slot_mapping) return PKV_ERR_NULL;
  const int64_t row = (int64_t)p->num_kv_heads * p->head_dim;
  if (k_token_stride == 0) k_token_stride = row;
  if (v_token_stride == 0) v_token_stride = row;
  if (k_token_stride < row || v_token_stride < row) return PKV_ERR_SHAPE;
  if (k_token_stride % 8 != 0 || v_token_stride % 8 != 0) return PKV_ERR_SHAPE;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16))
    return PKV_ERR_SHAPE;
  if ((int64_t)num_tokens * p->num_kv_heads * (p->head_dim / 8) > ((int64_t)1 << 40))
    return PKV_ERR_SHAPE;
  return hip_status(pkv::launch_reshape_and_cache(k_pool, v_pool, k, v, k_token_stride,
                                                  v_token_stride, slot_mapping, num_tokens,
                                                  p->num_kv_heads, p->block_size, p->head_dim,
                                                  p->num_blocks, (hipStream_t)stream));
}

int32_t pkv_decode_partition_size(int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                  const pkv_pool *p, int32_t partition_size) {
  Layout lay;
  if (decode_layout(num_seqs, num_heads, max_blocks_per_seq, p, partition_size, &lay) != PKV_OK)
    return 0;
  return lay.P;
}

size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                  const pkv_pool *p, int32_t partition_size) {
  Layout lay;
  if (decode_layout(num_seqs, num_heads, max_blocks_per_seq, p, partition_size, &lay) != PKV_OK)
    return 0;
  return lay.bytes;
}

pkv_status pkv_decode_partitions(void *out, const void *q, const void *k_pool, const void *v_pool,
                                 const int32_t *block_tables, const int32_t *context_lens,
                                 float scale, int32_t num_seqs, int32_t num_heads,
                                 int32_t max_blocks_per_seq, const pkv_pool *p,
                                 int32_t partition_size, void *workspace, size_t workspace_bytes,
                                 void *stream) {
  pkv::DecodeParams a;
  const pkv_status st = fill_params(out, q, k_pool, v_pool, block_tables, context_lens, scale,
                                    num_seqs, num_heads, max_blocks_per_seq, p, partition_size,
                                    workspace, workspace_bytes, true, &a);
  if (st != PKV_OK) return st;
  return hip_status(pkv::launch_decode_partitions(a, (hipStream_t)stream));
}

pkv_status pkv_decode_merge(void *out, const int32_t *context_lens, int32_t num_seqs,
                            int32_t num_heads, int32_t max_blocks_per_seq, const pkv_pool *p,
                            int32_t partition_size, const void *workspace, size_t workspace_bytes,
                            void *stream) {
  pkv::DecodeParams a;
  const pkv_status st = fill_params(out, nullptr, nullptr, nullptr, nullptr, context_lens, 1.0f,
                                    num_seqs, num_heads, max_blocks_per_seq, p, partition_size,
                                    workspace, workspace_bytes, false, &a);
  if (st != PKV_OK) return st;
  return hip_status(pkv::launch_decode_merge(a, (hipStream_t)stream));
}

pkv_status pkv_paged_attention_decode(void *out, const void *q, const void *k_pool,
                                      const void *v_pool, const int32_t *block_tables,
                                      const int32_t *context_lens, float scale, int32_t num_seqs,
                                      int32_t num_heads, int32_t max_blocks_per_seq,
                                      const pkv_pool *p, int32_t partition_size, void *workspace,
                                      size_t workspace_bytes, void *stream) {
  pkv::DecodeParams a;
  const pkv_status st = fill_params(out, q, k_pool, v_pool, block_tables, context_lens, scale,
                                    num_seqs, num_heads, max_blocks_per_seq, p, partition_size,
                                    workspace, workspace_bytes, true, &a);
  if (st != PKV_OK) return st;
  const pkv_status s1 = hip_status(pkv::launch_decode_partitions(a, (hipStream_t)stream));
  if (s1 != PKV_OK) return s1;
  return hip_status(pkv::launch_decode_merge(a, (hipStream_t)stream));
}

}  // extern "C"
