// C ABI of libpagedkv: argument validation, partition sizing, workspace
// layout and dispatch to the kernels.  Declarations and the contract of every
// entry point are in include/pagedkv.h.

#include "pagedkv.h"

#include <hip/hip_runtime.h>

#include <mutex>

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
  if ((p->flags & ~PKV_POOL_REUSE) != 0) return false;
  // every element index must fit in int64 (and slot numbers N * B as well)
  const double elems = (double)p->num_blocks * p->num_kv_heads * p->block_size * p->head_dim;
  return elems < 9.0e18;
}

int partition_unit(const pkv_pool *p) {
  const int tc = pkv::decode_chunk_tokens(p->head_dim);
  return p->block_size > tc ? p->block_size : tc;
}

bool aligned(const void *ptr, size_t a) { return ((uintptr_t)ptr & (a - 1)) == 0; }

// ---- static scratch of the no-allocation decode call
//
// Partial results and the chunk prefix of pkv_paged_attention_decode_noalloc
// live in this array instead of a caller workspace.  Every device the library
// runs on holds its own copy until the process ends.  In host code the name is
// only a stand-in: kernels get the device address that hipGetSymbolAddress
// returns, taken once per device with that device current.
constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// ---- device properties, cached per device (CU count, balanced-kernel occupancy)

struct OccEntry {
  int device;
  const void *kernel;
  size_t lds;
  int blocks;
};

std::mutex g_cache_mu;
int g_cus[64];            // 0 = not queried yet
void *g_scratch[64];      // device address of `scratch` per device; NULL = not taken yet
OccEntry g_occ[256];
int g_occ_n = 0;

int device_cus(int dev) {
  if (dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lk(g_cache_mu);
  if (g_cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    g_cus[dev] = n;
  }
  return g_cus[dev];
}

// Device address of `scratch` on device `dev` (the current device), taken on
// the first call for that device; NULL if the runtime refuses.
void *scratch_on(int dev) {
  if (dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lk(g_cache_mu);
  if (!g_scratch[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

int kernel_blocks_per_cu(int dev, const void *kernel, size_t lds) {
  {
    std::lock_guard<std::mutex> lk(g_cache_mu);
    for (int i = 0; i < g_occ_n; ++i)
      if (g_occ[i].device == dev && g_occ[i].kernel == kernel && g_occ[i].lds == lds) return g_occ[i].blocks;
  }
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, pkv::decode_waves() * 64, lds) != hipSuccess)
    return 0;
  std::lock_guard<std::mutex> lk(g_cache_mu);
  if (g_occ_n < 256) g_occ[g_occ_n++] = OccEntry{dev, kernel, lds, nb};
  return nb;
}

// Workers (wavefronts) the balanced split launches on the current device: as
// many as the device holds at once.  0 if the device cannot be queried.
int balanced_waves(const pkv_pool *p, int32_t num_seqs, bool group, bool fp8, bool suffix = false) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const int cus = device_cus(dev);
  if (cus <= 0) return 0;
  // occupancy for the LDS of this many sequences, rounded up to 4 KiB
  const size_t lds = align_up(group    ? pkv::group_lds_bytes(num_seqs)
                              : fp8    ? pkv::fp8_lds_bytes(num_seqs)
                              : suffix ? pkv::suffix_lds_bytes(num_seqs)
                                       : pkv::balanced_lds_bytes(num_seqs),
                              4096);
  // the smallest occupancy over the instances a call may launch (fused append
  // or not, streamed or cached K/V loads), so that the split and merge passes
  // agree on the worker count whatever the entry point and pool flags
  int nb = 1 << 30;
  for (int nt = 0; nt < 2; ++nt) {
    for (int app = 0; app < 2; ++app) {
      const void *k = group    ? pkv::group_kernel(p->dtype, p->head_dim, p->block_size, nt, fp8 ? 1 : 0)
                      : fp8    ? pkv::fp8_kernel(p->dtype, p->head_dim, p->block_size, nt, app)
                      : suffix ? pkv::suffix_kernel(p->dtype, p->head_dim, p->block_size, nt)
                               : pkv::balanced_kernel(p->dtype, p->head_dim, p->block_size, app, nt);
      if (!k) return 0;
      const int b = kernel_blocks_per_cu(dev, k, lds);
      if (b <= 0) return 0;
      nb = b < nb ? b : nb;
    }
  }
  long long g = (long long)cus * nb * pkv::decode_waves();
  if (g > pkv::kMaxWorkers) g = pkv::kMaxWorkers / pkv::decode_waves() * pkv::decode_waves();
  return (int)g;
}

struct Layout {
  bool balanced;
  bool group;  // several query rows per KV head (matrix-core kernel)
  int32_t P, MP;
  int64_t units;
  int64_t workers;  // balanced split: most workers the batch can use (slices of >= kMinWorkerChunks)
  size_t off_m, off_l, off_o, off_cum, bytes;
};

// fp8: e4m3 pools (head_dim 128, one query row per KV head, balanced split).
pkv_status decode_layout(int32_t num_seqs, int32_t num_heads, int32_t max_blocks,
                         const pkv_pool *p, int32_t partition_size, int32_t num_queries, Layout *lay,
                         bool fp8 = false) {
  if (!p) return PKV_ERR_NULL;
  if (!pool_ok(p)) return PKV_ERR_UNSUPPORTED;
  if (num_seqs < 0 || num_heads < 1 || max_blocks < 1 || num_queries < 1) return PKV_ERR_SHAPE;
  if ((int64_t)max_blocks * p->block_size > (1 << 30)) return PKV_ERR_SHAPE;
  if (num_heads % p->num_kv_heads != 0) return PKV_ERR_UNSUPPORTED;
  if (partition_size < 0) return PKV_ERR_UNSUPPORTED;
  const int64_t ctx = (int64_t)max_blocks * p->block_size;
  const int unit = partition_unit(p);
  *lay = Layout{};
  const int32_t rows = (num_heads / p->num_kv_heads) * num_queries;  // query rows per KV head
  if (fp8 && (partition_size != 0 || num_seqs > pkv::kBalancedMaxSeqs)) return PKV_ERR_UNSUPPORTED;
  if (rows > 1) {
    // several query rows per KV head: the matrix-core kernel, balanced split only
    if (rows > 16 || partition_size != 0 || num_seqs > pkv::kBalancedMaxSeqs) return PKV_ERR_UNSUPPORTED;
    const int64_t row_chunks = (ctx + 15) / 16;
    const int64_t most = (int64_t)num_seqs * p->num_kv_heads * row_chunks;
    if ((double)most >= 1.0e12) return PKV_ERR_SHAPE;
    lay->balanced = true;
    lay->group = true;
    const int64_t workers = (most + pkv::kMinWorkerChunks - 1) / pkv::kMinWorkerChunks;
    const int64_t units = (workers + (int64_t)num_seqs * p->num_kv_heads) * rows;
    lay->units = units;
    lay->workers = workers;
    const size_t cum = align_up((size_t)(num_seqs + 1) * sizeof(int64_t), kAlign);
    const size_t sec = align_up((size_t)units * sizeof(float), kAlign);
    lay->off_cum = 0;
    lay->off_m = cum;
    lay->off_l = cum + sec;
    lay->off_o = cum + 2 * sec;
    lay->bytes = cum + 2 * sec + align_up((size_t)units * p->head_dim * sizeof(float), kAlign);
    return PKV_OK;
  }
  if (partition_size == 0 && num_seqs <= pkv::kBalancedMaxSeqs) {
    // work-balanced split; the cost space (chunks) must stay far below 2^47
    const int tc = fp8 ? pkv::fp8_chunk_tokens(p->head_dim) : pkv::decode_chunk_tokens(p->head_dim);
    const int64_t row_chunks = (ctx + tc - 1) / tc;
    const double cost = (double)num_seqs * num_heads * (double)row_chunks;
    if (cost >= 1.0e12) return PKV_ERR_SHAPE;
    lay->balanced = true;
    // a worker's slice is at least kMinWorkerChunks long, which bounds the
    // workers; each (worker, row) pair it touches can hold a partial
    const int64_t most = (int64_t)num_seqs * num_heads * row_chunks;
    const int64_t workers = (most + pkv::kMinWorkerChunks - 1) / pkv::kMinWorkerChunks;
    const int64_t units = workers + (int64_t)num_seqs * num_heads;
    lay->units = units;
    lay->workers = workers;
    const size_t cum = align_up((size_t)(num_seqs + 1) * sizeof(int64_t), kAlign);
    const size_t sec = align_up((size_t)units * sizeof(float), kAlign);
    lay->off_cum = 0;
    lay->off_m = cum;
    lay->off_l = cum + sec;
    lay->off_o = cum + 2 * sec;
    lay->bytes = cum + 2 * sec + align_up((size_t)units * p->head_dim * sizeof(float), kAlign);
    return PKV_OK;
  }
  int64_t P = partition_size;
  if (P == 0) P = ctx <= 512 ? (ctx + unit - 1) / unit * unit : 512;
  if (P % unit != 0 || P / p->block_size > pkv::kTabMax) return PKV_ERR_UNSUPPORTED;
  const int32_t MP = (int32_t)((ctx + P - 1) / P);
  const int64_t units = (int64_t)num_seqs * num_heads * MP;
  if (units > (int64_t)0x7FFFFF00) return PKV_ERR_SHAPE;  // 1-D grid limit
  lay->P = (int32_t)P;
  lay->MP = MP;
  lay->units = units;
  if (MP >= 2 && units > 0) {
    const size_t sec = align_up((size_t)units * sizeof(float), kAlign);
    lay->off_m = 0;
    lay->off_l = sec;
    lay->off_o = 2 * sec;
    lay->bytes = 2 * sec + align_up((size_t)units * p->head_dim * sizeof(float), kAlign);
  }
  return PKV_OK;
}

// The balanced split's workspace sized for the G workers actually launched
// rather than for the most the batch could use: the chunk prefix, then (m, l,
// o) for each (worker, KV row) pair that can hold a partial, times the query
// rows per KV head.  A worker w < min(G, lay.workers) writes slot
// (w + s * Hkv + h) * rows + r at most, so this holds every partial.
void compact_layout(Layout *lay, int32_t G, int32_t num_seqs, int32_t num_kv_heads, int32_t rows,
                    int32_t head_dim) {
  const int64_t active = G < lay->workers ? (int64_t)G : lay->workers;
  const int64_t units = (active + (int64_t)num_seqs * num_kv_heads) * rows;
  const size_t cum = align_up((size_t)(num_seqs + 1) * sizeof(int64_t), kAlign);
  const size_t sec = align_up((size_t)units * sizeof(float), kAlign);
  lay->units = units;
  lay->off_cum = 0;
  lay->off_m = cum;
  lay->off_l = cum + sec;
  lay->off_o = cum + 2 * sec;
  lay->bytes = cum + 2 * sec + align_up((size_t)units * head_dim * sizeof(float), kAlign);
}

// Workers (wavefronts) the balanced split launches for these arguments, 0 if
// the device cannot be queried.  A small batch cannot use every resident
// wavefront: whole workgroups for the most workers it can use (the split and
// merge passes compute the same count from the same arguments).
int32_t balanced_workers(const pkv_pool *p, int32_t num_seqs, const Layout &lay, bool fp8) {
  int32_t G = balanced_waves(p, num_seqs, lay.group, fp8);
  if (G == 0) return 0;
  const int nw = pkv::decode_waves();
  const int64_t useful = (lay.workers + nw - 1) / nw * nw;
  if (useful < G) G = (int32_t)useful;
  return G;
}

pkv_status fill_params(void *out, const void *q, const void *k_pool, const void *v_pool,
                       const int32_t *block_tables, const int32_t *context_lens, float scale,
                       int32_t num_seqs, int32_t num_heads, int32_t max_blocks, const pkv_pool *p,
                       int32_t partition_size, const void *workspace, size_t workspace_bytes,
                       bool need_inputs, pkv::DecodeParams *a, int32_t num_queries = 1,
                       bool fp8 = false, bool no_alloc = false) {
  if (num_seqs == 0) {  // nothing to do; still validate the static arguments
    Layout lay;
    const pkv_status st = decode_layout(0, num_heads, max_blocks, p, partition_size, num_queries, &lay, fp8);
    *a = pkv::DecodeParams{};
    return st;
  }
  if (num_seqs < 0) return PKV_ERR_SHAPE;
  if (!p) return PKV_ERR_NULL;
  if (!pool_ok(p)) return PKV_ERR_UNSUPPORTED;
  if (num_heads < 1 || max_blocks < 1) return PKV_ERR_SHAPE;
  if (!out || !context_lens) return PKV_ERR_NULL;
  if (need_inputs && (!q || !k_pool || !v_pool || !block_tables)) return PKV_ERR_NULL;
  if (need_inputs && (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16)))
    return PKV_ERR_SHAPE;
  if (!aligned(out, 16)) return PKV_ERR_SHAPE;
  Layout lay;
  const pkv_status st = decode_layout(num_seqs, num_heads, max_blocks, p, partition_size, num_queries, &lay, fp8);
  if (st != PKV_OK) return st;
  int32_t G = 0;
  if (no_alloc) {
    // the static scratch of this device in place of a workspace
    if (!lay.balanced) return PKV_ERR_UNSUPPORTED;
    G = balanced_workers(p, num_seqs, lay, fp8);
    if (G == 0) return PKV_ERR_HIP;
    compact_layout(&lay, G, num_seqs, p->num_kv_heads, (num_heads / p->num_kv_heads) * num_queries,
                   p->head_dim);
    if (lay.bytes > kScratchBytes) return PKV_ERR_SCRATCH;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PKV_ERR_HIP;
    workspace = scratch_on(dev);
    if (!workspace) return PKV_ERR_HIP;
    workspace_bytes = kScratchBytes;
  }
  if (lay.bytes > 0) {
    if (!workspace || workspace_bytes < lay.bytes || !aligned(workspace, kAlign))
      return PKV_ERR_WORKSPACE;
  }
  char *ws = (char *)workspace;
  *a = pkv::DecodeParams{};
  a->out = out;
  a->q = q;
  a->k_pool = k_pool;
  a->v_pool = v_pool;
  a->tables = block_tables;
  a->lens = context_lens;
  if (lay.bytes) {
    a->ws_m = (float *)(ws + lay.off_m);
    a->ws_l = (float *)(ws + lay.off_l);
    a->ws_o = (float *)(ws + lay.off_o);
    a->ws_cum = lay.balanced ? (int64_t *)(ws + lay.off_cum) : nullptr;
  }
  if (lay.balanced && G == 0) {
    G = balanced_workers(p, num_seqs, lay, fp8);
    if (G == 0) return PKV_ERR_HIP;
  }
  a->G = G;
  a->nq = num_queries;
  a->group = lay.group ? 1 : 0;
  a->fp8 = fp8 ? 1 : 0;
  a->v_scale = 1.0f;
  a->stream_kv = (p->flags & PKV_POOL_REUSE) ? 0 : 1;
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
  a->items = lay.balanced ? 0 : (int32_t)lay.units;
  a->balanced = lay.balanced ? 1 : 0;
  a->dtype = p->dtype;
  return PKV_OK;
}

pkv_status hip_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_HIP; }

// Grouped rows take the append as its own launch (slots from the table)
// before the matrix-core split pass; one row per KV head fuses it into the
// split pass.
pkv_status append_if_separate(pkv::DecodeParams *a, hipStream_t stream) {
  if (!a->append || !a->group) return PKV_OK;
  const pkv_status st = hip_status(pkv::launch_append_last(*a, stream));
  a->append = 0;
  return st;
}

hipError_t launch_split(const pkv::DecodeParams &a, hipStream_t stream) {
  if (a.fp8 && !a.group) return pkv::launch_fp8_decode(a, stream);
  return a.group ? pkv::launch_group_decode(a, stream) : pkv::launch_decode_partitions(a, stream);
}

hipError_t launch_merge(const pkv::DecodeParams &a, hipStream_t stream) {
  return a.group ? pkv::launch_group_merge(a, stream) : pkv::launch_decode_merge(a, stream);
}

// Validation and parameters shared by the two fused-append entry points.
pkv_status fill_append(void *out, const void *q, const void *k_new, const void *v_new,
                       int64_t new_token_stride, void *k_pool, void *v_pool,
                       const int32_t *block_tables, const int32_t *context_lens, float scale,
                       int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                       const pkv_pool *p, int32_t partition_size, void *workspace,
                       size_t workspace_bytes, pkv::DecodeParams *a, bool fp8 = false) {
  const pkv_status st = fill_params(out, q, k_pool, v_pool, block_tables, context_lens, scale,
                                    num_seqs, num_heads, max_blocks_per_seq, p, partition_size,
                                    workspace, workspace_bytes, true, a, 1, fp8);
  if (st != PKV_OK || num_seqs == 0) return st;

  if (!k_new || !v_new) return PKV_ERR_NULL;
  const int64_t row = (int64_t)p->num_kv_heads * p->head_dim;
  if (new_token_stride == 0) new_token_stride = row;
  if (new_token_stride < row || new_token_stride % 8 != 0) return PKV_ERR_SHAPE;
  if (!aligned(k_new, 16) || !aligned(v_new, 16)) return PKV_ERR_SHAPE;
  a->append = 1;
  a->k_new = k_new;
  a->v_new = v_new;
  a->new_stride = new_token_stride;
  return PKV_OK;
}

// A per-pool FP8 scale: positive and finite, with a finite float32 reciprocal.
bool fp8_scale_ok(float s) { return s > 0.f && s <= 3.0e38f && 1.0f / s > 0.f && 1.0f / s <= 3.0e38f; }

// ---- shared prompt prefixes

// Workspace of pkv_paged_attention_decode_shared: the prefix pass's balanced
// layout (groups as sequences, their members as query rows), the prefix
// states of every (sequence, head) row, then the suffix pass's layout.
struct SharedLayout {
  Layout pre, suf;
  size_t off_pre, off_state_m, off_state_l, off_state_o, off_suf, bytes;
};

pkv_status shared_layout(int32_t num_seqs, int32_t num_heads, int32_t max_blocks, const pkv_pool *p,
                         int32_t group_size, SharedLayout *sl) {
  if (!p) return PKV_ERR_NULL;
  if (!pool_ok(p)) return PKV_ERR_UNSUPPORTED;
  if (num_seqs < 0 || num_heads < 1 || max_blocks < 1 || group_size < 1) return PKV_ERR_SHAPE;
  if (num_heads != p->num_kv_heads || group_size < 2 || group_size > 16 || num_seqs > pkv::kBalancedMaxSeqs)
    return PKV_ERR_UNSUPPORTED;
  if (num_seqs % group_size != 0) return PKV_ERR_SHAPE;
  if ((int64_t)max_blocks * p->block_size > (1 << 30)) return PKV_ERR_SHAPE;
  *sl = SharedLayout{};
  const int32_t groups = num_seqs / group_size;
  // prefix pass: the matrix-core kernel's layout for `groups` sequences of
  // group_size query rows per KV head
  const pkv_status st = decode_layout(groups, num_heads, max_blocks, p, 0, group_size, &sl->pre);
  if (st != PKV_OK) return st;
  const pkv_status st2 = decode_layout(num_seqs, num_heads, max_blocks, p, 0, 1, &sl->suf);
  if (st2 != PKV_OK) return st2;
  if (!sl->pre.group || !sl->suf.balanced || sl->suf.group) return PKV_ERR_UNSUPPORTED;
  const size_t rows = (size_t)num_seqs * num_heads;
  sl->off_pre = 0;
  sl->off_state_m = align_up(sl->pre.bytes, kAlign);
  sl->off_state_l = sl->off_state_m + align_up(rows * sizeof(float), kAlign);
  sl->off_state_o = sl->off_state_l + align_up(rows * sizeof(float), kAlign);
  sl->off_suf = sl->off_state_o + align_up(rows * p->head_dim * sizeof(float), kAlign);
  sl->bytes = sl->off_suf + align_up(sl->suf.bytes, kAlign);
  return PKV_OK;
}

void set_workspace(pkv::DecodeParams *a, const Layout &lay, char *base) {
  a->ws_m = (float *)(base + lay.off_m);
  a->ws_l = (float *)(base + lay.off_l);
  a->ws_o = (float *)(base + lay.off_o);
  a->ws_cum = (int64_t *)(base + lay.off_cum);
}

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
    case PKV_ERR_SCRATCH: return "the call needs more than the library's static scratch holds";
    default: return "unknown status";
  }
}

size_t pkv_pool_bytes(const pkv_pool *p) {
  if (!pool_ok(p)) return 0;
  return (size_t)p->num_blocks * p->num_kv_heads * p->block_size * p->head_dim * 2;
}

size_t pkv_fp8_pool_bytes(const pkv_pool *p) {
  if (!pool_ok(p)) return 0;
  return (size_t)p->num_blocks * p->num_kv_heads * p->block_size * p->head_dim;
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

pkv_status pkv_copy_blocks(void *k_pool, void *v_pool, const int64_t *block_pairs, int32_t num_pairs,
                           const pkv_pool *p, void *stream) {
  if (!p) return PKV_ERR_NULL;
  if (!pool_ok(p)) return PKV_ERR_UNSUPPORTED;
  if (num_pairs < 0) return PKV_ERR_SHAPE;
  if (num_pairs == 0) return PKV_OK;
  if (!k_pool || !v_pool || !block_pairs) return PKV_ERR_NULL;
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(block_pairs, 8)) return PKV_ERR_SHAPE;
  if (pkv::copy_blocks_workgroups(num_pairs, p->num_kv_heads, p->block_size, p->head_dim) > 0x7FFFFFFF)
    return PKV_ERR_SHAPE;
  return hip_status(pkv::launch_copy_blocks(k_pool, v_pool, block_pairs, num_pairs, p->num_kv_heads,
                                            p->block_size, p->head_dim, p->num_blocks,
                                            (hipStream_t)stream));
}

int32_t pkv_decode_partition_size(int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                  const pkv_pool *p, int32_t partition_size) {
  Layout lay;
  if (decode_layout(num_seqs, num_heads, max_blocks_per_seq, p, partition_size, 1, &lay) != PKV_OK)
    return -1;
  return lay.balanced ? 0 : lay.P;
}

size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                  const pkv_pool *p, int32_t partition_size) {
  Layout lay;
  if (decode_layout(num_seqs, num_heads, max_blocks_per_seq, p, partition_size, 1, &lay) != PKV_OK)
    return 0;
  return lay.bytes;
}

pkv_status pkv_decode_launch_info(int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                  const pkv_pool *p, int32_t partition_size, int32_t num_queries, int32_t fp8,
                                  int32_t append, pkv_launch_info *info) {
  if (!info) return PKV_ERR_NULL;
  *info = pkv_launch_info{};
  if (num_seqs < 1) return PKV_ERR_SHAPE;
  Layout lay;
  const pkv_status st =
      decode_layout(num_seqs, num_heads, max_blocks_per_seq, p, partition_size, num_queries, &lay, fp8 != 0);
  if (st != PKV_OK) return st;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PKV_ERR_HIP;
  const int cus = device_cus(dev);
  if (cus <= 0) return PKV_ERR_HIP;
  const int nw = pkv::decode_waves();
  const int nt = (p->flags & PKV_POOL_REUSE) ? 0 : 1;
  const void *k = nullptr;
  size_t lds = 0;
  int64_t wgs = 0;
  if (lay.balanced) {
    if (lay.group) {
      k = pkv::group_kernel(p->dtype, p->head_dim, p->block_size, nt, fp8 ? 1 : 0);
      lds = pkv::group_lds_bytes(num_seqs);
    } else if (fp8) {
      k = pkv::fp8_kernel(p->dtype, p->head_dim, p->block_size, nt, append ? 1 : 0);
      lds = pkv::fp8_lds_bytes(num_seqs);
    } else {
      k = pkv::balanced_kernel(p->dtype, p->head_dim, p->block_size, append ? 1 : 0, nt);
      lds = pkv::balanced_lds_bytes(num_seqs);
    }
    const int32_t G = balanced_workers(p, num_seqs, lay, fp8 != 0);
    if (G == 0) return PKV_ERR_HIP;
    wgs = G / nw;
  } else {
    k = pkv::partition_kernel(p->dtype, p->head_dim, p->block_size, nt);
    wgs = pkv::partition_grid(lay.units);
  }
  if (!k) return PKV_ERR_UNSUPPORTED;
  hipFuncAttributes attr;
  if (hipFuncGetAttributes(&attr, k) != hipSuccess) return PKV_ERR_HIP;
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k, nw * 64, lds) != hipSuccess) return PKV_ERR_HIP;
  info->workgroups = wgs > INT32_MAX ? INT32_MAX : (int32_t)wgs;
  info->waves_per_workgroup = nw;
  info->waves_per_simd = blocks * nw / 4;  // four SIMDs per compute unit
  info->compute_units = cus;
  info->registers = attr.numRegs;
  info->lds_static_bytes = (int32_t)attr.sharedSizeBytes;
  info->lds_dynamic_bytes = (int32_t)lds;
  info->scratch_bytes = (int32_t)attr.localSizeBytes;
  info->balanced = lay.balanced ? 1 : 0;
  info->partition_size = lay.balanced ? 0 : lay.P;
  return PKV_OK;
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
  return hip_status(launch_split(a, (hipStream_t)stream));
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
  return hip_status(launch_merge(a, (hipStream_t)stream));
}

pkv_status pkv_paged_attention_decode_append(void *out, const void *q, const void *k_new,
                                             const void *v_new, int64_t new_token_stride,
                                             void *k_pool, void *v_pool,
                                             const int32_t *block_tables,
                                             const int32_t *context_lens, float scale,
                                             int32_t num_seqs, int32_t num_heads,
                                             int32_t max_blocks_per_seq, const pkv_pool *p,
                                             int32_t partition_size, void *workspace,
                                             size_t workspace_bytes, void *stream) {
  pkv::DecodeParams a;
  const pkv_status st = fill_append(out, q, k_new, v_new, new_token_stride, k_pool, v_pool,
                                    block_tables, context_lens, scale, num_seqs, num_heads,
                                    max_blocks_per_seq, p, partition_size, workspace,
                                    workspace_bytes, &a);
  if (st != PKV_OK) return st;
  const pkv_status s0 = append_if_separate(&a, (hipStream_t)stream);
  if (s0 != PKV_OK) return s0;
  // balanced split, one row per KV head: the split pass substitutes the new
  // rows and the merge launch writes them to the pool
  if (a.append && a.balanced && !a.group) a.append_in_merge = 1;
  const pkv_status s1 = hip_status(launch_split(a, (hipStream_t)stream));
  if (s1 != PKV_OK) return s1;
  return hip_status(launch_merge(a, (hipStream_t)stream));
}

pkv_status pkv_decode_partitions_append(void *out, const void *q, const void *k_new,
                                        const void *v_new, int64_t new_token_stride, void *k_pool,
                                        void *v_pool, const int32_t *block_tables,
                                        const int32_t *context_lens, float scale, int32_t num_seqs,
                                        int32_t num_heads, int32_t max_blocks_per_seq,
                                        const pkv_pool *p, int32_t partition_size, void *workspace,
                                        size_t workspace_bytes, void *stream) {
  pkv::DecodeParams a;
  const pkv_status st = fill_append(out, q, k_new, v_new, new_token_stride, k_pool, v_pool,
                                    block_tables, context_lens, scale, num_seqs, num_heads,
                                    max_blocks_per_seq, p, partition_size, workspace,
                                    workspace_bytes, &a);
  if (st != PKV_OK) return st;
  const pkv_status s0 = append_if_separate(&a, (hipStream_t)stream);
  if (s0 != PKV_OK) return s0;
  return hip_status(launch_split(a, (hipStream_t)stream));
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
  const pkv_status s1 = hip_status(launch_split(a, (hipStream_t)stream));
  if (s1 != PKV_OK) return s1;
  return hip_status(launch_merge(a, (hipStream_t)stream));
}

pkv_status pkv_paged_attention_decode_noalloc(void *out, const void *q, const void *k_pool,
                                              const void *v_pool, const int32_t *block_tables,
                                              const int32_t *context_lens, float scale, int32_t num_seqs,
                                              int32_t num_heads, int32_t max_blocks_per_seq,
                                              const pkv_pool *p, void *stream) {
  pkv::DecodeParams a;
  const pkv_status st = fill_params(out, q, k_pool, v_pool, block_tables, context_lens, scale,
                                    num_seqs, num_heads, max_blocks_per_seq, p, 0, nullptr, 0, true, &a, 1,
                                    false, true);
  if (st != PKV_OK || num_seqs == 0) return st;
  const pkv_status s1 = hip_status(launch_split(a, (hipStream_t)stream));
  if (s1 != PKV_OK) return s1;
  return hip_status(launch_merge(a, (hipStream_t)stream));
}

size_t pkv_multi_workspace_bytes(int32_t num_seqs, int32_t num_queries, int32_t num_heads,
                                 int32_t max_blocks_per_seq, const pkv_pool *p) {
  Layout lay;
  if (decode_layout(num_seqs, num_heads, max_blocks_per_seq, p, 0, num_queries, &lay) != PKV_OK) return 0;
  return lay.bytes;
}

pkv_status pkv_paged_attention_multi(void *out, const void *q, const void *k_pool, const void *v_pool,
                                     const int32_t *block_tables, const int32_t *context_lens, float scale,
                                     int32_t num_seqs, int32_t num_queries, int32_t num_heads,
                                     int32_t max_blocks_per_seq, const pkv_pool *p, void *workspace,
                                     size_t workspace_bytes, void *stream) {
  pkv::DecodeParams a;
  const pkv_status st = fill_params(out, q, k_pool, v_pool, block_tables, context_lens, scale, num_seqs,
                                    num_heads, max_blocks_per_seq, p, 0, workspace, workspace_bytes, true, &a,
                                    num_queries);
  if (st != PKV_OK || num_seqs == 0) return st;
  const pkv_status s1 = hip_status(launch_split(a, (hipStream_t)stream));
  if (s1 != PKV_OK) return s1;
  return hip_status(launch_merge(a, (hipStream_t)stream));
}

pkv_status pkv_reshape_and_cache_fp8(void *k_pool, void *v_pool, const void *k, const void *v,
                                     int64_t k_token_stride, int64_t v_token_stride,
                                     const int64_t *slot_mapping, int32_t num_tokens, float k_scale,
                                     float v_scale, const pkv_pool *p, void *stream) {
  if (!p) return PKV_ERR_NULL;
  if (!pool_ok(p)) return PKV_ERR_UNSUPPORTED;
  if (num_tokens < 0) return PKV_ERR_SHAPE;
  if (!fp8_scale_ok(k_scale) || !fp8_scale_ok(v_scale)) return PKV_ERR_SHAPE;
  if (num_tokens == 0) return PKV_OK;
  if (!k_pool || !v_pool || !k || !v || !slot_mapping) return PKV_ERR_NULL;
  const int64_t row = (int64_t)p->num_kv_heads * p->head_dim;
  if (k_token_stride == 0) k_token_stride = row;
  if (v_token_stride == 0) v_token_stride = row;
  if (k_token_stride < row || v_token_stride < row) return PKV_ERR_SHAPE;
  if (k_token_stride % 8 != 0 || v_token_stride % 8 != 0) return PKV_ERR_SHAPE;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16))
    return PKV_ERR_SHAPE;
  if ((int64_t)num_tokens * p->num_kv_heads * (p->head_dim / 16) > ((int64_t)1 << 40))
    return PKV_ERR_SHAPE;
  return hip_status(pkv::launch_reshape_and_cache_fp8(
      k_pool, v_pool, k, v, k_token_stride, v_token_stride, slot_mapping, num_tokens, p->num_kv_heads,
      p->block_size, p->head_dim, p->num_blocks, p->dtype, 1.0f / k_scale, 1.0f / v_scale,
      (hipStream_t)stream));
}

size_t pkv_fp8_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                      const pkv_pool *p) {
  Layout lay;
  if (decode_layout(num_seqs, num_heads, max_blocks_per_seq, p, 0, 1, &lay, true) != PKV_OK) return 0;
  return lay.bytes;
}

pkv_status pkv_paged_attention_decode_fp8(void *out, const void *q, const void *k_pool, const void *v_pool,
                                          const int32_t *block_tables, const int32_t *context_lens, float scale,
                                          float k_scale, float v_scale, int32_t num_seqs, int32_t num_heads,
                                          int32_t max_blocks_per_seq, const pkv_pool *p, void *workspace,
                                          size_t workspace_bytes, void *stream) {
  if (!fp8_scale_ok(k_scale) || !fp8_scale_ok(v_scale)) return PKV_ERR_SHAPE;
  pkv::DecodeParams a;
  const pkv_status st = fill_params(out, q, k_pool, v_pool, block_tables, context_lens, scale, num_seqs,
                                    num_heads, max_blocks_per_seq, p, 0, workspace, workspace_bytes, true, &a, 1,
                                    true);
  if (st != PKV_OK || num_seqs == 0) return st;
  a.scale_log2 = scale * k_scale * 1.4426950408889634f;
  a.v_scale = v_scale;
  const pkv_status s1 = hip_status(launch_split(a, (hipStream_t)stream));
  if (s1 != PKV_OK) return s1;
  return hip_status(launch_merge(a, (hipStream_t)stream));
}

pkv_status pkv_paged_attention_decode_append_fp8(void *out, const void *q, const void *k_new, const void *v_new,
                                                 int64_t new_token_stride, void *k_pool, void *v_pool,
                                                 const int32_t *block_tables, const int32_t *context_lens,
                                                 float scale, float k_scale, float v_scale, int32_t num_seqs,
                                                 int32_t num_heads, int32_t max_blocks_per_seq, const pkv_pool *p,
                                                 void *workspace, size_t workspace_bytes, void *stream) {
  if (!fp8_scale_ok(k_scale) || !fp8_scale_ok(v_scale)) return PKV_ERR_SHAPE;
  pkv::DecodeParams a;
  const pkv_status st = fill_append(out, q, k_new, v_new, new_token_stride, k_pool, v_pool, block_tables,
                                    context_lens, scale, num_seqs, num_heads, max_blocks_per_seq, p, 0, workspace,
                                    workspace_bytes, &a, true);
  if (st != PKV_OK || num_seqs == 0) return st;
  a.scale_log2 = scale * k_scale * 1.4426950408889634f;
  a.v_scale = v_scale;
  a.k_inv = 1.0f / k_scale;
  a.v_inv = 1.0f / v_scale;
  if (a.group) {
    // grouped rows: the append as its own launch (slots from the table)
    const pkv_status s0 = hip_status(pkv::launch_append_last_fp8(a, a.k_inv, a.v_inv, (hipStream_t)stream));
    if (s0 != PKV_OK) return s0;
    a.append = 0;
  }
  // one row per KV head: the split pass quantises each row's new token in
  // place of its pool slot, and the merge launch writes the codes to the pool
  const pkv_status s1 = hip_status(launch_split(a, (hipStream_t)stream));
  if (s1 != PKV_OK) return s1;
  return hip_status(launch_merge(a, (hipStream_t)stream));
}

size_t pkv_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                         const pkv_pool *p, int32_t group_size) {
  SharedLayout sl;
  if (shared_layout(num_seqs, num_heads, max_blocks_per_seq, p, group_size, &sl) != PKV_OK) return 0;
  return sl.bytes;
}

pkv_status pkv_paged_attention_decode_shared(void *out, const void *q, const void *k_pool, const void *v_pool,
                                             const int32_t *block_tables, const int32_t *context_lens, float scale,
                                             int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                             const pkv_pool *p, int32_t group_size, const int32_t *prefix_lens,
                                             void *workspace, size_t workspace_bytes, void *stream) {
  SharedLayout sl;
  const pkv_status st = shared_layout(num_seqs, num_heads, max_blocks_per_seq, p, group_size, &sl);
  if (st != PKV_OK || num_seqs == 0) return st;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens || !prefix_lens) return PKV_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(out, 16)) return PKV_ERR_SHAPE;
  if (!workspace || workspace_bytes < sl.bytes || !aligned(workspace, kAlign)) return PKV_ERR_WORKSPACE;
  const int32_t groups = num_seqs / group_size;
  char *ws = (char *)workspace;
  float *st_m = (float *)(ws + sl.off_state_m);
  float *st_l = (float *)(ws + sl.off_state_l);
  float *st_o = (float *)(ws + sl.off_state_o);

  pkv::DecodeParams base{};
  base.out = out;
  base.q = q;
  base.k_pool = k_pool;
  base.v_pool = v_pool;
  base.tables = block_tables;
  base.scale_log2 = scale * 1.4426950408889634f;
  base.v_scale = 1.0f;
  base.num_blocks = p->num_blocks;
  base.H = num_heads;
  base.Hkv = p->num_kv_heads;
  base.maxb = max_blocks_per_seq;
  base.B = p->block_size;
  base.D = p->head_dim;
  base.dtype = p->dtype;
  base.balanced = 1;
  base.stream_kv = (p->flags & PKV_POOL_REUSE) ? 0 : 1;
  base.pfx_group = group_size;
  base.pfx_lens = prefix_lens;
  base.pfx_m = st_m;
  base.pfx_l = st_l;
  base.pfx_o = st_o;

  // prefix pass: groups as sequences, their members as the query rows of each
  // KV head, every row over the whole prefix; then its merge
  pkv::DecodeParams pre = base;
  pre.S = groups;
  pre.lens = prefix_lens;
  pre.nq = group_size;
  pre.group = 1;
  pre.pfx_pass = 1;
  set_workspace(&pre, sl.pre, ws + sl.off_pre);
  pre.G = balanced_workers(p, groups, sl.pre, false);
  if (pre.G == 0) return PKV_ERR_HIP;

  // suffix pass: every sequence from its group's prefix length on, starting
  // from the prefix state; then the merge of the rows it cuts
  pkv::DecodeParams suf = base;
  suf.S = num_seqs;
  suf.lens = context_lens;
  suf.nq = 1;
  suf.pfx_pass = 2;
  set_workspace(&suf, sl.suf, ws + sl.off_suf);
  {
    int32_t G = balanced_waves(p, num_seqs, false, false, true);
    if (G == 0) return PKV_ERR_HIP;
    const int nw = pkv::decode_waves();
    const int64_t useful = (sl.suf.workers + nw - 1) / nw * nw;
    suf.G = useful < G ? (int32_t)useful : G;
  }

  hipStream_t s = (hipStream_t)stream;
  pkv_status r = hip_status(pkv::launch_group_decode(pre, s));
  if (r == PKV_OK) r = hip_status(pkv::launch_group_merge(pre, s));
  if (r == PKV_OK) r = hip_status(pkv::launch_suffix(suf, s));
  if (r == PKV_OK) r = hip_status(pkv::launch_decode_merge(suf, s));
  return r;
}

size_t pkv_fp8_multi_workspace_bytes(int32_t num_seqs, int32_t num_queries, int32_t num_heads,
                                     int32_t max_blocks_per_seq, const pkv_pool *p) {
  Layout lay;
  if (decode_layout(num_seqs, num_heads, max_blocks_per_seq, p, 0, num_queries, &lay, true) != PKV_OK) return 0;
  return lay.bytes;
}

pkv_status pkv_paged_attention_multi_fp8(void *out, const void *q, const void *k_pool, const void *v_pool,
                                         const int32_t *block_tables, const int32_t *context_lens, float scale,
                                         float k_scale, float v_scale, int32_t num_seqs, int32_t num_queries,
                                         int32_t num_heads, int32_t max_blocks_per_seq, const pkv_pool *p,
                                         void *workspace, size_t workspace_bytes, void *stream) {
  if (!fp8_scale_ok(k_scale) || !fp8_scale_ok(v_scale)) return PKV_ERR_SHAPE;
  pkv::DecodeParams a;
  const pkv_status st = fill_params(out, q, k_pool, v_pool, block_tables, context_lens, scale, num_seqs,
                                    num_heads, max_blocks_per_seq, p, 0, workspace, workspace_bytes, true, &a,
                                    num_queries, true);
  if (st != PKV_OK || num_seqs == 0) return st;
  a.scale_log2 = scale * k_scale * 1.4426950408889634f;
  a.v_scale = v_scale;
  const pkv_status s1 = hip_status(launch_split(a, (hipStream_t)stream));
  if (s1 != PKV_OK) return s1;
  return hip_status(launch_merge(a, (hipStream_t)stream));
}

pkv_status pkv_decode_partitions_fp8(void *out, const void *q, const void *k_pool, const void *v_pool,
                                     const int32_t *block_tables, const int32_t *context_lens, float scale,
                                     float k_scale, float v_scale, int32_t num_seqs, int32_t num_queries,
                                     int32_t num_heads, int32_t max_blocks_per_seq, const pkv_pool *p,
                                     void *workspace, size_t workspace_bytes, void *stream) {
  if (!fp8_scale_ok(k_scale) || !fp8_scale_ok(v_scale)) return PKV_ERR_SHAPE;
  pkv::DecodeParams a;
  const pkv_status st = fill_params(out, q, k_pool, v_pool, block_tables, context_lens, scale, num_seqs,
                                    num_heads, max_blocks_per_seq, p, 0, workspace, workspace_bytes, true, &a,
                                    num_queries, true);
  if (st != PKV_OK || num_seqs == 0) return st;
  a.scale_log2 = scale * k_scale * 1.4426950408889634f;
  a.v_scale = v_scale;
  return hip_status(launch_split(a, (hipStream_t)stream));
}

pkv_status pkv_decode_merge_fp8(void *out, const int32_t *context_lens, int32_t num_seqs, int32_t num_queries,
                                int32_t num_heads, int32_t max_blocks_per_seq, const pkv_pool *p,
                                const void *workspace, size_t workspace_bytes, void *stream) {
  pkv::DecodeParams a;
  const pkv_status st = fill_params(out, nullptr, nullptr, nullptr, nullptr, context_lens, 1.0f, num_seqs,
                                    num_heads, max_blocks_per_seq, p, 0, workspace, workspace_bytes, false, &a,
                                    num_queries, true);
  if (st != PKV_OK || num_seqs == 0) return st;
  return hip_status(launch_merge(a, (hipStream_t)stream));
}

}  // extern "C"
