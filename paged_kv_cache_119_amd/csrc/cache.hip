// Cache append and slot translation for gfx950.
//
// Append ("PagedAttention 完全拆解", 原理详解（三）, item 1, fused reshape and
// block write): each new token's K and V rows, laid out [token][head][dim] as
// projected, are written to pool[slot / B][head][slot % B][:] in one kernel.
// Each thread moves one 16-byte piece of one (token, head) row of K and the
// same piece of V; consecutive threads cover consecutive pieces of a row, so
// reads and writes are both contiguous 16-byte accesses.
//
// Slot translation (iaim.asia block-table article, "KV Cache 如何按块分配",
// BLOCK_SIZE=16 table): slot = block_tables[s][pos / B] * B + pos % B.
//
// The decode step's append from the block table: row s of the new-token K/V
// becomes token L - 1 of sequence s, its slot found through the table (no
// slot list); used where the append is not fused into the split pass.
//
// Block copy ("PagedAttention 完全拆解", 内存共享 and Figure 8: a sequence about
// to write into a block it shares first gets a private copy of it): a batch
// of (src, dst) pairs is copied in one launch.  A pool block holds all heads
// ([Hkv][B][D]), so each copy is one contiguous run per pool, cut into runs of
// 16 KiB per workgroup.

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

namespace {

__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    uint16_t *__restrict__ kp, uint16_t *__restrict__ vp, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, int64_t k_stride, int64_t v_stride,
    const int64_t *__restrict__ slots, int32_t T, int32_t Hkv, int32_t B, int32_t D,
    int64_t num_blocks) {
  const int vpr = D / 8;                       // 16-byte pieces per head row
  const int64_t per_tok = (int64_t)Hkv * vpr;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)T * per_tok) return;
  const int t = (int)(idx / per_tok);
  const int r = (int)(idx - (int64_t)t * per_tok);
  const int h = r / vpr;
  const int piece = r - h * vpr;
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= num_blocks * B) return;
  const int64_t blk = slot / B;
  const int64_t off = slot - blk * B;
  const int64_t dst = ((blk * Hkv + h) * B + off) * D + piece * 8;
  const u32x4 kv = *reinterpret_cast<const u32x4 *>(k + (int64_t)t * k_stride + h * D + piece * 8);
  const u32x4 vv = *reinterpret_cast<const u32x4 *>(v + (int64_t)t * v_stride + h * D + piece * 8);
  *reinterpret_cast<u32x4 *>(kp + dst) = kv;
  *reinterpret_cast<u32x4 *>(vp + dst) = vv;
}

__global__ __launch_bounds__(256) void slot_mapping_kernel(int64_t *__restrict__ slots,
                                                           const int32_t *__restrict__ tables,
                                                           int32_t S, int32_t maxb,
                                                           const int32_t *__restrict__ seq,
                                                           const int32_t *__restrict__ pos,
                                                           int32_t T, int32_t B,
                                                           int64_t num_blocks) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  const int s = seq[t];
  const int x = pos[t];
  int64_t out = -1;
  if (s >= 0 && s < S && x >= 0 && x < maxb * B) {
    const int32_t blk = tables[(int64_t)s * maxb + x / B];
    if (blk >= 0 && (int64_t)blk < num_blocks) out = (int64_t)blk * B + x % B;
  }
  slots[t] = out;
}

// Workgroup w copies run w % per_pair of pair w / per_pair: kCopyUnroll
// 16-byte pieces per thread and tensor, all loads issued before the stores.
// Source and destination are touched once, so both go around the caches.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint16_t *__restrict__ kp,
                                                          uint16_t *__restrict__ vp,
                                                          const int64_t *__restrict__ pairs,
                                                          int64_t pieces,  // 16-byte pieces per block
                                                          uint32_t per_pair, int64_t num_blocks) {
  const uint32_t i = blockIdx.x / per_pair;
  const uint32_t run = blockIdx.x - i * per_pair;
  const int64_t src = pairs[2 * (int64_t)i];
  const int64_t dst = pairs[2 * (int64_t)i + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const int64_t first = (int64_t)run * (kCopyThreads * kCopyUnroll) + threadIdx.x;
  const uint16_t *ks = kp + (src * pieces + first) * 8, *vs = vp + (src * pieces + first) * 8;
  uint16_t *kd = kp + (dst * pieces + first) * 8, *vd = vp + (dst * pieces + first) * 8;
  constexpr int kStep = kCopyThreads * 8;  // elements between a thread's pieces
  if ((int64_t)(run + 1) * (kCopyThreads * kCopyUnroll) <= pieces) {
    // a whole run: every load in flight before the first store
    u32x4 kv[kCopyUnroll], vv[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      kv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(ks + u * kStep));
      vv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vs + u * kStep));
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      __builtin_nontemporal_store(kv[u], reinterpret_cast<u32x4 *>(kd + u * kStep));
      __builtin_nontemporal_store(vv[u], reinterpret_cast<u32x4 *>(vd + u * kStep));
    }
  } else {
    // the block's last, partial run
    for (int u = 0; u < kCopyUnroll && first + u * kCopyThreads < pieces; ++u) {
      const u32x4 kv = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(ks + u * kStep));
      const u32x4 vv = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vs + u * kStep));
      __builtin_nontemporal_store(kv, reinterpret_cast<u32x4 *>(kd + u * kStep));
      __builtin_nontemporal_store(vv, reinterpret_cast<u32x4 *>(vd + u * kStep));
    }
  }
}

// One thread per 16-byte piece of a (sequence, head) row, K and V; invalid
// contexts and table entries outside the pool write nothing.
__global__ __launch_bounds__(256) void append_last_kernel(DecodeParams a) {
  const int vpr = a.D / 8;
  const int64_t per_seq = (int64_t)a.Hkv * vpr;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)a.S * per_seq) return;
  const int s = (int)(idx / per_seq);
  const int r = (int)(idx - (int64_t)s * per_seq);
  const int h = r / vpr;
  const int piece = r - h * vpr;
  const int L = a.lens[s];
  if (L <= 0 || L > a.maxb * a.B) return;
  const int blk = a.tables[(int64_t)s * a.maxb + (L - 1) / a.B];
  if (blk < 0 || (int64_t)blk >= a.num_blocks) return;
  const int64_t dst = (((int64_t)blk * a.Hkv + h) * a.B + (L - 1) % a.B) * a.D + piece * 8;
  const int64_t src = (int64_t)s * a.new_stride + (int64_t)h * a.D + piece * 8;
  const u32x4 kv = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(a.k_new) + src);
  const u32x4 vv = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(a.v_new) + src);
  *reinterpret_cast<u32x4 *>(reinterpret_cast<uint16_t *>(const_cast<void *>(a.k_pool)) + dst) = kv;
  *reinterpret_cast<u32x4 *>(reinterpret_cast<uint16_t *>(const_cast<void *>(a.v_pool)) + dst) = vv;
}

}  // namespace

hipError_t launch_append_last(const DecodeParams &a, hipStream_t stream) {
  const int64_t threads = (int64_t)a.S * a.Hkv * (a.D / 8);
  if (threads == 0) return hipSuccess;
  const int64_t grid = (threads + 255) / 256;
  hipLaunchKernelGGL(append_last_kernel, dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

int64_t copy_blocks_workgroups(int64_t num_pairs, int32_t Hkv, int32_t B, int32_t D) {
  const int64_t pieces = (int64_t)Hkv * B * D / 8;
  return num_pairs * ((pieces + kCopyThreads * kCopyUnroll - 1) / (kCopyThreads * kCopyUnroll));
}

hipError_t launch_copy_blocks(void *k_pool, void *v_pool, const int64_t *pairs, int32_t n,
                              int32_t Hkv, int32_t B, int32_t D, int64_t num_blocks,
                              hipStream_t stream) {
  const int64_t pieces = (int64_t)Hkv * B * D / 8;
  const int64_t grid = copy_blocks_workgroups(n, Hkv, B, D);
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  const uint32_t per_pair = (uint32_t)(grid / n);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)grid), dim3(kCopyThreads), 0, stream,
                     reinterpret_cast<uint16_t *>(k_pool), reinterpret_cast<uint16_t *>(v_pool), pairs,
                     pieces, per_pair, num_blocks);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache(void *k_pool, void *v_pool, const void *k, const void *v,
                                    int64_t k_stride, int64_t v_stride, const int64_t *slots,
                                    int32_t T, int32_t Hkv, int32_t B, int32_t D,
                                    int64_t num_blocks, hipStream_t stream) {
  const int64_t threads = (int64_t)T * Hkv * (D / 8);
  if (threads == 0) return hipSuccess;
  const int64_t grid = (threads + 255) / 256;
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                     reinterpret_cast<uint16_t *>(k_pool), reinterpret_cast<uint16_t *>(v_pool),
                     reinterpret_cast<const uint16_t *>(k), reinterpret_cast<const uint16_t *>(v),
                     k_stride, v_stride, slots, T, Hkv, B, D, num_blocks);
  return hipGetLastError();
}

hipError_t launch_slot_mapping(int64_t *slots, const int32_t *tables, int32_t S, int32_t maxb,
                               const int32_t *seq, const int32_t *pos, int32_t T, int32_t B,
                               int64_t num_blocks, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int grid = (T + 255) / 256;
  hipLaunchKernelGGL(slot_mapping_kernel, dim3(grid), dim3(256), 0, stream, slots, tables, S,
                     maxb, seq, pos, T, B, num_blocks);
  return hipGetLastError();
}

}  // namespace pkv
