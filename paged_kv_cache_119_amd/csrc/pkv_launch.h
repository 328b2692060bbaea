// Internal launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Largest number of table entries one partition stages in LDS.
constexpr int kTabMax = 512;
// Consecutive logical work items kept on one XCD.
constexpr int kXcdGroup = 16;

struct DecodeParams {
  void *out;               // [S][H][D] 16-bit
  const void *q;           // [S][H][D] 16-bit
  const void *k_pool;      // [N][Hkv][B][D]
  const void *v_pool;
  const int32_t *tables;   // [S][maxb]
  const int32_t *lens;     // [S]
  float *ws_m;             // [S*H*MP]
  float *ws_l;             // [S*H*MP]
  float *ws_o;             // [S*H*MP*D]
  float scale_log2;        // scale * log2(e)
  int64_t num_blocks;      // N
  int32_t S, H, Hkv, maxb, B, D, P, MP;
  int32_t items;           // S * H * MP
  int32_t dtype;
};

// Number of waves per workgroup of the partition pass.
int decode_waves();

hipError_t launch_decode_partitions(const DecodeParams &a, hipStream_t stream);
hipError_t launch_decode_merge(const DecodeParams &a, hipStream_t stream);

hipError_t launch_reshape_and_cache(void *k_pool, void *v_pool, const void *k, const void *v,
                                    int64_t k_stride, int64_t v_stride, const int64_t *slots,
                                    int32_t T, int32_t Hkv, int32_t B, int32_t D,
                                    int64_t num_blocks, hipStream_t stream);

hipError_t launch_slot_mapping(int64_t *slots, const int32_t *tables, int32_t S, int32_t maxb,
                               const int32_t *seq, const int32_t *pos, int32_t T, int32_t B,
                               int64_t num_blocks, hipStream_t stream);

}  // namespace pkv
