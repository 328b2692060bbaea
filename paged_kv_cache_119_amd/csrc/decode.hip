// Paged decode attention for gfx950: partition pass + log-sum-exp merge pass.
//
// What is computed ("PagedAttention 完全拆解", 背景 attention equation and
// 原理详解（二） blockwise form): for each sequence s and head h,
//   o = sum_j exp(z_j - m) v_j / sum_j exp(z_j - m),   z_j = scale * q . k_j,
// over the sequence's logical tokens j < L, with k_j and v_j found through the
// block table.  Long contexts are cut into partitions of P tokens whose
// partial results are merged afterwards (iaim.asia block-table article,
// "vLLM 内核里的缓解写法": segments in parallel, then a reduction).
//
// Mapping to CDNA4 (this is our design, not the pages' warp-per-block one):
//  * One workgroup of NW wavefronts per (sequence, head, partition).  The
//    partition's table entries are staged in LDS with one coalesced load;
//    waves then read the (wave-uniform) block id from LDS, so the pool address
//    base lives in scalar registers.
//  * A wavefront step ("chunk") covers TC tokens: NL = 4 loads of 16 bytes per
//    lane from K and 4 from V.  With the [N][Hkv][B][D] layout a load
//    instruction reads 1 KiB of consecutive bytes (TPI whole token rows of one
//    block), so every load is fully coalesced however blocks are scattered.
//  * LPT = D / 8 lanes hold one token's row (8 elements each); the q.k partial
//    sums of those lanes are reduced with DPP inside the 16-lane row.  The TPI
//    token rows of a load stay in separate lane groups, and each group keeps
//    its own online-softmax state (running max m, sum l, 8 accumulators per
//    lane), so the hot loop has no cross-group traffic at all.  Groups and
//    waves are merged once at the end, by the same log-sum-exp rule.
//  * Chunks go round-robin over the waves; each wave double-buffers its
//    chunks (the loads of chunk c + NW are issued before chunk c is consumed).
//  * exp2 runs on v_exp_f32 with log2(e) folded into the scale.
//  * Unused slots of the last block are selected out (score -inf, V term
//    skipped), never multiplied by zero, so NaN in them cannot leak.
//  * The accumulation order depends only on logical positions, so results are
//    bitwise independent of where blocks sit in the pool.

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

namespace {

// Wavefronts per workgroup of the partition pass (build-time setting).
#ifndef PKV_DECODE_WAVES
#define PKV_DECODE_WAVES 4
#endif
constexpr int kNumWaves = PKV_DECODE_WAVES;
// 16-byte loads per lane per tensor in one wavefront step (build-time setting).
#ifndef PKV_DECODE_LOADS
#define PKV_DECODE_LOADS 4
#endif

template <int DT, int D, int B, int NW>
__global__ __launch_bounds__(NW * 64) void decode_partition_kernel(DecodeParams a) {
  constexpr int LPT = D / 8;    // lanes per token row
  constexpr int TPI = 64 / LPT; // token rows per load instruction
  constexpr int NL = PKV_DECODE_LOADS;  // load instructions per tensor per chunk
  constexpr int TC = NL * TPI;  // tokens per chunk
  static_assert(B % TPI == 0, "a load must not straddle two blocks");

  __shared__ int32_t s_tab[kTabMax];
  __shared__ float s_m[NW];
  __shared__ float s_l[NW];
  __shared__ float s_o[NW][D];

  const int item = xcd_remap<kXcdGroup>(blockIdx.x);
  if (item >= a.items) return;
  // logical order: sequence fastest, then head, then partition (last first)
  const int s = item % a.S;
  const int rest = item / a.S;
  const int h = rest % a.H;
  const int p = a.MP - 1 - rest / a.H;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int L = a.lens[s];
  uint16_t *out_row = reinterpret_cast<uint16_t *>(a.out) + ((int64_t)s * a.H + h) * D;

  if (L <= 0 || L > a.maxb * B) {
    // empty context -> zeros; invalid length -> NaN (written once, by p == 0)
    if (p == 0) {
      const uint16_t v = (L == 0) ? uint16_t(0) : to16<DT>(__builtin_nanf(""));
      for (int d = tid; d < D; d += NW * 64) out_row[d] = v;
    }
    return;
  }
  const int nparts = (L + a.P - 1) / a.P;
  if (p >= nparts) return;
  const int tok0 = p * a.P;
  const int n = min(a.P, L - tok0);  // tokens of this partition
  const int nblk = (n + B - 1) / B;

  // Stage this partition's table entries in LDS (one coalesced read).
  const int32_t *trow = a.tables + (int64_t)s * a.maxb + tok0 / B;
  for (int i = tid; i < nblk; i += NW * 64) s_tab[i] = trow[i];
  __syncthreads();

  const uint16_t *kp = reinterpret_cast<const uint16_t *>(a.k_pool);
  const uint16_t *vp = reinterpret_cast<const uint16_t *>(a.v_pool);
  const int64_t blk_stride = (int64_t)a.Hkv * B * D;  // elements per pool block
  const int64_t head_base = (int64_t)h * B * D;       // scalar part of the tile offset
  const int lane_off = lane * 8;                       // this lane's 8 elements
  const int row = lane / LPT;

  const u32x4 qv = *reinterpret_cast<const u32x4 *>(
      reinterpret_cast<const uint16_t *>(a.q) + ((int64_t)s * a.H + h) * D + (lane % LPT) * 8);

  bool bad = false;
  float m = kNegInf;
  float l = 0.f;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;

  // Issue the 2 * NL loads of chunk c.  Every address is a scalar base (block
  // id from LDS, moved to a scalar register) plus this lane's 16-byte offset.
  auto load_chunk = [&](int c, u32x4 (&kr)[NL], u32x4 (&vr)[NL]) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      int lb, off;
      if constexpr (TC >= B) {  // a chunk covers TC / B whole blocks
        lb = c * (TC / B) + (i * TPI) / B;
        off = (i * TPI) % B;
      } else {                  // a block holds B / TC chunks
        lb = c / (B / TC);
        off = (c % (B / TC)) * TC + i * TPI;
      }
      lb = min(lb, nblk - 1);   // tail loads stay inside the last block
      int blk = __builtin_amdgcn_readfirstlane(s_tab[lb]);
      if (blk < 0 || (int64_t)blk >= a.num_blocks) {
        bad = true;
        blk = 0;
      }
      const int64_t base = (int64_t)blk * blk_stride + head_base + off * D;
      kr[i] = *reinterpret_cast<const u32x4 *>(kp + base + lane_off);
      vr[i] = *reinterpret_cast<const u32x4 *>(vp + base + lane_off);
    }
  };

  // Fold chunk c into this lane group's online softmax.  Branch-free: rows at
  // or past n get score -inf and a zeroed V row (selected, never multiplied),
  // so the poison in unused slots cannot leak.
  auto consume = [&](int c, u32x4 (&kr)[NL], u32x4 (&vr)[NL]) {
    float z[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const bool valid = (c * TC + i * TPI + row) < n;
      const float d = group_sum<LPT>(dot8<DT>(qv, kr[i])) * a.scale_log2;
      z[i] = valid ? d : kNegInf;
      const u32x4 zero = {0u, 0u, 0u, 0u};
      vr[i] = valid ? vr[i] : zero;
    }
    float mx = z[0];
#pragma unroll
    for (int i = 1; i < NL; ++i) mx = fmaxf(mx, z[i]);
    const float mnew = fmaxf(m, mx);
    const float mref = (mnew == kNegInf) ? 0.f : mnew;  // no valid token yet
    const float alpha = fast_exp2(m - mref);             // m == -inf gives 0
    float pz[NL];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      pz[i] = fast_exp2(z[i] - mref);  // -inf gives 0
      psum += pz[i];
    }
    l = l * alpha + psum;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= alpha;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const uint32_t w[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] = fmaf(pz[i], lo16<DT>(w[j]), acc[2 * j]);
        acc[2 * j + 1] = fmaf(pz[i], hi16<DT>(w[j]), acc[2 * j + 1]);
      }
    }
    m = mnew;
  };

  // This wave's chunks are c_k = wave + k * NW, k < my_n; two are in flight at
  // a time.  The loop body always runs both halves and has a single back
  // edge, so the same loads are outstanding on every path into it and the
  // wait before each consume leaves the other chunk's 2 * NL loads in flight.
  const int nch = (n + TC - 1) / TC;
  if (wave < nch) {
    const int my_n = (nch - wave + NW - 1) / NW;
    u32x4 ka[NL], va[NL], kb[NL], vb[NL];
    load_chunk(wave, ka, va);
    int k = 0;
    for (; k + 2 < my_n; k += 2) {
      const int c = wave + k * NW;
      load_chunk(c + NW, kb, vb);
      // keep the prefetch ahead of the consume (the scheduler would sink it)
      __builtin_amdgcn_sched_barrier(0);
      consume(c, ka, va);
      load_chunk(c + 2 * NW, ka, va);
      __builtin_amdgcn_sched_barrier(0);
      consume(c + NW, kb, vb);
    }
    const int c = wave + k * NW;
    if (k + 1 < my_n) {
      load_chunk(c + NW, kb, vb);
      __builtin_amdgcn_sched_barrier(0);
      consume(c, ka, va);
      consume(c + NW, kb, vb);
    } else {
      consume(c, ka, va);
    }
  }

  // Merge the lane groups of this wave (same dims, different tokens).
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(m, off);
    const float l2 = __shfl_xor(l, off);
    const float mm = fmaxf(m, m2);
    const float f1 = (m == kNegInf) ? 0.f : fast_exp2(m - mm);
    const float f2 = (m2 == kNegInf) ? 0.f : fast_exp2(m2 - mm);
    l = l * f1 + l2 * f2;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float o2 = __shfl_xor(acc[j], off);
      acc[j] = acc[j] * f1 + o2 * f2;
    }
    m = mm;
  }
  if (lane < LPT) {
#pragma unroll
    for (int j = 0; j < 8; ++j) s_o[wave][lane * 8 + j] = acc[j];
    if (lane == 0) {
      s_m[wave] = m;
      s_l[wave] = l;
    }
  }
  const int any_bad = __syncthreads_or(bad ? 1 : 0);

  // Merge the waves; thread d owns output dimension d.
  for (int d = tid; d < D; d += NW * 64) {
    float M = s_m[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_m[w]);
    float lsum = 0.f;
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = (s_m[w] == kNegInf) ? 0.f : fast_exp2(s_m[w] - M);
      lsum += f * s_l[w];
      o += f * s_o[w][d];
    }
    if (any_bad) {
      M = __builtin_nanf("");
      lsum = __builtin_nanf("");
      o = __builtin_nanf("");
    }
    if (nparts == 1) {
      out_row[d] = to16<DT>(o / lsum);
    } else {
      const int64_t u = ((int64_t)s * a.H + h) * a.MP + p;
      a.ws_o[u * D + d] = o;
      if (d == 0) {
        a.ws_m[u] = M * kLn2;  // back to natural-log units
        a.ws_l[u] = lsum;
      }
    }
  }
}

template <int DT, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeParams a) {
  const int sh = blockIdx.x;  // s * H + h
  const int s = sh / a.H;
  const int L = a.lens[s];
  if (L <= 0 || L > a.maxb * a.B) return;
  const int n = (L + a.P - 1) / a.P;
  if (n < 2) return;
  const int64_t u0 = (int64_t)sh * a.MP;
  const float *mp = a.ws_m + u0;
  const float *lp = a.ws_l + u0;
  float M = mp[0];
  for (int p = 1; p < n; ++p) M = fmaxf(M, mp[p]);
  float lsum = 0.f;
  for (int p = 0; p < n; ++p) lsum += fast_exp2((mp[p] - M) * kLog2e) * lp[p];
  uint16_t *out_row = reinterpret_cast<uint16_t *>(a.out) + (int64_t)sh * D;
  for (int d = threadIdx.x; d < D; d += 64) {
    float o = 0.f;
    for (int p = 0; p < n; ++p) o += fast_exp2((mp[p] - M) * kLog2e) * a.ws_o[(u0 + p) * D + d];
    out_row[d] = to16<DT>(o / lsum);
  }
}

template <int DT, int D, int B>
hipError_t launch_partitions_t(const DecodeParams &a, hipStream_t stream) {
  const int group = 8 * kXcdGroup;
  const int grid = ((a.items + group - 1) / group) * group;
  hipLaunchKernelGGL((decode_partition_kernel<DT, D, B, kNumWaves>), dim3(grid),
                     dim3(kNumWaves * 64), 0, stream, a);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_partitions_b(const DecodeParams &a, hipStream_t stream) {
  switch (a.B) {
    case 8: return launch_partitions_t<DT, D, 8>(a, stream);
    case 16: return launch_partitions_t<DT, D, 16>(a, stream);
    case 32: return launch_partitions_t<DT, D, 32>(a, stream);
    case 64: return launch_partitions_t<DT, D, 64>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int decode_waves() { return kNumWaves; }

hipError_t launch_decode_partitions(const DecodeParams &a, hipStream_t stream) {
  if (a.items == 0) return hipSuccess;
  if (a.dtype == DT_F16) {
    if (a.D == 64) return launch_partitions_b<DT_F16, 64>(a, stream);
    if (a.D == 128) return launch_partitions_b<DT_F16, 128>(a, stream);
  } else {
    if (a.D == 64) return launch_partitions_b<DT_BF16, 64>(a, stream);
    if (a.D == 128) return launch_partitions_b<DT_BF16, 128>(a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_merge(const DecodeParams &a, hipStream_t stream) {
  const int grid = a.S * a.H;
  if (grid == 0 || a.MP < 2) return hipSuccess;
#define PKV_MERGE(DT, DD) \
  hipLaunchKernelGGL((decode_merge_kernel<DT, DD>), dim3(grid), dim3(64), 0, stream, a)
  if (a.dtype == DT_F16) {
    if (a.D == 64) PKV_MERGE(DT_F16, 64);
    else PKV_MERGE(DT_F16, 128);
  } else {
    if (a.D == 64) PKV_MERGE(DT_BF16, 64);
    else PKV_MERGE(DT_BF16, 128);
  }
#undef PKV_MERGE
  return hipGetLastError();
}

}  // namespace pkv
