// Paged decode attention for gfx950: split-context pass + log-sum-exp merge.
//
// What is computed ("PagedAttention 完全拆解", 背景 attention equation and
// 原理详解（二） blockwise form): for each sequence s and head h,
//   o = sum_j exp(z_j - m) v_j / sum_j exp(z_j - m),   z_j = scale * q . k_j,
// over the sequence's logical tokens j < L, with k_j and v_j found through the
// block table.  The context is cut into pieces processed in parallel whose
// partial results are merged afterwards (iaim.asia block-table article,
// "vLLM 内核里的缓解写法": segments in parallel, then a reduction).
//
// Two ways of cutting:
//  * Fixed partitions (partition_size P > 0): one workgroup of NW wavefronts
//    per (sequence, head, partition of P tokens); the partition's table
//    entries are staged in LDS once and the waves take chunks round-robin
//    (WaveAttn below).
//  * Work-balanced (partition_size 0): all chunks of the batch are cut into
//    equal slices, one per wavefront; each wavefront runs its slice as one
//    pipelined stream of chunks (Stream below).
//
// Inner engine of the fixed partitions (WaveAttn), per wavefront:
//  * A "chunk" covers TC tokens: NL loads of 16 bytes per lane from K and NL
//    from V.  With the [N][Hkv][B][D] pool layout one load instruction reads
//    1 KiB of consecutive bytes (TPI whole token rows of one block), so every
//    load is fully coalesced however the blocks are scattered.  Each address
//    is a scalar tile base (block id read from LDS, moved to a scalar
//    register) plus the lane's 16-byte offset.
//  * LPT = D / 8 lanes hold one token row (8 elements each); the q.k partial
//    sums of those lanes are reduced with DPP inside the 16-lane row.  The TPI
//    token rows of a load stay in separate lane groups, each with its own
//    online softmax (running max m, sum l, 8 accumulators per lane), so the
//    hot loop has no other cross-lane traffic.  Groups are merged once at the
//    end by the log-sum-exp rule.
//  * Chunks are double-buffered: the loads of the next chunk are issued before
//    the current one is consumed (a counted loop with one back edge keeps the
//    compiler's wait at exactly one chunk outstanding).
//  * exp2 runs on v_exp_f32 with log2(e) folded into the scale.
//  * Tokens outside the piece (the unused tail of a last block included) are
//    selected out -- score -inf, V row zeroed -- never multiplied by zero, so
//    NaN in unused slots cannot leak.
//  * The accumulation order depends only on logical positions, so results are
//    bitwise independent of where blocks sit in the pool.
//
// Both ways read K/V with non-temporal loads (each row is read once per call)
// unless the pool carries the reuse hint (blocks shared between sequences,
// whose later readers can then hit the last-level cache).  The load policy
// never changes a result bit.

#include <type_traits>

#include "pkv_device.h"
#include "pkv_launch.h"
#include "pkv_split.h"

namespace pkv {

namespace {

constexpr int kNumWaves = PKV_DECODE_WAVES;

template <int D>
struct Geo {
  static constexpr int LPT = D / 8;          // lanes per token row
  static constexpr int TPI = 64 / LPT;       // token rows per load instruction
  static constexpr int NL = kDecodeLoads;    // loads per tensor per chunk
  static constexpr int TC = NL * TPI;        // tokens per chunk
};

// One wavefront's online softmax over part of one (sequence, head).  NT:
// K/V rows are read with non-temporal loads.
template <int DT, int D, int B, bool NT>
struct WaveAttn {
  using G = Geo<D>;
  static constexpr int LPT = G::LPT, TPI = G::TPI, NL = G::NL, TC = G::TC;
  static_assert(B % TPI == 0, "a load must not straddle two blocks");

  const uint16_t *kp;
  const uint16_t *vp;
  int64_t blk_stride;   // elements per pool block (all heads)
  int64_t head_base;    // offset of this head's tile inside a block
  int64_t num_blocks;
  float scale_log2;
  int lane_off;         // this lane's 8 elements inside a 1 KiB load
  int row;              // lane group (token row of a load)
  u32x4 qv;
  bool bad;
  float m, l;
  float acc[8];
  // fused append: chunk and token holding the new row (-1: none), its data
  int app_c;
  int app_tok;
  u32x4 kn, vn;

  __device__ __forceinline__ void init(const DecodeParams &a, int s, int h, int lane) {
    kp = reinterpret_cast<const uint16_t *>(a.k_pool);
    vp = reinterpret_cast<const uint16_t *>(a.v_pool);
    blk_stride = (int64_t)a.Hkv * B * D;
    head_base = (int64_t)h * B * D;
    num_blocks = a.num_blocks;
    scale_log2 = a.scale_log2;
    lane_off = lane * 8;
    row = lane / LPT;
    qv = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(a.q) +
                                          ((int64_t)s * a.H + h) * D + (lane % LPT) * 8);
    bad = false;
    m = kNegInf;
    l = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.f;
    app_c = -1;
    app_tok = -1;
  }

  // Take token L - 1's K/V row from the new-token inputs (fused append).
  __device__ __forceinline__ void set_append(const DecodeParams &a, int s, int h, int L, int lane) {
    app_tok = L - 1;
    app_c = app_tok / TC;
    const int64_t e = (int64_t)s * a.new_stride + (int64_t)h * D + (lane % LPT) * 8;
    kn = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(a.k_new) + e);
    vn = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(a.v_new) + e);
  }

  // Write the new row to its pool slot (the lanes of its token row); `blk` is
  // the table entry of logical block app_tok / B.
  __device__ __forceinline__ void write_append(const DecodeParams &a, int blk) {
    if (blk < 0 || (int64_t)blk >= num_blocks) {
      bad = true;
      return;
    }
    if (row != (app_tok % TPI)) return;
    const int64_t base = (int64_t)blk * blk_stride + head_base + (app_tok % B) * D;
    uint16_t *kw = const_cast<uint16_t *>(kp) + base + (lane_off % (LPT * 8));
    uint16_t *vw = const_cast<uint16_t *>(vp) + base + (lane_off % (LPT * 8));
    *reinterpret_cast<u32x4 *>(kw) = kn;
    *reinterpret_cast<u32x4 *>(vw) = vn;
  }

  // Issue the 2 * NL loads of chunk c (tokens c*TC .. c*TC+TC-1 of the
  // sequence).  `tab` holds the table entries of logical blocks tab_base ..;
  // logical blocks past lb_max are clamped to it (their tokens are masked).
  __device__ __forceinline__ void load(int c, const int32_t *tab, int tab_base, int lb_max,
                                       u32x4 (&kr)[NL], u32x4 (&vr)[NL]) {
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
      lb = min(lb, lb_max);
      int blk = __builtin_amdgcn_readfirstlane(tab[lb - tab_base]);
      if (blk < 0 || (int64_t)blk >= num_blocks) {
        bad = true;
        blk = 0;
      }
      const int64_t base = (int64_t)blk * blk_stride + head_base + off * D;
      kr[i] = ld_kv<NT>(kp + base + lane_off);
      vr[i] = ld_kv<NT>(vp + base + lane_off);
    }
  }

  // Fold chunk c into this lane group's online softmax; tokens outside
  // [t_lo, t_hi) are selected out.  Branch-free.
  __device__ __forceinline__ void consume(int c, int t_lo, int t_hi, u32x4 (&kr)[NL],
                                          u32x4 (&vr)[NL]) {
    if (c == app_c) {  // the chunk holding the appended token: use the new row
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const bool sub = (c * TC + i * TPI + row) == app_tok;
        kr[i] = sub ? kn : kr[i];
        vr[i] = sub ? vn : vr[i];
      }
    }
    float z[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int tok = c * TC + i * TPI + row;
      const bool valid = tok >= t_lo && tok < t_hi;
      const float d = group_sum<LPT>(dot8<DT>(qv, kr[i])) * scale_log2;
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
  }

  // Chunks c0, c0 + stride, ... (count of them), two in flight.  The loop
  // body always runs both halves and has a single back edge, so the same loads
  // are outstanding on every path into it and the wait before each consume
  // leaves the other chunk's 2 * NL loads in flight.
  __device__ __forceinline__ void run(int c0, int stride, int count, const int32_t *tab,
                                      int tab_base, int lb_max, int t_lo, int t_hi) {
    if (count <= 0) return;
    u32x4 ka[NL], va[NL], kb[NL], vb[NL];
    load(c0, tab, tab_base, lb_max, ka, va);
    int k = 0;
    for (; k + 2 < count; k += 2) {
      const int c = c0 + k * stride;
      load(c + stride, tab, tab_base, lb_max, kb, vb);
      // keep the prefetch ahead of the consume (the scheduler would sink it)
      __builtin_amdgcn_sched_barrier(0);
      consume(c, t_lo, t_hi, ka, va);
      load(c + 2 * stride, tab, tab_base, lb_max, ka, va);
      __builtin_amdgcn_sched_barrier(0);
      consume(c + stride, t_lo, t_hi, kb, vb);
    }
    const int c = c0 + k * stride;
    if (k + 1 < count) {
      load(c + stride, tab, tab_base, lb_max, kb, vb);
      __builtin_amdgcn_sched_barrier(0);
      consume(c, t_lo, t_hi, ka, va);
      consume(c + stride, t_lo, t_hi, kb, vb);
    } else {
      consume(c, t_lo, t_hi, ka, va);
    }
  }

  // Merge the lane groups (same dims, different tokens); afterwards every lane
  // group holds the wave's (m, l, acc).
  __device__ __forceinline__ void merge_groups() {
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
  }
};

// ---------------------------------------------------------------------------
// Fixed partitions
// ---------------------------------------------------------------------------

template <int DT, int D, int B, int NW, bool NT>
__global__ __launch_bounds__(NW * 64) void decode_partition_kernel(DecodeParams a) {
  using WA = WaveAttn<DT, D, B, NT>;
  constexpr int TC = WA::TC;

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
  const int t_hi = min(tok0 + a.P, L);
  const int lb0 = tok0 / B;
  const int lb_max = (t_hi - 1) / B;

  // Stage this partition's table entries in LDS (one coalesced read).
  const int32_t *trow = a.tables + (int64_t)s * a.maxb + lb0;
  for (int i = tid; i <= lb_max - lb0; i += NW * 64) s_tab[i] = trow[i];
  __syncthreads();

  WA wa;
  wa.init(a, s, h, lane);
  const int c_first = tok0 / TC;
  const int nch = (t_hi - tok0 + TC - 1) / TC;
  const bool app = a.append && t_hi == L;  // this partition holds token L - 1
  if (app) wa.set_append(a, s, h, L, lane);
  if (wave < nch) {
    const int my_n = (nch - wave + NW - 1) / NW;
    wa.run(c_first + wave, NW, my_n, s_tab, lb0, lb_max, tok0, t_hi);
  }
  if (app && wave == 0) wa.write_append(a, __builtin_amdgcn_readfirstlane(s_tab[(L - 1) / B - lb0]));
  wa.merge_groups();

  if (lane < WA::LPT) {
#pragma unroll
    for (int j = 0; j < 8; ++j) s_o[wave][lane * 8 + j] = wa.acc[j];
    if (lane == 0) {
      s_m[wave] = wa.m;
      s_l[wave] = wa.l;
    }
  }
  const int any_bad = __syncthreads_or(wa.bad ? 1 : 0);

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
  const int lane = threadIdx.x;
  const int64_t u0 = (int64_t)sh * a.MP;
  const float *mp = a.ws_m + u0;
  const float *lp = a.ws_l + u0;
  // the partitions' maximum: 64 partitions per round of loads, then the wave
  float M = kNegInf;
  for (int p0 = 0; p0 < n; p0 += 64)
    if (p0 + lane < n) M = fmaxf(M, mp[p0 + lane]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  // each partition's weight, computed by one lane and read back by all,
  // then both sums in partition order (the o rows fetched 8 partitions a
  // round; each lane holds dims lane and lane + 64)
  constexpr int NDL = D / 64;
  float lsum = 0.f, o[NDL];
#pragma unroll
  for (int k = 0; k < NDL; ++k) o[k] = 0.f;
  for (int p0 = 0; p0 < n; p0 += 64) {
    const int pl = p0 + lane < n ? p0 + lane : n - 1;
    const float f = fast_exp2((mp[pl] - M) * kLog2e);
    const float fl = f * lp[pl];
    const int cnt = min(64, n - p0);
    int q0 = 0;
    for (; q0 + 8 <= cnt; q0 += 8) {  // whole batches: all 8 rows' loads, then the sums
      float ov[8][NDL];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
#pragma unroll
        for (int k = 0; k < NDL; ++k) ov[q][k] = a.ws_o[(u0 + p0 + q0 + q) * D + 64 * k + lane];
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float fq = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), q0 + q));
        lsum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fl), q0 + q));
#pragma unroll
        for (int k = 0; k < NDL; ++k) o[k] += fq * ov[q][k];
      }
    }
    for (; q0 < cnt; ++q0) {  // the rest, one by one
      const float fq = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), q0));
      lsum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fl), q0));
#pragma unroll
      for (int k = 0; k < NDL; ++k) o[k] += fq * a.ws_o[(u0 + p0 + q0) * D + 64 * k + lane];
    }
  }
  uint16_t *out_row = reinterpret_cast<uint16_t *>(a.out) + (int64_t)sh * D;
#pragma unroll
  for (int k = 0; k < NDL; ++k) out_row[64 * k + lane] = to16<DT>(o[k] / lsum);
}

// ---------------------------------------------------------------------------
// Work-balanced split
// ---------------------------------------------------------------------------
//
// Work is counted in chunks: the cost space [0, total) lists the chunks of
// every (sequence, head) row, rows in order (sequence major), where a row
// with L valid tokens has ceil(L / TC) chunks.  It is cut into equal slices,
// one per worker wavefront w.  The part of a row a slice covers is a
// "piece".  A piece that is the whole row writes the output row; any other
// writes a partial result to slot w + g (workers and rows both advance along
// the cost space, so the slot is unique) and the merge launch combines a
// row's partials in worker order.
//
// A wavefront runs its slice as one stream of chunks through three stages --
// table entries of chunk n + 2, K/V rows of chunk n + 1, arithmetic on chunk
// n -- so piece and row boundaries cost no exposed memory latency.  Every
// step issues the same loads (after the last chunk they repeat it and hit
// the cache), so the compiler's waits stay exact; the one exception, the new
// rows of the fused append, are loaded only with the chunk of token L - 1 and
// at worst make the wait before the next consume a little stricter.  A
// wavefront lowers its
// priority as it progresses through its slice, so wavefronts that share a
// SIMD finish together instead of in order of age.

// PFX: the suffix pass of the shared-prefix decode -- a row covers tokens
// t0 .. L - 1 and, when t0 > 0, starts from the softmax state the prefix pass
// left for it (lane group 0 takes it; the other groups start empty).
template <int DT, int D, int B, bool APP, bool NT, bool PFX = false>
struct Stream {
  using G = Geo<D>;
  static constexpr int LPT = G::LPT, TPI = G::TPI, NL = G::NL, TC = G::TC;
  static constexpr int NE = TC >= B ? TC / B : 1;  // table entries per chunk
  static_assert(B % TPI == 0, "a load must not straddle two blocks");

  struct PfxState {
    float m, l;
    u32x4 o0, o1;  // 8 float32 sums as bits
  };
  struct NoState {};
  struct Buf {
    u32x4 k[NL], v[NL];
    u32x4 q, kn, vn;
    int app_blk;
    bool bad;
    typename std::conditional<PFX, PfxState, NoState>::type ps;
  };

  // constants of the call
  const uint16_t *kp;
  const uint16_t *vp;
  const uint16_t *qp;
  const uint16_t *knp;
  const uint16_t *vnp;
  const int32_t *tables;
  uint16_t *outp;
  float *ws_m;
  float *ws_l;
  float *ws_o;
  int64_t blk_stride, num_blocks, new_stride;
  int S, H, maxb;
  float scale_log2;
  int lane, lane_off, row, qoff;
  int64_t worker;
  ChunkCursor<TC, PFX> cur;  // the slice, chunk by chunk
  const float *pfx_m;
  const float *pfx_l;
  const float *pfx_o;
  // running state of the current piece
  u32x4 qv;
  float m, l, acc[8];
  bool bad;
  bool store_new;  // fused append: write the new rows here (else the merge launch does)

  __device__ __forceinline__ void init(const DecodeParams &a, const int64_t *cum_, const int32_t *lens_,
                                       int lane_, const int32_t *starts_ = nullptr) {
    store_new = a.append_in_merge == 0;
    pfx_m = a.pfx_m;
    pfx_l = a.pfx_l;
    pfx_o = a.pfx_o;
    kp = reinterpret_cast<const uint16_t *>(a.k_pool);
    vp = reinterpret_cast<const uint16_t *>(a.v_pool);
    qp = reinterpret_cast<const uint16_t *>(a.q);
    knp = reinterpret_cast<const uint16_t *>(a.k_new);
    vnp = reinterpret_cast<const uint16_t *>(a.v_new);
    tables = a.tables;
    outp = reinterpret_cast<uint16_t *>(a.out);
    ws_m = a.ws_m;
    ws_l = a.ws_l;
    ws_o = a.ws_o;
    cur.init(cum_, lens_, a.S, a.H, lane_, starts_, a.maxb, a.B);
    blk_stride = (int64_t)a.Hkv * B * D;
    num_blocks = a.num_blocks;
    new_stride = a.new_stride;
    S = a.S;
    H = a.H;
    maxb = a.maxb;
    scale_log2 = a.scale_log2;
    lane = lane_;
    lane_off = lane * 8;
    row = lane / LPT;
    qoff = (lane % LPT) * 8;
  }

  __device__ __forceinline__ static int first_block(int c) { return TC >= B ? c * (TC / B) : c / (B / TC); }
  __device__ __forceinline__ static int last_block(const Chunk &d) { return (min(d.L, d.ce * TC) - 1) / B; }
  __device__ __forceinline__ static bool is_app_chunk(const Chunk &d) {
    return d.c == d.ce - 1 && d.ce * TC >= d.L;  // the chunk of token L - 1
  }

  // Stage 1: this lane's table entry of chunk d (entries past the piece's
  // last block are clamped to it; their tokens are masked).
  __device__ __forceinline__ uint32_t load_entries(const Chunk &d) const {
    const int lb = min(first_block(d.c) + min(lane, NE - 1), last_block(d));
    return (uint32_t)tables[(int64_t)d.s * maxb + lb];
  }

  // Stage 2: the K/V rows of chunk d, its query row and (fused append) the
  // new-token rows of its row.  Lanes of tokens past the context read the
  // row of token L - 1 instead (same cache lines as a valid row: the unused
  // tail of the last block costs no HBM traffic); their values are masked.
  __device__ __forceinline__ void load_kv(const Chunk &d, uint32_t e, Buf &b) const {
    const int64_t head_base = (int64_t)d.h * B * D;
    const int tail_off = ((d.L - 1) % B) * D + qoff;
    bool bd = false;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      int ei, off;
      if constexpr (TC >= B) {
        ei = (i * TPI) / B;
        off = (i * TPI) % B;
      } else {
        ei = 0;
        off = (d.c % (B / TC)) * TC + i * TPI;
      }
      int blk = __builtin_amdgcn_readlane((int)e, ei);
      if (blk < 0 || (int64_t)blk >= num_blocks) {
        bd = true;
        blk = 0;
      }
      const int64_t base = (int64_t)blk * blk_stride + head_base;
      const int lo = (d.c * TC + i * TPI + row < d.L) ? off * D + lane_off : tail_off;
      b.k[i] = ld_kv<NT>(kp + base + lo);
      b.v[i] = ld_kv<NT>(vp + base + lo);
    }
    b.bad = bd;
    // Issued for every chunk (an L2 hit after the first), so every chunk
    // issues the same loads.
    b.q = *reinterpret_cast<const u32x4 *>(qp + ((int64_t)d.s * H + d.h) * D + qoff);
    if constexpr (PFX) {
      // the prefix state of the row, with the row's first chunk
      if (d.c == d.c0 && d.t0 > 0) {
        const int64_t g = (int64_t)d.s * H + d.h;
        b.ps.m = pfx_m[g];
        b.ps.l = pfx_l[g];
        const u32x4 *po = reinterpret_cast<const u32x4 *>(pfx_o + g * D + qoff);
        b.ps.o0 = po[0];
        b.ps.o1 = po[1];
      }
    }
    if constexpr (APP) {
      // only the chunk of token L - 1 (once per row) loads the new rows
      if (is_app_chunk(d)) {
        const int64_t ne = (int64_t)d.s * new_stride + (int64_t)d.h * D + qoff;
        b.kn = *reinterpret_cast<const u32x4 *>(knp + ne);
        b.vn = *reinterpret_cast<const u32x4 *>(vnp + ne);
        const int ei = TC >= B ? min(NE - 1, max(0, (d.L - 1) / B - first_block(d.c))) : 0;
        b.app_blk = __builtin_amdgcn_readlane((int)e, ei);
      }
    }
  }

  // Stage 3: fold chunk d into the piece's online softmax; tokens outside the
  // piece are selected out (score -inf, V row zeroed).
  __device__ __forceinline__ void consume(const Chunk &d, Buf &b) {
    if (d.c == d.cb) {
      qv = b.q;
      m = kNegInf;
      l = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = 0.f;
      bad = false;
      if constexpr (PFX) {
        bad = d.t0 > d.L;  // the group's prefix is longer than this sequence
        if (d.c == d.c0 && d.t0 > 0 && row == 0) {
          m = b.ps.m;
          l = b.ps.l;
          const uint32_t w[8] = {b.ps.o0.x, b.ps.o0.y, b.ps.o0.z, b.ps.o0.w,
                                 b.ps.o1.x, b.ps.o1.y, b.ps.o1.z, b.ps.o1.w};
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[j] = __uint_as_float(w[j]);
        }
      }
    }
    bad = bad || b.bad;
    const bool app = APP && is_app_chunk(d);
    if (app) {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const bool sub = (d.c * TC + i * TPI + row) == d.L - 1;
        b.k[i] = sub ? b.kn : b.k[i];
        b.v[i] = sub ? b.vn : b.v[i];
      }
    }
    const int t_lo = PFX ? max(d.cb * TC, d.t0) : d.cb * TC;
    const int t_hi = min(d.L, d.ce * TC);
    float z[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int tok = d.c * TC + i * TPI + row;
      const bool valid = tok >= t_lo && tok < t_hi;
      const float dd = group_sum<LPT>(dot8<DT>(qv, b.k[i])) * scale_log2;
      z[i] = valid ? dd : kNegInf;
      const u32x4 zero = {0u, 0u, 0u, 0u};
      b.v[i] = valid ? b.v[i] : zero;
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
      const uint32_t w[4] = {b.v[i].x, b.v[i].y, b.v[i].z, b.v[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] = fmaf(pz[i], lo16<DT>(w[j]), acc[2 * j]);
        acc[2 * j + 1] = fmaf(pz[i], hi16<DT>(w[j]), acc[2 * j + 1]);
      }
    }
    m = mnew;
    if (d.c == d.ce - 1) finish_piece(d, b, app);
  }

  __device__ __forceinline__ void finish_piece(const Chunk &d, const Buf &b, bool app) {
    if (APP && app) {
      const int blk = b.app_blk;
      if (blk < 0 || (int64_t)blk >= num_blocks) {
        bad = true;
      } else if (store_new && row == (d.L - 1) % TPI) {
        const int64_t base = (int64_t)blk * blk_stride + (int64_t)d.h * B * D + ((d.L - 1) % B) * D + qoff;
        *reinterpret_cast<u32x4 *>(const_cast<uint16_t *>(kp) + base) = b.kn;
        *reinterpret_cast<u32x4 *>(const_cast<uint16_t *>(vp) + base) = b.vn;
      }
    }
    // merge the lane groups (same dims, different tokens)
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
    const int64_t g = (int64_t)d.s * H + d.h;
    if (lane < LPT) {
      const float nanv = bad ? __builtin_nanf("") : 0.f;
      if (d.cb == d.c0 && d.ce * TC >= d.L) {
        // the whole row: final output
        uint32_t packed[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t v0 = to16<DT>(acc[2 * j] / l + nanv);
          const uint32_t v1 = to16<DT>(acc[2 * j + 1] / l + nanv);
          packed[j] = v0 | (v1 << 16);
        }
        const u32x4 ov = {packed[0], packed[1], packed[2], packed[3]};
        *reinterpret_cast<u32x4 *>(outp + g * D + lane * 8) = ov;
      } else {
        const int64_t u = worker + g;
        float *o = ws_o + u * D + lane * 8;
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = acc[j] + nanv;
        if (lane == 0) {
          ws_m[u] = m * kLn2 + nanv;  // natural-log units
          ws_l[u] = l + nanv;
        }
      }
    }
  }
};

template <int DT, int D, int B, int NW, bool APP, bool NT, bool PFX = false>
__global__ __launch_bounds__(NW * 64) void decode_balanced_kernel(DecodeParams a) {
  using ST = Stream<DT, D, B, APP, NT, PFX>;
  constexpr int TC = ST::TC;

  extern __shared__ int64_t lds[];
  int64_t *cum = lds;                                         // [S + 1]
  int32_t *lens = reinterpret_cast<int32_t *>(lds + a.S + 1);  // [S]
  int32_t *starts = lens + a.S;                               // [S] (PFX)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (wave == 0) build_cost_prefix<TC, PFX>(a, a.H, cum, lens, lane, 1, starts);
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int i = tid; i <= a.S; i += NW * 64) a.ws_cum[i] = cum[i];
  }
  const uint64_t total = uni64((uint64_t)cum[a.S]);
  if (total == 0) return;

  const uint64_t slice = slice_of(total, a.G);
  const int w = blockIdx.x * NW + wave;
  const uint64_t lo = min(total, (uint64_t)w * slice);
  const uint64_t hi = min(total, lo + slice);
  if (lo >= hi) return;

  ST st;
  st.init(a, cum, lens, lane, starts);
  st.worker = w;
  st.cur.enter(lo, hi);
  __builtin_amdgcn_s_setprio(3);
  run_stream(st, (int)(hi - lo));
  __builtin_amdgcn_s_setprio(0);
}

// One wavefront per (sequence, head): rows of empty or invalid contexts, and
// the LSE merge of rows cut over several workers.  Two rounds of loads: the
// length and the chunk prefix; then every piece's (m, l) (lane j: piece j)
// together with the o rows of the first four pieces.  Pieces are combined in
// worker order.
// TC is the chunk length of the split pass that wrote the partials; F8: the
// pools hold e4m3 codes (the appended rows are quantised when written).
template <int DT, int D, int TC, bool F8>
__global__ __launch_bounds__(256) void decode_balanced_merge_kernel(DecodeParams a) {
  constexpr int V = D / 64;  // dims per lane
  const int lane = threadIdx.x & 63;
  const int64_t rows = (int64_t)a.S * a.H;
  // Decode step with the append (FP8 pools, or a 16-bit balanced split that
  // left the pool writes to this launch): the split pass attended over token
  // L - 1's row taken from k_new / v_new (FP8: quantised); the workgroups past
  // the merge's own write it to its pool slot, beside the merge instead of
  // ahead of it in its wavefronts.  16 bytes per lane: a row takes D / 8 lanes
  // (16-bit) or 8 lanes (FP8 codes, from 16-bit rows of 128); nothing for an
  // invalid context or an entry outside the pool.
  const int64_t merge_blocks = (rows + 3) / 4;
  if ((int64_t)blockIdx.x >= merge_blocks) {
    constexpr int LPR = F8 ? D / 16 : D / 8;  // lanes per row
    const int64_t row = (((int64_t)blockIdx.x - merge_blocks) * 4 + (threadIdx.x >> 6)) * (64 / LPR) + lane / LPR;
    const int p = lane % LPR;
    if (!a.append || row >= rows) return;
    const int s = (int)(row / a.H);
    const int h = (int)(row - (int64_t)s * a.H);
    const int L = a.lens[s];
    if (L < 1 || L > a.maxb * a.B) return;
    const int blk = a.tables[(int64_t)s * a.maxb + (L - 1) / a.B];
    if (blk < 0 || (int64_t)blk >= a.num_blocks) return;
    const int64_t slot = (((int64_t)blk * a.Hkv + h) * a.B + (L - 1) % a.B) * D;
    if constexpr (F8) {
      const int64_t src = (int64_t)s * a.new_stride + (int64_t)h * D + p * 16;
      const u32x4 *ks = reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(a.k_new) + src);
      const u32x4 *vs = reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(a.v_new) + src);
      *reinterpret_cast<u32x4 *>(reinterpret_cast<uint8_t *>(const_cast<void *>(a.k_pool)) + slot + p * 16) =
          quant16<DT>(ks[0], ks[1], a.k_inv);
      *reinterpret_cast<u32x4 *>(reinterpret_cast<uint8_t *>(const_cast<void *>(a.v_pool)) + slot + p * 16) =
          quant16<DT>(vs[0], vs[1], a.v_inv);
    } else {
      const int64_t src = (int64_t)s * a.new_stride + (int64_t)h * D + p * 8;
      const u32x4 kv = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(a.k_new) + src);
      const u32x4 vv = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(a.v_new) + src);
      *reinterpret_cast<u32x4 *>(reinterpret_cast<uint16_t *>(const_cast<void *>(a.k_pool)) + slot + p * 8) = kv;
      *reinterpret_cast<u32x4 *>(reinterpret_cast<uint16_t *>(const_cast<void *>(a.v_pool)) + slot + p * 8) = vv;
    }
    return;
  }
  const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (g >= rows) return;
  const int s = (int)(g / a.H);
  const int h = (int)(g - (int64_t)s * a.H);
  const int L = a.lens[s];
  const uint64_t cum_s = (uint64_t)a.ws_cum[s];
  const uint64_t total = (uint64_t)a.ws_cum[a.S];
  uint16_t *out_row = reinterpret_cast<uint16_t *>(a.out) + g * D;
  if (L <= 0 || L > a.maxb * a.B) {
    const uint16_t v = (L == 0) ? uint16_t(0) : to16<DT>(__builtin_nanf(""));
    for (int d = lane; d < D; d += 64) out_row[d] = v;
    return;
  }
  int nch = (L + TC - 1) / TC;
  if (a.pfx_pass == 2) {  // suffix pass of a shared prefix: the row's suffix
    int c0;
    suffix_span<TC>(L, a.pfx_lens[s / a.pfx_group], a.maxb, a.B, c0, nch);
  }
  const uint64_t seg = cum_s + (uint64_t)h * nch;
  const uint64_t end = seg + nch;  // the row's chunks are [seg, end)
  const uint64_t slice = slice_of(total, a.G);
  const int64_t t_a = (int64_t)udiv64(seg, slice);
  const int64_t n = (int64_t)udiv64(end - 1, slice) - t_a + 1;
  if (n <= 1) return;  // one piece: it wrote the row

  auto item = [&](int64_t j) { return t_a + j + g; };  // partial slot of piece j
  float m0 = kNegInf, l0 = 0.f;
  if (lane < n) {
    m0 = a.ws_m[item(lane)];
    l0 = a.ws_l[item(lane)];
  }
  float pre[4][V];  // o rows of pieces 0..3 (n >= 2; indexes past n repeat the last)
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t u = item(min((int64_t)q, n - 1));
#pragma unroll
    for (int k = 0; k < V; ++k) pre[q][k] = a.ws_o[u * D + lane + 64 * k];
  }
  float M = m0;
  for (int64_t j0 = 64; j0 < n; j0 += 64) {
    const int64_t j = j0 + lane;
    if (j < n) M = fmaxf(M, a.ws_m[item(j)]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));

  float lsum = 0.f;
  float o[V];
#pragma unroll
  for (int k = 0; k < V; ++k) o[k] = 0.f;
  for (int64_t j0 = 0; j0 < n; j0 += 64) {
    const int64_t j = j0 + lane;
    float f = 0.f, lw = 0.f;
    if (j0 == 0) {
      if (lane < n) {
        f = fast_exp2((m0 - M) * kLog2e);
        lw = l0;
      }
    } else if (j < n) {
      f = fast_exp2((a.ws_m[item(j)] - M) * kLog2e);
      lw = a.ws_l[item(j)];
    }
    const int cnt = (int)min((int64_t)64, n - j0);
    // workers in increasing order; their o rows are fetched 4 at a time
    for (int q0 = 0; q0 < cnt; q0 += 4) {
      float fj[4], vj[4][V];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int jj = min(q0 + q, cnt - 1);
        fj[q] = (q0 + q < cnt) ? __shfl(f, jj) : 0.f;
        if (j0 == 0 && q0 == 0) {
#pragma unroll
          for (int k = 0; k < V; ++k) vj[q][k] = pre[q][k];
        } else {
          const int64_t u = item(j0 + jj);
#pragma unroll
          for (int k = 0; k < V; ++k) vj[q][k] = a.ws_o[u * D + lane + 64 * k];
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (q0 + q >= cnt) break;
        lsum += fj[q] * __shfl(lw, q0 + q);
#pragma unroll
        for (int k = 0; k < V; ++k) o[k] += fj[q] * vj[q][k];
      }
    }
  }
#pragma unroll
  for (int k = 0; k < V; ++k) out_row[lane + 64 * k] = to16<DT>(o[k] / lsum);
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------

template <int DT, int D, int B>
struct PartitionsF {
  static hipError_t call(const DecodeParams &a, hipStream_t st) {
    const int grid = (int)partition_grid(a.items);
    if (a.stream_kv)
      hipLaunchKernelGGL((decode_partition_kernel<DT, D, B, kNumWaves, true>), dim3(grid),
                         dim3(kNumWaves * 64), 0, st, a);
    else
      hipLaunchKernelGGL((decode_partition_kernel<DT, D, B, kNumWaves, false>), dim3(grid),
                         dim3(kNumWaves * 64), 0, st, a);
    return hipGetLastError();
  }
};

template <int DT, int D, int B>
struct PartitionsPtrF {
  static const void *call(int nt) {
    return nt ? reinterpret_cast<const void *>(&decode_partition_kernel<DT, D, B, kNumWaves, true>)
              : reinterpret_cast<const void *>(&decode_partition_kernel<DT, D, B, kNumWaves, false>);
  }
};

template <int DT, int D, int B>
struct BalancedF {
  template <bool APP, bool NT>
  static void go(const DecodeParams &a, hipStream_t st) {
    hipLaunchKernelGGL((decode_balanced_kernel<DT, D, B, kNumWaves, APP, NT>), dim3(a.G / kNumWaves),
                       dim3(kNumWaves * 64), balanced_lds_bytes(a.S), st, a);
  }
  static hipError_t call(const DecodeParams &a, hipStream_t st) {
    if (a.append) {
      if (a.stream_kv) go<true, true>(a, st);
      else go<true, false>(a, st);
    } else {
      if (a.stream_kv) go<false, true>(a, st);
      else go<false, false>(a, st);
    }
    return hipGetLastError();
  }
};

template <int DT, int D, int B>
struct SuffixF {
  static hipError_t call(const DecodeParams &a, hipStream_t st) {
    if (a.stream_kv)
      hipLaunchKernelGGL((decode_balanced_kernel<DT, D, B, kNumWaves, false, true, true>), dim3(a.G / kNumWaves),
                         dim3(kNumWaves * 64), suffix_lds_bytes(a.S), st, a);
    else
      hipLaunchKernelGGL((decode_balanced_kernel<DT, D, B, kNumWaves, false, false, true>), dim3(a.G / kNumWaves),
                         dim3(kNumWaves * 64), suffix_lds_bytes(a.S), st, a);
    return hipGetLastError();
  }
};

template <int DT, int D, int B>
struct SuffixPtrF {
  static const void *call(int nt) {
    return nt ? reinterpret_cast<const void *>(&decode_balanced_kernel<DT, D, B, kNumWaves, false, true, true>)
              : reinterpret_cast<const void *>(&decode_balanced_kernel<DT, D, B, kNumWaves, false, false, true>);
  }
};

template <int DT, int D, int B>
struct BalancedPtrF {
  static const void *call(int append, int nt) {
    if (append)
      return nt ? reinterpret_cast<const void *>(&decode_balanced_kernel<DT, D, B, kNumWaves, true, true>)
                : reinterpret_cast<const void *>(&decode_balanced_kernel<DT, D, B, kNumWaves, true, false>);
    return nt ? reinterpret_cast<const void *>(&decode_balanced_kernel<DT, D, B, kNumWaves, false, true>)
              : reinterpret_cast<const void *>(&decode_balanced_kernel<DT, D, B, kNumWaves, false, false>);
  }
};

// Call F<DT, D, B>::call(args...) for the runtime (dtype, D, B).
template <template <int, int, int> class F, typename R, typename... Args>
R dispatch(int dtype, int D, int B, R fail, Args... args) {
#define PKV_B(DT, DD)                             \
  switch (B) {                                    \
    case 8: return F<DT, DD, 8>::call(args...);   \
    case 16: return F<DT, DD, 16>::call(args...); \
    case 32: return F<DT, DD, 32>::call(args...); \
    case 64: return F<DT, DD, 64>::call(args...); \
    default: return fail;                         \
  }
  if (dtype == DT_F16) {
    if (D == 64) { PKV_B(DT_F16, 64) }
    if (D == 128) { PKV_B(DT_F16, 128) }
  } else {
    if (D == 64) { PKV_B(DT_BF16, 64) }
    if (D == 128) { PKV_B(DT_BF16, 128) }
  }
#undef PKV_B
  return fail;
}

}  // namespace

const void *suffix_kernel(int dtype, int head_dim, int block_size, int nt) {
  return dispatch<SuffixPtrF, const void *>(dtype, head_dim, block_size, nullptr, nt);
}

size_t suffix_lds_bytes(int num_seqs) {
  return (size_t)(num_seqs + 1) * sizeof(int64_t) + 2 * (size_t)num_seqs * sizeof(int32_t);
}

hipError_t launch_suffix(const DecodeParams &a, hipStream_t stream) {
  if (a.S == 0 || a.G == 0) return hipSuccess;
  return dispatch<SuffixF, hipError_t>(a.dtype, a.D, a.B, hipErrorInvalidValue, a, stream);
}

int decode_waves() { return kNumWaves; }

int decode_chunk_tokens(int head_dim) {
  return head_dim == 64 ? Geo<64>::TC : Geo<128>::TC;
}

size_t balanced_lds_bytes(int num_seqs) {
  return (size_t)(num_seqs + 1) * sizeof(int64_t) + (size_t)num_seqs * sizeof(int32_t);
}

const void *partition_kernel(int dtype, int head_dim, int block_size, int nt) {
  return dispatch<PartitionsPtrF, const void *>(dtype, head_dim, block_size, nullptr, nt);
}

int64_t partition_grid(int64_t items) {
  const int64_t group = 8 * kXcdGroup;
  return (items + group - 1) / group * group;
}

const void *balanced_kernel(int dtype, int head_dim, int block_size, int append, int nt) {
  return dispatch<BalancedPtrF, const void *>(dtype, head_dim, block_size, nullptr, append, nt);
}

hipError_t launch_decode_partitions(const DecodeParams &a, hipStream_t stream) {
  if (a.S == 0) return hipSuccess;
  if (a.balanced) {
    if (a.G == 0) return hipSuccess;
    return dispatch<BalancedF, hipError_t>(a.dtype, a.D, a.B, hipErrorInvalidValue, a, stream);
  }
  if (a.items == 0) return hipSuccess;
  return dispatch<PartitionsF, hipError_t>(a.dtype, a.D, a.B, hipErrorInvalidValue, a, stream);
}

hipError_t launch_decode_merge(const DecodeParams &a, hipStream_t stream) {
  if (a.S == 0) return hipSuccess;
  if (a.balanced) {
    const int64_t segs = (int64_t)a.S * a.H;
    const int grid = (int)((segs + 3) / 4);
    // a 16-bit split that left the pool writes to this launch: one more
    // workgroup per 4 * 64 / (D / 8) rows writes them
    const int rows_per_wg = 4 * 64 / (a.D / 8);
    const int hgrid = grid + (a.append && a.append_in_merge ? (int)((segs + rows_per_wg - 1) / rows_per_wg) : 0);
#define PKV_BMERGE(DT, DD) \
  hipLaunchKernelGGL((decode_balanced_merge_kernel<DT, DD, Geo<DD>::TC, false>), dim3(hgrid), dim3(256), 0, stream, a)
    if (a.fp8) {
      if (a.D != 64 && a.D != 128) return hipErrorInvalidValue;
      // with the append: one more workgroup per 4 * 64 / (D / 16) rows writes
      // the new codes
      const int frows = 4 * 64 / (a.D / 16);
      const int fgrid = grid + (a.append ? (int)((segs + frows - 1) / frows) : 0);
      // the e4m3 split pass's chunks: 32 tokens at head_dim 128, 64 at 64
#define PKV_FMERGE(DT, DD, TCC) \
  hipLaunchKernelGGL((decode_balanced_merge_kernel<DT, DD, TCC, true>), dim3(fgrid), dim3(256), 0, stream, a)
      if (fp8_chunk_tokens(a.D) != (a.D == 64 ? 64 : 32)) return hipErrorInvalidValue;
      if (a.dtype == DT_F16) {
        if (a.D == 64) PKV_FMERGE(DT_F16, 64, 64);
        else PKV_FMERGE(DT_F16, 128, 32);
      } else {
        if (a.D == 64) PKV_FMERGE(DT_BF16, 64, 64);
        else PKV_FMERGE(DT_BF16, 128, 32);
      }
#undef PKV_FMERGE
    } else if (a.dtype == DT_F16) {
      if (a.D == 64) PKV_BMERGE(DT_F16, 64);
      else PKV_BMERGE(DT_F16, 128);
    } else {
      if (a.D == 64) PKV_BMERGE(DT_BF16, 64);
      else PKV_BMERGE(DT_BF16, 128);
    }
#undef PKV_BMERGE
    return hipGetLastError();
  }
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
