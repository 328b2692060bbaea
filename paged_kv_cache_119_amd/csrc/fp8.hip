// FP8 KV cache for gfx950: the K and V pools hold OCP e4m3 codes (one byte per
// element) with one float32 scale per pool; a stored code c means the value
// e4m3(c) * scale.  Half the bytes of a 16-bit cache for the same tokens.
//
//  * Append (the cache append of "PagedAttention 完全拆解", 原理详解（三）, item
//    1, with a quantising store): code = e4m3(x * (1 / scale)), the product
//    rounded in float32, saturated to +-448, then rounded to the nearest e4m3
//    value, ties to even (v_cvt_pk_fp8_f32); NaN stays NaN.
//  * Append of each sequence's new token (the decode step): the same
//    quantisation, the slot of token L - 1 taken from the block table.  With
//    one row per KV head the split pass quantises the new token itself and
//    uses those codes in place of the pool's, and the merge launch writes
//    them to the pool afterwards: no launch of its own, and no stores from
//    inside the long stream kernel (they measured far slower than a separate
//    launch on large pools).  Grouped rows use a separate launch with no slot
//    list before the split pass.
//  * Decode (the attention equation of the same page, 背景): the balanced
//    split and pipelined chunk stream of the 16-bit kernel, with 32-token
//    chunks: 8 lanes hold a token row (16 codes each), a load instruction
//    reads 8 whole rows (1 KiB).  Codes are widened in pairs by gfx950's
//    packed conversions, exactly: K to the query's 16-bit type, so q.k runs
//    on v_dot2c with exact products as in the 16-bit kernel; V to binary16,
//    accumulated in float32 by mixed-precision FMAs.  The K scale is folded
//    into the score scale and the V scale applied to the weighted V sum.

#include <type_traits>

#include "pkv_device.h"
#include "pkv_launch.h"
#include "pkv_split.h"

namespace pkv {

namespace {

constexpr int kFp8Waves = PKV_DECODE_WAVES;
constexpr int FD = 128;               // head_dim of this path
constexpr int FLPT = 8;               // lanes per token row
constexpr int FTPI = 64 / FLPT;       // token rows per load instruction
constexpr int FNL = 4;                // loads per tensor per chunk
constexpr int FTC = FNL * FTPI;       // tokens per chunk

// Two e4m3 codes (bytes 0, 1 or, hi, bytes 2, 3 of w) -> a packed pair of the
// 16-bit type, exactly (gfx950's packed conversion at unit scale).
template <int DT>
__device__ __forceinline__ uint32_t pair16(uint32_t w, bool hi) {
  if constexpr (DT == DT_F16) {
    return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true))
              : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
  } else {
    return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true))
              : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  }
}

// 16 elements of a K row and of a V row (16-bit, 32 bytes each) -> 16 codes
// each, written at element offset dst of the pools.
template <int DT>
__device__ __forceinline__ void quantise_piece(uint8_t *kp, uint8_t *vp, const uint16_t *ksrc, const uint16_t *vsrc,
                                               int64_t dst, float k_inv, float v_inv) {
  const u32x4 *ks = reinterpret_cast<const u32x4 *>(ksrc);
  const u32x4 *vs = reinterpret_cast<const u32x4 *>(vsrc);
  *reinterpret_cast<u32x4 *>(kp + dst) = quant16<DT>(ks[0], ks[1], k_inv);
  *reinterpret_cast<u32x4 *>(vp + dst) = quant16<DT>(vs[0], vs[1], v_inv);
}

// One thread per 16 elements of a (token, head) row, slots from a list.
template <int DT>
__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(
    uint8_t *__restrict__ kp, uint8_t *__restrict__ vp, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, int64_t k_stride, int64_t v_stride, const int64_t *__restrict__ slots,
    int32_t T, int32_t Hkv, int32_t B, int32_t D, int64_t num_blocks, float k_inv, float v_inv) {
  const int per_row = D / 16;
  const int64_t per_tok = (int64_t)Hkv * per_row;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)T * per_tok) return;
  const int t = (int)(idx / per_tok);
  const int r = (int)(idx - (int64_t)t * per_tok);
  const int h = r / per_row;
  const int piece = r - h * per_row;
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= num_blocks * B) return;
  const int64_t blk = slot / B;
  const int64_t off = slot - blk * B;
  const int64_t dst = ((blk * Hkv + h) * B + off) * D + piece * 16;
  quantise_piece<DT>(kp, vp, k + (int64_t)t * k_stride + h * D + piece * 16, v + (int64_t)t * v_stride + h * D + piece * 16,
                     dst, k_inv, v_inv);
}

// The decode step's append: row s of k_new / v_new becomes token L - 1 of
// sequence s, its slot from the block table.  One thread per 16 elements of
// a (sequence, head) row; invalid contexts and out-of-pool entries write
// nothing.
template <int DT>
__global__ __launch_bounds__(256) void append_last_fp8_kernel(DecodeParams a, float k_inv, float v_inv) {
  const int per_row = FD / 16;
  const int64_t per_seq = (int64_t)a.Hkv * per_row;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)a.S * per_seq) return;
  const int s = (int)(idx / per_seq);
  const int r = (int)(idx - (int64_t)s * per_seq);
  const int h = r / per_row;
  const int piece = r - h * per_row;
  const int L = a.lens[s];
  if (L <= 0 || L > a.maxb * a.B) return;
  const int blk = a.tables[(int64_t)s * a.maxb + (L - 1) / a.B];
  if (blk < 0 || (int64_t)blk >= a.num_blocks) return;
  const int64_t dst = (((int64_t)blk * a.Hkv + h) * a.B + (L - 1) % a.B) * FD + piece * 16;
  const int64_t src = (int64_t)s * a.new_stride + (int64_t)h * FD + piece * 16;
  quantise_piece<DT>(reinterpret_cast<uint8_t *>(const_cast<void *>(a.k_pool)),
                     reinterpret_cast<uint8_t *>(const_cast<void *>(a.v_pool)),
                     reinterpret_cast<const uint16_t *>(a.k_new) + src,
                     reinterpret_cast<const uint16_t *>(a.v_new) + src, dst, k_inv, v_inv);
}

// APP: the decode step's append -- token L - 1 of every row is taken from
// k_new / v_new, quantised here exactly as the append quantises it, in place
// of the pool's codes (the merge launch writes the codes to the pool after
// this pass has run).
template <int DT, int B, bool NT, bool APP>
struct Fp8Stream {
  static constexpr int NE = FTC >= B ? FTC / B : 1;  // table entries per chunk
  static_assert(B % FTPI == 0, "a load must not straddle two blocks");

  struct BufP {
    u32x4 k[FNL], v[FNL];
    u32x4 q0, q1;
    bool bad;
  };
  struct BufA {
    u32x4 k[FNL], v[FNL];
    u32x4 q0, q1;
    // chunk of token L - 1 only: the new-token rows spread over the wave,
    // lane l < 32 holding K elements 4l .. 4l+3, lane 32 + l V elements
    // 4l .. 4l+3 (8 bytes a lane)
    uint32_t nw0, nw1;
    bool bad;
  };
  using Buf = typename std::conditional<APP, BufA, BufP>::type;

  const uint8_t *kp;
  const uint8_t *vp;
  const uint16_t *qp;
  const int32_t *tables;
  uint16_t *outp;
  float *ws_m;
  float *ws_l;
  float *ws_o;
  int64_t blk_stride, num_blocks;
  int H, maxb;
  float scale_log2, v_scale;
  const uint16_t *knp;  // APP: new-token rows and quantisation factors
  const uint16_t *vnp;
  int64_t new_stride;
  float k_inv, v_inv;
  int lane, lane_off, row, qoff;
  int64_t worker;
  ChunkCursor<FTC> cur;
  u32x4 qa, qb;  // this lane's 16 query elements as packed pairs
  float m, l, acc[16];
  bool bad;

  __device__ __forceinline__ void init(const DecodeParams &a, const int64_t *cum_, const int32_t *lens_, int lane_) {
    kp = reinterpret_cast<const uint8_t *>(a.k_pool);
    vp = reinterpret_cast<const uint8_t *>(a.v_pool);
    qp = reinterpret_cast<const uint16_t *>(a.q);
    tables = a.tables;
    outp = reinterpret_cast<uint16_t *>(a.out);
    ws_m = a.ws_m;
    ws_l = a.ws_l;
    ws_o = a.ws_o;
    blk_stride = (int64_t)a.Hkv * B * FD;
    num_blocks = a.num_blocks;
    H = a.H;
    maxb = a.maxb;
    scale_log2 = a.scale_log2;
    v_scale = a.v_scale;
    knp = reinterpret_cast<const uint16_t *>(a.k_new);
    vnp = reinterpret_cast<const uint16_t *>(a.v_new);
    new_stride = a.new_stride;
    k_inv = a.k_inv;
    v_inv = a.v_inv;
    lane = lane_;
    lane_off = lane * 16;
    row = lane / FLPT;
    qoff = (lane % FLPT) * 16;
    cur.init(cum_, lens_, a.S, a.H, lane_);
  }

  __device__ __forceinline__ static int first_block(int c) { return FTC >= B ? c * (FTC / B) : c / (B / FTC); }
  __device__ __forceinline__ static int last_block(const Chunk &d) { return (min(d.L, d.ce * FTC) - 1) / B; }
  __device__ __forceinline__ static bool is_app_chunk(const Chunk &d) {
    return d.c == d.ce - 1 && d.ce * FTC >= d.L;  // the chunk of token L - 1
  }

  __device__ __forceinline__ uint32_t load_entries(const Chunk &d) const {
    const int lb = min(first_block(d.c) + min(lane, NE - 1), last_block(d));
    return (uint32_t)tables[(int64_t)d.s * maxb + lb];
  }

  // Tokens past the context read the row of token L - 1 instead (cache lines
  // already fetched); they are masked.
  __device__ __forceinline__ void load_kv(const Chunk &d, uint32_t e, Buf &b) const {
    const int64_t head_base = (int64_t)d.h * B * FD;
    const int tail_off = ((d.L - 1) % B) * FD + qoff;
    bool bd = false;
#pragma unroll
    for (int i = 0; i < FNL; ++i) {
      int ei, off;
      if constexpr (FTC >= B) {
        ei = (i * FTPI) / B;
        off = (i * FTPI) % B;
      } else {
        ei = 0;
        off = (d.c % (B / FTC)) * FTC + i * FTPI;
      }
      int blk = __builtin_amdgcn_readlane((int)e, ei);
      if (blk < 0 || (int64_t)blk >= num_blocks) {
        bd = true;
        blk = 0;
      }
      const int64_t base = (int64_t)blk * blk_stride + head_base;
      const int lo = (d.c * FTC + i * FTPI + row < d.L) ? off * FD + lane_off : tail_off;
      b.k[i] = ld_kv<NT>(kp + base + lo);
      b.v[i] = ld_kv<NT>(vp + base + lo);
    }
    b.bad = bd;
    const uint16_t *q = qp + ((int64_t)d.s * H + d.h) * FD + qoff;
    b.q0 = *reinterpret_cast<const u32x4 *>(q);
    b.q1 = *reinterpret_cast<const u32x4 *>(q + 8);
    if constexpr (APP) {
      // only the chunk of token L - 1 (once per row) loads the new rows
      if (is_app_chunk(d)) {
        const int64_t src = (int64_t)d.s * new_stride + (int64_t)d.h * FD + 4 * (lane & 31);
        const uint64_t w = *reinterpret_cast<const uint64_t *>((lane < 32 ? knp : vnp) + src);
        b.nw0 = (uint32_t)w;
        b.nw1 = (uint32_t)(w >> 32);
      }
    }
  }

  __device__ __forceinline__ void consume(const Chunk &d, Buf &b) {
    if (d.c == d.cb) {
      qa = b.q0;
      qb = b.q1;
      m = kNegInf;
      l = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[j] = 0.f;
      bad = false;
    }
    bad = bad || b.bad;
    if constexpr (APP) {
      if (is_app_chunk(d)) {
        // each lane quantises its 4 elements (the same quant4 steps as the
        // append's); the lanes of token L - 1's row gather their 16 codes
        // of K (from lanes 4(l%8) .. +3) and of V (32 + the same)
        const float inv = lane < 32 ? k_inv : v_inv;
        const int qd = (int)quant4(lo16<DT>(b.nw0) * inv, hi16<DT>(b.nw0) * inv, lo16<DT>(b.nw1) * inv,
                                   hi16<DT>(b.nw1) * inv);
        const int sl = (lane & 7) * 4;
        u32x4 kc, vc;
        kc.x = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * sl, qd);
        kc.y = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (sl + 1), qd);
        kc.z = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (sl + 2), qd);
        kc.w = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (sl + 3), qd);
        vc.x = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (32 + sl), qd);
        vc.y = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (33 + sl), qd);
        vc.z = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (34 + sl), qd);
        vc.w = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (35 + sl), qd);
#pragma unroll
        for (int i = 0; i < FNL; ++i) {
          const bool sub = (d.c * FTC + i * FTPI + row) == d.L - 1;
          b.k[i] = sub ? kc : b.k[i];
          b.v[i] = sub ? vc : b.v[i];
        }
      }
    }
    const int t_lo = d.cb * FTC;
    const int t_hi = min(d.L, d.ce * FTC);
    float z[FNL];
#pragma unroll
    for (int i = 0; i < FNL; ++i) {
      const int tok = d.c * FTC + i * FTPI + row;
      const bool valid = tok >= t_lo && tok < t_hi;
      const uint32_t w[4] = {b.k[i].x, b.k[i].y, b.k[i].z, b.k[i].w};
      const uint32_t qw[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
      float dot = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // four codes -> two pairs of the query's type (exact), two dot2 steps
        dot = dot2<DT>(qw[2 * j], pair16<DT>(w[j], false), dot);
        dot = dot2<DT>(qw[2 * j + 1], pair16<DT>(w[j], true), dot);
      }
      const float dd = group_sum<FLPT>(dot) * scale_log2;
      z[i] = valid ? dd : kNegInf;
      const u32x4 zero = {0u, 0u, 0u, 0u};
      b.v[i] = valid ? b.v[i] : zero;
    }
    float mx = z[0];
#pragma unroll
    for (int i = 1; i < FNL; ++i) mx = fmaxf(mx, z[i]);
    const float mnew = fmaxf(m, mx);
    const float mref = (mnew == kNegInf) ? 0.f : mnew;
    const float alpha = fast_exp2(m - mref);
    float pz[FNL];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < FNL; ++i) {
      pz[i] = fast_exp2(z[i] - mref);
      psum += pz[i];
    }
    l = l * alpha + psum;
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] *= alpha;
#pragma unroll
    for (int i = 0; i < FNL; ++i) {
      const uint32_t w[4] = {b.v[i].x, b.v[i].y, b.v[i].z, b.v[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // four codes -> two binary16 pairs (exact), mixed-precision FMAs
        const uint32_t h0 = pair16<DT_F16>(w[j], false), h1 = pair16<DT_F16>(w[j], true);
        acc[4 * j] = fmaf(pz[i], lo16<DT_F16>(h0), acc[4 * j]);
        acc[4 * j + 1] = fmaf(pz[i], hi16<DT_F16>(h0), acc[4 * j + 1]);
        acc[4 * j + 2] = fmaf(pz[i], lo16<DT_F16>(h1), acc[4 * j + 2]);
        acc[4 * j + 3] = fmaf(pz[i], hi16<DT_F16>(h1), acc[4 * j + 3]);
      }
    }
    m = mnew;
    if (d.c == d.ce - 1) finish_piece(d);
  }

  __device__ __forceinline__ void finish_piece(const Chunk &d) {
#pragma unroll
    for (int off = FLPT; off < 64; off <<= 1) {
      const float m2 = __shfl_xor(m, off);
      const float l2 = __shfl_xor(l, off);
      const float mm = fmaxf(m, m2);
      const float f1 = (m == kNegInf) ? 0.f : fast_exp2(m - mm);
      const float f2 = (m2 == kNegInf) ? 0.f : fast_exp2(m2 - mm);
      l = l * f1 + l2 * f2;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float o2 = __shfl_xor(acc[j], off);
        acc[j] = acc[j] * f1 + o2 * f2;
      }
      m = mm;
    }
    const int64_t g = (int64_t)d.s * H + d.h;
    if (lane < FLPT) {
      const float nanv = bad ? __builtin_nanf("") : 0.f;
      if (d.cb == 0 && d.ce * FTC >= d.L) {
        const float f = v_scale / l;
        uint32_t w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          w[j] = (uint32_t)to16<DT>(acc[2 * j] * f + nanv) | ((uint32_t)to16<DT>(acc[2 * j + 1] * f + nanv) << 16);
        uint16_t *o = outp + g * FD + qoff;
        *reinterpret_cast<u32x4 *>(o) = u32x4{w[0], w[1], w[2], w[3]};
        *reinterpret_cast<u32x4 *>(o + 8) = u32x4{w[4], w[5], w[6], w[7]};
      } else {
        const int64_t u = worker + g;
        float *o = ws_o + u * FD + qoff;
#pragma unroll
        for (int j = 0; j < 16; ++j) o[j] = acc[j] * v_scale + nanv;
        if (lane == 0) {
          ws_m[u] = m * kLn2 + nanv;  // natural-log units
          ws_l[u] = l + nanv;
        }
      }
    }
  }
};

template <int DT, int B, int NW, bool NT, bool APP>
__global__ __launch_bounds__(NW * 64) void decode_fp8_kernel(DecodeParams a) {
  using ST = Fp8Stream<DT, B, NT, APP>;
  extern __shared__ int64_t lds[];
  int64_t *cum = lds;                                         // [S + 1]
  int32_t *lens = reinterpret_cast<int32_t *>(lds + a.S + 1);  // [S]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (wave == 0) build_cost_prefix<FTC>(a, a.H, cum, lens, lane);
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
  st.init(a, cum, lens, lane);
  st.worker = w;
  st.cur.enter(lo, hi);
  __builtin_amdgcn_s_setprio(3);
  run_stream(st, (int)(hi - lo));
  __builtin_amdgcn_s_setprio(0);
}

template <int DT, bool NT, bool APP>
const void *fp8_ptr(int B) {
  switch (B) {
    case 8: return reinterpret_cast<const void *>(&decode_fp8_kernel<DT, 8, kFp8Waves, NT, APP>);
    case 16: return reinterpret_cast<const void *>(&decode_fp8_kernel<DT, 16, kFp8Waves, NT, APP>);
    case 32: return reinterpret_cast<const void *>(&decode_fp8_kernel<DT, 32, kFp8Waves, NT, APP>);
    case 64: return reinterpret_cast<const void *>(&decode_fp8_kernel<DT, 64, kFp8Waves, NT, APP>);
    default: return nullptr;
  }
}

template <int DT, int B, bool APP>
void launch_fp8_app(const DecodeParams &a, hipStream_t st) {
  if (a.stream_kv)
    hipLaunchKernelGGL((decode_fp8_kernel<DT, B, kFp8Waves, true, APP>), dim3(a.G / kFp8Waves),
                       dim3(kFp8Waves * 64), fp8_lds_bytes(a.S), st, a);
  else
    hipLaunchKernelGGL((decode_fp8_kernel<DT, B, kFp8Waves, false, APP>), dim3(a.G / kFp8Waves),
                       dim3(kFp8Waves * 64), fp8_lds_bytes(a.S), st, a);
}

template <int DT, int B>
hipError_t launch_fp8(const DecodeParams &a, hipStream_t st) {
  if (a.append) launch_fp8_app<DT, B, true>(a, st);
  else launch_fp8_app<DT, B, false>(a, st);
  return hipGetLastError();
}

}  // namespace

int fp8_chunk_tokens() { return FTC; }

size_t fp8_lds_bytes(int num_seqs) {
  return (size_t)(num_seqs + 1) * sizeof(int64_t) + (size_t)num_seqs * sizeof(int32_t);
}

const void *fp8_kernel(int dtype, int block_size, int nt, int append) {
  if (append) {
    if (nt) return dtype == DT_F16 ? fp8_ptr<DT_F16, true, true>(block_size) : fp8_ptr<DT_BF16, true, true>(block_size);
    return dtype == DT_F16 ? fp8_ptr<DT_F16, false, true>(block_size) : fp8_ptr<DT_BF16, false, true>(block_size);
  }
  if (nt) return dtype == DT_F16 ? fp8_ptr<DT_F16, true, false>(block_size) : fp8_ptr<DT_BF16, true, false>(block_size);
  return dtype == DT_F16 ? fp8_ptr<DT_F16, false, false>(block_size) : fp8_ptr<DT_BF16, false, false>(block_size);
}

hipError_t launch_fp8_decode(const DecodeParams &a, hipStream_t stream) {
  if (a.S == 0 || a.G == 0) return hipSuccess;
#define PKV_F(DT)                                 \
  switch (a.B) {                                  \
    case 8: return launch_fp8<DT, 8>(a, stream);   \
    case 16: return launch_fp8<DT, 16>(a, stream); \
    case 32: return launch_fp8<DT, 32>(a, stream); \
    case 64: return launch_fp8<DT, 64>(a, stream); \
    default: return hipErrorInvalidValue;         \
  }
  if (a.dtype == DT_F16) { PKV_F(DT_F16) }
  PKV_F(DT_BF16)
#undef PKV_F
}

hipError_t launch_append_last_fp8(const DecodeParams &a, float k_inv, float v_inv, hipStream_t stream) {
  const int64_t threads = (int64_t)a.S * a.Hkv * (FD / 16);
  if (threads == 0) return hipSuccess;
  const int64_t grid = (threads + 255) / 256;
  if (a.dtype == DT_F16)
    hipLaunchKernelGGL((append_last_fp8_kernel<DT_F16>), dim3((unsigned)grid), dim3(256), 0, stream, a, k_inv, v_inv);
  else
    hipLaunchKernelGGL((append_last_fp8_kernel<DT_BF16>), dim3((unsigned)grid), dim3(256), 0, stream, a, k_inv,
                       v_inv);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache_fp8(void *k_pool, void *v_pool, const void *k, const void *v, int64_t k_stride,
                                        int64_t v_stride, const int64_t *slots, int32_t T, int32_t Hkv, int32_t B,
                                        int32_t D, int64_t num_blocks, int dtype, float k_inv, float v_inv,
                                        hipStream_t stream) {
  const int64_t threads = (int64_t)T * Hkv * (D / 16);
  if (threads == 0) return hipSuccess;
  const int64_t grid = (threads + 255) / 256;
#define PKV_Q(DT)                                                                                             \
  hipLaunchKernelGGL((reshape_and_cache_fp8_kernel<DT>), dim3((unsigned)grid), dim3(256), 0, stream,           \
                     reinterpret_cast<uint8_t *>(k_pool), reinterpret_cast<uint8_t *>(v_pool),                 \
                     reinterpret_cast<const uint16_t *>(k), reinterpret_cast<const uint16_t *>(v), k_stride, \
                     v_stride, slots, T, Hkv, B, D, num_blocks, k_inv, v_inv)
  if (dtype == DT_F16) PKV_Q(DT_F16);
  else PKV_Q(DT_BF16);
#undef PKV_Q
  return hipGetLastError();
}

}  // namespace pkv
