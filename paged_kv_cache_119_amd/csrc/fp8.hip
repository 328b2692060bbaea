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
//    split and pipelined chunk stream of the 16-bit kernel.  8 lanes hold a
//    token row and a load instruction reads 8 whole rows: at head_dim 128,
//    16 codes a lane (1 KiB an instruction) and 32-token chunks; at head_dim
//    64, 8 codes a lane and 64-token chunks (4 KiB of each tensor per chunk
//    either way).  Codes are widened in pairs by gfx950's
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

// Decode geometry for head_dim D: a lane loads BPL codes of a token row (16
// at D = 128, 8 at D = 64), LPT = 8 lanes hold a row, a load instruction
// reads 8 whole rows, and NL loads per tensor make a chunk of TC tokens, so
// a chunk keeps 4 KiB of each tensor in flight at either head_dim.
template <int D>
struct F8Geo {
  static constexpr int BPL = D == 128 ? 16 : 8;  // code bytes per lane per load
  static constexpr int LPT = D / BPL;            // lanes per token row
  static constexpr int TPI = 64 / LPT;           // token rows per load instruction
  static constexpr int NL = 4096 / (64 * BPL);   // loads per tensor per chunk
  static constexpr int TC = NL * TPI;            // tokens per chunk
  static constexpr int NQ = BPL / 8;             // 16-byte pieces of 16-bit query per lane
  static_assert(LPT == 8, "8 lanes per token row");
};

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
  const int per_row = a.D / 16;
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
  const int64_t dst = (((int64_t)blk * a.Hkv + h) * a.B + (L - 1) % a.B) * a.D + piece * 16;
  const int64_t src = (int64_t)s * a.new_stride + (int64_t)h * a.D + piece * 16;
  quantise_piece<DT>(reinterpret_cast<uint8_t *>(const_cast<void *>(a.k_pool)),
                     reinterpret_cast<uint8_t *>(const_cast<void *>(a.v_pool)),
                     reinterpret_cast<const uint16_t *>(a.k_new) + src,
                     reinterpret_cast<const uint16_t *>(a.v_new) + src, dst, k_inv, v_inv);
}

// APP: the decode step's append -- token L - 1 of every row is taken from
// k_new / v_new, quantised here exactly as the append quantises it, in place
// of the pool's codes (the merge launch writes the codes to the pool after
// this pass has run).
template <int DT, int D, int B, bool NT, bool APP>
struct Fp8Stream {
  using GM = F8Geo<D>;
  static constexpr int FLPT = GM::LPT, FTPI = GM::TPI, FNL = GM::NL, FTC = GM::TC, BPL = GM::BPL, NQ = GM::NQ;
  static constexpr int NE = FTC >= B ? FTC / B : 1;  // table entries per chunk
  static constexpr int NWD = BPL / 4;                // dwords of codes per lane per load
  static_assert(B % FTPI == 0, "a load must not straddle two blocks");
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  using kv_t = typename std::conditional<BPL == 16, u32x4, u32x2_t>::type;

  struct BufP {
    kv_t k[FNL], v[FNL];
    u32x4 q[NQ];
    bool bad;
  };
  struct BufA {
    kv_t k[FNL], v[FNL];
    u32x4 q[NQ];
    // chunk of token L - 1 only: the new-token rows spread over the wave,
    // lane l < D / 4 holding K elements 4l .. 4l+3, lane D / 4 + l V
    // elements 4l .. 4l+3 (8 bytes a lane; lanes past D / 2 repeat them)
    uint32_t nw0, nw1;
    bool bad;
  };
  using Buf = typename std::conditional<APP, BufA, BufP>::type;

  __device__ __forceinline__ static kv_t ld_codes(const uint8_t *p) {
    if constexpr (BPL == 16) return ld_kv<NT>(p);
    else return ld_kv8<NT>(p);
  }

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
  u32x4 qv[NQ];  // this lane's BPL query elements as packed pairs
  float m, l, acc[BPL];
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
    blk_stride = (int64_t)a.Hkv * B * D;
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
    lane_off = lane * BPL;
    row = lane / FLPT;
    qoff = (lane % FLPT) * BPL;
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
    const int64_t head_base = (int64_t)d.h * B * D;
    const int tail_off = ((d.L - 1) % B) * D + qoff;
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
      const int lo = (d.c * FTC + i * FTPI + row < d.L) ? off * D + lane_off : tail_off;
      b.k[i] = ld_codes(kp + base + lo);
      b.v[i] = ld_codes(vp + base + lo);
    }
    b.bad = bd;
    const uint16_t *q = qp + ((int64_t)d.s * H + d.h) * D + qoff;
#pragma unroll
    for (int j = 0; j < NQ; ++j) b.q[j] = *reinterpret_cast<const u32x4 *>(q + 8 * j);
    if constexpr (APP) {
      // only the chunk of token L - 1 (once per row) loads the new rows
      if (is_app_chunk(d)) {
        constexpr int QL = D / 4;  // lanes quantising one tensor's row
        const int ql = lane % (2 * QL);
        const int64_t src = (int64_t)d.s * new_stride + (int64_t)d.h * D + 4 * (ql % QL);
        const uint64_t w = *reinterpret_cast<const uint64_t *>((ql < QL ? knp : vnp) + src);
        b.nw0 = (uint32_t)w;
        b.nw1 = (uint32_t)(w >> 32);
      }
    }
  }

  __device__ __forceinline__ void consume(const Chunk &d, Buf &b) {
    if (d.c == d.cb) {
#pragma unroll
      for (int j = 0; j < NQ; ++j) qv[j] = b.q[j];
      m = kNegInf;
      l = 0.f;
#pragma unroll
      for (int j = 0; j < BPL; ++j) acc[j] = 0.f;
      bad = false;
    }
    bad = bad || b.bad;
    if constexpr (APP) {
      if (is_app_chunk(d)) {
        // each lane quantises its 4 elements (the same quant4 steps as the
        // append's); the lanes of token L - 1's row gather their BPL codes
        // of K (from lanes NWD(l%8) .. +NWD-1) and of V (D / 4 + the same)
        constexpr int QL = D / 4;
        const float inv = (lane % (2 * QL)) < QL ? k_inv : v_inv;
        const int qd = (int)quant4(lo16<DT>(b.nw0) * inv, hi16<DT>(b.nw0) * inv, lo16<DT>(b.nw1) * inv,
                                   hi16<DT>(b.nw1) * inv);
        const int sl = (lane & 7) * NWD;
        kv_t kc, vc;
#pragma unroll
        for (int j = 0; j < NWD; ++j) {
          kc[j] = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (sl + j), qd);
          vc[j] = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (QL + sl + j), qd);
        }
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
      float dot = 0.f;
#pragma unroll
      for (int j = 0; j < NWD; ++j) {
        // four codes -> two pairs of the query's type (exact), two dot2 steps
        const uint32_t w = b.k[i][j];
        dot = dot2<DT>(qv[j / 2][2 * (j & 1)], pair16<DT>(w, false), dot);
        dot = dot2<DT>(qv[j / 2][2 * (j & 1) + 1], pair16<DT>(w, true), dot);
      }
      const float dd = group_sum<FLPT>(dot) * scale_log2;
      z[i] = valid ? dd : kNegInf;
      const kv_t zero = {};
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
    for (int j = 0; j < BPL; ++j) acc[j] *= alpha;
#pragma unroll
    for (int i = 0; i < FNL; ++i) {
#pragma unroll
      for (int j = 0; j < NWD; ++j) {
        // four codes -> two binary16 pairs (exact), mixed-precision FMAs
        const uint32_t w = b.v[i][j];
        const uint32_t h0 = pair16<DT_F16>(w, false), h1 = pair16<DT_F16>(w, true);
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
      for (int j = 0; j < BPL; ++j) {
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
        uint32_t w[BPL / 2];
#pragma unroll
        for (int j = 0; j < BPL / 2; ++j)
          w[j] = (uint32_t)to16<DT>(acc[2 * j] * f + nanv) | ((uint32_t)to16<DT>(acc[2 * j + 1] * f + nanv) << 16);
        uint16_t *o = outp + g * D + qoff;
#pragma unroll
        for (int j = 0; j < NQ; ++j)
          *reinterpret_cast<u32x4 *>(o + 8 * j) = u32x4{w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]};
      } else {
        const int64_t u = worker + g;
        float *o = ws_o + u * D + qoff;
#pragma unroll
        for (int j = 0; j < BPL; ++j) o[j] = acc[j] * v_scale + nanv;
        if (lane == 0) {
          ws_m[u] = m * kLn2 + nanv;  // natural-log units
          ws_l[u] = l + nanv;
        }
      }
    }
  }
};

template <int DT, int D, int B, int NW, bool NT, bool APP>
__global__ __launch_bounds__(NW * 64) void decode_fp8_kernel(DecodeParams a) {
  using ST = Fp8Stream<DT, D, B, NT, APP>;
  constexpr int FTC = ST::FTC;
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

template <int DT, int D, bool NT, bool APP>
const void *fp8_ptr(int B) {
  switch (B) {
    case 8: return reinterpret_cast<const void *>(&decode_fp8_kernel<DT, D, 8, kFp8Waves, NT, APP>);
    case 16: return reinterpret_cast<const void *>(&decode_fp8_kernel<DT, D, 16, kFp8Waves, NT, APP>);
    case 32: return reinterpret_cast<const void *>(&decode_fp8_kernel<DT, D, 32, kFp8Waves, NT, APP>);
    case 64: return reinterpret_cast<const void *>(&decode_fp8_kernel<DT, D, 64, kFp8Waves, NT, APP>);
    default: return nullptr;
  }
}

template <int DT, int D, int B, bool APP>
void launch_fp8_app(const DecodeParams &a, hipStream_t st) {
  if (a.stream_kv)
    hipLaunchKernelGGL((decode_fp8_kernel<DT, D, B, kFp8Waves, true, APP>), dim3(a.G / kFp8Waves),
                       dim3(kFp8Waves * 64), fp8_lds_bytes(a.S), st, a);
  else
    hipLaunchKernelGGL((decode_fp8_kernel<DT, D, B, kFp8Waves, false, APP>), dim3(a.G / kFp8Waves),
                       dim3(kFp8Waves * 64), fp8_lds_bytes(a.S), st, a);
}

template <int DT, int B>
hipError_t launch_fp8(const DecodeParams &a, hipStream_t st) {
  if (a.D == 64) {
    if (a.append) launch_fp8_app<DT, 64, B, true>(a, st);
    else launch_fp8_app<DT, 64, B, false>(a, st);
  } else {
    if (a.append) launch_fp8_app<DT, 128, B, true>(a, st);
    else launch_fp8_app<DT, 128, B, false>(a, st);
  }
  return hipGetLastError();
}

}  // namespace

int fp8_chunk_tokens(int head_dim) { return head_dim == 64 ? F8Geo<64>::TC : F8Geo<128>::TC; }

size_t fp8_lds_bytes(int num_seqs) {
  return (size_t)(num_seqs + 1) * sizeof(int64_t) + (size_t)num_seqs * sizeof(int32_t);
}

const void *fp8_kernel(int dtype, int head_dim, int block_size, int nt, int append) {
  if (head_dim != 64 && head_dim != 128) return nullptr;
#define PKV_P(DT, D)                                                                                   \
  if (append) return nt ? fp8_ptr<DT, D, true, true>(block_size) : fp8_ptr<DT, D, false, true>(block_size); \
  return nt ? fp8_ptr<DT, D, true, false>(block_size) : fp8_ptr<DT, D, false, false>(block_size);
  if (dtype == DT_F16) {
    if (head_dim == 64) { PKV_P(DT_F16, 64) }
    PKV_P(DT_F16, 128)
  }
  if (head_dim == 64) { PKV_P(DT_BF16, 64) }
  PKV_P(DT_BF16, 128)
#undef PKV_P
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
  const int64_t threads = (int64_t)a.S * a.Hkv * (a.D / 16);
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
