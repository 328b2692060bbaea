// Paged attention for several query rows per KV head, on the matrix cores.
//
// Two cases share one kernel: grouped-query decode (G query heads read the
// same KV head, the Llama-2-70B shape of the iaim.asia block-table article,
// "末尾块的内部碎片") and multi-token queries (the last Q tokens of each
// sequence attend causally over its paged context, as when several new
// tokens are verified or prefilled in one step).  A KV head's row of the
// batch is streamed once for all its M = G * Q query rows (M <= 16), so the
// K/V bytes per query row drop by M, and the per-chunk products become small
// real contractions:
//   S^T (16 tokens x 16 rows) = K (16 x 128) * Q^T (128 x 16)  -- 4 x v_mfma_f32_16x16x32
//   O^T (128 dims x 16 rows) += V^T (128 x 16 tokens) * P^T   -- 8 x v_mfma_f32_16x16x16
// What is computed is the attention equation of "PagedAttention 完全拆解",
// 背景, per query row, over the tokens its position may see.
//
// Register layouts (checked on the device):
//  * K operand: lane l holds token l%16, dims 32j + 8(l/16) .. +8 for k-slice
//    j -- the 16x16x32 A operand (row l%16, k-group l/16).  Loaded that way a
//    load instruction would touch 16 rows x 64 bytes (half cache lines), so
//    16-bit K is loaded as whole rows (lane l of load j: token 4j + l/16,
//    dims 8(l%16) .. +8) and transposed through a per-wavefront LDS tile
//    before the products (5% faster on the Llama-2-70B shape).
//  * Q: lane l holds query row l%16, the same dims -- the B operand of Q^T.
//  * S^T result: lane l holds tokens 4(l/16) .. +4 of row l%16 -- the B
//    operand P^T of the 16x16x16 product (k = tokens 4(l/16) .. +4).
//  * V: lane l loads tokens 4(l/16) + t (t < 4), dims 8(l%16) .. +8; element
//    s of those four rows is the A operand V^T for output dims 8r + s.
//  * O^T result for slice s: lane l holds dims 8(4(l/16) + i) + s of row l%16,
//    so a lane ends with four runs of 8 consecutive dims of its row.
// Each row's online softmax (max, sum) lives in the four lanes holding it.
//
// FP8 (e4m3) pools (F8): K and V codes are widened in registers to the query's
// 16-bit type (every e4m3 value is exact in binary16 and bfloat16) and go
// through the same products.  K: lane l loads bytes 32(l/16) .. +32 of token
// l%16 and takes dims 32(l/16) + 8j .. +8 as k-slice j; the query fragment
// uses the same dims (a dot product does not depend on how dims are assigned
// to k-slots).  V: lane l loads bytes 8(l%16) .. +8 of tokens 4(l/16) + t.
// The K scale is folded into the score scale, the V scale multiplies the V
// sums when a piece is written.  The weighted V sum of e4m3 pools runs in
// binary16 whatever the query type (V is exact in it, the weights round to
// 11 bits as on the binary16 path): one product per slice.
// The work split, the pipeline (table entries two chunks ahead, K/V one
// chunk ahead, arithmetic on the current chunk; a piece's query fragments come
// with its first chunk) and the partial results / merge follow the balanced
// decode kernel; rows are (sequence, KV head).

#include <type_traits>

#include "pkv_device.h"
#include "pkv_launch.h"
#include "pkv_split.h"

namespace pkv {

namespace {

constexpr int kGroupWaves = PKV_DECODE_WAVES;
constexpr int GTC = 16;  // tokens per MFMA tile (and per chunk of 16-bit pools)

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float f4_t __attribute__((ext_vector_type(4)));

// S^T += K * Q^T for one 32-dim slice (operands as loaded: 8 elements a lane).
template <int DT>
__device__ __forceinline__ f4_t mfma_qk(const u32x4 &k, const u32x4 &q, f4_t c) {
  if constexpr (DT == DT_F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, k), __builtin_bit_cast(half8_t, q),
                                                  c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8_t, k), __builtin_bit_cast(bf8_t, q), c,
                                                   0, 0, 0);
}

// f32 pair -> packed 16-bit pair of the element type, round to nearest even.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return (uint32_t)to16<DT>(a) | ((uint32_t)to16<DT>(b) << 16);
}

// Eight e4m3 codes (two dwords) -> eight values of the 16-bit type, exactly
// (every e4m3 value is a binary16 and a bfloat16 value): gfx950's packed
// conversions, two codes per instruction, with a unit scale.
template <int DT>
__device__ __forceinline__ u32x4 widen8(uint32_t w0, uint32_t w1) {
  typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
  if constexpr (DT == DT_F16) {
    return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true))};
  } else {
    return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true))};
  }
}

// O^T += V^T * P^T for one 16-dim slice; p holds 4 weights as two packed
// 16-bit pairs (f16: one product; bf16: the weights are split into a bf16
// high part and a bf16 remainder, two products, so the weights keep 16 bits).
template <int DT>
__device__ __forceinline__ f4_t mfma_pv(uint32_t v01, uint32_t v23, uint32_t p01, uint32_t p23, uint32_t r01,
                                        uint32_t r23, f4_t c) {
  const uint32_t va[2] = {v01, v23};
  if constexpr (DT == DT_F16) {
    const uint32_t pa[2] = {p01, p23};
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4_t, va), __builtin_bit_cast(half4_t, pa), c,
                                                 0, 0, 0);
  } else {
    const uint32_t pa[2] = {p01, p23};
    const uint32_t ra[2] = {r01, r23};
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4_t, va), __builtin_bit_cast(short4_t, pa),
                                                  c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4_t, va),
                                                     __builtin_bit_cast(short4_t, ra), c, 0, 0, 0);
  }
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// GDIM: head_dim, 128 or (16-bit pools) 64.  At 64, K rows are 8 lanes x 16
// bytes (8 rows per load instruction, two loads per 16-token tile), S^T takes
// 2 k-slices, and O^T 4 slices: slice s gives output dim 8(m % 8) + 2s +
// m / 8 to operand row m, so that a lane (r, g) of the V load, which holds
// dims 8(r % 8) .. +8, supplies element 2s + r / 8 of them.
template <int DT, int B, bool NT, bool F8, int GDIM = 128>
struct GroupStream {
  static_assert(GDIM == 128 || GDIM == 64, "head_dim 64 or 128");
  static constexpr int KPT = GDIM / 64;  // e4m3: 16-byte K loads per lane per 16-token tile
  static constexpr int NKS = GDIM / 32;  // k-slices of S^T (and whole-row K loads per 16-token tile)
  static constexpr int NS = GDIM / 16;   // 16-dim slices of O^T
  // tokens per chunk: e4m3 chunks hold two 16-token tiles, so that a stage
  // keeps as many bytes in flight as a 16-bit one
  static constexpr int TC = F8 ? 2 * GTC : GTC;
  static constexpr int NSUB = TC / GTC;
  static constexpr int NE = TC >= B ? TC / B : 1;  // table entries per chunk

  struct Buf16 {
    u32x4 k[NKS], v[4], q[NKS];
    bool bad;
  };
  struct Buf8 {
    u32x4 k[2 * KPT];  // 16 KPT codes of token r of each tile (k[KPT u] ..: tile u)
    u32x2 v[8];        // 8 codes of each of tokens 4g .. 4g+3 of each tile (v[4u + t])
    u32x4 q[NKS];
    bool bad;
  };
  using Buf = typename std::conditional<F8, Buf8, Buf16>::type;

  // constants of the call
  const char *kp;  // pools as bytes
  const char *vp;
  const uint16_t *qp;
  const int32_t *tables;
  uint16_t *outp;
  float *ws_m;
  float *ws_l;
  float *ws_o;
  int64_t blk_stride, num_blocks;
  int64_t tstride;  // table entries between the rows of two sequences of this launch
  bool pfx;         // the prefix pass of a shared-prefix decode
  float *pfx_m;
  float *pfx_l;
  float *pfx_o;
  int S, Hkv, H, maxb, nq, gq, M;
  float scale_log2, v_scale;
  int lane, g, r;
  int64_t worker;
  // 16-bit pools: this wavefront's K transpose tile (16 token rows of kKRow
  // 16-byte pieces; the padding piece keeps 16 lanes' reads off one bank).
  static constexpr int kKRow = GDIM / 8 + 1;
  static constexpr int kTile = 16 * kKRow;
  // A whole row's output (M rows of GDIM 16-bit values): with 16-bit pools
  // at head_dim 128 (kTileOut) and M > 8 it passes through the K tile, so
  // that a store instruction writes whole rows; stored from the lanes' runs,
  // an instruction puts 16 bytes in each of 32 lines (16 query tokens: split
  // pass 94 against 91.5 us).  Otherwise the lanes store their runs: with
  // M <= 8, and over e4m3 pools, the tiled stores measured no faster, and at
  // head_dim 64 their registers would cost a wave per SIMD.  Keeping a whole
  // row's output in LDS until the stream ends (as the first cut piece is)
  // gained nothing either.
  static constexpr bool kTileOut = !F8 && GDIM == 128;
  u32x4 *ktile;
  ChunkCursor<TC> cur;  // the slice, chunk by chunk
  // running state of the current piece (row r of this lane)
  f4_t acc[NS];
  // The piece's query fragments, loaded with its first chunk and held for
  // the rest (this saves the query re-reads, up to 4 KiB per chunk, that
  // otherwise queue beside the K/V reads).  e4m3 at head_dim 64 re-reads them
  // with every chunk instead: holding them costs the register room of its
  // third wave per SIMD, which is worth more there.
  static constexpr bool kHoldQ = !(F8 && GDIM == 64);
  u32x4 qf[NKS];
  float m, lp;
  bool bad;
  // The wavefront's first cut piece (a slice that starts inside a row)
  // finishes in the middle of its stream.  Its partial results are kept in
  // LDS (row i at stage + i * kStageRow floats) and written to the workspace
  // when the stream ends: stores issued mid-stream would hold up the
  // wavefront's later loads until they complete (the vector memory counter
  // counts loads and stores in one order).  At most two pieces of a slice are
  // cut, the first and the last, and the last ends the stream anyway.
  // e4m3 pools at head_dim 64 store the piece directly: the stage's
  // registers would cost that kernel its third wave per SIMD (measured
  // slower).
  static constexpr bool kStage = !(F8 && GDIM == 64);
  static constexpr int kStageRow = GDIM + 4;  // +16 bytes: rows start in different banks
  float *stage;
  bool staged;     // wave-uniform: the stage holds a piece
  int64_t st_u0;   // its first workspace slot (row 0)
  float st_m, st_l;  // its max (natural-log units) and sum, for this lane's row

  __device__ __forceinline__ void init(const DecodeParams &a, const int64_t *cum_, const int32_t *lens_, int lane_) {
    kp = reinterpret_cast<const char *>(a.k_pool);
    vp = reinterpret_cast<const char *>(a.v_pool);
    qp = reinterpret_cast<const uint16_t *>(a.q);
    tables = a.tables;
    outp = reinterpret_cast<uint16_t *>(a.out);
    ws_m = a.ws_m;
    ws_l = a.ws_l;
    ws_o = a.ws_o;
    cur.init(cum_, lens_, a.S, a.Hkv, lane_);
    blk_stride = (int64_t)a.Hkv * B * GDIM;
    num_blocks = a.num_blocks;
    S = a.S;
    Hkv = a.Hkv;
    H = a.H;
    maxb = a.maxb;
    pfx = a.pfx_pass == 1;
    // prefix pass: group i reads the table row of its first sequence
    tstride = (int64_t)a.maxb * (pfx ? a.pfx_group : 1);
    pfx_m = a.pfx_m;
    pfx_l = a.pfx_l;
    pfx_o = a.pfx_o;
    nq = a.nq;
    gq = a.H / a.Hkv;
    M = gq * nq;
    scale_log2 = a.scale_log2;
    v_scale = a.v_scale;
    lane = lane_;
    g = lane >> 4;
    r = lane & 15;
  }

  __device__ __forceinline__ static int first_block(int c) { return TC >= B ? c * (TC / B) : c / (B / TC); }
  __device__ __forceinline__ static int last_block(const Chunk &d) { return (min(d.L, d.ce * TC) - 1) / B; }

  // Stage 1: this lane's table entry of chunk d (clamped to the piece's last
  // block; tokens past it are masked).
  __device__ __forceinline__ uint32_t load_entries(const Chunk &d) const {
    const int lb = min(first_block(d.c) + min(lane, NE - 1), last_block(d));
    return (uint32_t)tables[(int64_t)d.s * tstride + lb];
  }

  // The chunk's blocks (NE <= 4 wave-uniform block numbers, from its table
  // entries); an entry outside the pool marks the chunk bad and reads block 0
  // instead.  Named values rather than an array, and 32-bit: the per-token
  // selection below then stays in registers.
  struct Blocks {
    int b0, b1, b2, b3;
  };

  __device__ __forceinline__ int block_of(uint32_t e, int i, bool &bd) const {
    const int blk = __builtin_amdgcn_readlane((int)e, i);
    const bool out = blk < 0 || (int64_t)blk >= num_blocks;
    bd = bd || out;
    return out ? 0 : blk;
  }

  __device__ __forceinline__ Blocks chunk_blocks(uint32_t e, bool &bd) const {
    static_assert(NE == 1 || NE == 2 || NE == 4, "1, 2 or 4 blocks per chunk");
    Blocks bk;
    bk.b0 = block_of(e, 0, bd);
    bk.b1 = bk.b2 = bk.b3 = bk.b0;
    if constexpr (NE > 1) bk.b1 = block_of(e, 1, bd);
    if constexpr (NE > 2) {
      bk.b2 = block_of(e, 2, bd);
      bk.b3 = block_of(e, 3, bd);
    }
    return bk;
  }

  // Element offset of token t (0 <= t < TC) of chunk d.
  __device__ __forceinline__ int64_t token_off(const Chunk &d, Blocks bk, int t) const {
    const int64_t hoff = (int64_t)d.h * B * GDIM;
    if constexpr (TC >= B) {
      const int i = t / B;
      int blk = bk.b0;
      if constexpr (NE > 1) blk = i == 1 ? bk.b1 : blk;
      if constexpr (NE > 2) {
        blk = i == 2 ? bk.b2 : blk;
        blk = i == 3 ? bk.b3 : blk;
      }
      return (int64_t)blk * blk_stride + hoff + (int64_t)(t & (B - 1)) * GDIM;
    } else {
      return (int64_t)bk.b0 * blk_stride + hoff + (int64_t)((d.c % (B / TC)) * TC + t) * GDIM;
    }
  }

  // Stage 2: K rows (16-bit: whole rows of tokens 4j + g; e4m3: token r), V
  // rows (tokens 4g .. 4g+3) of chunk d, and with the first chunk of a piece
  // its query rows (the same for all its chunks).
  // Tokens past the context read the row of token L - 1 instead (cache
  // lines already fetched: the unused tail of the last block costs no HBM
  // traffic); they are masked.
  __device__ __forceinline__ void load_kv(const Chunk &d, uint32_t e, Buf &b) const {
    bool bd = false;
    const Blocks bb = chunk_blocks(e, bd);
    const int last = d.L - 1 - d.c * TC;  // token L - 1 relative to the chunk
    // query row r of this KV head (rows >= M read row 0; their results are
    // never written)
    const int rr = r < M ? r : 0;
    const int qi = rr / gq, gi = rr - (rr / gq) * gq;
    const int64_t qrow = (((int64_t)d.s * nq + qi) * H + (int64_t)d.h * gq + gi) * GDIM;
    if constexpr (F8) {
      // K: lane (r, g) takes codes 16 KPT g .. +16 KPT of token r (dims of
      // k-slices j: 16 KPT g + 8j .. +8, and the query fragment the same);
      // V: 8 codes of tokens 4g + t at dims 8(r % (GDIM / 8))
#pragma unroll
      for (int u = 0; u < NSUB; ++u) {
        const int64_t kb = token_off(d, bb, min(GTC * u + r, last)) + 16 * KPT * g;
#pragma unroll
        for (int i = 0; i < KPT; ++i) b.k[KPT * u + i] = ld_kv<NT>(kp + kb + 16 * i);
        // four consecutive tokens from a multiple of 4 lie in one block
        const int t0 = min(GTC * u + 4 * g, last);
        const int64_t vb = token_off(d, bb, t0) + 8 * (r % (GDIM / 8));
#pragma unroll
        for (int t = 0; t < 4; ++t)
          b.v[4 * u + t] = ld_kv8<NT>(vp + vb + (int64_t)(min(GTC * u + 4 * g + t, last) - t0) * GDIM);
      }
      if (!kHoldQ || d.c == d.cb) {
#pragma unroll
        for (int j = 0; j < NKS; ++j)
          b.q[j] = *reinterpret_cast<const u32x4 *>(qp + qrow + 16 * KPT * g + 8 * j);
      }
    } else {
      // whole token rows (GDIM / 8 lanes a row): lane l of load j gets token
      // j * RPL + l / (GDIM / 8), dims 8(l % (GDIM / 8)) .. +8; consume
      // transposes them into the matrix-core layout through LDS
      constexpr int LPR = GDIM / 8;  // lanes per row
      constexpr int RPL = 64 / LPR;  // rows per load
#pragma unroll
      for (int j = 0; j < NKS; ++j) {
        const int64_t kb = token_off(d, bb, min(RPL * j + lane / LPR, last)) + 8 * (lane % LPR);
        b.k[j] = ld_kv<NT>(kp + 2 * kb);
      }
      const int t0 = min(4 * g, last);
      const int64_t vb = token_off(d, bb, t0) + 8 * (r % LPR);
#pragma unroll
      for (int t = 0; t < 4; ++t) b.v[t] = ld_kv<NT>(vp + 2 * (vb + (int64_t)(min(4 * g + t, last) - t0) * GDIM));
      if (d.c == d.cb) {
#pragma unroll
        for (int j = 0; j < NKS; ++j) b.q[j] = *reinterpret_cast<const u32x4 *>(qp + qrow + 8 * g + 32 * j);
      }
    }
    b.bad = bd;
  }

  // One 16-token tile starting at token t0: scores, online softmax and the
  // weighted V sum.  The running max m is the reference the weights are
  // taken against; it is raised, and the sums rescaled, only on tiles where
  // some row's score passes it by more than kRaise (log2 units): the
  // conditional rescaling of FlashAttention-4, which gives the same softmax
  // up to rounding, keeps every weight below 2^kRaise and lets most tiles
  // skip the rescale of the 4 x NS accumulators.
  static constexpr float kRaise = 8.f;

  __device__ __forceinline__ void tile(const Chunk &d, int t0, const u32x4 (&kk)[NKS], const u32x4 (&vv)[4],
                                       const u32x4 (&q)[NKS]) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    f4_t st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NKS; ++j) st = mfma_qk<DT>(kk[j], q[j], st);
    // row r sees tokens [t_lo, min(t_hi, its causal limit)); rows >= M
    // follow row 0 (prefix pass: every row sees the whole shared prefix)
    const int t_lo = d.cb * TC;
    const int t_hi = min(d.L, d.ce * TC);
    const int lim0 = pfx ? d.L : d.L - nq + 1;
    float sc[4];
    u32x4 v[4];
    if (t0 >= t_lo && t0 + GTC <= min(t_hi, lim0)) {
      // a tile inside every row's range: nothing masked
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[i] = st[i] * scale_log2;
#pragma unroll
      for (int t = 0; t < 4; ++t) v[t] = vv[t];
    } else {
      const int t_row = min(t_hi, pfx || r >= M ? lim0 : lim0 + r / gq);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = t0 + 4 * g + i;
        sc[i] = (tok >= t_lo && tok < t_row) ? st[i] * scale_log2 : kNegInf;
      }
      // V rows of tokens outside [t_lo, t_hi) are zeroed (unused slots may hold NaN)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int tok = t0 + 4 * g + t;
        v[t] = (tok >= t_lo && tok < t_hi) ? vv[t] : zero;
      }
    }
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const bool raise = mx > m + kRaise;  // m == -inf: any valid score
    if (__ballot(raise) != 0) {
      const float alpha = raise ? fast_exp2(m - mx) : 1.f;  // m == -inf gives 0
      lp *= alpha;
#pragma unroll
      for (int s_ = 0; s_ < NS; ++s_) acc[s_] *= alpha;
      m = raise ? mx : m;
    }
    const float mref = (m == kNegInf) ? 0.f : m;  // no valid token yet
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = fast_exp2(sc[i] - mref);  // -inf gives 0
    lp += (p[0] + p[1]) + (p[2] + p[3]);
    constexpr int PT = F8 ? DT_F16 : DT;  // type of the weighted V sum's operands
    uint32_t p01, p23, r01 = 0, r23 = 0;
    if constexpr (PT == DT_F16) {
      p01 = pack2<PT>(p[0], p[1]);
      p23 = pack2<PT>(p[2], p[3]);
    } else {
      p01 = pack2<PT>(p[0], p[1]);
      p23 = pack2<PT>(p[2], p[3]);
      r01 = pack2<PT>(p[0] - lo16<PT>(p01), p[1] - hi16<PT>(p01));
      r23 = pack2<PT>(p[2] - lo16<PT>(p23), p[3] - hi16<PT>(p23));
    }
#pragma unroll
    for (int s_ = 0; s_ < NS; ++s_) {
      // element e of the four V rows: dword e / 2, low or high half (e = s_
      // at head_dim 128; 2 s_ + r / 8 at 64)
      const int hi = GDIM == 128 ? (s_ & 1) : (r >> 3);
      const int dw = GDIM == 128 ? (s_ >> 1) : s_;
      const uint32_t sel = hi ? 0x07060302u : 0x05040100u;
      const uint32_t v01 = __builtin_amdgcn_perm(v[1][dw], v[0][dw], sel);
      const uint32_t v23 = __builtin_amdgcn_perm(v[3][dw], v[2][dw], sel);
      acc[s_] = mfma_pv<PT>(v01, v23, p01, p23, r01, r23, acc[s_]);
    }
  }

  // Stage 3: scores, online softmax and the weighted V sum of chunk d.
  __device__ __forceinline__ void consume(const Chunk &d, Buf &b) {
    if (d.c == d.cb) {
      m = kNegInf;
      lp = 0.f;
#pragma unroll
      for (int s_ = 0; s_ < NS; ++s_) acc[s_] = f4_t{0.f, 0.f, 0.f, 0.f};
      bad = false;
#pragma unroll
      for (int j = 0; j < NKS; ++j) qf[j] = b.q[j];
    }
    bad = bad || b.bad;
#pragma unroll
    for (int u = 0; u < NSUB; ++u) {
      u32x4 kk[NKS], vv[4];  // K and V fragments of tile u in the 16-bit type
      if constexpr (F8) {
#pragma unroll
        for (int j = 0; j < NKS; ++j)
          kk[j] = widen8<DT>(b.k[KPT * u + (j >> 1)][2 * (j & 1)], b.k[KPT * u + (j >> 1)][2 * (j & 1) + 1]);
#pragma unroll
        for (int t = 0; t < 4; ++t) vv[t] = widen8<DT_F16>(b.v[4 * u + t][0], b.v[4 * u + t][1]);
      } else {
        // K rows -> this wavefront's LDS tile -> lane (r, g) reads token r's
        // dims 32j + 8g .. +8 for k-slice j (rows padded by one 16-byte piece,
        // so neither the writes nor the reads of 16 lanes share a bank)
        constexpr int LPR = GDIM / 8, RPL = 64 / LPR;
#pragma unroll
        for (int j = 0; j < NKS; ++j) ktile[(RPL * j + lane / LPR) * kKRow + lane % LPR] = b.k[j];
#pragma unroll
        for (int j = 0; j < NKS; ++j) kk[j] = ktile[r * kKRow + 4 * j + g];
#pragma unroll
        for (int t = 0; t < 4; ++t) vv[t] = b.v[t];
      }
      tile(d, d.c * TC + GTC * u, kk, vv, kHoldQ ? qf : b.q);
    }
    if (d.c == d.ce - 1) finish_piece(d);
  }

  __device__ __forceinline__ void finish_piece(const Chunk &d) {
    lp += __shfl_xor(lp, 16);
    lp += __shfl_xor(lp, 32);
    const bool cut = !(d.cb == 0 && d.ce * TC >= d.L);
    const bool to_stage = kStage && cut && !staged;
    staged = staged || to_stage;
    // every lane takes part in flush(): the slot is set here, before the
    // lanes of rows >= M leave
    if (to_stage) st_u0 = (worker + (int64_t)d.s * Hkv + d.h) * M;
    if constexpr (F8) {
#pragma unroll
      for (int s_ = 0; s_ < NS; ++s_) acc[s_] *= v_scale;
    }
    if constexpr (GDIM == 128) {
      // slice s_, value i: dim 8(4g + i) + s_ -- four runs of 8 dims per lane
      float run[4][8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int s_ = 0; s_ < 8; ++s_) run[i][s_] = acc[s_][i];
      }
      const int run_dim[4] = {8 * (4 * g), 8 * (4 * g + 1), 8 * (4 * g + 2), 8 * (4 * g + 3)};
      end_piece<4>(d, run, run_dim, cut, to_stage);
    } else {
      // slice s_, value i: element 2 s_ + (g / 2) of the block 4(g % 2) + i,
      // so lanes (r, g) and (r, g ^ 2) hold the even and the odd elements of
      // the same four blocks; they swap halves and keep two whole blocks each
      const bool even = g < 2;
      float recv[8];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
#pragma unroll
        for (int t = 0; t < 4; ++t) recv[4 * k + t] = __shfl_xor(even ? acc[t][2 + k] : acc[t][k], 32);
      }
      float run[2][8];
      int run_dim[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        run_dim[k] = 8 * (4 * (g & 1) + (even ? k : 2 + k));
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          run[k][2 * t] = even ? acc[t][k] : recv[4 * k + t];
          run[k][2 * t + 1] = even ? recv[4 * k + t] : acc[t][2 + k];
        }
      }
      end_piece<2>(d, run, run_dim, cut, to_stage);
    }
  }

  // Eight output values of a run, normalised and rounded to the element type.
  __device__ __forceinline__ static u32x4 pack8(const float (&v)[8], float inv, float nanv) {
    u32x4 w;
    w.x = pack2<DT>(v[0] * inv + nanv, v[1] * inv + nanv);
    w.y = pack2<DT>(v[2] * inv + nanv, v[3] * inv + nanv);
    w.z = pack2<DT>(v[4] * inv + nanv, v[5] * inv + nanv);
    w.w = pack2<DT>(v[6] * inv + nanv, v[7] * inv + nanv);
    return w;
  }

  // A whole row (not a prefix pass, kTileOut, M > 8): its final output
  // through the tile, with every lane; otherwise the lanes of rows < M write
  // the piece.
  template <int NR>
  __device__ __forceinline__ void end_piece(const Chunk &d, const float (&run)[NR][8], const int (&run_dim)[NR],
                                            bool cut, bool to_stage) {
    if constexpr (kTileOut) {
      if (!cut && !pfx && M > 8) {
        // lane (r, g) leaves its runs at piece run_dim / 8 of tile row r
        if (r < M) {
          const float nanv = bad ? __builtin_nanf("") : 0.f;
          const float inv = 1.f / lp;
#pragma unroll
          for (int i = 0; i < NR; ++i) ktile[r * kKRow + run_dim[i] / 8] = pack8(run[i], inv, nanv);
        }
        store_out_rows(((int64_t)d.s * nq * H + (int64_t)d.h * gq) * GDIM,
                       [&](int rr, int p) { return ktile[rr * kKRow + p]; });
        return;
      }
    }
    if (r >= M) return;
    write_piece<NR>(d, run, run_dim, to_stage);
  }

  // Lane l stores piece l % PPR of query row RPI j + l / PPR of the output
  // rows whose pieces src(rr, p) returns (rr < 16), so that a store
  // instruction writes RPI whole rows; row (qi, gi) lies (qi H + gi) GDIM
  // elements past row (0, 0) at o_base.
  template <class Src>
  __device__ __forceinline__ void store_out_rows(int64_t o_base, Src src) {
    constexpr int PPR = GDIM / 8;  // 16-byte pieces per row
    constexpr int RPI = 64 / PPR;  // rows per store instruction
    const int p = lane % PPR;
    const float inv_gq = 1.f / (float)gq;
#pragma unroll 1  // unrolled, the rounds' registers cost a wave per SIMD
    for (int j = 0; j < 16 / RPI; ++j) {
      if (RPI * j >= M) break;
      const int rr = RPI * j + lane / PPR;
      const u32x4 w = src(min(rr, 15), p);
      // rr / gq: (rr + 1/2) / gq lies at least 1/32 from an integer
      const int qi = (int)(((float)rr + 0.5f) * inv_gq);
      const int gi = rr - qi * gq;
      if (rr < M) *reinterpret_cast<u32x4 *>(outp + o_base + (qi * H + gi) * GDIM + 8 * p) = w;
    }
  }

  // The staged piece to the workspace: its M rows of GDIM floats are
  // contiguous there (slots st_u0 ..), so every store instruction writes
  // whole lines.
  __device__ __forceinline__ void flush() {
    if (!staged) return;
    constexpr int PR = GDIM / 4;  // 16-byte pieces per row
    f4_t *dst = reinterpret_cast<f4_t *>(ws_o + st_u0 * GDIM);
    for (int i = lane; i < M * PR; i += 64) {
      const int row = i / PR, col = i - (i / PR) * PR;
      dst[i] = *reinterpret_cast<const f4_t *>(stage + row * kStageRow + 4 * col);
    }
    if (g == 0 && r < M) {
      ws_m[st_u0 + r] = st_m;
      ws_l[st_u0 + r] = st_l;
    }
  }

  // The finished piece of this lane's row r (a cut piece, or a whole row not
  // stored through the tile): runs of 8 consecutive dims.
  template <int NR>
  __device__ __forceinline__ void write_piece(const Chunk &d, const float (&run)[NR][8], const int (&run_dim)[NR],
                                              bool to_stage) {
    const int qi = r / gq, gi = r - (r / gq) * gq;
    const float nanv = bad ? __builtin_nanf("") : 0.f;
    if (pfx && d.cb == 0 && d.ce * TC >= d.L) {
      // the whole row of a prefix pass: its softmax state (max in log2
      // units, sum, unnormalised V sums) for the suffix pass
      const int64_t pi = ((int64_t)d.s * nq + qi) * H + (int64_t)d.h * gq + gi;
      float *o = pfx_o + pi * GDIM;
#pragma unroll
      for (int i = 0; i < NR; ++i) {
#pragma unroll
        for (int e = 0; e < 8; ++e) o[run_dim[i] + e] = run[i][e] + nanv;
      }
      if (g == 0) {
        pfx_m[pi] = m + nanv;
        pfx_l[pi] = lp + nanv;
      }
    } else if (d.cb == 0 && d.ce * TC >= d.L) {
      // the whole row: final output
      uint16_t *o = outp + (((int64_t)d.s * nq + qi) * H + (int64_t)d.h * gq + gi) * GDIM;
      const float inv = 1.f / lp;
#pragma unroll
      for (int i = 0; i < NR; ++i) *reinterpret_cast<u32x4 *>(o + run_dim[i]) = pack8(run[i], inv, nanv);
    } else if (to_stage) {
      float *o = stage + r * kStageRow;
#pragma unroll
      for (int i = 0; i < NR; ++i) {
#pragma unroll
        for (int e = 0; e < 8; ++e) o[run_dim[i] + e] = run[i][e] + nanv;
      }
      st_m = m * kLn2 + nanv;
      st_l = lp + nanv;
    } else {
      const int64_t u = (worker + (int64_t)d.s * Hkv + d.h) * M + r;
      float *o = ws_o + u * GDIM;
#pragma unroll
      for (int i = 0; i < NR; ++i) {
#pragma unroll
        for (int e = 0; e < 8; ++e) o[run_dim[i] + e] = run[i][e] + nanv;
      }
      if (g == 0) {
        ws_m[u] = m * kLn2 + nanv;  // natural-log units
        ws_l[u] = lp + nanv;
      }
    }
  }
};

template <int DT, int B, int NW, bool NT, bool F8, int GDIM = 128>
__global__ __launch_bounds__(NW * 64) void decode_group_kernel(DecodeParams a) {
  using ST = GroupStream<DT, B, NT, F8, GDIM>;
  extern __shared__ int64_t lds[];
  int64_t *cum = lds;                                         // [S + 1]
  int32_t *lens = reinterpret_cast<int32_t *>(lds + a.S + 1);  // [S]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (wave == 0) build_cost_prefix<ST::TC>(a, a.Hkv, cum, lens, lane, a.pfx_pass == 1 ? 1 : a.nq);
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

  __shared__ u32x4 ktiles[F8 ? 1 : NW * ST::kTile];
  __shared__ float stages[ST::kStage ? NW * 16 * ST::kStageRow : 1];
  ST st;
  st.init(a, cum, lens, lane);
  st.ktile = ktiles + (F8 ? 0 : wave * ST::kTile);
  st.stage = stages + (ST::kStage ? wave * 16 * ST::kStageRow : 0);
  st.staged = false;
  st.worker = w;
  st.cur.enter(lo, hi);
  __builtin_amdgcn_s_setprio(3);
  run_stream(st, (int)(hi - lo));
  __builtin_amdgcn_s_setprio(0);
  st.flush();
}

// One wavefront per (sequence, KV head), for its M query rows: rows of empty
// or invalid contexts, and the LSE merge of rows cut over several workers.
// A row takes LPR lanes (16 when M <= 4, 8 when M <= 8, else 4), so that
// the wavefront's lanes are busy and a load instruction reads whole lines:
// lane c of a row takes dims 4c + 4 LPR k .. +4 (k < GDIM / (4 LPR)) of the
// pieces' partial results.  The pieces' (m, l) and o rows are fetched four
// pieces at a time (rows cut into more pieces: every piece's m first, 4 LPR
// a round).  The compiler issues each piece's loads inside the test for that
// piece, so a row's pieces are loaded one after another; holding all four in
// flight (selects instead of the test, with or without loads of absent
// pieces, 2 or 3 waves per SIMD) measured slower: the merge is bound by the
// cache lines its loads touch more than by their round trips.  With 4 lanes
// a row holding runs of 32 dims, a load instruction touched 16 bytes of 64
// lines; interleaving the dims made the merge 13-26% faster.
// TC: the chunk length of the split pass that wrote the partials; GDIM:
// head_dim.
template <int DT, int TC, int GDIM, int LPR>
__device__ __forceinline__ void merge_rows(const DecodeParams &a, int lane, int64_t grow) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  static_assert(GDIM % (4 * LPR) == 0, "whole float4s per lane");
  const int gq = a.H / a.Hkv;
  const int M = gq * a.nq;
  const int s = (int)(grow / a.Hkv);
  const int h = (int)(grow - (int64_t)s * a.Hkv);
  const int r = lane / LPR;            // this lane's query row
  const int c = lane % LPR;            // and its place among the row's lanes
  constexpr int NV = GDIM / (4 * LPR);  // float4s of this lane's dims
  constexpr int DS = 4 * LPR;           // dims between them
  const int d0 = 4 * c;                 // the first of them
  const bool live = r < M;
  const int qi = r / gq, gi = r - (r / gq) * gq;
  uint16_t *out_row = reinterpret_cast<uint16_t *>(a.out) +
                      (((int64_t)s * a.nq + qi) * a.H + (int64_t)h * gq + gi) * GDIM + d0;
  const int L = a.lens[s];
  const uint64_t cum_s = (uint64_t)a.ws_cum[s];
  const uint64_t total = (uint64_t)a.ws_cum[a.S];
  const bool pfx = a.pfx_pass == 1;
  // prefix pass: a group without a valid prefix leaves no state (the suffix
  // pass then reads none, or marks the row invalid)
  if (pfx && (L <= 0 || L > a.maxb * a.B)) return;
  if (L <= 0 || L > a.maxb * a.B || L < a.nq) {
    const uint32_t v = (L == 0) ? 0u : 0x00010001u * to16<DT>(__builtin_nanf(""));
    if (live) {
#pragma unroll
      for (int k = 0; k < NV; ++k) *reinterpret_cast<u32x2 *>(out_row + DS * k) = u32x2{v, v};
    }
    return;
  }
  const int nch = (L + TC - 1) / TC;
  const uint64_t seg = cum_s + (uint64_t)h * nch;
  const uint64_t end = seg + nch;
  const uint64_t slice = slice_of(total, a.G);
  const int64_t t_a = (int64_t)udiv64(seg, slice);
  const int64_t n = (int64_t)udiv64(end - 1, slice) - t_a + 1;
  if (n <= 1 || !live) return;  // one piece: it wrote the rows
  auto slot = [&](int64_t j) { return (t_a + j + grow) * M + r; };
  // pieces combined in worker order, with the row's max over its pieces
  float mx = kNegInf;
  float lsum = 0.f;
  f4 o[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) o[k] = f4{0.f, 0.f, 0.f, 0.f};
  auto fold = [&](const float (&mv)[4], const float (&lv)[4], const f4 (&ov)[4][NV], int64_t j0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (j0 + q >= n) break;
      const float f = (mv[q] == kNegInf) ? 0.f : fast_exp2((mv[q] - mx) * kLog2e);
      lsum += f * lv[q];
#pragma unroll
      for (int k = 0; k < NV; ++k) o[k] += f * ov[q][k];
    }
  };
  auto fetch = [&](float (&mv)[4], float (&lv)[4], f4 (&ov)[4][NV], int64_t j0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t u = slot(min(j0 + q, n - 1));
      mv[q] = a.ws_m[u];
      lv[q] = a.ws_l[u];
      const float *src = a.ws_o + u * GDIM + d0;
#pragma unroll
      for (int k = 0; k < NV; ++k) ov[q][k] = *reinterpret_cast<const f4 *>(src + DS * k);
    }
  };
  if (n <= 4) {
    // the usual case: every piece in one round of loads
    float mv[4], lv[4];
    f4 ov[4][NV];
    fetch(mv, lv, ov, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) mx = fmaxf(mx, mv[q]);
    fold(mv, lv, ov, 0);
  } else {
    // the max first (the row's lanes take every LPR-th piece, 4 LPR pieces
    // a round), then the sums, four pieces per round
    for (int64_t j0 = 0; j0 < n; j0 += 4 * LPR) {
      float mm[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) mm[i] = a.ws_m[slot(min(j0 + LPR * i + c, n - 1))];
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, mm[i]);
    }
    // across the row's lanes (all live or all not)
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    for (int64_t j0 = 0; j0 < n; j0 += 4) {
      float mv[4], lv[4];
      f4 ov[4][NV];
      fetch(mv, lv, ov, j0);
      fold(mv, lv, ov, j0);
    }
  }
  if (pfx) {
    // the merged softmax state of the prefix (max in log2 units)
    const int64_t pi = ((int64_t)s * a.nq + qi) * a.H + (int64_t)h * gq + gi;
    float *dst = a.pfx_o + pi * GDIM + d0;
#pragma unroll
    for (int k = 0; k < NV; ++k) *reinterpret_cast<f4_t *>(dst + DS * k) = o[k];
    if (c == 0) {
      a.pfx_m[pi] = mx * kLog2e;
      a.pfx_l[pi] = lsum;
    }
    return;
  }
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const uint32_t w0 = (uint32_t)to16<DT>(o[k][0] / lsum) | ((uint32_t)to16<DT>(o[k][1] / lsum) << 16);
    const uint32_t w1 = (uint32_t)to16<DT>(o[k][2] / lsum) | ((uint32_t)to16<DT>(o[k][3] / lsum) << 16);
    *reinterpret_cast<u32x2 *>(out_row + DS * k) = u32x2{w0, w1};
  }
}

template <int DT, int TC, int GDIM = 128>
__global__ __launch_bounds__(256) void decode_group_merge_kernel(DecodeParams a) {
  const int lane = threadIdx.x & 63;
  const int64_t grow = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // s * Hkv + h
  if (grow >= (int64_t)a.S * a.Hkv) return;
  const int M = (a.H / a.Hkv) * a.nq;
  if (M <= 4)
    merge_rows<DT, TC, GDIM, 16>(a, lane, grow);
  else if (M <= 8)
    merge_rows<DT, TC, GDIM, 8>(a, lane, grow);
  else
    merge_rows<DT, TC, GDIM, 4>(a, lane, grow);
}

template <int DT, int B, bool NT, bool F8, int GDIM>
void go_group(const DecodeParams &a, hipStream_t st) {
  hipLaunchKernelGGL((decode_group_kernel<DT, B, kGroupWaves, NT, F8, GDIM>), dim3(a.G / kGroupWaves),
                     dim3(kGroupWaves * 64), group_lds_bytes(a.S), st, a);
}

template <int DT, int B>
hipError_t launch_group(const DecodeParams &a, hipStream_t st) {
  if (a.fp8 && a.D == 64) {
    if (a.stream_kv) go_group<DT, B, true, true, 64>(a, st);
    else go_group<DT, B, false, true, 64>(a, st);
  } else if (a.fp8) {
    if (a.stream_kv) go_group<DT, B, true, true, 128>(a, st);
    else go_group<DT, B, false, true, 128>(a, st);
  } else if (a.D == 64) {
    if (a.stream_kv) go_group<DT, B, true, false, 64>(a, st);
    else go_group<DT, B, false, false, 64>(a, st);
  } else {
    if (a.stream_kv) go_group<DT, B, true, false, 128>(a, st);
    else go_group<DT, B, false, false, 128>(a, st);
  }
  return hipGetLastError();
}

template <int DT, bool NT, bool F8, int GDIM>
const void *group_ptr(int B) {
  switch (B) {
    case 8: return reinterpret_cast<const void *>(&decode_group_kernel<DT, 8, kGroupWaves, NT, F8, GDIM>);
    case 16: return reinterpret_cast<const void *>(&decode_group_kernel<DT, 16, kGroupWaves, NT, F8, GDIM>);
    case 32: return reinterpret_cast<const void *>(&decode_group_kernel<DT, 32, kGroupWaves, NT, F8, GDIM>);
    case 64: return reinterpret_cast<const void *>(&decode_group_kernel<DT, 64, kGroupWaves, NT, F8, GDIM>);
    default: return nullptr;
  }
}

}  // namespace

size_t group_lds_bytes(int num_seqs) {
  return (size_t)(num_seqs + 1) * sizeof(int64_t) + (size_t)num_seqs * sizeof(int32_t);
}

const void *group_kernel(int dtype, int head_dim, int block_size, int nt, int fp8) {
  if (fp8 && head_dim == 64) {
    if (nt) return dtype == DT_F16 ? group_ptr<DT_F16, true, true, 64>(block_size)
                                   : group_ptr<DT_BF16, true, true, 64>(block_size);
    return dtype == DT_F16 ? group_ptr<DT_F16, false, true, 64>(block_size)
                           : group_ptr<DT_BF16, false, true, 64>(block_size);
  }
  if (fp8) {
    if (head_dim != 128) return nullptr;
    if (nt) return dtype == DT_F16 ? group_ptr<DT_F16, true, true, 128>(block_size)
                                   : group_ptr<DT_BF16, true, true, 128>(block_size);
    return dtype == DT_F16 ? group_ptr<DT_F16, false, true, 128>(block_size)
                           : group_ptr<DT_BF16, false, true, 128>(block_size);
  }
  if (head_dim == 64) {
    if (nt) return dtype == DT_F16 ? group_ptr<DT_F16, true, false, 64>(block_size)
                                   : group_ptr<DT_BF16, true, false, 64>(block_size);
    return dtype == DT_F16 ? group_ptr<DT_F16, false, false, 64>(block_size)
                           : group_ptr<DT_BF16, false, false, 64>(block_size);
  }
  if (head_dim != 128) return nullptr;
  if (nt) return dtype == DT_F16 ? group_ptr<DT_F16, true, false, 128>(block_size)
                                 : group_ptr<DT_BF16, true, false, 128>(block_size);
  return dtype == DT_F16 ? group_ptr<DT_F16, false, false, 128>(block_size)
                         : group_ptr<DT_BF16, false, false, 128>(block_size);
}

hipError_t launch_group_decode(const DecodeParams &a, hipStream_t stream) {
  if (a.S == 0 || a.G == 0) return hipSuccess;
#define PKV_G(DT)                                   \
  switch (a.B) {                                    \
    case 8: return launch_group<DT, 8>(a, stream);   \
    case 16: return launch_group<DT, 16>(a, stream); \
    case 32: return launch_group<DT, 32>(a, stream); \
    case 64: return launch_group<DT, 64>(a, stream); \
    default: return hipErrorInvalidValue;           \
  }
  if (a.dtype == DT_F16) { PKV_G(DT_F16) }
  PKV_G(DT_BF16)
#undef PKV_G
}

hipError_t launch_group_merge(const DecodeParams &a, hipStream_t stream) {
  if (a.S == 0) return hipSuccess;
  const int64_t groups = (int64_t)a.S * a.Hkv;  // one wavefront per (sequence, KV head)
  const int grid = (int)((groups + 3) / 4);
  if (a.fp8 && a.D == 64) {
    if (a.dtype == DT_F16)
      hipLaunchKernelGGL((decode_group_merge_kernel<DT_F16, 2 * GTC, 64>), dim3(grid), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_group_merge_kernel<DT_BF16, 2 * GTC, 64>), dim3(grid), dim3(256), 0, stream, a);
  } else if (a.fp8) {
    if (a.dtype == DT_F16)
      hipLaunchKernelGGL((decode_group_merge_kernel<DT_F16, 2 * GTC>), dim3(grid), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_group_merge_kernel<DT_BF16, 2 * GTC>), dim3(grid), dim3(256), 0, stream, a);
  } else if (a.D == 64) {
    if (a.dtype == DT_F16)
      hipLaunchKernelGGL((decode_group_merge_kernel<DT_F16, GTC, 64>), dim3(grid), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_group_merge_kernel<DT_BF16, GTC, 64>), dim3(grid), dim3(256), 0, stream, a);
  } else if (a.dtype == DT_F16) {
    hipLaunchKernelGGL((decode_group_merge_kernel<DT_F16, GTC>), dim3(grid), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL((decode_group_merge_kernel<DT_BF16, GTC>), dim3(grid), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace pkv
