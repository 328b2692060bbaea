// Work-balanced split shared by the decode kernels: the batch's chunks, row
// by row (sequence major), cut into equal slices, one per worker wavefront.
#pragma once

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

// Chunks of a row of L tokens; invalid and empty contexts have none.
template <int TC>
__device__ __forceinline__ int row_chunks(int L, int maxb, int B, int min_len = 1) {
  return (L >= min_len && L > 0 && L <= maxb * B) ? (L + TC - 1) / TC : 0;
}

// floor(x / d) for d >= 1 without the slow 64-bit integer division: a double
// estimate corrected to the exact quotient with 64-bit multiplies.
__device__ __forceinline__ uint64_t udiv64(uint64_t x, uint64_t d) {
  uint64_t q = (uint64_t)((double)x / (double)d);
  while (q > 0 && q * d > x) --q;
  while ((q + 1) * d <= x) ++q;
  return q;
}

__device__ __forceinline__ uint64_t uni64(uint64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// Workers share the cost space in equal slices: worker w owns positions
// [min(total, w * slice), min(total, (w + 1) * slice)).  At most G workers,
// each slice at least kMinWorkerChunks long.
__device__ __forceinline__ uint64_t slice_of(uint64_t total, int G) {
  const uint64_t want = total / (uint64_t)kMinWorkerChunks;  // constant divisor
  const uint64_t workers = max((uint64_t)1, min((uint64_t)G, want));
  return max((uint64_t)1, udiv64(total + workers - 1, workers));
}

// Suffix pass of the shared-prefix decode: a row of L tokens whose first
// `st` tokens were done by the prefix pass covers chunks c0 .. c0 + n - 1
// (chunks of TC tokens from token 0).  A row with nothing left (L == st)
// keeps one chunk, all of it masked, so that its output is still written from
// the prefix state; st > L (a broken group) keeps one chunk and gives NaN.
// Invalid contexts have no chunks.
template <int TC>
__device__ __forceinline__ void suffix_span(int L, int st, int maxb, int B, int &c0, int &n) {
  if (L < 1 || L > maxb * B) {
    c0 = 0;
    n = 0;
  } else if (st <= 0) {
    c0 = 0;
    n = (L + TC - 1) / TC;
  } else if (st > L) {
    c0 = (L - 1) / TC;
    n = 1;
  } else {
    c0 = st / TC;
    n = max(1, (L + TC - 1) / TC - c0);
  }
}

// Prefix of the chunk count over sequences into LDS (cum[0] = 0, cum[S] =
// total; a sequence has `rows` rows of row_chunks chunks each) and a copy of
// the context lengths, computed by one wavefront: each lane sums a contiguous
// run, then a scan.  Contexts shorter than min_len count as invalid.  PFX
// (suffix pass): rows cover their suffix (suffix_span) and `starts` gets
// each sequence's first token.
template <int TC, bool PFX = false>
__device__ __forceinline__ void build_cost_prefix(const DecodeParams &a, int rows, int64_t *cum, int32_t *lens,
                                                  int lane, int min_len = 1, int32_t *starts = nullptr) {
  const int S = a.S;
  const int per = (S + 63) / 64;
  const int s0 = min(S, lane * per);
  const int s1 = min(S, s0 + per);
  int64_t run = 0;
  for (int s = s0; s < s1; ++s) {
    const int L = a.lens[s];
    lens[s] = L;
    if constexpr (PFX) {
      const int st = a.pfx_lens[s / a.pfx_group];
      starts[s] = st;
      int c0, n;
      suffix_span<TC>(L, st, a.maxb, a.B, c0, n);
      run += (int64_t)rows * n;
    } else {
      run += (int64_t)rows * row_chunks<TC>(L, a.maxb, a.B, min_len);
    }
  }
  int64_t incl = run;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  int64_t x = incl - run;  // exclusive prefix of this lane's run
  if (lane == 0) cum[0] = 0;
  for (int s = s0; s < s1; ++s) {
    if constexpr (PFX) {
      int c0, n;
      suffix_span<TC>(lens[s], starts[s], a.maxb, a.B, c0, n);
      x += (int64_t)rows * n;
    } else {
      x += (int64_t)rows * row_chunks<TC>(lens[s], a.maxb, a.B, min_len);
    }
    cum[s + 1] = x;
  }
}

// One chunk of a stream: chunk c of row (s, h), in the piece [cb, ce) of that
// row the slice covers.  Chunk indexes count TC-token chunks from token 0;
// the row's chunks start at c0 (0 except in the suffix pass of a shared
// prefix, whose rows start at token t0).  `valid` is false once the stream
// has ended; the other fields then repeat the last chunk (so its loads stay
// in bounds).
struct Chunk {
  int s, h, L, c, cb, ce, c0, t0;
  bool valid;
};

// Walks a wavefront's slice of the cost space chunk by chunk: sequences of
// `rows` rows of ceil(L / TC) chunks each (PFX: their suffix, suffix_span),
// with the chunk prefix `cum`, the lengths `lens` (and PFX: the first tokens
// `starts`) in LDS.
template <int TC, bool PFX = false>
struct ChunkCursor {
  const int64_t *cum;
  const int32_t *lens;
  const int32_t *starts;
  int S, rows, lane, maxb, B;
  uint64_t it_hi;
  int cs_, ch_, cL, cn, cc, ccb, cce;  // s, h, L, chunks of row, chunk, piece [cb, ce) (from the row's first)
  int cc0, ct0;                       // row's first chunk and first token
  uint64_t cseg;                      // cost position of the first chunk of row (s, h)
  bool cvalid;
  Chunk last;

  __device__ __forceinline__ void init(const int64_t *cum_, const int32_t *lens_, int S_, int rows_, int lane_,
                                       const int32_t *starts_ = nullptr, int maxb_ = 0, int B_ = 0) {
    cum = cum_;
    lens = lens_;
    starts = starts_;
    S = S_;
    rows = rows_;
    lane = lane_;
    maxb = maxb_;
    B = B_;
    cvalid = false;
  }

  __device__ __forceinline__ uint64_t cum_at(int s) const { return uni64((uint64_t)cum[s]); }
  __device__ __forceinline__ int len_at(int s) const { return __builtin_amdgcn_readfirstlane(lens[s]); }

  // Chunks of the rows of sequence s (which has some) and where they start.
  __device__ __forceinline__ void span_of(int s) {
    cL = len_at(s);
    if constexpr (PFX) {
      ct0 = __builtin_amdgcn_readfirstlane(starts[s]);
      suffix_span<TC>(cL, ct0, maxb, B, cc0, cn);
      ct0 = max(ct0, 0);
    } else {
      cc0 = 0;
      ct0 = 0;
      cn = (cL + TC - 1) / TC;
    }
  }

  // Largest s < S with cum[s] <= p (p < total): 64 samples per round.
  __device__ __forceinline__ int find_seq(uint64_t p) const {
    int base = 0, span = S;
    while (span > 1) {
      const int step = (span + 63) >> 6;
      const int idx = base + lane * step;
      const bool ok = idx < base + span && (uint64_t)cum[idx] <= p;
      const uint64_t mask = __ballot(ok);
      const int j = __builtin_amdgcn_readfirstlane(__popcll(mask)) - 1;
      base += j * step;
      span = min(step, span - j * step);
    }
    return base;
  }

  // Start the slice [lo, hi) (lo < hi <= total).
  __device__ __forceinline__ void enter(uint64_t lo, uint64_t hi) {
    it_hi = hi;
    const int s = find_seq(lo);
    const uint64_t base = cum_at(s);
    cs_ = s;
    span_of(s);  // sequence s has chunks: cum[s + 1] > lo >= cum[s]
    const uint64_t off = lo - base;  // < rows * cn
    const uint32_t h = off < (1ull << 32) ? (uint32_t)off / (uint32_t)cn : (uint32_t)udiv64(off, (uint64_t)cn);
    ch_ = (int)h;
    cseg = base + (uint64_t)h * cn;
    ccb = (int)(lo - cseg);
    cc = ccb;
    cce = (int)min((uint64_t)cn, hi - cseg);
    cvalid = true;
  }

  // Move to the row after (s, h) inside the slice, or end the slice.
  __device__ __forceinline__ void next_row() {
    const uint64_t pos = cseg + cn;
    if (pos >= it_hi) {
      cvalid = false;
      return;
    }
    if (ch_ + 1 < rows) {
      ++ch_;
    } else {
      int s = cs_ + 1;
      while (cum_at(s + 1) == pos) ++s;  // sequences without chunks
      cs_ = s;
      ch_ = 0;
      span_of(s);
    }
    cseg = pos;
    ccb = 0;
    cc = 0;
    cce = (int)min((uint64_t)cn, it_hi - cseg);
  }

  // The next chunk of the stream.
  __device__ __forceinline__ Chunk produce() {
    if (!cvalid) {
      Chunk none = last;
      none.valid = false;
      return none;
    }
    Chunk ch;
    ch.s = cs_;
    ch.h = ch_;
    ch.L = cL;
    ch.c = cc + cc0;
    ch.cb = ccb + cc0;
    ch.ce = cce + cc0;
    ch.c0 = cc0;
    ch.t0 = ct0;
    ch.valid = true;
    last = ch;
    if (cc + 1 < cce) ++cc;
    else next_row();
    return ch;
  }
};

// Runs a wavefront's stream of n chunks (n >= 1) through the three stages
// of ST: load_entries (the chunk's table entries), load_kv (its K/V rows)
// and consume (fold it into the running softmax).  Stage 1 of chunk i + 2,
// stage 2 of chunk i + 1 and stage 3 of chunk i overlap.  The loop body
// handles two chunks, one per buffer, runs a counted number of times and has
// its only exit at the bottom; the prologue issues its loads in the loop's
// order.  Every path into the loop top therefore carries the same
// outstanding loads, so the compiler's wait before each consume leaves the
// younger chunk's loads in flight.  An odd last chunk is consumed after the
// loop; past the end of the slice the cursor repeats its last chunk, whose
// loads stay in bounds and are never consumed.  The priority falls from 3 to
// 0 as the wavefront passes quarters of its slice, so wavefronts that share
// a SIMD progress together instead of in order of age.
template <class ST>
__device__ __forceinline__ void run_stream(ST &st, int n) {
  const int th1 = n / 4, th2 = n / 2, th3 = (3 * n) / 4;
  typename ST::Buf ba, bb;
  Chunk d0 = st.cur.produce();
  uint32_t ea = st.load_entries(d0);
  Chunk d1 = st.cur.produce();
  uint32_t eb = st.load_entries(d1);
  __builtin_amdgcn_sched_barrier(0);
  st.load_kv(d0, ea, ba);
  __builtin_amdgcn_sched_barrier(0);
  for (int done = 0; done + 2 <= n; done += 2) {
    const Chunk d2 = st.cur.produce();
    ea = st.load_entries(d2);
    st.load_kv(d1, eb, bb);
    __builtin_amdgcn_sched_barrier(0);
    st.consume(d0, ba);
    if (done + 1 == th1) __builtin_amdgcn_s_setprio(2);
    if (done + 1 == th2) __builtin_amdgcn_s_setprio(1);
    if (done + 1 == th3) __builtin_amdgcn_s_setprio(0);
    const Chunk d3 = st.cur.produce();
    eb = st.load_entries(d3);
    st.load_kv(d2, ea, ba);
    __builtin_amdgcn_sched_barrier(0);
    st.consume(d1, bb);
    if (done + 2 == th1) __builtin_amdgcn_s_setprio(2);
    if (done + 2 == th2) __builtin_amdgcn_s_setprio(1);
    if (done + 2 == th3) __builtin_amdgcn_s_setprio(0);
    d0 = d2;
    d1 = d3;
  }
  if (n & 1) st.consume(d0, ba);
}

}  // namespace pkv
