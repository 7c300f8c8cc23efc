// dkv_decomp.h - how a decode call's tokens are cut into work items.
//
// Shared, word for word, by the decode kernel (which derives every item from
// the sequence lengths in device memory, so a captured graph stays valid as
// the cache grows) and by the host-side plan introspection that the CPU tests
// check for coverage.  Integer arithmetic only, so both sides agree exactly.
//
// Terms.  Each sequence's attended tokens fall into two tiers (host-pinned
// memory and HBM); a tier's tokens are numbered in tier order ("ordinals":
// contiguous layout, the tier's rows in order; paged layout, the tier's pages
// in logical order).  An item is a run of ordinals of one sequence in one
// tier, processed once per KV head.  Each tier has `team` workgroups per KV
// head (Hkv * team in all), which take the tier's (item, KV head) units in
// order, KV head fastest, from one queue.
// SplitKernel README, Overview: both tiers stream at the same time; Key
// Features: attention over a host/device partitioned KV cache.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define DKV_HD __host__ __device__
#else
#define DKV_HD
#endif

namespace dkv {

// Longest sequence batch the decode kernel derives items for (its per-sequence
// prefix arrays live in LDS).
constexpr int kDecodeMaxBatch = 512;
// Longest item (tokens): bounds the item count by the pool capacity.
constexpr int32_t kDecodeChunkCap = 1 << 22;

// Fixed on the host from the call's shape alone (no lengths).
struct DecodeTemplate {
  int32_t hkv;      // KV heads
  int32_t team_h;   // host-tier workgroups per KV head (0: no host tier)
  int32_t team_d;   // HBM-tier workgroups per KV head (0: no HBM tier)
  int32_t upw_h;    // items per workgroup the host chunk size aims at
  int32_t upw_d;    // items per workgroup the HBM chunk size aims at
  int32_t floor_h;  // fewest tokens per host item
  int32_t floor_d;  // fewest tokens per HBM item
  int32_t align;    // item granularity: a power of two, 64 or the page size
  int32_t guided;   // 1: the end of each long HBM range is cut finer
  int32_t tuned_h;  // > 0: fixed host item length (tokens, multiple of align)
  int32_t tuned_d;  // > 0: fixed HBM item length
  int32_t pad;
};

// Item lengths of one call, from the tier totals.
struct DecodeSizes {
  int32_t ch;        // tokens per host item
  int32_t cd;        // tokens per HBM item
  int32_t cs;        // tokens per HBM tail item
  int32_t guided;    // 1 when HBM ranges end in a tail of cs-token items
  int64_t tail_num;  // tail tokens of a range of n HBM tokens:
  int64_t tail_den;  //   floor(floor(n * tail_num / tail_den) / align) * align
};

// Items of one sequence.
struct DecodeSeqItems {
  int32_t uh;        // host items
  int32_t um;        // HBM items before the tail
  int32_t ut;        // HBM tail items
  int32_t pad;
  int64_t t0;        // first tail ordinal of the HBM range (= its length when no tail)
};

// Quotient of a >= 0 by b > 0: a 32-bit division when both fit in 32 bits (on
// the GPU a 64-bit division is a long software sequence, a 32-bit one a
// short one), else a 64-bit one; the same exact result either way.
DKV_HD inline int64_t decomp_div(int64_t a, int64_t b) {
  if ((((uint64_t)a | (uint64_t)b) >> 32) == 0) return (int64_t)((uint32_t)a / (uint32_t)b);
  return a / b;
}

DKV_HD inline int64_t decomp_cdiv(int64_t a, int64_t b) {
  if (a < 0) return (a + b - 1) / b;
  const int64_t q = decomp_div(a, b);
  return q * b == a ? q : q + 1;
}

// x >= 0 rounded up / down to a multiple of align, a power of two.
DKV_HD inline int64_t decomp_round_up(int64_t x, int32_t align) { return (x + align - 1) & ~(int64_t)(align - 1); }
DKV_HD inline int64_t decomp_round_down(int64_t x, int32_t align) { return x & ~(int64_t)(align - 1); }

// Tokens per item: enough that a tier's `team` workgroups see about `upw`
// items each, at least floor_tok, a multiple of align, at most the cap.
DKV_HD inline int32_t decode_chunk(int64_t tokens, int32_t team, int32_t upw, int32_t floor_tok, int32_t align,
                                   int32_t tuned) {
  if (tuned > 0) return (int32_t)decomp_round_up(tuned, align);
  int64_t c = (team > 0 && tokens > 0) ? decomp_cdiv(tokens, (int64_t)team * (upw > 0 ? upw : 1)) : 1;
  if (c < floor_tok) c = floor_tok;
  c = decomp_round_up(c, align);
  const int64_t cap = decomp_round_down(kDecodeChunkCap, align);
  return (int32_t)(c < cap ? c : cap);
}

// tot_h / tot_d: tokens per KV head in each tier, summed over the batch.
DKV_HD inline DecodeSizes decode_sizes(const DecodeTemplate& t, int64_t tot_h, int64_t tot_d) {
  DecodeSizes z{};
  z.ch = decode_chunk(tot_h, t.team_h, t.upw_h, t.floor_h, t.align, t.tuned_h);
  z.cd = decode_chunk(tot_d, t.team_d, t.upw_d, t.floor_d, t.align, t.tuned_d);
  z.cs = (int32_t)decomp_round_up(z.cd / 4, t.align);
  // Guided tail: with items of a few thousand tokens the workgroups of a tier
  // run out of work up to one item apart, so the last part of every HBM range
  // (about two tail items per workgroup in all) is cut into quarter-size
  // items that come after every other HBM item.
  z.guided = (t.guided && t.tuned_d <= 0 && z.cs >= 512 && t.team_d > 0 &&
              tot_d >= (int64_t)z.cd * t.team_d * 4) ? 1 : 0;
  if (z.guided) {
    const int64_t want = 4 * (int64_t)t.team_d * z.cs;  // twice the tail tokens, per KV head
    z.tail_num = tot_d < want ? tot_d : want;           // fraction min(1/2, 2 team cs / tot)
    z.tail_den = 2 * tot_d;
  } else {
    z.tail_num = 0;
    z.tail_den = 1;
  }
  return z;
}

// nh, nd: the sequence's host and HBM tokens (ordinals); both < 2^31.
DKV_HD inline DecodeSeqItems decode_seq_items(const DecodeSizes& z, int32_t align, int64_t nh, int64_t nd) {
  DecodeSeqItems s{};
  s.uh = nh > 0 ? (int32_t)decomp_cdiv(nh, z.ch) : 0;
  // nd < 2^31 and tail_num <= 4 * team * cs <= 2^32 keep the product in range
  const int64_t tail = z.guided ? decomp_round_down(decomp_div(nd * z.tail_num, z.tail_den), align) : 0;
  s.t0 = nd - tail;
  s.um = s.t0 > 0 ? (int32_t)decomp_cdiv(s.t0, z.cd) : 0;
  s.ut = tail > 0 ? (int32_t)decomp_cdiv(tail, z.cs) : 0;
  return s;
}

// Host and HBM tokens attended of a contiguous-split sequence: `attended`
// cached tokens, of which the oldest floor(r * placed) are host-resident
// (placed = attended, plus one when the call appends a token first).
DKV_HD inline void contig_tiers(double ratio, int64_t attended, int64_t placed, int64_t* nh, int64_t* nd,
                                int64_t* n_host_placed) {
  const double prod = ratio * (double)placed;
  int64_t p = (int64_t)prod;  // prod >= 0: truncation is the floor
  if (p > placed) p = placed;
  *n_host_placed = p;
  *nh = p < attended ? p : attended;
  *nd = attended > p ? attended - p : 0;
}

// Split slots per sequence written by the split (unfused) form: one per item.
DKV_HD inline int32_t decode_seq_splits(const DecodeSeqItems& s) { return s.uh + s.um + s.ut; }

// Upper bound of the split count of a call over tiers holding at most
// host_cap / dev_cap tokens per KV head (the pool capacities), for `batch`
// sequences: the item length never falls below tot / (team * upw) before the
// cap, and the tail holds at most 2 team cs tokens.
DKV_HD inline int64_t decode_max_splits(const DecodeTemplate& t, int32_t batch, int64_t host_cap, int64_t dev_cap) {
  int64_t s = 0;
  if (t.team_h > 0) {
    const int64_t by_len = t.tuned_h > 0 ? decomp_cdiv(host_cap, t.tuned_h) : (int64_t)t.team_h * t.upw_h;
    s += by_len + host_cap / decomp_round_down(kDecodeChunkCap, t.align) + batch;
  }
  if (t.team_d > 0) {
    const int64_t by_len = t.tuned_d > 0 ? decomp_cdiv(dev_cap, t.tuned_d) : (int64_t)t.team_d * t.upw_d;
    s += by_len + dev_cap / decomp_round_down(kDecodeChunkCap, t.align) + batch;  // main items
    if (t.guided && t.tuned_d <= 0) s += 2 * (int64_t)t.team_d + batch;   // tail items
  }
  return s;
}

}  // namespace dkv
