// dkv_decode.hip - gfx950 decode kernels: split decode attention over a KV
// cache held partly in host-pinned memory (read in place over the host link)
// and partly in HBM, with the work split derived on the device.
//
//   decode_tiers_kernel  paged layout: each sequence's pages sorted by tier
//                        (physical page numbers in logical order) and its
//                        tokens per tier, for the sequence lengths of this call
//   decode_kernel        rotate the query heads (Neox RoPE, fp64 angle), stream
//                        K/V tiles of one tier into LDS, Q.K on MFMA, online
//                        softmax, P.V on the vector ALUs, one normalised
//                        partial per (work item, KV head); fused, the
//                        partials are merged by log-sum-exp in the same
//                        launch, after each sequence's new token is appended
//
// Method sources (page, section): DirectKV README, introduction (one kernel
// projects the new token's K/V, rotates keys with Neox RoPE and attends over
// KV read from CPU-pinned buffers) and Attribution (online softmax over KV
// streamed from CPU memory with no GPU staging buffer); SplitKernel README,
// Overview and Key Features (direct access of the remote tier into on-chip
// memory; attention over a host/device partitioned KV cache; both tiers'
// bandwidth used at once).
//
// Design for CDNA4:
//   * No host plan.  Every workgroup reads the lengths (and, paged, the tier
//     counts) from device memory and derives the same items (dkv_decomp.h), so
//     a call captured in a graph stays valid while the cache grows, and a step
//     needs no host work beyond argument checks.
//   * Queues.  Each tier has one queue of (item, KV head) units with the KV
//     head fastest, taken in order (first by index, then by an atomic
//     counter, or round-robin when a tier has at most two units per
//     workgroup), so the workgroups of a tier stream neighbouring rows of the
//     same token range at once (DRAM page locality).  Fused form: the
//     appended tokens, one unit per (sequence, KV head), follow the HBM
//     tier's attention units in its queue, so the first workgroups to run out
//     of attention take them.
//   * Fused form.  Each unit's partial goes to its slot in the workspace; a
//     sequence's slots (its appended token, then its items) form groups of
//     kMergeGroup.  The last unit of a group to finish merges the group into
//     its first slot, and the last group of a (sequence, KV head) merges the
//     group results into the output, so no workgroup folds more than a few
//     dozen partials.  Partials are written and read with agent-coherent
//     (sc1) buffer accesses and each count is bumped after the stores are
//     acknowledged, which orders them across XCDs without an L2 write-back.
//   * Tiles: 64 tokens of one KV head, D/32 coalesced 16-byte loads of K and
//     of V per thread (non-temporal: the KV is read once), staged in LDS with a
//     16-byte row pad; the next tile is in flight while one is computed.
//   * Q.K^T on v_mfma_f32_16x16x32_bf16: A = 16 keys x 32 dims from LDS, B =
//     the group's rotated queries, each fp32 query split into high and low bf16
//     parts in columns h and h+8 (~16 bits of the query, fp32 accumulation).
//   * P.V on the vector ALUs (two output dims per lane at D = 128).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "dkv_decomp.h"
#include "dkv_device.h"
#include "dkv_internal.h"

namespace dkv {

template <int D>
struct AttnShape {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kPitch = kRowBytes + 16;          // LDS row pitch (bytes)
  static constexpr int kChunksPerRow = D / 8;            // 16-byte chunks per row
  static constexpr int kChunksPerThread = kTile * kChunksPerRow / kThreads;  // D/32
  static constexpr int kKSteps = D / 32;                 // MFMA k-steps per key
  static constexpr int kDimsPerLane = D / 64;            // P.V output dims per lane
};


// ---------------------------------------------------------------------------
// Paged layout: per sequence, the physical pages of each tier in logical order
// and the tokens each tier holds among the sequence's first seq_lens[b].
// Grid (chunks, batch): workgroup (c, b) places page entries [c CH, (c+1) CH)
// of sequence b, CH = 1024 threads x 16 entries.  It first counts the valid
// host and HBM entries before its chunk (strided loads, many in flight), so
// the chunks of a long sequence run side by side with no dependency between
// workgroups; then each thread takes 16 consecutive entries (all loads issued
// before any is used) and places them with a block-wide scan.  Entries that
// are negative or beyond their tier's pool are left out (and flagged by the
// chunk that holds them).  The last chunk writes the sequence's counts.
// ---------------------------------------------------------------------------
constexpr int kTierThreads = 1024;
constexpr int kTierPer = 16;
constexpr int kTierChunk = kTierThreads * kTierPer;

__global__ __launch_bounds__(kTierThreads) void decode_tiers_kernel(DecodeArgs a, int32_t* __restrict__ counts,
                                                                   int32_t* __restrict__ pages) {
  constexpr int NW = kTierThreads / 64;
  __shared__ int32_t s_wh[NW], s_wd[NW];
  __shared__ int32_t s_base[2];
  __shared__ int32_t s_last;  // tier of the sequence's final page: 1 host, 0 HBM, -1 none
  const int c = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int P = 1 << a.page_shift;
  int64_t A = a.seq_lens[b];
  if (A < 0) A = 0;
  int64_t npg = (A + P - 1) >> a.page_shift;
  int err = 0;
  if (npg > a.max_pages) {
    err |= kDecodeErrPage;
    npg = a.max_pages;
    A = npg * P;
  }
  const int64_t last_chunk = npg > 0 ? (npg - 1) / kTierChunk : 0;
  if (c > last_chunk) return;  // workgroup-uniform
  if (c > 0) err = 0;          // the length is flagged once
  const int32_t* __restrict__ row = a.page_table + (int64_t)b * a.max_pages;
  int32_t* __restrict__ hl = pages + (int64_t)b * a.max_pages;
  int32_t* __restrict__ dl = pages + ((int64_t)a.batch + b) * a.max_pages;
  const int64_t host_pages_cap = a.host_k ? (a.host_rows >> a.page_shift) : 0;
  const int64_t dev_pages_cap = a.dev_k ? (a.dev_rows >> a.page_shift) : 0;
  auto valid = [&](int32_t x) {
    const bool host = (x & 1) != 0;
    return x >= 0 && (int64_t)(x >> 1) < (host ? host_pages_cap : dev_pages_cap);
  };

  // valid host / HBM entries before this chunk
  const int64_t j0 = (int64_t)c * kTierChunk;
  int ch0 = 0, cd0 = 0;
  constexpr int U = 8;
  auto count = [&](int32_t x) {
    if (valid(x)) {
      if (x & 1) ++ch0;
      else ++cd0;
    }
  };
  if (((uintptr_t)row & 15) == 0) {
    // 16-byte loads (j0 is a multiple of 4 entries), U per thread in flight
    const u32x4* row4 = reinterpret_cast<const u32x4*>(row);
    const int64_t n4 = j0 >> 2;
    for (int64_t j = tid; j < n4; j += (int64_t)kTierThreads * U) {
      u32x4 e[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t idx = j + (int64_t)u * kTierThreads;
        e[u] = idx < n4 ? row4[idx] : u32x4{~0u, ~0u, ~0u, ~0u};
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) count((int32_t)e[u][q]);
    }
  } else {
    for (int64_t j = tid; j < j0; j += (int64_t)kTierThreads * U) {
      int32_t e[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t idx = j + (int64_t)u * kTierThreads;
        e[u] = idx < j0 ? row[idx] : -1;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) count(e[u]);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    ch0 += __shfl_xor(ch0, o);
    cd0 += __shfl_xor(cd0, o);
  }
  if (lane == 0) {
    s_wh[wave] = ch0;
    s_wd[wave] = cd0;
  }
  if (tid == 0) s_last = -1;
  __syncthreads();
  if (tid == 0) {
    int th = 0, td = 0;
    for (int w = 0; w < NW; ++w) {
      th += s_wh[w];
      td += s_wd[w];
    }
    s_base[0] = th;
    s_base[1] = td;
  }
  __syncthreads();

  // this chunk: wave w takes entries [w*64*16, (w+1)*64*16) of it in 16
  // rounds of 64 consecutive entries (lane = entry: coalesced loads and, per
  // tier, consecutive stores); per-wave counts, one scan over the waves, then
  // each round places its entries by ballot.
  constexpr int WPE = 64 * kTierPer;  // entries per wave
  const int64_t jw = j0 + (int64_t)wave * WPE + lane;
  int32_t e[kTierPer];
#pragma unroll
  for (int k = 0; k < kTierPer; ++k) e[k] = (jw + 64 * k < npg) ? row[jw + 64 * k] : -1;
  uint32_t hm = 0, dm = 0;  // per lane: rounds whose entry is a valid host / HBM page
#pragma unroll
  for (int k = 0; k < kTierPer; ++k) {
    const int64_t j = jw + 64 * k;
    if (j >= npg) continue;
    const int32_t x = e[k];
    if (!valid(x)) {
      err |= kDecodeErrPage;
      continue;
    }
    const bool host = (x & 1) != 0;
    if (host) hm |= 1u << k;
    else dm |= 1u << k;
    if (j == npg - 1) s_last = host ? 1 : 0;
  }
  int ch = __builtin_popcount(hm), cd = __builtin_popcount(dm);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    ch += __shfl_xor(ch, o);
    cd += __shfl_xor(cd, o);
  }
  __syncthreads();  // s_wh / s_wd of the count phase are read
  if (lane == 0) {
    s_wh[wave] = ch;
    s_wd[wave] = cd;
  }
  __syncthreads();
  int ph = s_base[0], pd = s_base[1];
  for (int w = 0; w < wave; ++w) {
    ph += s_wh[w];
    pd += s_wd[w];
  }
#pragma unroll
  for (int k = 0; k < kTierPer; ++k) {
    const uint64_t bh = __ballot((hm >> k) & 1u), bd = __ballot((dm >> k) & 1u);
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    if ((hm >> k) & 1u) hl[ph + __popcll(bh & below)] = e[k] >> 1;
    if ((dm >> k) & 1u) dl[pd + __popcll(bd & below)] = e[k] >> 1;
    ph += __popcll(bh);
    pd += __popcll(bd);
  }
  if (err) atomicOr(&a.counters[decode_error_word()], err);
  if (c == last_chunk && tid == 0) {
    int th = s_base[0], td = s_base[1];
    for (int w = 0; w < NW; ++w) {
      th += s_wh[w];
      td += s_wd[w];
    }
    const int64_t deficit = npg > 0 ? P - (A - (npg - 1) * P) : 0;
    const int64_t nh = (int64_t)th * P - (s_last == 1 ? deficit : 0);
    const int64_t nd = (int64_t)td * P - (s_last == 0 ? deficit : 0);
    counts[4 * b + 0] = th;
    counts[4 * b + 1] = td;
    counts[4 * b + 2] = (int32_t)nh;
    counts[4 * b + 3] = (int32_t)nd;
  }
}

// ---------------------------------------------------------------------------
// Decode kernel.
// ---------------------------------------------------------------------------

// Fused form: partial slots per merge group (a group's last unit to finish
// folds them; the last group of a (sequence, KV head) folds the groups).
constexpr int kMergeGroup = 16;

// One work item as the kernel sees it.
struct DItem {
  int32_t b;      // sequence
  int32_t n_tok;  // tokens
  int32_t slot;   // split form: partial slot
  int32_t pad;
  int64_t k0;     // first ordinal of the item in its tier
};

// Per-sequence prefix arrays of the current call (LDS), built by wave 0.
struct DecodeLds {
  int32_t ph[kDecodeMaxBatch + 1];   // host items before sequence b
  int32_t pm[kDecodeMaxBatch + 1];   // HBM items (before the tail) before b
  int32_t pt[kDecodeMaxBatch + 1];   // HBM tail items before b
  int32_t off[kDecodeMaxBatch + 1];  // split slots before b
  int32_t nh[kDecodeMaxBatch];       // host tokens attended
  int32_t nd[kDecodeMaxBatch];       // HBM tokens attended
  int32_t t0[kDecodeMaxBatch];       // first tail ordinal of the HBM range
  DecodeSizes z;
};

// Largest b in [0, B) with arr[b] <= i (arr non-decreasing, arr[0] = 0, i < arr[B]).
__device__ __forceinline__ int seq_of(const int32_t* arr, int B, int i) {
  int lo = 0, hi = B;  // arr[lo] <= i < arr[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (arr[mid] <= i) lo = mid;
    else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ DItem item_at(const DecodeLds& L, int B, bool host, int i) {
  DItem it{};
  if (host) {
    const int b = seq_of(L.ph, B, i);
    const int c = i - L.ph[b];
    it.b = b;
    it.k0 = (int64_t)c * L.z.ch;
    it.n_tok = (int32_t)min((int64_t)L.z.ch, (int64_t)L.nh[b] - it.k0);
    it.slot = L.off[b] + c;
  } else {
    const int M = L.pm[B];
    if (i < M) {
      const int b = seq_of(L.pm, B, i);
      const int c = i - L.pm[b];
      it.b = b;
      it.k0 = (int64_t)c * L.z.cd;
      it.n_tok = (int32_t)min((int64_t)L.z.cd, (int64_t)L.t0[b] - it.k0);
      it.slot = L.off[b] + (L.ph[b + 1] - L.ph[b]) + c;
    } else {
      const int i2 = i - M;
      const int b = seq_of(L.pt, B, i2);
      const int c = i2 - L.pt[b];
      it.b = b;
      it.k0 = (int64_t)L.t0[b] + (int64_t)c * L.z.cs;
      it.n_tok = (int32_t)min((int64_t)L.z.cs, (int64_t)L.nd[b] - it.k0);
      it.slot = L.off[b] + (L.ph[b + 1] - L.ph[b]) + (L.pm[b + 1] - L.pm[b]) + c;
    }
  }
  return it;
}

// Inclusive scan of v over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

__device__ __forceinline__ long long wave_sum64(long long v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Wave 0 reads the lengths, derives each sequence's tier tokens and items and
// writes the prefix arrays; the caller synchronises the workgroup afterwards.
template <bool PAGED>
__device__ void build_prefix(const DecodeArgs& a, DecodeLds& L) {
  const int lane = threadIdx.x & 63;
  const int B = a.batch;
  long long th = 0, td = 0;
  int err = 0;
  for (int b = lane; b < B; b += 64) {
    int64_t nh, nd;
    if (PAGED) {
      nh = a.tier_counts[4 * b + 2];
      nd = a.tier_counts[4 * b + 3];
    } else {
      int64_t Lb = a.seq_lens[b];
      if (Lb < 0) Lb = 0;
      int64_t placed_host;
      contig_tiers(a.ratio, Lb, Lb + a.new_tokens, &nh, &nd, &placed_host);
      const int64_t placed_dev = Lb + a.new_tokens - placed_host;
      const bool bad = (placed_host > 0 && (placed_host > a.host_stride || !a.host_k ||
                                            (int64_t)b * a.host_stride + placed_host > a.host_rows)) ||
                       (placed_dev > 0 && (placed_dev > a.dev_stride || !a.dev_k ||
                                           (int64_t)b * a.dev_stride + placed_dev > a.dev_rows));
      if (bad) {  // rows beyond the layout: the sequence is not read (and is flagged)
        err |= kDecodeErrLayout;
        nh = 0;
        nd = 0;
      }
    }
    L.nh[b] = (int32_t)nh;
    L.nd[b] = (int32_t)nd;
    th += nh;
    td += nd;
  }
  if (B == 1) {  // one sequence (workgroup-uniform): lane 0 holds the totals
    th = __shfl(th, 0);
    td = __shfl(td, 0);
  } else {
    th = wave_sum64(th);
    td = wave_sum64(td);
  }
  const DecodeSizes z = decode_sizes(a.tmpl, th, td);
  if (B == 1) {  // no scans: the prefix of one sequence is its item counts
    if (lane == 0) {
      const DecodeSeqItems s = decode_seq_items(z, a.tmpl.align, L.nh[0], L.nd[0]);
      L.ph[0] = 0;
      L.pm[0] = 0;
      L.pt[0] = 0;
      L.off[0] = 0;
      L.t0[0] = (int32_t)s.t0;
      L.ph[1] = s.uh;
      L.pm[1] = s.um;
      L.pt[1] = s.ut;
      L.off[1] = s.uh + s.um + s.ut;
      L.z = z;
    }
    if (err) atomicOr(&a.counters[decode_error_word()], err);
    return;
  }
  int ch = 0, cm = 0, ct = 0, cs = 0;  // running totals of earlier chunks of 64 sequences
  for (int base = 0; base < B; base += 64) {
    const int b = base + lane;
    DecodeSeqItems s{};
    if (b < B) s = decode_seq_items(z, a.tmpl.align, L.nh[b], L.nd[b]);
    const int nsp = s.uh + s.um + s.ut;
    const int ih = wave_incl_scan(s.uh), im = wave_incl_scan(s.um), it = wave_incl_scan(s.ut),
              is = wave_incl_scan(nsp);
    if (b < B) {
      L.ph[b] = ch + ih - s.uh;
      L.pm[b] = cm + im - s.um;
      L.pt[b] = ct + it - s.ut;
      L.off[b] = cs + is - nsp;
      L.t0[b] = (int32_t)s.t0;
    }
    ch += __shfl(ih, 63);
    cm += __shfl(im, 63);
    ct += __shfl(it, 63);
    cs += __shfl(is, 63);
  }
  if (lane == 0) {
    L.ph[B] = ch;
    L.pm[B] = cm;
    L.pt[B] = ct;
    L.off[B] = cs;
    L.z = z;
  }
  if (err) atomicOr(&a.counters[decode_error_word()], err);
}

template <int D, int G, bool PAGED, bool FUSED>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  using S = AttnShape<D>;
  constexpr int NC = S::kChunksPerThread;
  constexpr int KS = S::kKSteps;
  constexpr int DPL = S::kDimsPerLane;
  static_assert(G >= 1 && G <= 8, "group size");
  static_assert(4 * G * (D + 2) * 4 <= kTile * S::kPitch, "epilogue scratch");
  static_assert(2 * D * 4 <= kTile * S::kPitch, "appended token scratch");

  __shared__ __attribute__((aligned(16))) uint8_t k_lds[kTile * S::kPitch];
  __shared__ __attribute__((aligned(16))) uint8_t v_lds[kTile * S::kPitch];
  __shared__ __attribute__((aligned(16))) float p_lds[4][16][8];
  __shared__ float a_lds[4][8];
  __shared__ __attribute__((aligned(16))) float q_lds[G][D];  // rotated query heads of q_b
  __shared__ DecodeLds L;
  __shared__ int s_next;
  __shared__ int s_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15;     // MFMA column / row-in-tile
  const int j4 = lane >> 4;    // 0..3
  const int B = a.batch;

  const bool traced = a.wg_trace && (int)blockIdx.x < a.wg_trace_cap && tid == 0;
  const uint64_t t_start = traced ? wall_clock64() : 0;

  if (wave == 0) build_prefix<PAGED>(a, L);
  __syncthreads();

  // Role: host-tier workgroups first.  One queue per tier whose units are
  // (item, KV head) with the KV head fastest, so the heads of a token range
  // are read together.
  const DecodeTemplate& T = a.tmpl;
  const bool host_role = (int)blockIdx.x < a.hkv * T.team_h;
  const int r_idx = host_role ? (int)blockIdx.x : (int)blockIdx.x - a.hkv * T.team_h;
  const int role_wgs = a.hkv * (host_role ? T.team_h : T.team_d);
  const int n_items = host_role ? L.ph[B] : L.pm[B] + L.pt[B];
  // the call's partial slots must fit the arrays it was given; otherwise
  // nothing is computed and the call is flagged (the host's bound on the slot
  // count makes this unreachable for lengths that fit the pools)
  const bool fits = L.off[B] + (FUSED ? B * a.new_tokens : 0) <= a.max_slots;
  const int n_units = fits ? n_items * a.hkv : 0;
  const uint16_t* __restrict__ kpool = host_role ? a.host_k : a.dev_k;
  const uint16_t* __restrict__ vpool = host_role ? a.host_v : a.dev_v;
  const int64_t stride = host_role ? a.host_stride : a.dev_stride;
  const int32_t* __restrict__ tier_list =
      PAGED ? a.tier_pages + (host_role ? 0 : (int64_t)B * a.max_pages) : nullptr;
  int* qctr = a.counters + decode_queue(host_role);
  int kvh = 0;

  if (!fits && blockIdx.x == 0 && tid == 0) atomicOr(&a.counters[decode_error_word()], kDecodeErrCapacity);
  if (!FUSED && blockIdx.x == 0 && a.split_offsets)
    for (int i = tid; i <= B; i += kThreads) a.split_offsets[i] = L.off[i];

  // Rotated query heads of sequence b for this KV head into q_lds: one Neox pair
  // per thread, angle q_pos[b] * f_i with sin and cos in fp64, rounded once to
  // fp32 with scale * log2(e) folded in.
  int q_b = -1, q_kvh = -1;
  auto rotate_q = [&](int b) {
    __syncthreads();  // earlier readers of q_lds are done
    const int pos = a.q_pos[b];
    const uint16_t* qh = a.q + ((size_t)b * a.hq + (size_t)kvh * G) * D;
    for (int idx = tid; idx < G * (D / 2); idx += kThreads) {
      const int h = idx / (D / 2), i = idx - h * (D / 2);
      double sn, cs;
      sincos((double)pos * a.freq.f[i], &sn, &cs);
      const double xl = (double)bf16_to_f32(qh[h * D + i]);
      const double xh = (double)bf16_to_f32(qh[h * D + i + D / 2]);
      q_lds[h][i] = (float)(xl * cs - xh * sn) * a.scale_log2;
      q_lds[h][i + D / 2] = (float)(xh * cs + xl * sn) * a.scale_log2;
    }
    __syncthreads();
    q_b = b;
    q_kvh = kvh;
  };

  // Fused form.  Sequence b owns slots [seq_first(b), seq_first(b) +
  // seq_slots(b)): first its appended token's, then one per item.  Partials
  // are [slot][Hq][D] (lse [slot][Hq]); offsets fit 31 bits (checked on the
  // host).
  auto seq_slots = [&](int b) -> int {
    return (L.off[b + 1] - L.off[b]) + a.new_tokens;
  };
  auto seq_first = [&](int b) -> int { return L.off[b] + b * a.new_tokens; };

  // Fold n partials of (b, kvh), at slots s0, s0 + step, ..., by log-sum-exp
  // into slot dst or, with dst < 0, into the output.  The lse values of up to
  // CAPN partials at a time are staged in LDS (the K tile buffer); pass 1
  // gives each head's maximum and sum of exp(lse - max), pass 2 turns the
  // staged values into weights and folds the outputs, the threads of each
  // float4 of the output splitting the partials between them.
  auto merge = [&](int b, int s0, int step, int n, int dst) {
    const __amdgpu_buffer_rsrc_t pr_o = coherent_rsrc(a.part_o);
    const __amdgpu_buffer_rsrc_t pr_l = coherent_rsrc(a.part_lse);
    constexpr int CAPN = (kTile * S::kPitch) / (G * 4);
    constexpr int NCH = G * D / 4;           // float4 chunks of a partial (<= 256)
    constexpr int NSG = kThreads / NCH;      // threads per chunk
    static_assert(NCH <= kThreads && NSG * NCH == kThreads, "merge layout");
    static_assert(NSG * G * D * 4 <= kTile * S::kPitch, "merge reduction scratch");
    constexpr int U = 8;                     // loads in flight per thread
    float* wl = reinterpret_cast<float*>(k_lds);   // [CAPN][G]
    float* red = reinterpret_cast<float*>(v_lds);  // [NSG][G * D]
    const int hq0 = kvh * G;
    const int c = tid % NCH, sg = tid / NCH;
    const int hc = (c * 4) / D;
    auto o_off = [&](int k) { return (((s0 + k * step) * a.hq + hq0) * D + c * 4) * 4; };
    auto stage = [&](int c0, int cn) {
      for (int idx = tid; idx < cn * G; idx += kThreads) {
        const int k = idx / G, h = idx - k * G;
        wl[idx] = coherent_load1(pr_l, ((s0 + (c0 + k) * step) * a.hq + hq0 + h) * 4);
      }
    };
    // A fold whose partials fit U per thread (a group of 16 at D = 128,
    // G = 4) issues their output loads before the lse values are staged, so
    // both arrive in one round trip; indices past n reload partial n - 1,
    // which the accumulation skips.  Contiguous layout only: the registers
    // would take the paged kernels past 256 (one wave per SIMD).
    const bool pre = !PAGED && n <= U * NSG && n <= CAPN;
    floatx4 opre[U];
    if (pre) {
#pragma unroll
      for (int u = 0; u < U; ++u) opre[u] = coherent_load4(pr_o, o_off(min(sg + u * NSG, n - 1)));
    }
    __syncthreads();  // earlier users of the tile buffers and a_lds are done
    for (int c0 = 0; c0 < n; c0 += CAPN) {
      const int cn = min(CAPN, n - c0);
      if (c0 > 0) __syncthreads();
      stage(c0, cn);
      __syncthreads();
      for (int h = wave; h < G; h += 4) {
        float m = -INFINITY;
        for (int k = lane; k < cn; k += 64) m = fmaxf(m, wl[k * G + h]);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
        float w = 0.f;
        for (int k = lane; k < cn; k += 64) {
          const float x = wl[k * G + h];
          w += (x == -INFINITY) ? 0.f : expf(x - m);
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) w += __shfl_xor(w, o);
        if (lane == 0) {
          const float mp = c0 > 0 ? a_lds[0][h] : -INFINITY;
          const float wp = c0 > 0 ? a_lds[1][h] : 0.f;
          const float M = fmaxf(mp, m);
          a_lds[0][h] = M;
          a_lds[1][h] = (M == -INFINITY) ? 0.f
                                          : (mp == -INFINITY ? 0.f : wp * expf(mp - M)) +
                                                (m == -INFINITY ? 0.f : w * expf(m - M));
        }
      }
      __syncthreads();
    }
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < n; c0 += CAPN) {
      const int cn = min(CAPN, n - c0);
      if (n > CAPN) {  // restage this chunk (pass 1 left the last one)
        __syncthreads();
        stage(c0, cn);
        __syncthreads();
      }
      for (int idx = tid; idx < cn * G; idx += kThreads) {
        const int h = idx % G;
        const float x = wl[idx], M = a_lds[0][h];
        wl[idx] = (M == -INFINITY || x == -INFINITY) ? 0.f : expf(x - M) / a_lds[1][h];
      }
      __syncthreads();
      if (pre) {  // one chunk (n <= CAPN), outputs already in registers
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int kk = sg + u * NSG;
          if (kk < cn) {
            const float w = wl[kk * G + hc];
            if (w != 0.f) acc += w * opre[u];
          }
        }
        continue;
      }
      // U loads in flight per thread in every round, the last one included:
      // indices past the chunk reload its last partial and are skipped
      for (int k = sg; k < cn; k += U * NSG) {
        floatx4 o[U];
#pragma unroll
        for (int u = 0; u < U; ++u) o[u] = coherent_load4(pr_o, o_off(c0 + min(k + u * NSG, cn - 1)));
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int kk = k + u * NSG;
          if (kk < cn) {
            const float w = wl[kk * G + hc];
            if (w != 0.f) acc += w * o[u];
          }
        }
      }
    }
    *reinterpret_cast<floatx4*>(red + sg * G * D + c * 4) = acc;
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += kThreads) {
      float o = 0.f;
#pragma unroll
      for (int k = 0; k < NSG; ++k) o += red[k * G * D + idx];
      const int h = idx / D;
      if (a_lds[0][h] == -INFINITY) o = 0.f;
      if (dst < 0) a.out_o[((size_t)b * a.hq + hq0) * D + idx] = o;
      else coherent_store1(pr_o, ((dst * a.hq + hq0) * D + idx) * 4, o);
    }
    if (tid < G) {
      const float M = a_lds[0][tid];
      const float lse = (M == -INFINITY) ? -INFINITY : M + logf(a_lds[1][tid]);
      if (dst < 0) {
        if (a.out_lse) a.out_lse[(size_t)b * a.hq + hq0 + tid] = lse;
      } else {
        coherent_store1(pr_l, (dst * a.hq + hq0 + tid) * 4, lse);
      }
    }
  };

  // Fused form: the partial at relative slot rel of (b, kvh) is written and
  // acknowledged.  Count it in its group; the group's last arrival merges the
  // group into the group's first slot (or, for a single group, into the
  // output) and counts the group; the last group merges the group results.
  auto arrive = [&](int b, int rel) {
    const int S_b = seq_slots(b), first = seq_first(b);
    const int gk = rel / kMergeGroup;
    const int gs = first + gk * kMergeGroup;
    const int gn = min(kMergeGroup, S_b - gk * kMergeGroup);
    const int ng = (S_b + kMergeGroup - 1) / kMergeGroup;
    int* c1 = a.group_cnt + (size_t)gs * a.hkv + kvh;
    int* c2 = a.group_cnt + (size_t)a.max_slots * a.hkv + (size_t)b * a.hkv + kvh;
    if (gn > 1) {  // a group of one slot is its own result
      if (tid == 0) s_flag = atomicAdd(c1, 1) + 1 == gn;
      __syncthreads();
      if (!s_flag) return;
      if (tid == 0) __hip_atomic_store(c1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (ng == 1) {
      merge(b, gs, 1, gn, -1);
      return;
    }
    if (gn > 1) {
      merge(b, gs, 1, gn, gs);
      wait_stores();
    }
    __syncthreads();
    if (tid == 0) s_flag = atomicAdd(c2, 1) + 1 == ng;
    __syncthreads();
    if (!s_flag) return;
    if (tid == 0) __hip_atomic_store(c2, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    merge(b, first, kMergeGroup, ng, -1);
  };

  // Fused form, appended token of (b, kvh): rotate its key at pos_new[b]
  // (fp64, one bf16 rounding), write its one-token partial (o = v, lse = its
  // scaled score) into the sequence's first slot, count it, and store K and V
  // in the token's cache slot.  The token's own loads are issued before the
  // query rotation, and the cache stores after the count: nothing in this
  // launch reads the cache row, and waiting for their acknowledgement (a PCIe
  // write for a host slot) would delay the count.
  auto new_token = [&](int b) {
    const int kvd = a.hkv * D;
    const int p = a.pos_new ? a.pos_new[b] : a.seq_lens[b];
    int64_t Lb = PAGED ? 0 : a.seq_lens[b];
    // this thread's inputs: K pair (i, i + D/2) for tid < D/2, V dims (i, i + D/2) for D/2 <= tid < D
    const int i = tid < D / 2 ? tid : tid - D / 2;
    float in0 = 0.f, in1 = 0.f;
    if (tid < D) {
      const size_t base = tid < D / 2 ? (size_t)kvh * D : (size_t)kvd + kvh * D;  // projection: K then V
      if (a.kv_proj) {
        const float* src = a.kv_proj + (size_t)b * 2 * kvd + base;
        in0 = src[i];
        in1 = src[i + D / 2];
      } else {
        const uint16_t* src = (tid < D / 2 ? a.k_new : a.v_new) + (size_t)b * kvd + kvh * D;
        in0 = bf16_to_f32(src[i]);
        in1 = bf16_to_f32(src[i + D / 2]);
      }
    }
    if (q_b != b || q_kvh != kvh) rotate_q(b);
    float* kr = reinterpret_cast<float*>(k_lds);  // rotated key (bf16 values) [D]
    float* vr = kr + D;                           // value [D]
    // slot of (b, p)
    uint16_t* sk = nullptr;
    uint16_t* sv = nullptr;
    if (p >= 0) {
      if (PAGED) {
        const int lp = p >> a.page_shift;
        if (lp < a.max_pages) {
          const int32_t e = a.page_table[(int64_t)b * a.max_pages + lp];
          const bool host = (e & 1) != 0;
          const int64_t row = ((int64_t)(e >> 1) << a.page_shift) | (p & ((1 << a.page_shift) - 1));
          if (e >= 0 && row < (host ? a.host_rows : a.dev_rows) && (host ? a.host_k : a.dev_k)) {
            sk = (host ? a.host_k : a.dev_k) + row * kvd + kvh * D;
            sv = (host ? a.host_v : a.dev_v) + row * kvd + kvh * D;
          }
        }
      } else {
        if (Lb < 0) Lb = 0;
        int64_t nh, nd, ph;
        contig_tiers(a.ratio, Lb, Lb + 1, &nh, &nd, &ph);
        const bool host = p < ph;
        if (p <= Lb) {
          const int64_t row = host ? (int64_t)b * a.host_stride + p : (int64_t)b * a.dev_stride + (p - ph);
          const bool fits_row = host ? (ph <= a.host_stride && row < a.host_rows && a.host_k)
                                     : (Lb + 1 - ph <= a.dev_stride && row < a.dev_rows && a.dev_k);
          if (fits_row) {
            sk = (host ? a.host_k : a.dev_k) + row * kvd + kvh * D;
            sv = (host ? a.host_v : a.dev_v) + row * kvd + kvh * D;
          }
        }
      }
    }
    if (!sk && tid == 0) atomicOr(&a.counters[decode_error_word()], kDecodeErrSlot);
    // bf16 bits this thread stores into the cache row after the count
    uint32_t out0 = 0, out1 = 0;
    if (tid < D / 2) {
      double sn, cs;
      sincos((double)p * a.freq.f[i], &sn, &cs);
      const double xl = (double)in0, xh = (double)in1;
      out0 = f64_to_bf16(xl * cs - xh * sn);
      out1 = f64_to_bf16(xh * cs + xl * sn);
      kr[i] = bf16_to_f32(out0);
      kr[i + D / 2] = bf16_to_f32(out1);
    } else if (tid < D) {
      // V is stored as given (bf16), or rounded once from the fp32 projection
      out0 = a.kv_proj ? f32_to_bf16(in0) : (__float_as_uint(in0) >> 16);
      out1 = a.kv_proj ? f32_to_bf16(in1) : (__float_as_uint(in1) >> 16);
      vr[i] = bf16_to_f32(out0);
      vr[i + D / 2] = bf16_to_f32(out1);
    }
    __syncthreads();
    const int slot = seq_first(b);
    const __amdgpu_buffer_rsrc_t pr_o = coherent_rsrc(a.part_o);
    const __amdgpu_buffer_rsrc_t pr_l = coherent_rsrc(a.part_lse);
    // scores: 32 lanes per head
    {
      const int h = tid >> 5, l32 = tid & 31;
      float s = 0.f;
      if (h < G)
        for (int d = l32; d < D; d += 32) s = fmaf(q_lds[h][d], kr[d], s);
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) s += __shfl_xor(s, o);
      if (h < G && l32 == 0)  // log2 units -> natural log
        coherent_store1(pr_l, (slot * a.hq + kvh * G + h) * 4, s * 0.69314718055994530942f);
    }
    for (int idx = tid; idx < G * D; idx += kThreads)
      coherent_store1(pr_o, ((slot * a.hq + kvh * G) * D + idx) * 4, vr[idx % D]);
    wait_stores();
    __syncthreads();
    arrive(b, 0);
    if (tid < D / 2) {
      if (sk) {
        sk[i] = (uint16_t)out0;
        sk[i + D / 2] = (uint16_t)out1;
      }
    } else if (tid < D) {
      if (sv) {
        sv[i] = (uint16_t)out0;
        sv[i + D / 2] = (uint16_t)out1;
      }
    }
  };

  int units_done = 0;
  // Appended tokens (fused form): one (sequence, KV head) pair each, queued
  // after the attention units of the HBM tier (of the host tier when there is
  // no HBM tier), so the first workgroups to run out of units take them.
  const int n_new = (FUSED && a.new_tokens && fits && (T.team_d > 0 ? !host_role : host_role)) ? B * a.hkv : 0;
  // A tier with at most two units per workgroup deals them round-robin (the
  // next unit of a workgroup is its current one plus the workgroup count):
  // with so few, the queue balances nothing, and its atomic would put a round
  // trip at the end of every unit.
  const bool dealt = n_units + n_new <= 2 * role_wgs;

  u32x4 kreg[NC], vreg[NC];
  // Paged: the physical page of each of this thread's chunks of a tile, from
  // the tier list, issued right before the tile's loads.  One form for every
  // page size (vector loads, lanes of a page share a line): a runtime choice
  // between scalar and vector lookups left loads of one branch pending on
  // registers the other reuses, which made the compiler wait for the whole
  // tile in flight before every tile's compute.
  auto lookup = [&](const DItem& it, int tile, int32_t* pte) {
    const int32_t* pl = tier_list + (int64_t)it.b * a.max_pages;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int tok = min(tile * kTile + (tid + c * kThreads) / S::kChunksPerRow, it.n_tok - 1);
      pte[c] = pl[(it.k0 + tok) >> a.page_shift];
    }
  };
  auto load_tile = [&](const DItem& it, int kv, int tile, const int32_t* pte) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int chunk = tid + c * kThreads;
      const int r = chunk / S::kChunksPerRow;
      const int col = chunk - r * S::kChunksPerRow;
      // rows past the item's end load its last token again (real data whose
      // scores the mask removes, so p = 0 exactly): every load is issued
      // unconditionally and none waits for another
      const int tok = min(tile * kTile + r, it.n_tok - 1);
      int64_t row;
      if (PAGED) {
        const int64_t k = it.k0 + tok;
        row = ((int64_t)pte[c] << a.page_shift) | (k & ((1 << a.page_shift) - 1));
      } else {
        row = (int64_t)it.b * stride + it.k0 + tok;
      }
      const int64_t off = (row * a.hkv + kv) * D + col * 8;
      // KV is read once per step: non-temporal loads on both tiers
      kreg[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kpool + off));
      vreg[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vpool + off));
    }
  };

  // unit u: its item and KV head
  auto unit_item = [&](int u, int* kv) -> DItem {
    const int item = u / a.hkv;
    *kv = u - item * a.hkv;
    return item_at(L, B, host_role, item);
  };
  int i = r_idx;
  DItem it{};
  int32_t pte[NC] = {};
  // paged: pte holds the pages of the next tile to load (looked up one tile
  // ahead of its loads; past an item's last tile it repeats the last one)
  if (i < n_units) {
    it = unit_item(i, &kvh);
    if (PAGED) lookup(it, 0, pte);
    load_tile(it, kvh, 0, pte);
    if (PAGED) lookup(it, min(1, (it.n_tok - 1) / kTile), pte);
  }
  float acc[G][DPL];
  bf16x8_t qb[KS];
  while (i < n_units) {
    ++units_done;
    const int ntiles = (it.n_tok + kTile - 1) / kTile;
    if (q_b != it.b || q_kvh != kvh) rotate_q(it.b);
    {
      // query operand: columns h (high bf16 part) and h+8 (low part)
      const int hsel = n & 7;
      const bool active = hsel < G;
      const float* qr = &q_lds[active ? hsel : 0][0];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const floatx4 lo4 = *reinterpret_cast<const floatx4*>(qr + ks * 32 + j4 * 8);
        const floatx4 hi4 = *reinterpret_cast<const floatx4*>(qr + ks * 32 + j4 * 8 + 4);
        const float x8[8] = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = active ? x8[2 * e] : 0.f;
          const float x1 = active ? x8[2 * e + 1] : 0.f;
          uint32_t b0 = f32_to_bf16(x0), b1 = f32_to_bf16(x1);
          if (n >= 8) {  // low part: residual after the high part
            b0 = f32_to_bf16(x0 - bf16_to_f32(b0));
            b1 = f32_to_bf16(x1 - bf16_to_f32(b1));
          }
          w[e] = b0 | (b1 << 16);
        }
        u32x4 wv = {w[0], w[1], w[2], w[3]};
        qb[ks] = __builtin_bit_cast(bf16x8_t, wv);
      }
    }
    float m_run = -INFINITY;  // per lane: state of head (n & 7)
    float l_run = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[h][e] = 0.f;
    int next_i = n_units;
    int nkvh = kvh;
    DItem nit{};
    for (int tile = 0; tile < ntiles; ++tile) {
      __syncthreads();  // previous tile's readers are done
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int chunk = tid + c * kThreads;
        const int r = chunk / S::kChunksPerRow;
        const int col = chunk - r * S::kChunksPerRow;
        *reinterpret_cast<u32x4*>(k_lds + r * S::kPitch + col * 16) = kreg[c];
        *reinterpret_cast<u32x4*>(v_lds + r * S::kPitch + col * 16) = vreg[c];
      }
      const bool last = tile + 1 == ntiles;
      if (last && tid == 0) s_next = dealt ? i + role_wgs : role_wgs + atomicAdd(qctr, 1);
      __syncthreads();
      // keep one tile in flight: the next tile of this item, or the first
      // tile of the next item while this item's last tile is computed
      if (!last) {
        load_tile(it, kvh, tile + 1, pte);
        if (PAGED) lookup(it, min(tile + 2, ntiles - 1), pte);
      } else {
        next_i = __builtin_amdgcn_readfirstlane(s_next);
        if (next_i < n_units) {
          nit = unit_item(next_i, &nkvh);
          if (PAGED) lookup(nit, 0, pte);
          load_tile(nit, nkvh, 0, pte);
          if (PAGED) lookup(nit, min(1, (nit.n_tok - 1) / kTile), pte);
        }
      }

      // ---- scores for this wave's 16 tokens: rows = tokens, columns = heads
      floatx4 sc = {0.f, 0.f, 0.f, 0.f};
      const uint8_t* krow = k_lds + (wave * 16 + n) * S::kPitch + j4 * 16;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 kv = *reinterpret_cast<const u32x4*>(krow + ks * 64);
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kv), qb[ks], sc, 0, 0, 0);
      }
      const int tok0 = tile * kTile + wave * 16 + j4 * 4;
      float s[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float v = sc[q] + __shfl_xor(sc[q], 8);
        s[q] = (tok0 + q < it.n_tok) ? v : -INFINITY;
      }
      float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_run - m_new);
      float p[4], ps = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        p[q] = (s[q] == -INFINITY) ? 0.f : exp2f(s[q] - m_new);
        ps += p[q];
      }
      ps += __shfl_xor(ps, 16);
      ps += __shfl_xor(ps, 32);
      l_run = l_run * alpha + ps;
      m_run = m_new;
      if (n < G) {
#pragma unroll
        for (int q = 0; q < 4; ++q) p_lds[wave][j4 * 4 + q][n] = p[q];
        if (j4 == 0) a_lds[wave][n] = alpha;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

      // ---- P.V: lane owns dims lane*DPL .. lane*DPL+DPL-1
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float al = a_lds[wave][h];
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[h][e] *= al;
      }
      const uint8_t* vbase = v_lds + (wave * 16) * S::kPitch + lane * DPL * 2;
#pragma unroll 4
      for (int t = 0; t < 16; ++t) {
        float vv[DPL];
        if (DPL == 2) {
          const uint32_t w = *reinterpret_cast<const uint32_t*>(vbase + t * S::kPitch);
          vv[0] = __uint_as_float(w << 16);
          vv[DPL - 1] = __uint_as_float(w & 0xffff0000u);
        } else {
          const uint32_t w = *reinterpret_cast<const uint16_t*>(vbase + t * S::kPitch);
          vv[0] = __uint_as_float(w << 16);
        }
        float pp[G];
#pragma unroll
        for (int h = 0; h < G; ++h) pp[h] = p_lds[wave][t][h];
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < DPL; ++e) acc[h][e] = fmaf(pp[h], vv[e], acc[h][e]);
      }
      __builtin_amdgcn_wave_barrier();
    }

    // ---- end of the unit: combine the four waves and write its partial
    __syncthreads();
    {
      float* sm_m = reinterpret_cast<float*>(k_lds);   // [4][G]
      float* sm_l = sm_m + 4 * G;                      // [4][G]
      float* sm_acc = sm_l + 4 * G;                    // [4][G][D]
      if (lane < G) {
        sm_m[wave * G + lane] = m_run;
        sm_l[wave * G + lane] = l_run;
      }
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < DPL; ++e) sm_acc[(wave * G + h) * D + lane * DPL + e] = acc[h][e];
      __syncthreads();
      const int slot = FUSED ? it.slot + (it.b + 1) * a.new_tokens : it.slot;
      for (int idx = tid; idx < G * D; idx += kThreads) {
        const int h = idx / D, d = idx - h * D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w * G + h]);
        float o = 0.f, lsum = 0.f;
        if (M != -INFINITY) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float mw = sm_m[w * G + h];
            const float sw = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
            lsum += sw * sm_l[w * G + h];
            o += sw * sm_acc[(w * G + h) * D + d];
          }
          o = o / lsum;
        }
        const float lse = (M == -INFINITY) ? -INFINITY : (M + log2f(lsum)) * 0.69314718055994530942f;
        const int hq_idx = kvh * G + h;
        if (FUSED) {
          coherent_store1(coherent_rsrc(a.part_o), ((slot * a.hq + hq_idx) * D + d) * 4, o);
          if (d == 0) coherent_store1(coherent_rsrc(a.part_lse), (slot * a.hq + hq_idx) * 4, lse);
        } else {
          a.part_o[((size_t)slot * a.hq + hq_idx) * D + d] = o;
          if (d == 0) a.part_lse[(size_t)slot * a.hq + hq_idx] = lse;
        }
      }
      if (FUSED) {
        wait_stores();
        __syncthreads();
        arrive(it.b, a.new_tokens + it.slot - L.off[it.b]);
      }
    }
    // the next item's first tile is already in registers
    i = next_i;
    it = nit;
    kvh = nkvh;
  }
  // appended tokens: queue indices [n_units, n_units + n_new)
  if constexpr (FUSED) {
    while (i < n_units + n_new) {
      const int pr = i - n_units;
      kvh = pr % a.hkv;
      new_token(pr / a.hkv);
      if (tid == 0) s_next = dealt ? i + role_wgs : role_wgs + atomicAdd(qctr, 1);
      __syncthreads();
      i = __builtin_amdgcn_readfirstlane(s_next);
    }
  }

  // Fused form: sequences with nothing to merge (no tokens and no appended token).
  if (FUSED && !a.new_tokens && fits && blockIdx.x == 0) {
    for (int b = 0; b < B; ++b)
      if (L.off[b + 1] == L.off[b])
        for (int idx = tid; idx < a.hq * D; idx += kThreads) {
          a.out_o[(size_t)b * a.hq * D + idx] = 0.f;
          if (idx < a.hq && a.out_lse) a.out_lse[(size_t)b * a.hq + idx] = -INFINITY;
        }
  }

  // Last workgroup out clears the item queues for the next call on this
  // workspace.  When neither tier took units from its queue (both dealt
  // round-robin, as every workgroup finds from the same lengths), no counter
  // moved and the exit count, a round trip at the end of the launch, is
  // skipped.
  const auto queue_used = [&](bool host) {
    const int wgs = a.hkv * (host ? T.team_h : T.team_d);
    const int units = fits ? (host ? L.ph[B] : L.pm[B] + L.pt[B]) * a.hkv : 0;
    const int news = (FUSED && a.new_tokens && fits && (T.team_d > 0 ? !host : host)) ? B * a.hkv : 0;
    return wgs > 0 && units + news > 2 * wgs;
  };
  const bool queues = queue_used(true) || queue_used(false);
  __syncthreads();
  if (tid == 0 && queues) {
    wait_stores();
    const int ec = decode_exit_counter();
    const int done = atomicAdd(&a.counters[ec], 1) + 1;
    if (done == (int)gridDim.x) {
      for (int k = decode_queue(true); k < decode_counter_words(); ++k)
        __hip_atomic_store(&a.counters[k], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.counters[ec], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (traced) {
    uint64_t* t = a.wg_trace + 4 * (size_t)blockIdx.x;
    t[0] = t_start;
    t[1] = wall_clock64();
    t[2] = host_role ? 1 : 0;
    t[3] = (uint64_t)units_done;
  }
}

// ---------------------------------------------------------------------------
// Static scratch for callers that cannot allocate device memory (the
// allocation-free decode step): a file-scope device array, one copy on every
// GPU the library runs on, zero when the code object loads.  Its first
// kDecodeStaticCounterBytes hold the counters of every call and nothing else;
// every completed call leaves them at zero again and rewrites everything else
// it reads, so calls of any shape follow each other on it; calls that overlap
// on one GPU race.  Host code never uses the array's name as an address: the
// per-device address comes from hipGetSymbolAddress.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[kDecodeStaticScratchBytes];

int decode_static_scratch(void** ptr, size_t* bytes) {
  static std::mutex mu;
  static void* per_device[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!per_device[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  *bytes = kDecodeStaticScratchBytes;
  return (int)hipSuccess;
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
int launch_decode_tiers(const DecodeArgs& a, int32_t* tier_counts, int32_t* tier_pages, void* stream) {
  if (a.batch < 1) return (int)hipSuccess;
  const int chunks = (int)std::max<int64_t>(1, ((int64_t)a.max_pages + kTierChunk - 1) / kTierChunk);
  hipLaunchKernelGGL(decode_tiers_kernel, dim3(chunks, a.batch), dim3(kTierThreads), 0, (hipStream_t)stream, a,
                     tier_counts, tier_pages);
  return (int)hipGetLastError();
}

template <int D, int G, bool FUSED>
static hipError_t launch_decode_dgf(const DecodeArgs& a, hipStream_t s) {
  const int grid = a.hkv * (a.tmpl.team_h + a.tmpl.team_d);
  if (grid < 1) return hipErrorInvalidValue;
  if (a.page_shift >= 0)
    hipLaunchKernelGGL((decode_kernel<D, G, true, FUSED>), dim3(grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((decode_kernel<D, G, false, FUSED>), dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int D, int G>
static hipError_t launch_decode_dg(const DecodeArgs& a, hipStream_t s) {
  return a.fused ? launch_decode_dgf<D, G, true>(a, s) : launch_decode_dgf<D, G, false>(a, s);
}

template <int D>
static hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t s) {
  switch (a.hq / a.hkv) {
    case 1: return launch_decode_dg<D, 1>(a, s);
    case 2: return launch_decode_dg<D, 2>(a, s);
    case 4: return launch_decode_dg<D, 4>(a, s);
    case 8: return launch_decode_dg<D, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

int launch_decode(const DecodeArgs& a, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (a.head_dim == 64) return (int)launch_decode_d<64>(a, s);
  if (a.head_dim == 128) return (int)launch_decode_d<128>(a, s);
  return (int)hipErrorInvalidValue;
}

}  // namespace dkv
