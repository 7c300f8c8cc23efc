// dkv_plan.cpp - split planner: offload ratio / page tiers -> per-tier work
// items, split slots and the workgroup split between the host and HBM tiers.
//
// SplitKernel README, Overview: prefetching designs leave the aggregate
// bandwidth of the local and remote tiers unused; here both tiers stream at
// once, each on its own set of workgroups.  SplitKernel README, Usage: the
// offloading ratio places the oldest floor(r * L) tokens in host memory.
//
// Pure C++: no HIP calls, so CPU tests can exercise it.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>

#include "dkv_internal.h"

namespace dkv {
namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int64_t round_up(int64_t a, int64_t m) { return ceil_div(a, m) * m; }

bool fail(std::string* err, const char* fmt, long long a = 0, long long b = 0, long long c = 0) {
  char buf[256];
  snprintf(buf, sizeof buf, fmt, a, b, c);
  *err = buf;
  return false;
}

// Attention workgroups the planner places per CU.  Two per CU stream HBM at
// its best measured rate; more only lengthen the tail of the persistent loop.
constexpr int kSlotsPerCu = 2;

// Tokens per work item.  Workgroups take units dynamically, so several units
// per workgroup even out per-CU speed differences; the floor keeps each unit
// long enough that its fixed cost (query operand, epilogue, partial write)
// stays small next to its KV stream.
int32_t choose_chunk(int64_t tier_token_heads, int32_t wgs, int32_t units_per_wg, int32_t floor_tok,
                     int32_t cap_tok, int32_t align, int32_t tuned) {
  if (tuned > 0) return (int32_t)round_up(tuned, align);
  if (tier_token_heads <= 0 || wgs <= 0) return align;
  int64_t c = ceil_div(tier_token_heads, (int64_t)wgs * units_per_wg);
  c = std::max<int64_t>(c, floor_tok);
  c = std::min<int64_t>(c, cap_tok);
  return (int32_t)round_up(c, align);
}

// Workgroups per tier for a launch whose tiers stream host_units and
// dev_units (any common unit).  Measured on MI355X: 48-64 workgroups keep
// PCIe 5.0 x16 full for a host tier alone; while HBM streams at the same
// time, every extra host workgroup costs HBM throughput, so a balanced split
// uses cus/16 (never below the bandwidth-proportional share of the resident
// slots); HBM workgroups fill the remaining slots.
void split_workgroups(const PlanInput& in, int64_t host_units, int64_t dev_units, int32_t* wh_out,
                      int32_t* wd_out) {
  const int32_t cus = std::max(1, in.num_cus);
  const int32_t resident = cus * kSlotsPerCu;
  const double bw_h = in.host_bw > 0 ? in.host_bw : 57.0;
  const double bw_d = in.dev_bw > 0 ? in.dev_bw : 5300.0;
  int32_t wh = 0, wd = 0;
  if (host_units > 0 && dev_units > 0) {
    const bool host_dominant = (double)host_units / bw_h > 1.5 * (double)dev_units / bw_d;
    const int32_t want_h = in.host_wgs > 0 ? in.host_wgs : (host_dominant ? std::max(8, cus * 3 / 16) : std::max(4, cus / 16));
    wh = std::max(want_h, (int32_t)std::lround(resident * bw_h / (bw_h + bw_d)));
    wh = std::min(wh, resident / 2);
    wd = in.dev_wgs > 0 ? in.dev_wgs : resident - wh;
  } else if (host_units > 0) {
    wh = in.host_wgs > 0 ? in.host_wgs : std::max(8, cus / 4);
  } else if (dev_units > 0) {
    wd = in.dev_wgs > 0 ? in.dev_wgs : resident;
  }
  *wh_out = wh;
  *wd_out = wd;
}

}  // namespace

// ---------------------------------------------------------------- decode
//
// The decode kernel derives its items on the device (dkv_decomp.h); the host
// only fixes the shape of the launch: workgroups per tier and per KV head, and
// the item-length rules.  Nothing here depends on the sequence lengths.
DecodeTemplate decode_template(const PlanInput& in, bool host_tier, bool dev_tier, double host_frac) {
  DecodeTemplate t{};
  t.hkv = std::max(1, in.hkv);
  const int32_t cus = std::max(1, in.num_cus);
  const int32_t resident = cus * kSlotsPerCu;
  // the same workgroup split as the other split kernels, with an expected
  // host share in place of the byte counts
  int32_t wh = 0, wd = 0;
  const double f = std::min(1.0, std::max(0.0, host_frac));
  split_workgroups(in, host_tier ? (int64_t)std::llround(f * 1e9) : 0,
                   dev_tier ? (int64_t)std::llround((1.0 - f) * 1e9) : 0, &wh, &wd);
  if (host_tier && wh < 1) wh = 1;
  if (dev_tier && wd < 1) wd = 1;
  t.team_h = host_tier ? (int32_t)ceil_div(wh, t.hkv) : 0;
  t.team_d = dev_tier ? (int32_t)std::max<int64_t>(1, (in.dev_wgs > 0 ? ceil_div(wd, t.hkv)
                                                                        : (resident - t.team_h * t.hkv) / t.hkv))
                      : 0;
  const bool mixed = host_tier && dev_tier;
  t.upw_h = mixed ? 4 : 2;
  t.upw_d = 6;
  // host items as short as one tile when the tier is small (a PCIe round trip
  // per tile: many short items in flight beat a few long ones); HBM items of
  // at least 512 tokens (the 32k-token layer from HBM: 0.032 ms as 512-token
  // units against 0.038 ms as 1024-token units on MI355X)
  t.floor_h = kTile;
  t.floor_d = 512;
  t.align = (int32_t)std::max<int64_t>(kTile, in.page_size > 0 ? in.page_size : 1);
  t.guided = 1;
  t.tuned_h = in.host_chunk > 0 ? (int32_t)round_up(in.host_chunk, t.align) : 0;
  t.tuned_d = in.dev_chunk > 0 ? (int32_t)round_up(in.dev_chunk, t.align) : 0;
  return t;
}

bool decode_tiers_host(const PlanInput& in, int64_t b, int64_t attended, std::vector<int32_t>* host_pages,
                       std::vector<int32_t>* dev_pages, int64_t* nh, int64_t* nd) {
  const int64_t P = in.page_size;
  int64_t A = std::max<int64_t>(0, attended);
  int64_t npg = ceil_div(A, P);
  bool ok = true;
  if (npg > in.max_pages) {
    ok = false;
    npg = in.max_pages;
    A = npg * P;
  }
  host_pages->clear();
  dev_pages->clear();
  int last = -1;
  for (int64_t j = 0; j < npg; ++j) {
    const int32_t e = in.page_table_host[b * in.max_pages + j];
    const bool host = (e & 1) != 0;
    const int64_t cap = host ? (in.host_rows / P) : (in.dev_rows / P);
    if (e < 0 || (int64_t)(e >> 1) >= cap) {
      ok = false;
      continue;
    }
    (host ? host_pages : dev_pages)->push_back((int32_t)j);
    if (j == npg - 1) last = host ? 1 : 0;
  }
  const int64_t deficit = npg > 0 ? P - (A - (npg - 1) * P) : 0;
  *nh = (int64_t)host_pages->size() * P - (last == 1 ? deficit : 0);
  *nd = (int64_t)dev_pages->size() * P - (last == 0 ? deficit : 0);
  return ok;
}

void decode_enumerate(const DecodeTemplate& t, int B, const int64_t* nh, const int64_t* nd,
                      std::vector<DecodeHostItem>* items, std::vector<int32_t>* offsets, DecodeSizes* zout) {
  int64_t th = 0, td = 0;
  for (int b = 0; b < B; ++b) {
    th += nh[b];
    td += nd[b];
  }
  const DecodeSizes z = decode_sizes(t, th, td);
  if (zout) *zout = z;
  std::vector<DecodeSeqItems> s(B);
  offsets->assign(B + 1, 0);
  for (int b = 0; b < B; ++b) {
    s[b] = decode_seq_items(z, t.align, nh[b], nd[b]);
    (*offsets)[b + 1] = (*offsets)[b] + decode_seq_splits(s[b]);
  }
  items->clear();
  // host items, then HBM items before the tail, then the tail (the order the
  // kernel's queues hand them out)
  for (int b = 0; b < B; ++b)
    for (int c = 0; c < s[b].uh; ++c) {
      const int64_t k0 = (int64_t)c * z.ch;
      items->push_back({1, b, (*offsets)[b] + c, (int32_t)std::min<int64_t>(z.ch, nh[b] - k0), k0});
    }
  for (int b = 0; b < B; ++b)
    for (int c = 0; c < s[b].um; ++c) {
      const int64_t k0 = (int64_t)c * z.cd;
      items->push_back({0, b, (*offsets)[b] + s[b].uh + c, (int32_t)std::min<int64_t>(z.cd, s[b].t0 - k0), k0});
    }
  for (int b = 0; b < B; ++b)
    for (int c = 0; c < s[b].ut; ++c) {
      const int64_t k0 = s[b].t0 + (int64_t)c * z.cs;
      items->push_back(
          {0, b, (*offsets)[b] + s[b].uh + s[b].um + c, (int32_t)std::min<int64_t>(z.cs, nd[b] - k0), k0});
    }
}

}  // namespace dkv

namespace dkv {

// ---------------------------------------------------------------- prefill
//
// DirectKV README, Step 6 ("Prefill (all new KV)"): new tokens attend
// causally to the cache.  A block of QB = 128/G consecutive query rows of one
// sequence shares one stream of its KV prefix [0, last row's position]; that
// prefix is cut by tier and into chunks, one work item per (block, chunk).
bool build_prefill_plan(const PlanInput& in, const int32_t* q_start, const int32_t* q_pos0,
                        PlanLayout* out, std::vector<uint8_t>* blob, std::string* err) {
  *out = PlanLayout{};
  const int B = in.batch;
  if (B < 1) return fail(err, "batch must be >= 1 (got %lld)", B);
  if (!in.seq_lens || !q_start || !q_pos0) return fail(err, "seq_lens, q_start and q_pos0 are required");
  if (in.hkv < 1 || in.hq % in.hkv) return fail(err, "num_q_heads must be a multiple of num_kv_heads");
  const int G = in.hq / in.hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(err, "query group size %lld not built", G);
  const int QB = kPrefillRows / G;
  const bool paged = in.page_size > 0;
  const int64_t P = paged ? in.page_size : 1;
  const int64_t row_bytes = (int64_t)in.hkv * in.head_dim * 2;
  if (q_start[0] != 0) return fail(err, "q_start[0] must be 0");

  // ---- per-sequence placement (validated exactly as for decode)
  std::vector<int64_t> nh(B, 0);
  std::vector<std::vector<int32_t>> host_pages(paged ? B : 0), dev_pages(paged ? B : 0);
  std::vector<int64_t> emax(B, 0);
  std::vector<int64_t> pre(B, 0);    // tokens below pre[b] come from the tiers
  std::vector<int32_t> nblk(B, 0);
  for (int b = 0; b < B; ++b) {
    const int64_t L = in.seq_lens[b];
    const int64_t n = (int64_t)q_start[b + 1] - q_start[b];
    if (n < 0) return fail(err, "q_start must be non-decreasing (sequence %lld)", b);
    if (L < 1) return fail(err, "seq_lens[%lld] must be >= 1", b);
    if (q_pos0[b] < 0 || (int64_t)q_pos0[b] + n > L)
      return fail(err, "sequence %lld: query rows at positions %lld.. exceed the %lld cached tokens", b,
                  q_pos0[b], L);
    emax[b] = n > 0 ? (int64_t)q_pos0[b] + n : 0;
    pre[b] = in.prefill_fresh ? (int64_t)q_pos0[b] : L;
    nblk[b] = (int32_t)ceil_div(n, QB);
    if (!paged) {
      const int64_t h = (int64_t)std::floor(in.ratio * (double)L);
      nh[b] = h;
      if (h > 0 && (h > in.host_stride || (int64_t)b * in.host_stride + h > in.host_rows))
        return fail(err, "sequence %lld: host rows needed beyond host_stride/host_rows", b);
      if (L - h > 0 && (L - h > in.dev_stride || (int64_t)b * in.dev_stride + (L - h) > in.dev_rows))
        return fail(err, "sequence %lld: device rows needed beyond dev_stride/dev_rows", b);
    } else {
      if (!in.page_table_host) return fail(err, "paged layout needs page_table_host");
      const int64_t npg = ceil_div(L, P);
      if (npg > in.max_pages) return fail(err, "sequence %lld needs %lld pages > max_pages", b, npg);
      for (int64_t j = 0; j < npg; ++j) {
        const int32_t e = in.page_table_host[(int64_t)b * in.max_pages + j];
        if (e < 0) return fail(err, "page_table[%lld][%lld] is negative", b, j);
        const bool host = (e & 1) != 0;
        if (((int64_t)(e >> 1) + 1) * P > (host ? in.host_rows : in.dev_rows))
          return fail(err, "page_table[%lld][%lld]: page beyond its tier's pool", b, j);
        (host ? host_pages[b] : dev_pages[b]).push_back((int32_t)j);
      }
    }
  }

  // tokens of tier `host` below position E (pages of the tier are in logical order)
  auto tier_tokens = [&](int b, int64_t E, bool host) -> int64_t {
    if (!paged) return host ? std::min<int64_t>(nh[b], E) : std::max<int64_t>(0, E - nh[b]);
    int64_t t = 0;
    for (int32_t j : (host ? host_pages[b] : dev_pages[b])) {
      if ((int64_t)j * P >= E) break;
      t += std::min<int64_t>(P, E - (int64_t)j * P);
    }
    return t;
  };
  auto tier_pages_below = [&](int b, int64_t E, bool host) -> size_t {
    const std::vector<int32_t>& pg = host ? host_pages[b] : dev_pages[b];
    size_t k = 0;
    while (k < pg.size() && (int64_t)pg[k] * P < E) ++k;
    return k;
  };

  // ---- staging: host rows that two or more row blocks read are copied once
  // into an HBM pool, within the byte budget, in sequence order.
  const int64_t budget = in.stage_max_bytes;
  std::vector<int64_t> stage_base(B, -1);
  std::vector<StageTile> tiles;
  int64_t stage_rows = 0;
  for (int b = 0; b < B; ++b) {
    if (budget <= 0 || nblk[b] < 2) continue;
    const int64_t lim = std::min(emax[b], pre[b]);
    const int64_t rows = paged ? (int64_t)tier_pages_below(b, lim, true) * P : std::min<int64_t>(nh[b], lim);
    if (rows <= 0 || (stage_rows + rows) * row_bytes * 2 > budget) continue;
    stage_base[b] = stage_rows;
    if (!paged) {
      for (int64_t r = 0; r < rows; r += kStageTileRows) {
        StageTile t{};
        t.src_row = (int64_t)b * in.host_stride + r;
        t.dst_row = stage_rows + r;
        t.n_rows = (int32_t)std::min<int64_t>(kStageTileRows, rows - r);
        tiles.push_back(t);
      }
    } else {
      const int64_t np = rows / P;
      for (int64_t i = 0; i < np; ++i) {
        const int32_t e = in.page_table_host[(int64_t)b * in.max_pages + host_pages[b][i]];
        StageTile t{};
        t.src_row = (int64_t)(e >> 1) * P;
        t.dst_row = stage_rows + i * P;
        t.n_rows = (int32_t)P;
        tiles.push_back(t);
      }
    }
    stage_rows += rows;
  }

  // ---- row blocks and the tokens each reads per pool
  struct Blk { int b, row0, n_rows, pos0; int64_t end; };
  std::vector<Blk> blocks;
  int64_t host_reads = 0, dev_reads = 0;
  for (int b = 0; b < B; ++b) {
    const int n = q_start[b + 1] - q_start[b];
    for (int r0 = 0; r0 < n; r0 += QB) {
      Blk k{b, q_start[b] + r0, std::min(QB, n - r0), q_pos0[b] + r0, 0};
      k.end = (int64_t)k.pos0 + k.n_rows;  // tokens [0, end) are visible to some row
      const int64_t te = std::min(k.end, pre[b]);
      const int64_t th = tier_tokens(b, te, true);
      (stage_base[b] >= 0 ? dev_reads : host_reads) += th;
      dev_reads += tier_tokens(b, te, false) + std::max<int64_t>(0, k.end - pre[b]);
      blocks.push_back(k);
    }
  }

  // ---- workgroup split (same rules as decode) and chunk sizes
  int32_t wh = 0, wd = 0;
  split_workgroups(in, host_reads, dev_reads, &wh, &wd);
  const int32_t align = (int32_t)std::max<int64_t>(kPfTile, P);  // whole prefill tiles per item
  const int32_t ch = choose_chunk(host_reads * in.hkv, wh, 4, 256, 16384, align, in.host_chunk);
  // A prefill token-head costs a full 128-row MFMA pass, so HBM units are
  // long: fewer partials to write and merge (none when every block fits one
  // unit), longest-first order evens out the tail.  On the LLaMA-3-8B
  // 2048-row case 2048-token units beat 1024 (0.105 vs 0.112 ms).
  const int32_t cd = choose_chunk(dev_reads * in.hkv, wd, 2, 2048, 1 << 16, align, in.dev_chunk);

  // ---- items, split slots, row offsets and positions
  const int64_t T = q_start[B];
  std::vector<PrefillItem> hitems, ditems;
  std::vector<int32_t> pages, rowpos(T), offsets(T + 1, 0);
  int64_t slot = 0;
  for (const Blk& k : blocks) {
    std::vector<PrefillItem> items;
    const bool staged = stage_base[k.b] >= 0;
    const int64_t te = std::min(k.end, pre[k.b]);  // end of the tier tokens
    for (int64_t t = pre[k.b]; t < k.end; t += cd) {  // new rows: fresh pool
      PrefillItem it{};
      it.n_tok = (int32_t)std::min<int64_t>(cd, k.end - t);
      it.tok0 = (int32_t)t;
      it.pool = kPoolFresh;
      it.row_pool = (int64_t)q_start[k.b] + (t - pre[k.b]);
      items.push_back(it);
    }
    for (int tier = 1; tier >= 0; --tier) {
      const int32_t pool = tier ? (staged ? kPoolStaged : kPoolHost) : kPoolDev;
      const int64_t chunk = pool == kPoolHost ? ch : cd;
      if (!paged) {
        const int64_t t0 = tier ? 0 : nh[k.b];
        const int64_t t1 = tier ? std::min<int64_t>(nh[k.b], te) : te;
        for (int64_t t = t0; t < t1; t += chunk) {
          PrefillItem it{};
          it.n_tok = (int32_t)std::min<int64_t>(chunk, t1 - t);
          it.tok0 = (int32_t)t;
          it.pool = pool;
          it.row_pool = pool == kPoolHost ? (int64_t)k.b * in.host_stride + t
                      : pool == kPoolStaged ? stage_base[k.b] + t
                                            : (int64_t)k.b * in.dev_stride + (t - nh[k.b]);
          items.push_back(it);
        }
      } else {
        const std::vector<int32_t>& pg = tier ? host_pages[k.b] : dev_pages[k.b];
        const size_t npg = tier_pages_below(k.b, te, tier == 1);
        const size_t per = (size_t)(chunk / P);
        for (size_t p0 = 0; p0 < npg; p0 += per) {
          const size_t p1 = std::min(npg, p0 + per);
          PrefillItem it{};
          int64_t nt = 0;
          for (size_t q = p0; q < p1; ++q) nt += std::min<int64_t>(P, te - (int64_t)pg[q] * P);
          it.n_tok = (int32_t)nt;
          it.plist = (int32_t)(pages.size() / 2);
          it.pool = pool;
          for (size_t q = p0; q < p1; ++q) {
            const int32_t e = in.page_table_host[(int64_t)k.b * in.max_pages + pg[q]];
            pages.push_back(pg[q]);
            pages.push_back(pool == kPoolStaged ? (int32_t)(stage_base[k.b] / P + (int64_t)q) : (e >> 1));
          }
          items.push_back(it);
        }
      }
    }
    const int32_t S_k = (int32_t)items.size();
    for (int32_t s = 0; s < S_k; ++s) {
      PrefillItem& it = items[s];
      it.b = k.b;
      it.row0 = k.row0;
      it.n_rows = k.n_rows;
      it.pos0 = k.pos0;
      it.split_idx = s;
      it.n_splits = S_k;
      it.base = (int32_t)slot;
      (it.pool == kPoolHost ? hitems : ditems).push_back(it);
    }
    for (int r = 0; r < k.n_rows; ++r) {
      offsets[k.row0 + r] = (int32_t)(slot + (int64_t)r * S_k);
      rowpos[k.row0 + r] = k.pos0 + r;
    }
    slot += (int64_t)k.n_rows * S_k;
    if (slot > INT32_MAX) return fail(err, "too many prefill splits");
  }
  offsets[T] = (int32_t)slot;
  if ((int64_t)(hitems.size() + ditems.size()) * in.hkv > INT32_MAX) return fail(err, "too many work units");
  if ((int64_t)pages.size() > INT32_MAX) return fail(err, "page list too long");
  // longest items first: workgroups take units in list order, so the tail of
  // the persistent loop is made of short units
  auto longer = [](const PrefillItem& x, const PrefillItem& y) { return x.n_tok > y.n_tok; };
  std::stable_sort(hitems.begin(), hitems.end(), longer);
  std::stable_sort(ditems.begin(), ditems.end(), longer);

  out->n_host_items = (int32_t)hitems.size();
  out->n_dev_items = (int32_t)ditems.size();
  out->num_splits = (int32_t)slot;
  out->batch = B;
  out->n_rows = (int32_t)T;
  out->host_wgs = hitems.empty() ? 0 : (int32_t)std::min<int64_t>(wh, (int64_t)hitems.size() * in.hkv);
  out->dev_wgs = ditems.empty() ? 0 : (int32_t)std::min<int64_t>(std::max(wd, 1), (int64_t)ditems.size() * in.hkv);
  // HBM queues per XCD (8 of them, workgroups dealt round-robin): queue q
  // owns the KV heads h = q mod 8, so workgroups of one L2 re-read the same
  // heads.  Both workgroup counts become multiples of 8 so that blockIdx
  // mod 8 is the queue of every HBM-role workgroup.
  out->dev_queues = 1;
  if (in.hkv % kPfMaxQueues == 0 && out->dev_wgs >= kPfMaxQueues) {
    out->dev_queues = kPfMaxQueues;
    out->host_wgs = out->host_wgs / kPfMaxQueues * kPfMaxQueues + (out->host_wgs % kPfMaxQueues ? kPfMaxQueues : 0);
    out->dev_wgs = out->dev_wgs / kPfMaxQueues * kPfMaxQueues;
  }
  out->host_chunk = hitems.empty() ? 0 : ch;
  out->dev_chunk = ditems.empty() ? 0 : cd;
  out->stage_rows = stage_rows;
  out->staged_bytes = stage_rows * row_bytes * 2;
  out->n_stage_tiles = (int32_t)tiles.size();
  out->host_reads = host_reads * row_bytes * 2;
  out->dev_reads = dev_reads * row_bytes * 2;
  out->host_bytes = out->host_reads + out->staged_bytes;
  out->dev_bytes = out->dev_reads;
  out->n_plist = (int32_t)(pages.size() / 2);
  out->items_off = 0;
  out->plist_off = (hitems.size() + ditems.size()) * sizeof(PrefillItem);
  out->stage_tiles_off = round_up(out->plist_off + pages.size() * sizeof(int32_t), 32);
  out->rowpos_off = round_up(out->stage_tiles_off + tiles.size() * sizeof(StageTile), 16);
  out->rowseq_off = round_up(out->rowpos_off + T * sizeof(int32_t), 16);
  out->seqlens_off = round_up(out->rowseq_off + T * sizeof(int32_t), 16);
  out->offsets_off = round_up(out->seqlens_off + B * sizeof(int32_t), 16);
  out->counters_off = round_up(out->offsets_off + (T + 1) * sizeof(int32_t), 16);
  out->blob_bytes = round_up(out->counters_off + (kPfMaxQueues + 1) * sizeof(int32_t), 256);
  if (blob) {
    blob->assign(out->blob_bytes, 0);
    uint8_t* p = blob->data();
    if (!hitems.empty()) memcpy(p, hitems.data(), hitems.size() * sizeof(PrefillItem));
    if (!ditems.empty())
      memcpy(p + hitems.size() * sizeof(PrefillItem), ditems.data(), ditems.size() * sizeof(PrefillItem));
    if (!pages.empty()) memcpy(p + out->plist_off, pages.data(), pages.size() * sizeof(int32_t));
    if (!tiles.empty()) memcpy(p + out->stage_tiles_off, tiles.data(), tiles.size() * sizeof(StageTile));
    if (T) memcpy(p + out->rowpos_off, rowpos.data(), T * sizeof(int32_t));
    int32_t* rs = reinterpret_cast<int32_t*>(p + out->rowseq_off);
    for (int b = 0; b < B; ++b)
      for (int32_t r = q_start[b]; r < q_start[b + 1]; ++r) rs[r] = b;
    memcpy(p + out->seqlens_off, in.seq_lens, B * sizeof(int32_t));
    memcpy(p + out->offsets_off, offsets.data(), offsets.size() * sizeof(int32_t));
  }
  return true;
}

// ---------------------------------------------------------------- linear
//
// SplitKernel README, Overview / Key Features: an offloaded linear layer reads
// its weights directly from the remote tier.  W [N][K] is split by output
// rows: rows [0, floor(r N)) in host memory, the rest in HBM.  An item is a
// block of up to kLinRows rows of one tier and a range of the reduction
// dimension.  With at least a quarter as many row blocks as workgroups K
// stays whole (no partials); with fewer, K is cut so that a tier has about
// two items per workgroup, ranges of at least 1024, and the ranges of a block
// are summed by the last of them to finish, in the same launch.  Measured on
// MI355X for the 14336 x 4096 MLP up-projection from HBM (224 row blocks),
// 1 token, one call after a cache flush: 0.031 ms unsplit on 224 workgroups,
// 0.035 ms in 2 ranges, 0.036 in 4, 0.044 in 8.
bool linear_shape(const PlanInput& in, int32_t N, int32_t K, LinearShape* out, std::string* err) {
  *out = LinearShape{};
  if (N < 1 || K < 1) return fail(err, "out_features and in_features must be >= 1");
  if (K % 8) return fail(err, "in_features must be a multiple of 8 (got %lld)", K);
  const int64_t nh = (int64_t)std::floor(in.ratio * (double)N);
  const int64_t nd = N - nh;
  const int64_t bh = ceil_div(nh, kLinRows), bd = ceil_div(nd, kLinRows);
  int32_t wh = 0, wd = 0;
  split_workgroups(in, nh * K, nd * K, &wh, &wd);
  auto kchunk = [&](int64_t blocks, int32_t wgs, int32_t tuned) -> int64_t {
    if (tuned > 0) return std::min<int64_t>(round_up(tuned, 32), round_up(K, 32));
    if (blocks == 0 || 4 * blocks >= (int64_t)wgs) return round_up(K, 32);
    const int64_t c = std::min<int64_t>(ceil_div(2 * (int64_t)wgs, blocks), std::max<int64_t>(1, K / 1024));
    return round_up(ceil_div(K, c), 32);
  };
  const int64_t kh = kchunk(bh, wh, in.host_chunk), kd = kchunk(bd, wd, in.dev_chunk);
  const int64_t sh = ceil_div(K, kh), sd = ceil_div(K, kd);
  const int64_t ih = bh * sh, id = bd * sd;
  // a tier whose blocks are not split writes y directly
  const int64_t ph = sh > 1 ? ih : 0, pd = sd > 1 ? id : 0;
  const bool partial = ph + pd > 0;
  // partial byte offsets are 32-bit buffer offsets
  if (ph + pd > INT32_MAX / (kLinRows * kLinMaxTokens * 4)) return fail(err, "too many linear K ranges");
  if (ih + id > INT32_MAX / 2) return fail(err, "too many linear items");
  out->n_host = (int32_t)nh;
  out->bh = (int32_t)bh;
  out->bd = (int32_t)bd;
  out->kc_host = (int32_t)kh;
  out->kc_dev = (int32_t)kd;
  out->sp_host = (int32_t)sh;
  out->sp_dev = (int32_t)sd;
  out->n_host_items = (int32_t)ih;
  out->n_dev_items = (int32_t)id;
  out->host_wgs = ih == 0 ? 0 : (int32_t)std::min<int64_t>(wh, ih);
  out->dev_wgs = id == 0 ? 0 : (int32_t)std::min<int64_t>(std::max(wd, 1), id);
  out->num_splits = partial ? (int32_t)(ph + pd) : 0;
  out->host_bytes = nh * K * 2;
  out->dev_bytes = nd * K * 2;
  out->part_off = (size_t)round_up((4 + bh + bd) * (int64_t)sizeof(int32_t), 256);
  out->ws_bytes = out->part_off + (size_t)out->num_splits * kLinMaxTokens * kLinRows * 4;
  return true;
}

void linear_items(const LinearShape& z, int32_t N, int32_t K, std::vector<LinearItem>* items) {
  items->clear();
  int32_t slot = 0;
  for (int tier = 1; tier >= 0; --tier) {
    const int64_t r0 = tier ? 0 : z.n_host, r1 = tier ? z.n_host : N;
    const int64_t kc = tier ? z.kc_host : z.kc_dev;
    for (int64_t r = r0; r < r1; r += kLinRows)
      for (int64_t k = 0; k < K; k += kc) {
        LinearItem it{};
        it.row0 = (int32_t)r;
        it.n_rows = (int32_t)std::min<int64_t>(kLinRows, r1 - r);
        it.k0 = (int32_t)k;
        it.k1 = (int32_t)std::min<int64_t>(K, k + kc);
        it.slot = (tier ? z.sp_host : z.sp_dev) > 1 ? slot++ : -1;
        it.pool = tier ? kPoolHost : kPoolDev;
        items->push_back(it);
      }
  }
}

}  // namespace dkv
