// Paged KV allocator: two page pools (host-pinned, HBM) with a LIFO free
// list each and the page table the paged kernels read.  Host bookkeeping
// only; see include/dkv.h for the placement rule and the error behaviour.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <new>
#include <vector>

#include "dkv.h"
#include "dkv_internal.h"

struct dkv_pager {
  int32_t page_size;
  int32_t max_seqs;
  int32_t max_pages;
  double host_fraction;
  std::vector<int32_t> free_list[2];  // [0] HBM, [1] host; back() is the next page handed out
  int32_t pool_pages[2];
  std::vector<int32_t> table;          // [max_seqs][max_pages]
  std::vector<int32_t> n_pages;        // pages held per sequence
  int32_t spilled = 0;
};

namespace {

// Tier the placement rule gives logical page j: 1 (host) iff the count of
// host pages floor(f * n) grows when page j is added.
int policy_tier(double f, int64_t j) {
  return std::floor(f * (double)(j + 1)) > std::floor(f * (double)j) ? 1 : 0;
}

}  // namespace

extern "C" {

dkv_status dkv_pager_create(int32_t n_host_pages, int32_t n_dev_pages, int32_t page_size,
                            int32_t max_seqs, int32_t max_pages, double host_fraction, dkv_pager** out) {
  if (!out) return dkv::error(DKV_ERR_INVALID, "out is NULL");
  *out = nullptr;
  if (n_host_pages < 0 || n_dev_pages < 0)
    return dkv::error(DKV_ERR_INVALID, "page counts must be >= 0");
  if (page_size <= 0 || page_size > 1024 || (page_size & (page_size - 1)))
    return dkv::error(DKV_ERR_INVALID, "page_size must be a power of two <= 1024");
  if (max_seqs < 1 || max_pages < 1)
    return dkv::error(DKV_ERR_INVALID, "max_seqs and max_pages must be >= 1");
  if ((int64_t)max_seqs * max_pages > (int64_t)1 << 28)
    return dkv::error(DKV_ERR_INVALID, "max_seqs * max_pages is too large");
  if (!(host_fraction >= 0.0 && host_fraction <= 1.0))
    return dkv::error(DKV_ERR_INVALID, "host_fraction must be in [0, 1]");
  // an entry is phys << 1 | tier in an int32, and physical page p of a pool
  // holds rows p*page_size ..: both must stay below 2^31
  if (std::max(n_host_pages, n_dev_pages) >= (1 << 30) ||
      (int64_t)std::max(n_host_pages, n_dev_pages) * page_size > ((int64_t)1 << 31) - 1)
    return dkv::error(DKV_ERR_INVALID, "pool pages must be < 2^30 and pool rows < 2^31");
  dkv_pager* p = new (std::nothrow) dkv_pager();
  if (!p) return dkv::error(DKV_ERR_NOMEM, "pager allocation failed");
  try {
    p->page_size = page_size;
    p->max_seqs = max_seqs;
    p->max_pages = max_pages;
    p->host_fraction = host_fraction;
    p->pool_pages[0] = n_dev_pages;
    p->pool_pages[1] = n_host_pages;
    for (int t = 0; t < 2; ++t) {
      p->free_list[t].resize(p->pool_pages[t]);
      for (int32_t i = 0; i < p->pool_pages[t]; ++i) p->free_list[t][i] = p->pool_pages[t] - 1 - i;
    }
    p->table.assign((size_t)max_seqs * max_pages, -1);
    p->n_pages.assign(max_seqs, 0);
  } catch (const std::bad_alloc&) {
    delete p;
    return dkv::error(DKV_ERR_NOMEM, "pager tables do not fit in host memory");
  }
  *out = p;
  return dkv::success();
}

dkv_status dkv_pager_destroy(dkv_pager* pager) {
  delete pager;
  return dkv::success();
}

dkv_status dkv_pager_reserve(dkv_pager* p, int32_t seq, int64_t n_tokens) {
  if (!p) return dkv::error(DKV_ERR_INVALID, "pager is NULL");
  if (seq < 0 || seq >= p->max_seqs) return dkv::error(DKV_ERR_INVALID, "seq out of range");
  if (n_tokens < 0) return dkv::error(DKV_ERR_INVALID, "n_tokens must be >= 0");
  const int64_t want = (n_tokens + p->page_size - 1) / p->page_size;
  if (want > p->max_pages) return dkv::error(DKV_ERR_INVALID, "n_tokens exceeds max_pages * page_size");
  const int32_t have = p->n_pages[seq];
  if (want <= have) return dkv::success();
  // count first, so that a failure changes nothing
  int64_t need[2] = {0, 0};
  for (int64_t j = have; j < want; ++j) ++need[policy_tier(p->host_fraction, j)];
  const int64_t free_total = (int64_t)p->free_list[0].size() + (int64_t)p->free_list[1].size();
  if (need[0] + need[1] > free_total)
    return dkv::error(DKV_ERR_NOMEM, "not enough free pages in the two pools");
  int32_t* row = p->table.data() + (size_t)seq * p->max_pages;
  for (int64_t j = have; j < want; ++j) {
    int tier = policy_tier(p->host_fraction, j);
    if (p->free_list[tier].empty()) {
      tier ^= 1;
      ++p->spilled;
    }
    const int32_t phys = p->free_list[tier].back();
    p->free_list[tier].pop_back();
    row[j] = (phys << 1) | tier;
  }
  p->n_pages[seq] = (int32_t)want;
  return dkv::success();
}

dkv_status dkv_pager_release(dkv_pager* p, int32_t seq) {
  if (!p) return dkv::error(DKV_ERR_INVALID, "pager is NULL");
  if (seq < 0 || seq >= p->max_seqs) return dkv::error(DKV_ERR_INVALID, "seq out of range");
  int32_t* row = p->table.data() + (size_t)seq * p->max_pages;
  // pages go back in reverse order, so the next reserve reuses them in order
  for (int32_t j = p->n_pages[seq] - 1; j >= 0; --j) {
    p->free_list[row[j] & 1].push_back(row[j] >> 1);
    row[j] = -1;
  }
  p->n_pages[seq] = 0;
  return dkv::success();
}

dkv_status dkv_pager_table(const dkv_pager* p, const int32_t** table, const int32_t** pages_of_seq) {
  if (!p || !table) return dkv::error(DKV_ERR_INVALID, "pager or table is NULL");
  *table = p->table.data();
  if (pages_of_seq) *pages_of_seq = p->n_pages.data();
  return dkv::success();
}

dkv_status dkv_pager_stats_get(const dkv_pager* p, dkv_pager_stats* st) {
  if (!p || !st) return dkv::error(DKV_ERR_INVALID, "pager or stats is NULL");
  st->free_dev_pages = (int32_t)p->free_list[0].size();
  st->free_host_pages = (int32_t)p->free_list[1].size();
  st->used_dev_pages = p->pool_pages[0] - st->free_dev_pages;
  st->used_host_pages = p->pool_pages[1] - st->free_host_pages;
  st->spilled_pages = p->spilled;
  st->reserved = 0;
  return dkv::success();
}

}  // extern "C"
