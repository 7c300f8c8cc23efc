// dkv_kernels.hip - gfx950 kernels of the prefill, linear and helper paths
// (the decode attention kernels are in dkv_decode.hip).
//
//   merge_lse_kernel      combine per-split partials by log-sum-exp (one workgroup
//   merge_lse_wave_kernel   per pair for few long lists, one wave per pair for many)
//   append_kernel         Neox RoPE of new keys (fp64) + bf16 store into the cache slot
//   proj_kernel           new-token K/V projection on MFMA (split over the hidden dim)
//   proj_reduce_kernel    sum of the projection's hidden-dim partials
//   rope_table_kernel     (cos, sin) of every prefill row's angles, fp64
//   append_rows_kernel    fused prefill step: append of the new rows + their rotation table
//   prefill_split_kernel  causal prefill attention over both tiers, both products on MFMA
//   stage_copy_kernel     copy of host-tier rows that prefill re-reads into HBM
//   linear_split_kernel   y = x W^T with W split by rows between host memory and HBM
//   probe_read_kernel     streaming-read bandwidth probe (grid-stride, blocked, or
//                         row segments like the attention tiles)
//
// Method sources (page, section): DirectKV README, introduction (fused projection,
// Neox RoPE and attention reading KV from CPU-pinned buffers) and Attribution
// (online softmax; KV streamed from CPU memory with no GPU staging buffer);
// SplitKernel README, Overview and Key Features (direct access of the remote
// tier into on-chip memory; attention over a host/device partitioned KV cache).
//
// Design notes for CDNA4:
//   * 64-lane waves, 256-thread workgroups (4 waves).  Prefill tiles are 64
//     keys of one KV head: each thread moves D/32 16-byte chunks of K and of V
//     per tile with coalesced loads (host-tier loads are non-temporal) into LDS.
//   * Both prefill products run on v_mfma_f32_16x16x32_bf16; operands that are
//     not exact in bf16 (rotated queries, softmax weights) are split into a high
//     and a low bf16 part so the product keeps ~16 bits and fp32 accumulation.
//   * Host-role and HBM-role workgroups are disjoint (blockIdx below / above the
//     host workgroup count) so both tiers stream concurrently.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "dkv_internal.h"
#include "dkv_device.h"

namespace dkv {

// (cos, sin) of every prefill row's rotation angles, fp64, computed once per
// call; the prefill kernel rotates its query columns with them.
__global__ __launch_bounds__(kThreads) void rope_table_kernel(const int32_t* __restrict__ rowpos, int n_rows,
                                                              int half, RopeFreq freq, double2* __restrict__ cs,
                                                              const int32_t* __restrict__ plan_offsets,
                                                              int32_t* __restrict__ split_offsets) {
  if (blockIdx.x == 0 && split_offsets)
    for (int i = threadIdx.x; i <= n_rows; i += blockDim.x) split_offsets[i] = plan_offsets[i];
  const int64_t total = (int64_t)n_rows * half;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = idx / half;
    const int i = (int)(idx - row * half);
    double sn, c;
    sincos((double)rowpos[row] * freq.f[i], &sn, &c);
    cs[idx] = make_double2(c, sn);
  }
}

// ---------------------------------------------------------------------------
// Prefill: causal attention of blocks of new query rows over the cache.
//
// A unit = (row block of kPrefillRows/G query rows of one sequence, run of
// cached tokens in one pool, KV head).  Its 128 query-head rows are the
// (row, head) pairs of the group, 32 per wave as two 16-column MFMA tiles.
// Both contractions are dense and run on v_mfma_f32_16x16x32_bf16 in the
// transposed form, so the probabilities never leave registers:
//   S^T = K . Q^T   A = 16 keys x 32 dims (LDS), B = query columns (the fp32
//                   rotated query split into high and low bf16 parts)
//   O^T += V^T . P^T A = V transposed into LDS at staging time, B = the
//                   probabilities (high and low bf16 parts) taken straight
//                   from the S^T accumulators: accumulator lane group j holds
//                   keys 4j..4j+3 of each 16-key tile, so a 32-key k-step
//                   pairs two tiles and V^T is read in the same key order.
// Causal mask: token t is visible to a row at position p iff t <= p; tiles
// entirely below the block's first position skip the mask.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float x, float y) {
  const bf16x2_t v = {(__bf16)x, (__bf16)y};
  return __builtin_bit_cast(uint32_t, v);
}

// x = hi + lo with hi, lo bf16: pack (x0, x1) into hi and lo words.
__device__ __forceinline__ void split_bf16(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16(x0, x1);
  lo = pack_bf16(x0 - __uint_as_float(hi << 16), x1 - __uint_as_float(hi & 0xffff0000u));
}

// 16-column MFMA tiles per prefill wave (8 waves of 16 columns measured faster
// than 4 waves of 32 columns on MI355X).
constexpr int kPfNtw = 1;

// Cache slot of new token i of an append (contiguous split or paged); shared
// by the append kernel and the prefill kernel's writer role.
struct Slot {
  uint16_t* k;
  uint16_t* v;
  bool ok;
};

__device__ __forceinline__ Slot append_slot(const AppendArgs& a, int i) {
  Slot s{nullptr, nullptr, false};
  const int b = a.seq_idx[i];
  const int p = a.pos[i];
  if (b < 0 || b >= a.batch || p < 0) return s;
  int64_t row;
  bool host;
  if (a.page_size == 0) {
    const int L = a.seq_lens[b];
    if (p >= L) return s;
    const int64_t nh = (int64_t)floor(a.ratio * (double)L);
    host = p < nh;
    if (host) {
      if (nh > a.host_stride) return s;
      row = (int64_t)b * a.host_stride + p;
    } else {
      if (L - nh > a.dev_stride) return s;
      row = (int64_t)b * a.dev_stride + (p - nh);
    }
  } else {
    const int lp = p / a.page_size;
    if (lp >= a.max_pages) return s;
    const int32_t e = a.page_table[(int64_t)b * a.max_pages + lp];
    if (e < 0) return s;
    host = (e & 1) != 0;
    row = (int64_t)(e >> 1) * a.page_size + (p % a.page_size);
  }
  const int64_t cap = host ? a.host_rows : a.dev_rows;
  if (row < 0 || row >= cap) return s;
  const int64_t off = row * (int64_t)a.hkv * a.head_dim;
  s.k = (host ? a.host_k : a.dev_k) + off;
  s.v = (host ? a.host_v : a.dev_v) + off;
  s.ok = (host ? a.host_k : a.dev_k) != nullptr;
  return s;
}

// Reductions over the four 16-lane groups of a wave (lanes n, n+16, n+32,
// n+48), with the gfx950 lane-swap instructions: permlane16_swap pairs rows
// 0-1 and 2-3, permlane32_swap the two halves.
__device__ __forceinline__ float wave_max_rows4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float wave_sum_rows4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Key order inside a V^T row: within each 32-key step, lane group j of an
// MFMA operand takes keys 4j..4j+3 and 16+4j..16+4j+3 (the keys its S^T
// accumulators hold), so those eight keys are stored next to each other and
// the operand is one 16-byte LDS read.  Keys of one aligned quad stay
// contiguous.
__device__ __forceinline__ int vt_slot(int key) {
  const int q = (key & 31) >> 2;
  return (key & ~31) + ((q & 3) << 3) + ((q >> 2) << 2) + (key & 3);
}

// A plan item at a workgroup-uniform address, read through the constant
// address space: scalar loads, counted apart from the vector loads in flight,
// so fetching the next unit's item does not wait for the tile loads.
__device__ __forceinline__ PrefillItem load_item_uniform(const PrefillItem* p) {
  static_assert(sizeof(PrefillItem) == 64, "item size");
  typedef __attribute__((address_space(4))) const u32x4 ConstVec;
  const ConstVec* w = (const ConstVec*)p;
  struct Raw {
    u32x4 v[4];
  } t;
#pragma unroll
  for (int i = 0; i < 4; ++i) t.v[i] = w[i];
  return __builtin_bit_cast(PrefillItem, t);
}

// Headroom of the lazily updated softmax reference maximum (log2 units).
constexpr float kRescaleSlack = 8.f;

template <int NTW>
constexpr int pf_threads() { return kPrefillRows / (16 * NTW) * 64; }

// NTW: 16-column MFMA tiles (query-head rows / 16) per wave; the workgroup
// holds kPrefillRows / (16 NTW) waves.  With 64-key tiles, one column tile
// per wave (8 waves, two per SIMD) measured faster than two per wave (4
// waves, one per SIMD) on the LLaMA-3-8B 2048-row prefill: 0.105 vs 0.131 ms,
// also when the two-per-wave form interleaves one group's softmax with the
// other group's MFMAs; 64-row workgroups (two per CU) gave 0.111 ms.  With
// 128-key tiles one column tile per wave takes 254 VGPRs.
template <int D, int G, bool PAGED, int NTW>
__global__ __launch_bounds__(pf_threads<NTW>()) void prefill_split_kernel(PrefillArgs a) {
  constexpr int NT = pf_threads<NTW>();
  constexpr int PT = kPfTile;                  // keys per tile
  constexpr int HT = PT / 64;                  // 64-key halves per tile
  constexpr int MT = PT / 16;                  // 16-key blocks per tile
  constexpr int KT = PT / 32;                  // 32-key k-steps of P.V per tile
  constexpr int KS = D / 32;                   // k-steps of Q.K over the head dim
  constexpr int DT = D / 16;                   // 16-row d tiles of O^T
  // Row pitches padded by 32 bytes: the MFMA operand reads (16 rows x 16 B at
  // four column offsets per instruction) then hit distinct banks of the
  // 64-bank LDS, which serves them at ~245 B/clk per CU on MI355X against
  // ~126 B/clk with a 16-byte pad (measured).
  constexpr int KPITCH = D * 2 + 32;           // bytes per K row in LDS
  constexpr int VPB = PT * 2 + 32;             // bytes per V^T row (one d, PT keys)
  constexpr int CPR = D / 8;                   // 16-byte chunks per KV row
  constexpr int NCK = PT * CPR / NT;           // K chunks per thread
  constexpr int TPT = NCK;                     // V keys per thread (one 8-dim chunk)
  constexpr int KQ = PT / TPT;                 // V key groups per tile
  static_assert(TPT == 1 || TPT == 2 || TPT == 4, "tile shape");
  static_assert(KQ * CPR == NT, "V staging covers the tile");

  __shared__ __attribute__((aligned(16))) uint8_t k_lds[PT * KPITCH];
  __shared__ __attribute__((aligned(16))) uint8_t vt_lds[D * VPB];
  __shared__ int tpos_lds[PT];
  __shared__ int s_next;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15;
  const int j4 = lane >> 4;
  // V staging: consecutive lanes take consecutive key groups of one 8-dim
  // chunk, so the transposed LDS writes of a wave hit distinct banks
  const int vq = tid % KQ;
  const int vc = tid / KQ;

  // Work queues: the host role has one; the HBM role has one per queue id
  // (blockIdx mod dev_queues), each owning the KV heads congruent to it, so
  // the workgroups that share an L2 share KV heads.
  // Writer role (fused step only): the first writer_wgs workgroups copy the
  // new rows from their HBM copy into their cache slots (PCIe writes when the
  // slots are host-resident) while the other workgroups attend.
  if ((int)blockIdx.x < a.writer_wgs) {
    // (row, 16-byte chunk) pairs of the K and V rows, NT per pass, two passes
    // in flight per thread
    const int64_t chunks = (int64_t)a.hkv * D / 8;
    const int64_t total = (int64_t)a.app.n_new * chunks;
    const int64_t stride = (int64_t)a.writer_wgs * NT;
    for (int64_t f0 = (int64_t)blockIdx.x * NT + tid; f0 < total; f0 += 2 * stride) {
      u32x4 kv[2][2];
      Slot sl[2];
      int64_t c[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t f = f0 + j * stride;
        sl[j] = Slot{nullptr, nullptr, false};
        if (f < total) {
          const int i = (int)(f / chunks);
          c[j] = f - (int64_t)i * chunks;
          sl[j] = append_slot(a.app, i);
          const size_t src = (size_t)i * chunks * 8 + c[j] * 8;
          kv[j][0] = *reinterpret_cast<const u32x4*>(a.fresh_k + src);
          kv[j][1] = *reinterpret_cast<const u32x4*>(a.fresh_v + src);
        }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
        if (sl[j].ok) {
          *reinterpret_cast<u32x4*>(sl[j].k + c[j] * 8) = kv[j][0];
          *reinterpret_cast<u32x4*>(sl[j].v + c[j] * 8) = kv[j][1];
        }
    }
    return;
  }
  const int bid = (int)blockIdx.x - a.writer_wgs;
  const bool host_role = bid < a.host_wgs;
  const int wg = host_role ? bid : bid - a.host_wgs;
  const int nq = host_role ? 1 : a.dev_queues;
  const int q = wg % nq;
  const int nwg = (host_role ? a.host_wgs : a.dev_wgs) / nq;
  const int hpq = a.hkv / nq;  // KV heads per queue
  const int nunits = (host_role ? a.n_host_items : a.n_dev_items) * hpq;
  const PrefillItem* items = host_role ? a.host_items : a.dev_items;
  int* counter = a.unit_counters + (host_role ? kPfHostCounter : q);

  struct Src {
    const uint16_t* k;
    const uint16_t* v;
  };
  auto src_of = [&](const PrefillItem& it) -> Src {
    if (it.pool == kPoolHost) return Src{a.host_k, a.host_v};
    if (it.pool == kPoolDev) return Src{a.dev_k, a.dev_v};
    if (it.pool == kPoolFresh) return Src{a.fresh_k, a.fresh_v};
    return Src{a.stage_k, a.stage_v};
  };
  // pool row of token `tok` of an item (tokens past the end read token 0);
  // fresh rows are contiguous in either layout
  auto row_of = [&](const PrefillItem& it, int tok) -> int64_t {
    tok = tok < it.n_tok ? tok : 0;
    if (PAGED && it.pool != kPoolFresh) {
      const int pg = tok >> a.page_shift;
      return ((int64_t)a.pages[2 * (it.plist + pg) + 1] << a.page_shift) | (tok & ((1 << a.page_shift) - 1));
    }
    return it.row_pool + tok;
  };
  auto pos_of = [&](const PrefillItem& it, int tok) -> int {
    if (tok >= it.n_tok) return -1;
    if (PAGED && it.pool != kPoolFresh) {
      const int pg = tok >> a.page_shift;
      return (a.pages[2 * (it.plist + pg)] << a.page_shift) + (tok & ((1 << a.page_shift) - 1));
    }
    return it.tok0 + tok;
  };

  // A thread's share of the next tile is loaded into registers while the
  // current tile is reduced out of LDS; the registers carry the unit and tile
  // index their data belongs to.
  struct TileRegs {
    u32x4 k[NCK];
    u32x4 v[TPT];
    int tpos;
    int u;     // unit, nunits when the stream has ended
    int tile;  // tile index inside the unit
  };
  // Element offsets of this thread's K and V loads for the prefetch cursor's
  // current tile.  Rows past the item's end are clamped to its first token:
  // real data whose keys the mask removes (p = 0 exactly).
  int64_t koff[NCK], voff[TPT];
  auto set_offsets = [&](const PrefillItem& it, int kvh, int tile) {
    const int t0 = tile * PT;
#pragma unroll
    for (int c = 0; c < NCK; ++c) {
      const int chunk = tid + c * NT;
      koff[c] = (row_of(it, t0 + chunk / CPR) * a.hkv + kvh) * D + (chunk % CPR) * 8;
    }
#pragma unroll
    for (int e = 0; e < TPT; ++e) voff[e] = (row_of(it, t0 + vq * TPT + e) * a.hkv + kvh) * D + vc * 8;
  };
  // Loads of the prefetch cursor's next tile into r.  Every call issues the
  // same loads, so no path through a step lacks them: once the stream has
  // ended the addresses fall back to the first bytes of the query rows (the
  // tags mark such a tile as empty).
  auto load_tile = [&](TileRegs& r, bool live, const PrefillItem& it, const Src& sp, int kvh, int tile) {
    const int t0 = tile * PT;
    if (live) {
      // contiguous items step the offsets by whole tiles except where the
      // tile runs past the item (clamping) ; paged items look up every tile
      if ((PAGED && it.pool != kPoolFresh) || tile == 0 || t0 + PT > it.n_tok) {
        set_offsets(it, kvh, tile);
      } else {
        const int64_t step = (int64_t)PT * a.hkv * D;
#pragma unroll
        for (int c = 0; c < NCK; ++c) koff[c] += step;
#pragma unroll
        for (int e = 0; e < TPT; ++e) voff[e] += step;
      }
    }
    const uint16_t* dummy = a.q;
#pragma unroll
    for (int c = 0; c < NCK; ++c)
      r.k[c] = *reinterpret_cast<const u32x4*>(live ? sp.k + koff[c] : dummy + c * 8);
#pragma unroll
    for (int e = 0; e < TPT; ++e)
      r.v[e] = *reinterpret_cast<const u32x4*>(live ? sp.v + voff[e] : dummy + (NCK + e) * 8);
    r.tpos = (live && tid < PT) ? pos_of(it, t0 + tid) : -1;
  };

  // ---- prefetch cursor: the unit and tile whose loads are issued next.
  // A workgroup's first unit is wg / nq; later ones come from the queue's
  // counter (claimed by thread 0, read by all after a barrier).
  int pu = wg / nq;
  PrefillItem pit{};
  Src psrc{};
  int pkvh = 0, ptile = 0, pntiles = 0;
  auto open_unit = [&]() {
    if (pu < nunits) {
      pit = load_item_uniform(items + pu / hpq);
      pkvh = q + nq * (pu % hpq);
      psrc = src_of(pit);
      ptile = 0;
      pntiles = (pit.n_tok + PT - 1) / PT;
    }
  };
  auto needs_claim = [&]() { return pu < nunits && ptile == pntiles; };  // workgroup-uniform
  auto claim = [&](bool c) {  // between two barriers
    if (c && tid == 0) s_next = nwg + atomicAdd(counter, 1);
  };
  auto after_claim = [&](bool c) {  // after the barrier that follows claim()
    if (c) {
      pu = __builtin_amdgcn_readfirstlane(s_next);
      open_unit();
    }
  };
  auto issue = [&](TileRegs& r) {
    const bool live = pu < nunits;
    load_tile(r, live, pit, psrc, pkvh, ptile);
    r.u = live ? pu : nunits;
    r.tile = live ? ptile++ : 0;
  };

  TileRegs ra;
  open_unit();
  issue(ra);

  // ---- compute cursor: the unit whose tiles are being reduced
  PrefillItem it{};
  int kvh = 0, ntiles = 0;
  // query operand (B of S^T): column n of tile nt = query-head row
  // rho = 16*(NTW*wave + nt) + n = (row rho/G, head rho%G)
  uint32_t qb_hi[NTW][KS][4], qb_lo[NTW][KS][4];
  int rpos[NTW];
  bool rvalid[NTW];
  // m_run: reference maximum of the scores (log2 units); it only moves when
  // the running maximum exceeds it by more than kRescaleSlack, so most tiles
  // skip rescaling O (probabilities then stay <= 2^kRescaleSlack).
  float m_run[NTW], l_run[NTW];
  floatx4 ot[NTW][DT];

  auto begin_unit = [&](int u) {
    it = load_item_uniform(items + u / hpq);
    kvh = q + nq * (u % hpq);
    ntiles = (it.n_tok + PT - 1) / PT;
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      const int rho = (wave * NTW + nt) * 16 + n;
      const int r = rho / G, h = rho % G;
      rvalid[nt] = r < it.n_rows;
      rpos[nt] = it.pos0 + r;
      // rotate the column's query (Neox pairs d, d + D/2) with the row's fp64
      // (cos, sin), round once to fp32, fold in scale * log2(e)
      const size_t row = (size_t)it.row0 + (rvalid[nt] ? r : 0);
      const uint16_t* qr = a.q + (row * a.hq + kvh * G + h) * D;
      const double2* cs = reinterpret_cast<const double2*>(a.rope_cs) + row * (D / 2);
#pragma unroll
      for (int ks = 0; ks < KS / 2; ++ks) {
        const int d0 = ks * 32 + j4 * 8;  // dims d0 .. d0+7 and their partners d0+D/2 ..
        const u32x4 lo16 = *reinterpret_cast<const u32x4*>(qr + d0);
        const u32x4 hi16 = *reinterpret_cast<const u32x4*>(qr + d0 + D / 2);
        float yl[8], yh[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double2 t = cs[d0 + e];
          const double xl = (double)bf16_to_f32((uint16_t)((lo16[e >> 1] >> ((e & 1) * 16)) & 0xffffu));
          const double xh = (double)bf16_to_f32((uint16_t)((hi16[e >> 1] >> ((e & 1) * 16)) & 0xffffu));
          yl[e] = rvalid[nt] ? (float)(xl * t.x - xh * t.y) * a.scale_log2 : 0.f;
          yh[e] = rvalid[nt] ? (float)(xh * t.x + xl * t.y) * a.scale_log2 : 0.f;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          split_bf16(yl[2 * e], yl[2 * e + 1], qb_hi[nt][ks][e], qb_lo[nt][ks][e]);
          split_bf16(yh[2 * e], yh[2 * e + 1], qb_hi[nt][ks + KS / 2][e], qb_lo[nt][ks + KS / 2][e]);
        }
      }
      m_run[nt] = -INFINITY;
      l_run[nt] = 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) ot[nt][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
  };

  // ---- this unit's partial for every valid row
  auto end_unit = [&]() {
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      const float l = wave_sum_rows4(l_run[nt]);
      if (!rvalid[nt]) continue;
      const int rho = (wave * NTW + nt) * 16 + n;
      const int r = rho / G, h = rho % G;
      const size_t slot = (size_t)it.base + (size_t)r * it.n_splits + it.split_idx;
      const size_t head = slot * a.hq + kvh * G + h;
      const bool empty = m_run[nt] == -INFINITY;
      const float inv = empty ? 0.f : 1.f / l;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<floatx4*>(a.part_o + head * D + dt * 16 + j4 * 4) = ot[nt][dt] * inv;
      if (j4 == 0)
        a.part_lse[head] = empty ? -INFINITY : (m_run[nt] + log2f(l)) * 0.69314718055994530942f;
    }
  };

  // One tile: stage r in LDS, refill r with the next tile, reduce.  A tile
  // past the end of the stream is staged and refilled (with the same loads as
  // any other) but not reduced.
  auto step = [&](TileRegs& r) {
    const int tile = r.tile;
    const bool work = r.u < nunits;
    if (work && tile == 0) begin_unit(r.u);
    __syncthreads();  // previous tile's readers are done
#pragma unroll
    for (int c = 0; c < NCK; ++c) {
      const int chunk = tid + c * NT;
      *reinterpret_cast<u32x4*>(k_lds + (chunk / CPR) * KPITCH + (chunk % CPR) * 16) = r.k[c];
    }
    // V^T: row d = 8*vc + e holds keys vq*TPT .. vq*TPT + TPT-1
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int w = e >> 1, sh = (e & 1) * 16;
      uint8_t* dst = vt_lds + (vc * 8 + e) * VPB + vt_slot(vq * TPT) * 2;
      if constexpr (TPT == 1) {
        *reinterpret_cast<uint16_t*>(dst) = (uint16_t)((r.v[0][w] >> sh) & 0xffffu);
      } else {
        const uint32_t k01 = ((r.v[0][w] >> sh) & 0xffffu) | (((r.v[TPT > 1 ? 1 : 0][w] >> sh) & 0xffffu) << 16);
        if constexpr (TPT == 4) {
          const uint32_t k23 = ((r.v[2][w] >> sh) & 0xffffu) | (((r.v[3][w] >> sh) & 0xffffu) << 16);
          *reinterpret_cast<u32x2*>(dst) = u32x2{k01, k23};
        } else {
          *reinterpret_cast<uint32_t*>(dst) = k01;
        }
      }
    }
    if (tid < PT) tpos_lds[tid] = r.tpos;
    const bool c = needs_claim();
    claim(c);
    __syncthreads();
    after_claim(c);
    issue(r);

    if (!work) return;

    // ---- per-tile compute, in pieces per 16-column group nt:
    //   S^T = K . Q^T (64 keys x 16 columns), causal mask, softmax with the
    //   lazily moved reference maximum, P^T into B operands, O^T += V^T . P^T.
    // High-part MFMAs of all tiles are issued before the low-part ones so no
    // MFMA waits on the one before it.
    floatx4 st[MT][NTW];
    uint32_t pb_hi[NTW][KT][4], pb_lo[NTW][KT][4];
    const bool need_mask = (tile + 1) * PT > it.n_tok || tpos_lds[PT - 1] > it.pos0;
    // K operands of the 64 keys of half h
    auto load_k = [&](bf16x8_t (&kf)[KS][4], int h) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          kf[ks][mt] = __builtin_bit_cast(
              bf16x8_t,
              *reinterpret_cast<const u32x4*>(k_lds + (h * 64 + mt * 16 + n) * KPITCH + ks * 64 + j4 * 16));
    };
    auto s_mfma = [&](int nt, const bf16x8_t (&kf)[KS][4], int h) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) st[4 * h + mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 qh = {qb_hi[nt][ks][0], qb_hi[nt][ks][1], qb_hi[nt][ks][2], qb_hi[nt][ks][3]};
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          st[4 * h + mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              kf[ks][mt], __builtin_bit_cast(bf16x8_t, qh), st[4 * h + mt][nt], 0, 0, 0);
        const u32x4 ql = {qb_lo[nt][ks][0], qb_lo[nt][ks][1], qb_lo[nt][ks][2], qb_lo[nt][ks][3]};
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          st[4 * h + mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              kf[ks][mt], __builtin_bit_cast(bf16x8_t, ql), st[4 * h + mt][nt], 0, 0, 0);
      }
    };
    // causal mask and the reference-maximum update of column group nt
    auto mask_rescale = [&](int nt) {
      if (need_mask) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tp = tpos_lds[mt * 16 + j4 * 4 + i];
            st[mt][nt][i] = (tp >= 0 && tp <= rpos[nt]) ? st[mt][nt][i] : -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, st[mt][nt][i]);
      mx = wave_max_rows4(mx);  // over the four lane groups of column n
      const float m_new = (mx > m_run[nt] + kRescaleSlack) ? mx : m_run[nt];
      if (__builtin_amdgcn_ballot_w64(m_new != m_run[nt]) != 0) {  // wave-uniform
        // 1 if this column kept its reference (also while it is still -inf),
        // 0 on its first finite maximum
        const float alpha = m_new == m_run[nt] ? 1.f : exp2f(m_run[nt] - m_new);
        l_run[nt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) ot[nt][dt] *= alpha;
        m_run[nt] = m_new;
      }
    };
    // probabilities of column group nt, split into high/low bf16 B operands
    auto probs = [&](int nt) {
      const float m_use = m_run[nt] == -INFINITY ? 0.f : m_run[nt];
      float ps = 0.f;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        float pv[2][4];
#pragma unroll
        for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pv[m2][i] = __builtin_amdgcn_exp2f(st[2 * kt + m2][nt][i] - m_use);  // -inf -> 0
            ps += pv[m2][i];
          }
        split_bf16(pv[0][0], pv[0][1], pb_hi[nt][kt][0], pb_lo[nt][kt][0]);
        split_bf16(pv[0][2], pv[0][3], pb_hi[nt][kt][1], pb_lo[nt][kt][1]);
        split_bf16(pv[1][0], pv[1][1], pb_hi[nt][kt][2], pb_lo[nt][kt][2]);
        split_bf16(pv[1][2], pv[1][3], pb_hi[nt][kt][3], pb_lo[nt][kt][3]);
      }
      l_run[nt] += ps;
    };
    // V^T operands of the two 32-key k-steps of half h
    auto load_v = [&](bf16x8_t (&va)[2][DT], int h) {
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          va[k2][dt] = __builtin_bit_cast(
              bf16x8_t,
              *reinterpret_cast<const u32x4*>(vt_lds + (dt * 16 + n) * VPB + ((2 * h + k2) * 32 + j4 * 8) * 2));
        }
    };
    auto pv_mfma = [&](int nt, const bf16x8_t (&va)[2][DT], int h) {
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const int kt = 2 * h + k2;
        const u32x4 ph = {pb_hi[nt][kt][0], pb_hi[nt][kt][1], pb_hi[nt][kt][2], pb_hi[nt][kt][3]};
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          ot[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[k2][dt], __builtin_bit_cast(bf16x8_t, ph),
                                                               ot[nt][dt], 0, 0, 0);
        const u32x4 pl = {pb_lo[nt][kt][0], pb_lo[nt][kt][1], pb_lo[nt][kt][2], pb_lo[nt][kt][3]};
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          ot[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[k2][dt], __builtin_bit_cast(bf16x8_t, pl),
                                                               ot[nt][dt], 0, 0, 0);
      }
    };
#pragma unroll
    for (int h = 0; h < HT; ++h) {
      bf16x8_t kf[KS][4];
      load_k(kf, h);
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) s_mfma(nt, kf, h);
    }
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) mask_rescale(nt);
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) probs(nt);
#pragma unroll
    for (int h = 0; h < HT; ++h) {
      bf16x8_t va[2][DT];
      load_v(va, h);
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) pv_mfma(nt, va, h);
    }

    if (tile + 1 == ntiles) end_unit();
  };
  // the stream ends when the registers carry no unit
  while (ra.u < nunits) step(ra);
}

// ---------------------------------------------------------------------------
// Offloaded linear y = x W^T with W [N][K] split by output rows between host
// memory (read in place) and HBM.  Workgroup = 4 waves; an item is up to 64
// rows (16 per wave) x a K range, walked in 256-wide chunks.  A chunk of W
// (64 rows x 512 B, each 32 lanes reading one row's 512 contiguous bytes)
// and the chunk of x are loaded into registers one chunk ahead, stay in
// flight while the current chunk's MFMAs run, and are then staged in LDS.
// Per 32-wide k-step each wave issues v_mfma_f32_16x16x32_bf16 with A = 16
// tokens of x and B = its 16 rows of W, both read from LDS; MT row tiles
// cover up to 16*MT tokens per W read.  Measured on MI355X for the
// 14336 x 4096 MLP up-projection from HBM, 1 token: 0.024 ms with the loads
// in flight across the MFMAs, 0.035 ms when each chunk's loads were waited
// for right after issue; 512-wide chunks were no faster (0.026 ms).  The
// host tier runs at the link rate either way.
//
// No host plan: item i of a tier is derived from the call's shape (row block
// i / sp, K range i % sp).  When K is split, each range writes its partial
// with agent-coherent stores, and the last range of a row block to finish
// (per-block counter) sums the block's partials in slot order into y.  The
// last workgroup to exit sets the queue and block counters back to zero, so
// the workspace needs no upload or clear between calls.
// ---------------------------------------------------------------------------
constexpr int kLinKC = 256;  // K per chunk (8 k-steps)

struct LinItem {
  int row0, n_rows, k0, k1;
  int slot;   // partial slot, < 0: y written directly
  int blk;    // row block over both tiers (index of its counter)
  int sp;     // K ranges of the block
  int first;  // the block's first partial slot
};

__device__ __forceinline__ LinItem linear_item(const LinearArgs& a, bool host, int i) {
  const int sp = host ? a.sp_host : a.sp_dev, kc = host ? a.kc_host : a.kc_dev;
  const int blk = i / sp, s = i - blk * sp;
  const int r0 = host ? 0 : a.n_host, r1 = host ? a.n_host : a.n;
  LinItem it;
  it.row0 = r0 + blk * kLinRows;
  it.n_rows = min(kLinRows, r1 - it.row0);
  it.k0 = s * kc;
  it.k1 = min(a.k, it.k0 + kc);
  it.slot = sp > 1 ? (host ? i : a.p_host + i) : -1;
  it.blk = host ? blk : a.bh + blk;
  it.sp = sp;
  it.first = it.slot - s;
  return it;
}

template <int MT, bool HOST>
__device__ __forceinline__ void linear_stream(const LinearArgs& a, uint8_t* x_lds, uint8_t* w_lds, int* s_next_p,
                                              int* s_last_p) {
  constexpr int XP = kLinKC * 2 + 16;                   // bytes per staged row (x token or W row)
  constexpr int CPR = kLinKC * 2 / 16;                  // 16-byte columns per staged row
  constexpr int PASSES = kLinRows * CPR / kThreads;     // 16-byte W loads per thread per chunk
  constexpr int XPASSES = MT * 16 * CPR / kThreads;     // 16-byte x loads per thread per chunk
  constexpr int RPP = kThreads / CPR;                   // rows per pass
  static_assert(kThreads % CPR == 0 && (kLinRows * CPR) % kThreads == 0 && (MT * 16 * CPR) % kThreads == 0);
  int& s_next = *s_next_p;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n = lane & 15, j4 = lane >> 4;
  const int wr = tid / CPR;  // staging: row within a pass
  const int wc = tid % CPR;  //          16-byte column
  constexpr bool host_role = HOST;
  const int wg = host_role ? (int)blockIdx.x : (int)blockIdx.x - a.host_wgs;
  const int nwg = host_role ? a.host_wgs : a.dev_wgs;
  const int nunits = host_role ? a.n_host_items : a.n_dev_items;
  int* counter = a.counters + (host_role ? 1 : 0);
  const uint16_t* __restrict__ wpool = host_role ? a.host_w : a.dev_w;
  const int row_shift = host_role ? 0 : a.n_host;
  const __amdgpu_buffer_rsrc_t part_rsrc = coherent_rsrc(a.part);

  u32x4 wreg[PASSES], xreg[XPASSES];
  // Columns past k1 read the item's first column for W and are zeroed when
  // staged (a select right after the load would wait for it); x tokens past
  // m and columns past k1 are not loaded and stay zero.
  bool wz = false;
  auto load_chunk = [&](const LinItem& it, int kc) {
    const int k = kc + wc * 8;
    const bool kok = k < it.k1;
    wz = !kok;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int r = p * RPP + wr;
      const int64_t row = (int64_t)(it.row0 - row_shift + (r < it.n_rows ? r : 0));
      const u32x4* src = reinterpret_cast<const u32x4*>(wpool + row * a.k + (kok ? k : it.k0));
      wreg[p] = *src;
    }
#pragma unroll
    for (int p = 0; p < XPASSES; ++p) {
      const int tok = p * RPP + wr;
      xreg[p] = u32x4{0u, 0u, 0u, 0u};
      if (tok < a.m && kok) xreg[p] = *reinterpret_cast<const u32x4*>(a.x + (size_t)tok * a.k + k);
    }
  };

  int u = wg;
  LinItem it{};
  if (u < nunits) {
    it = linear_item(a, host_role, u);
    load_chunk(it, it.k0);
  }
  while (u < nunits) {
    floatx4 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
    int next_u = nunits;
    LinItem nit{};
    for (int kc = it.k0; kc < it.k1; kc += kLinKC) {
      __syncthreads();  // previous chunk's readers are done
#pragma unroll
      for (int p = 0; p < PASSES; ++p)
        *reinterpret_cast<u32x4*>(w_lds + (p * RPP + wr) * XP + wc * 16) = wz ? u32x4{0u, 0u, 0u, 0u} : wreg[p];
#pragma unroll
      for (int p = 0; p < XPASSES; ++p)
        *reinterpret_cast<u32x4*>(x_lds + (p * RPP + wr) * XP + wc * 16) = xreg[p];
      const bool last = kc + kLinKC >= it.k1;
      if (last && tid == 0) s_next = nwg + atomicAdd(counter, 1);
      __syncthreads();
      // one call site for the next chunk's loads, so that they land in the
      // same registers on both paths and stay in flight through the MFMAs
      LinItem lit = it;
      int lkc = kc + kLinKC;
      bool more = true;
      if (last) {
        next_u = s_next;
        more = next_u < nunits;
        if (more) {
          nit = linear_item(a, host_role, next_u);
          lit = nit;
          lkc = nit.k0;
        }
      }
      if (more) load_chunk(lit, lkc);
#pragma unroll
      for (int s = 0; s < kLinKC / 32; ++s) {
        const bf16x8_t wb = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const u32x4*>(w_lds + (wave * 16 + n) * XP + (s * 32 + j4 * 8) * 2));
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const bf16x8_t xa = __builtin_bit_cast(
              bf16x8_t, *reinterpret_cast<const u32x4*>(x_lds + (t * 16 + n) * XP + (s * 32 + j4 * 8) * 2));
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, wb, acc[t], 0, 0, 0);
        }
      }
    }
    // lane (n + 16 j4) holds y[token 16 t + 4 j4 + i][row n of this wave]
    const int r = wave * 16 + n;
    if (r < it.n_rows) {
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = t * 16 + j4 * 4 + i;
          if (tok >= a.m) continue;
          if (it.slot < 0)
            a.y[(size_t)tok * a.n + it.row0 + r] = acc[t][i];
          else
            coherent_store1(part_rsrc, ((it.slot * kLinMaxTokens + tok) * kLinRows + r) * 4, acc[t][i]);
        }
    }
    if (it.slot >= 0) {
      // the last K range of this row block to finish sums the block's
      // partials, in slot order, into y
      wait_stores();
      __syncthreads();
      if (tid == 0) {
        int* done = a.counters + 4 + it.blk;
        const int prev = atomicAdd(done, 1);
        const bool fin = prev == it.sp - 1;
        if (fin) __hip_atomic_store(done, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_last_p = fin;
      }
      __syncthreads();
      if (*s_last_p) {
        for (int e = tid; e < a.m * kLinRows; e += kThreads) {
          const int rr = e % kLinRows, tok = e / kLinRows;
          if (rr >= it.n_rows) continue;
          float sum = 0.f;
          for (int j = 0; j < it.sp; ++j)
            sum += coherent_load1(part_rsrc, (((it.first + j) * kLinMaxTokens + tok) * kLinRows + rr) * 4);
          a.y[(size_t)tok * a.n + it.row0 + rr] = sum;
        }
      }
    }
    u = next_u;
    it = nit;
  }
}

template <int MT>
__global__ __launch_bounds__(kThreads) void linear_split_kernel(LinearArgs a) {
  constexpr int XP = kLinKC * 2 + 16;
  __shared__ __attribute__((aligned(16))) uint8_t x_lds[MT * 16 * XP];
  __shared__ __attribute__((aligned(16))) uint8_t w_lds[kLinRows * XP];
  __shared__ int s_next, s_last;
  if ((int)blockIdx.x < a.host_wgs)
    linear_stream<MT, true>(a, x_lds, w_lds, &s_next, &s_last);
  else
    linear_stream<MT, false>(a, x_lds, w_lds, &s_next, &s_last);
  // the last workgroup out sets the queues back to zero (every workgroup
  // has taken its last item before it gets here)
  if (threadIdx.x == 0 && atomicAdd(a.counters + 2, 1) == (int)gridDim.x - 1) {
    __hip_atomic_store(a.counters + 0, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.counters + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.counters + 2, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Staging copy of host-tier rows into the HBM pool: tile after tile, 16-byte
// non-temporal loads from the mapped host memory, eight in flight per lane.
__global__ __launch_bounds__(kThreads) void stage_copy_kernel(StageArgs a) {
  constexpr int U = 8;
  for (int t = blockIdx.x; t < a.n_tiles; t += gridDim.x) {
    const StageTile tl = a.tiles[t];
    const int64_t per = (int64_t)tl.n_rows * a.row_chunks;  // chunks per tensor
    const u32x4* src[2] = {reinterpret_cast<const u32x4*>(a.src_k) + tl.src_row * a.row_chunks,
                           reinterpret_cast<const u32x4*>(a.src_v) + tl.src_row * a.row_chunks};
    u32x4* dst[2] = {reinterpret_cast<u32x4*>(a.dst_k) + tl.dst_row * a.row_chunks,
                     reinterpret_cast<u32x4*>(a.dst_v) + tl.dst_row * a.row_chunks};
    for (int64_t c0 = threadIdx.x; c0 < 2 * per; c0 += (int64_t)kThreads * U) {
      u32x4 v[U];
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const int64_t c = c0 + (int64_t)k * kThreads;
        const int w = c >= per;
        v[k] = c < 2 * per ? __builtin_nontemporal_load(src[w] + (c - w * per)) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const int64_t c = c0 + (int64_t)k * kThreads;
        const int w = c >= per;
        if (c < 2 * per) dst[w][c - w * per] = v[k];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// LSE merge: the maximum and the weight sum of the split LSEs are block
// reductions, then every split's partial is folded with weight exp(lse - M).
// ---------------------------------------------------------------------------
template <int NT>
__device__ __forceinline__ float block_reduce_n(float v, bool is_max, float* sm) {
  for (int o = 32; o >= 1; o >>= 1) {
    const float w = __shfl_xor(v, o);
    v = is_max ? fmaxf(v, w) : v + w;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sm[wave] = v;
  __syncthreads();
  v = sm[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) v = is_max ? fmaxf(v, sm[w]) : v + sm[w];
  return v;
}

// Workgroup = (b, h, slice of DS), 1024 threads: D/(4 DS) lanes each own 4
// of the slice's dims (one 16-byte load per split), the rest of the threads
// form groups that fold every group-th split with several loads in flight,
// then the groups combine through LDS.  With few (b, h) pairs (one sequence)
// the dims are sliced over DS workgroups so that more CUs read the partials;
// each slice recomputes the maximum and the sum from the lse list.
constexpr int kMergeThreads = 1024;

template <int D, int DS>
__global__ __launch_bounds__(kMergeThreads) void merge_lse_kernel(MergeArgs a) {
  constexpr int DW = D / DS;  // dims of this workgroup
  constexpr int LANES = DW / 4;
  constexpr int NG = kMergeThreads / LANES;
  constexpr int U = 4;
  __shared__ float sm_red[kMergeThreads / 64];
  __shared__ __attribute__((aligned(16))) float sm_o[NG][DW];
  const int bh = blockIdx.x / DS, slice = blockIdx.x - bh * DS;
  const int b = bh / a.hq, h = bh - b * a.hq;
  const int tid = threadIdx.x;
  const int s0 = a.split_offsets[b], s1 = a.split_offsets[b + 1];
  const float* lse = a.part_lse + h;
  float m = -INFINITY;
  for (int s = s0 + tid; s < s1; s += kMergeThreads) m = fmaxf(m, lse[(size_t)s * a.hq]);
  const float M = block_reduce_n<kMergeThreads>(m, true, sm_red);
  float* out = a.out_o + ((size_t)b * a.hq + h) * D + slice * DW;
  if (M == -INFINITY) {  // no finite split
    if (tid < DW) out[tid] = 0.f;
    if (slice == 0 && tid == 0 && a.out_lse) a.out_lse[(size_t)b * a.hq + h] = -INFINITY;
    return;
  }
  float l = 0.f;
  for (int s = s0 + tid; s < s1; s += kMergeThreads) {
    const float x = lse[(size_t)s * a.hq];
    l += (x == -INFINITY) ? 0.f : expf(x - M);
  }
  const float Lsum = block_reduce_n<kMergeThreads>(l, false, sm_red);
  const int g = tid / LANES, d4 = (tid - g * LANES) * 4;
  const float* po = a.part_o + (size_t)h * D + slice * DW + d4;
  const size_t srow = (size_t)a.hq * D;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // U splits in flight per thread in every round, the last one included:
  // indices past the list reload its last split and are skipped
  for (int s = s0 + g; s < s1; s += U * NG) {
    float x[U];
    float4 o[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int sk = min(s + k * NG, s1 - 1);
      x[k] = lse[(size_t)sk * a.hq];
      o[k] = *reinterpret_cast<const float4*>(po + (size_t)sk * srow);
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
      if (s + k * NG >= s1) continue;
      const float w = (x[k] == -INFINITY) ? 0.f : expf(x[k] - M);
      acc.x += w * o[k].x; acc.y += w * o[k].y; acc.z += w * o[k].z; acc.w += w * o[k].w;
    }
  }
  *reinterpret_cast<float4*>(&sm_o[g][d4]) = acc;
  __syncthreads();
  // combine the NG groups in two passes: every thread first sums PER groups
  // of one dim, then DW threads sum the kMergeThreads / DW results
  constexpr int R = kMergeThreads / DW, PER = NG / R;
  static_assert(NG % R == 0, "merge combine");
  {
    const int col = tid % DW, gs = tid / DW;
    float o = 0.f;
#pragma unroll
    for (int k = 0; k < PER; ++k) o += sm_o[gs * PER + k][col];
    __syncthreads();
    sm_o[gs][col] = o;
    __syncthreads();
  }
  if (tid < DW) {
    float o = 0.f;
#pragma unroll 8
    for (int k = 0; k < R; ++k) o += sm_o[k][tid];
    out[tid] = o / Lsum;
    if (slice == 0 && tid == 0 && a.out_lse) a.out_lse[(size_t)b * a.hq + h] = M + logf(Lsum);
  }
}

// Many (b, h) pairs with few splits each (prefill rows): one wave per pair,
// each lane owns D/64 dims, splits folded in order with several loads in
// flight.  A single split is returned exactly (weight exp(0) = 1, sum 1).
constexpr int kMergeWaveThreads = 256;
constexpr int64_t kMergeWaveMinPairs = 2048;

template <int D>
__global__ __launch_bounds__(kMergeWaveThreads) void merge_lse_wave_kernel(MergeArgs a) {
  constexpr int E = D / 64;
  constexpr int U = 4;
  const int lane = threadIdx.x & 63;
  const int64_t bh = (int64_t)blockIdx.x * (kMergeWaveThreads / 64) + (threadIdx.x >> 6);
  if (bh >= (int64_t)a.batch * a.hq) return;
  const int b = (int)(bh / a.hq), h = (int)(bh - (int64_t)b * a.hq);
  const int s0 = a.split_offsets[b], s1 = a.split_offsets[b + 1];
  const float* lse = a.part_lse + h;
  float m = -INFINITY;
  for (int s = s0 + lane; s < s1; s += 64) m = fmaxf(m, lse[(size_t)s * a.hq]);
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  float* out = a.out_o + (size_t)bh * D + lane * E;
  if (m == -INFINITY) {
#pragma unroll
    for (int e = 0; e < E; ++e) out[e] = 0.f;
    if (lane == 0 && a.out_lse) a.out_lse[bh] = -INFINITY;
    return;
  }
  float l = 0.f;
  for (int s = s0 + lane; s < s1; s += 64) {
    const float x = lse[(size_t)s * a.hq];
    l += (x == -INFINITY) ? 0.f : expf(x - m);
  }
  for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o);
  const float* po = a.part_o + (size_t)h * D + lane * E;
  const size_t srow = (size_t)a.hq * D;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  // (pairs here have one split or a few: the leftovers are loaded one at a
  // time, since a full round of U would mostly reload the last split)
  int s = s0;
  for (; s + U <= s1; s += U) {
    float x[U], v[U][E];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      x[k] = lse[(size_t)(s + k) * a.hq];
#pragma unroll
      for (int e = 0; e < E; ++e) v[k][e] = po[(size_t)(s + k) * srow + e];
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const float w = (x[k] == -INFINITY) ? 0.f : expf(x[k] - m);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += w * v[k][e];
    }
  }
  for (; s < s1; ++s) {
    const float x = lse[(size_t)s * a.hq];
    const float w = (x == -INFINITY) ? 0.f : expf(x - m);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += w * po[(size_t)s * srow + e];
  }
#pragma unroll
  for (int e = 0; e < E; ++e) out[e] = acc[e] / l;
  if (lane == 0 && a.out_lse) a.out_lse[bh] = m + logf(l);
}

// ---------------------------------------------------------------------------
// Append: slot of (b, p) from the placement, K rotated in fp64 and rounded
// once to bf16, V stored as is.  Thread = (token, group of 8 rotation pairs);
// it loops over the KV heads so each angle's sin/cos is computed once.
// ---------------------------------------------------------------------------

// Fused prefill step: the rotation table of the new rows and their keys and
// values.  One thread per (row, group of QP pairs, hpt KV heads): it computes
// the pairs' (cos, sin) once, stores them in the table (first head chunk;
// the prefill kernel rotates the queries with them) and rotates that slice of
// the row's key for its heads.  Rows go to the HBM copy (fresh_k/fresh_v) and, unless skip_slots,
// to their cache slots; projection mode reads kv_proj as append_kernel does.
__global__ __launch_bounds__(kThreads) void append_rows_kernel(AppendArgs a, double2* __restrict__ table,
                                                               const int32_t* __restrict__ plan_offsets,
                                                               int32_t* __restrict__ split_offsets, int hpt) {
  constexpr int QP = 4;  // rotation pairs per thread
  if (blockIdx.x == 0 && split_offsets)
    for (int i = threadIdx.x; i <= a.n_new; i += blockDim.x) split_offsets[i] = plan_offsets[i];
  const int D = a.head_dim, half = D / 2, groups = half / QP;
  const int kvd = a.hkv * D;
  const int hchunks = (a.hkv + hpt - 1) / hpt;  // threads per (row, pair group)
  const int64_t total = (int64_t)a.n_new * groups * hchunks;
  for (int64_t gidx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gidx < total;
       gidx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t ig = gidx / hchunks;
    const int hc = (int)(gidx - ig * hchunks);
    const int i = (int)(ig / groups);
    const int p0 = (int)(ig - (int64_t)i * groups) * QP;
    const double pos = (double)a.pos[i];
    double cs[QP], sn[QP];
#pragma unroll
    for (int e = 0; e < QP; ++e) {
      sincos(pos * a.freq.f[p0 + e], &sn[e], &cs[e]);
      if (hc == 0) table[(size_t)i * half + p0 + e] = make_double2(cs[e], sn[e]);
    }
    const Slot sl = a.skip_slots ? Slot{nullptr, nullptr, false} : append_slot(a, i);
    const int h1 = min(a.hkv, (hc + 1) * hpt);
    for (int h = hc * hpt; h < h1; ++h) {
      double xl[QP], xh[QP];
      uint2 v0, v1;
      if (a.kv_proj) {
        const float* kp = a.kv_proj + (size_t)i * 2 * kvd + h * D;
        const float* vp = kp + kvd;
#pragma unroll
        for (int e = 0; e < QP; ++e) {
          xl[e] = (double)kp[p0 + e];
          xh[e] = (double)kp[half + p0 + e];
        }
        v0 = make_uint2(f32_to_bf16(vp[p0]) | (f32_to_bf16(vp[p0 + 1]) << 16),
                        f32_to_bf16(vp[p0 + 2]) | (f32_to_bf16(vp[p0 + 3]) << 16));
        v1 = make_uint2(f32_to_bf16(vp[half + p0]) | (f32_to_bf16(vp[half + p0 + 1]) << 16),
                        f32_to_bf16(vp[half + p0 + 2]) | (f32_to_bf16(vp[half + p0 + 3]) << 16));
      } else {
        const uint16_t* kp = a.k_new + (size_t)i * kvd + h * D;
        const uint16_t* vs = a.v_new + (size_t)i * kvd + h * D;
        const uint2 lo = *reinterpret_cast<const uint2*>(kp + p0);
        const uint2 hi = *reinterpret_cast<const uint2*>(kp + half + p0);
        v0 = *reinterpret_cast<const uint2*>(vs + p0);
        v1 = *reinterpret_cast<const uint2*>(vs + half + p0);
        xl[0] = (double)bf16_to_f32(lo.x & 0xffffu);
        xl[1] = (double)bf16_to_f32(lo.x >> 16);
        xl[2] = (double)bf16_to_f32(lo.y & 0xffffu);
        xl[3] = (double)bf16_to_f32(lo.y >> 16);
        xh[0] = (double)bf16_to_f32(hi.x & 0xffffu);
        xh[1] = (double)bf16_to_f32(hi.x >> 16);
        xh[2] = (double)bf16_to_f32(hi.y & 0xffffu);
        xh[3] = (double)bf16_to_f32(hi.y >> 16);
      }
      uint32_t yl[QP / 2], yh[QP / 2];
#pragma unroll
      for (int e = 0; e < QP / 2; ++e) {
        const int e0 = 2 * e, e1 = 2 * e + 1;
        yl[e] = f64_to_bf16(xl[e0] * cs[e0] - xh[e0] * sn[e0]) |
                (f64_to_bf16(xl[e1] * cs[e1] - xh[e1] * sn[e1]) << 16);
        yh[e] = f64_to_bf16(xh[e0] * cs[e0] + xl[e0] * sn[e0]) |
                (f64_to_bf16(xh[e1] * cs[e1] + xl[e1] * sn[e1]) << 16);
      }
      uint16_t* fk = a.fresh_k + (size_t)i * kvd + h * D;
      uint16_t* fv = a.fresh_v + (size_t)i * kvd + h * D;
      *reinterpret_cast<uint2*>(fk + p0) = make_uint2(yl[0], yl[1]);
      *reinterpret_cast<uint2*>(fk + half + p0) = make_uint2(yh[0], yh[1]);
      *reinterpret_cast<uint2*>(fv + p0) = v0;
      *reinterpret_cast<uint2*>(fv + half + p0) = v1;
      if (sl.ok) {
        *reinterpret_cast<uint2*>(sl.k + h * D + p0) = make_uint2(yl[0], yl[1]);
        *reinterpret_cast<uint2*>(sl.k + h * D + half + p0) = make_uint2(yh[0], yh[1]);
        *reinterpret_cast<uint2*>(sl.v + h * D + p0) = v0;
        *reinterpret_cast<uint2*>(sl.v + h * D + half + p0) = v1;
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void append_kernel(AppendArgs a) {
  constexpr int QP = 4;  // rotation pairs per thread
  const int D = a.head_dim, half = D / 2, groups = half / QP;
  const int kvd = a.hkv * D;
  const int per_tok = a.hkv * groups;
  const int64_t total = (int64_t)a.n_new * per_tok;
  for (int64_t gidx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gidx < total;
       gidx += (int64_t)gridDim.x * blockDim.x) {
    const int i = (int)(gidx / per_tok);
    const int r = (int)(gidx - (int64_t)i * per_tok);
    const int h = r / groups;
    const int p0 = (r - h * groups) * QP;
    const Slot sl = append_slot(a, i);
    if (!sl.ok) continue;
    const double pos = (double)a.pos[i];
    double xl[QP], xh[QP];
    if (a.kv_proj) {
      const float* kp = a.kv_proj + (size_t)i * 2 * kvd + h * D;
#pragma unroll
      for (int e = 0; e < QP; ++e) {
        xl[e] = (double)kp[p0 + e];
        xh[e] = (double)kp[half + p0 + e];
      }
    } else {
      const uint16_t* kp = a.k_new + (size_t)i * kvd + h * D;
      const uint2 lo = *reinterpret_cast<const uint2*>(kp + p0);
      const uint2 hi = *reinterpret_cast<const uint2*>(kp + half + p0);
      xl[0] = (double)bf16_to_f32(lo.x & 0xffffu);
      xl[1] = (double)bf16_to_f32(lo.x >> 16);
      xl[2] = (double)bf16_to_f32(lo.y & 0xffffu);
      xl[3] = (double)bf16_to_f32(lo.y >> 16);
      xh[0] = (double)bf16_to_f32(hi.x & 0xffffu);
      xh[1] = (double)bf16_to_f32(hi.x >> 16);
      xh[2] = (double)bf16_to_f32(hi.y & 0xffffu);
      xh[3] = (double)bf16_to_f32(hi.y >> 16);
    }
    double cs[QP], sn[QP];
#pragma unroll
    for (int e = 0; e < QP; ++e) sincos(pos * a.freq.f[p0 + e], &sn[e], &cs[e]);
    uint32_t yl[QP / 2], yh[QP / 2];
#pragma unroll
    for (int e = 0; e < QP / 2; ++e) {
      const int e0 = 2 * e, e1 = 2 * e + 1;
      yl[e] = f64_to_bf16(xl[e0] * cs[e0] - xh[e0] * sn[e0]) |
              (f64_to_bf16(xl[e1] * cs[e1] - xh[e1] * sn[e1]) << 16);
      yh[e] = f64_to_bf16(xh[e0] * cs[e0] + xl[e0] * sn[e0]) |
              (f64_to_bf16(xh[e1] * cs[e1] + xl[e1] * sn[e1]) << 16);
    }
    uint16_t* dst = sl.k + h * D;
    if (!a.skip_slots) {
      *reinterpret_cast<uint2*>(dst + p0) = make_uint2(yl[0], yl[1]);
      *reinterpret_cast<uint2*>(dst + half + p0) = make_uint2(yh[0], yh[1]);
    }
    if (a.fresh_k) {
      uint16_t* fk = a.fresh_k + (size_t)i * kvd + h * D;
      *reinterpret_cast<uint2*>(fk + p0) = make_uint2(yl[0], yl[1]);
      *reinterpret_cast<uint2*>(fk + half + p0) = make_uint2(yh[0], yh[1]);
    }
    // V: the same thread moves the matching 2 x 4 values of this head
    uint16_t* vd = sl.v + h * D;
    if (a.kv_proj) {
      const float* vp = a.kv_proj + (size_t)i * 2 * kvd + kvd + h * D;
      uint32_t w0[2], w1[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        w0[e] = f32_to_bf16(vp[p0 + 2 * e]) | (f32_to_bf16(vp[p0 + 2 * e + 1]) << 16);
        w1[e] = f32_to_bf16(vp[half + p0 + 2 * e]) | (f32_to_bf16(vp[half + p0 + 2 * e + 1]) << 16);
      }
      if (!a.skip_slots) {
        *reinterpret_cast<uint2*>(vd + p0) = make_uint2(w0[0], w0[1]);
        *reinterpret_cast<uint2*>(vd + half + p0) = make_uint2(w1[0], w1[1]);
      }
      if (a.fresh_v) {
        uint16_t* fv = a.fresh_v + (size_t)i * kvd + h * D;
        *reinterpret_cast<uint2*>(fv + p0) = make_uint2(w0[0], w0[1]);
        *reinterpret_cast<uint2*>(fv + half + p0) = make_uint2(w1[0], w1[1]);
      }
    } else {
      const uint16_t* vs = a.v_new + (size_t)i * kvd + h * D;
      const uint2 v0 = *reinterpret_cast<const uint2*>(vs + p0);
      const uint2 v1 = *reinterpret_cast<const uint2*>(vs + half + p0);
      if (!a.skip_slots) {
        *reinterpret_cast<uint2*>(vd + p0) = v0;
        *reinterpret_cast<uint2*>(vd + half + p0) = v1;
      }
      if (a.fresh_v) {
        uint16_t* fv = a.fresh_v + (size_t)i * kvd + h * D;
        *reinterpret_cast<uint2*>(fv + p0) = v0;
        *reinterpret_cast<uint2*>(fv + half + p0) = v1;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Projection [n_new x hidden] . [hidden x 2*kv_dim] on MFMA 16x16x32 bf16.
// Workgroup = 64 output columns x one slice of the hidden dim; the W slice is
// transposed into LDS ([col][k]) on its way in so each lane reads its B operand
// (8 consecutive k of one column) with one 16-byte LDS read.  Partials per
// slice go to `partial`; the append kernel's reader sums them in slice order.
// ---------------------------------------------------------------------------
constexpr int kProjCols = 64;
constexpr int kProjK = 256;  // hidden-dim slice per workgroup

__global__ __launch_bounds__(kThreads) void proj_kernel(ProjArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t wt[kProjCols][kProjK + 8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, j4 = lane >> 4;
  const int ncols = 2 * a.kv_dim;
  const int col0 = blockIdx.x * kProjCols;
  const int ks = blockIdx.y;            // hidden slice
  const int k0 = ks * kProjK;
  // ---- stage W[k0 .. k0+kProjK)[col0 .. col0+64) transposed; every load of
  // the thread is issued before the first is used (one round trip, not one
  // per load)
  constexpr int WPT = kProjK * (kProjCols / 8) / kThreads;  // 16-byte loads per thread
  static_assert(WPT * kThreads == kProjK * (kProjCols / 8), "staging split");
  u32x4 w[WPT];
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int c = tid + i * kThreads;
    const int kr = c / (kProjCols / 8);
    const int gcol = col0 + (c - kr * (kProjCols / 8)) * 8;
    const uint16_t* src = (gcol < a.kv_dim) ? a.wk + (size_t)(k0 + kr) * a.kv_dim + gcol
                                            : a.wv + (size_t)(k0 + kr) * a.kv_dim + (gcol - a.kv_dim);
    w[i] = *reinterpret_cast<const u32x4*>(src);
  }
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int c = tid + i * kThreads;
    const int kr = c / (kProjCols / 8);
    const int cc = (c - kr * (kProjCols / 8)) * 8;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      wt[cc + 2 * e][kr] = (uint16_t)(w[i][e] & 0xffffu);
      wt[cc + 2 * e + 1][kr] = (uint16_t)(w[i][e] >> 16);
    }
  }
  __syncthreads();
  // ---- wave w computes columns col0 + 16w .. +16 for every 16-token tile
  const int ctile = wave * 16;
  for (int m0 = 0; m0 < a.n_new; m0 += 16) {
    floatx4 c = {0.f, 0.f, 0.f, 0.f};
    const int row = m0 + n;
    const bool rv = row < a.n_new;
    // x rows past n_new read row 0 and are zeroed when used
    const uint16_t* xr = a.x + (size_t)(rv ? row : 0) * a.hidden + k0 + j4 * 8;
    u32x4 xv[kProjK / 32];
#pragma unroll
    for (int s = 0; s < kProjK / 32; ++s) xv[s] = *reinterpret_cast<const u32x4*>(xr + s * 32);
#pragma unroll
    for (int s = 0; s < kProjK / 32; ++s) {
      const u32x4 av = rv ? xv[s] : u32x4{0u, 0u, 0u, 0u};
      const u32x4 bv = *reinterpret_cast<const u32x4*>(&wt[ctile + n][s * 32 + j4 * 8]);
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                  __builtin_bit_cast(bf16x8_t, bv), c, 0, 0, 0);
    }
    // D layout: lane holds rows j4*4 + i, column n
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = m0 + j4 * 4 + i;
      if (r < a.n_new)
        a.partial[((size_t)ks * a.n_pad + r) * ncols + col0 + ctile + n] = c[i];
    }
  }
}

// Sum of the hidden-slice partials (fixed order) into [n_new][2*kv_dim].
__global__ __launch_bounds__(kThreads) void proj_reduce_kernel(ProjArgs a) {
  const int ncols = 2 * a.kv_dim;
  const int64_t total = (int64_t)a.n_new * ncols;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int r = (int)(idx / ncols), c = (int)(idx - (int64_t)r * ncols);
    float s = 0.f;
    // unrolled so that several slices' loads are in flight; sums stay in
    // slice order
#pragma unroll 8
    for (int k = 0; k < a.ksplit; ++k) s += a.partial[((size_t)k * a.n_pad + r) * ncols + c];
    a.out[idx] = s;
  }
}

// ---------------------------------------------------------------------------
// Streaming read probe: 16 B per lane per load, coalesced, U loads in flight
// per thread.  Grid-stride: consecutive workgroups read neighbouring 4 KiB
// blocks.  Blocked: each workgroup streams its own contiguous slice, as the
// attention kernel streams a work item.  Segments: the buffer is rows of
// kProbeRow bytes cut into kProbeSeg-byte segments, and a workgroup streams one
// segment of every row of its slice (the attention kernel's reads of one KV
// head: 256 bytes of each 2 KiB token row of the LLaMA-3-8B layer).
// ---------------------------------------------------------------------------
constexpr int kProbeRow = 2048;
constexpr int kProbeSeg = 256;

template <bool NT, int MODE>
__global__ __launch_bounds__(kThreads) void probe_read_kernel(const u32x4* __restrict__ src,
                                                             const u32x4* __restrict__ src2, int64_t n16,
                                                             float* sink) {
  constexpr int U = 8;  // 16-byte loads in flight per thread
  // with a second buffer, odd workgroups read it and even ones the first
  const int nb = src2 ? 2 : 1;
  int wg = (int)blockIdx.x / nb, nwg = (int)gridDim.x / nb;
  const u32x4* __restrict__ p = (src2 && (blockIdx.x & 1)) ? src2 : src;
  uint32_t acc = 0;
  if (MODE == 2) {
    constexpr int SPR = kProbeRow / kProbeSeg;   // segments per row
    constexpr int CPS = kProbeSeg / 16;          // 16-byte chunks per segment
    constexpr int RPI = kThreads / CPS;          // rows per load instruction
    const int seg = wg % SPR;
    wg /= SPR;
    nwg = max(1, nwg / SPR);
    const int64_t rows = n16 * 16 / kProbeRow;
    const int64_t per = (rows + nwg - 1) / nwg;
    const int64_t r0 = (int64_t)wg * per, r1 = min(rows, r0 + per);
    const int rr = threadIdx.x / CPS, cc = threadIdx.x % CPS;
    auto at = [&](int64_t row) { return p + row * (kProbeRow / 16) + seg * CPS + cc; };
    int64_t r = r0 + rr;
    for (; r + (U - 1) * RPI < r1; r += U * RPI) {
      u32x4 v[U];
#pragma unroll
      for (int k = 0; k < U; ++k) v[k] = NT ? __builtin_nontemporal_load(at(r + k * RPI)) : *at(r + k * RPI);
#pragma unroll
      for (int k = 0; k < U; ++k) acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
    }
    for (; r < r1; r += RPI) {
      const u32x4 v = NT ? __builtin_nontemporal_load(at(r)) : *at(r);
      acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
  } else {
    int64_t i, end, stride;
    if (MODE == 1) {
      const int64_t per = (n16 + nwg - 1) / nwg;
      i = (int64_t)wg * per + threadIdx.x;
      end = min(n16, (int64_t)(wg + 1) * per);
      stride = blockDim.x;
    } else {
      i = (int64_t)wg * blockDim.x + threadIdx.x;
      end = n16;
      stride = (int64_t)nwg * blockDim.x;
    }
    for (; i + (U - 1) * stride < end; i += U * stride) {
      u32x4 v[U];
#pragma unroll
      for (int k = 0; k < U; ++k) v[k] = NT ? __builtin_nontemporal_load(p + i + k * stride) : p[i + k * stride];
#pragma unroll
      for (int k = 0; k < U; ++k) acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
    }
    for (; i < end; i += stride) {
      const u32x4 v = NT ? __builtin_nontemporal_load(p + i) : p[i];
      acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
  }
  if (acc == 0x9e3779b9u) sink[0] = (float)acc;  // keeps the loads alive
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <int D, int G>
static hipError_t launch_prefill_dg(const PrefillArgs& a, hipStream_t s) {
  const int grid = a.writer_wgs + a.host_wgs + a.dev_wgs;
  if (grid <= 0) return hipSuccess;
  if (a.pages)
    hipLaunchKernelGGL((prefill_split_kernel<D, G, true, kPfNtw>), dim3(grid), dim3(pf_threads<kPfNtw>()), 0, s, a);
  else
    hipLaunchKernelGGL((prefill_split_kernel<D, G, false, kPfNtw>), dim3(grid), dim3(pf_threads<kPfNtw>()), 0, s, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_prefill_d(const PrefillArgs& a, hipStream_t s) {
  switch (a.hq / a.hkv) {
    case 1: return launch_prefill_dg<D, 1>(a, s);
    case 2: return launch_prefill_dg<D, 2>(a, s);
    case 4: return launch_prefill_dg<D, 4>(a, s);
    case 8: return launch_prefill_dg<D, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

int launch_prefill(const PrefillArgs& a, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (a.host_wgs + a.dev_wgs <= 0) return (int)hipSuccess;
  if (a.head_dim == 64) return (int)launch_prefill_d<64>(a, s);
  if (a.head_dim == 128) return (int)launch_prefill_d<128>(a, s);
  return (int)hipErrorInvalidValue;
}

int launch_rope_table(const int32_t* rowpos, int n_rows, int d, const RopeFreq& freq, double* cs,
                      const int32_t* plan_offsets, int32_t* split_offsets, void* stream) {
  const int64_t total = (int64_t)n_rows * (d / 2);
  const int bx = (int)std::max<int64_t>(1, std::min<int64_t>((total + kThreads - 1) / kThreads, 16384));
  hipLaunchKernelGGL(rope_table_kernel, dim3(bx), dim3(kThreads), 0, (hipStream_t)stream, rowpos, n_rows, d / 2,
                     freq, reinterpret_cast<double2*>(cs), plan_offsets, split_offsets);
  return (int)hipGetLastError();
}

int launch_stage(const StageArgs& a, int nwg, void* stream) {
  if (a.n_tiles <= 0) return (int)hipSuccess;
  nwg = std::max(1, std::min(nwg, a.n_tiles));
  hipLaunchKernelGGL(stage_copy_kernel, dim3(nwg), dim3(kThreads), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

int launch_linear(const LinearArgs& a, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const int grid = a.host_wgs + a.dev_wgs;
  if (grid <= 0 || a.m < 1 || a.m > kLinMaxTokens) return (int)hipErrorInvalidValue;
  if (a.m <= 16)
    hipLaunchKernelGGL(linear_split_kernel<1>, dim3(grid), dim3(kThreads), 0, s, a);
  else if (a.m <= 32)
    hipLaunchKernelGGL(linear_split_kernel<2>, dim3(grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(linear_split_kernel<4>, dim3(grid), dim3(kThreads), 0, s, a);
  return (int)hipGetLastError();
}

int launch_merge(const MergeArgs& a, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const int64_t grid = (int64_t)a.batch * a.hq;
  if (grid > 0x7fffffff) return (int)hipErrorInvalidValue;
  if (grid >= kMergeWaveMinPairs) {  // enough pairs to fill the chip one wave each
    const int64_t per = kMergeWaveThreads / 64;
    const unsigned wg = (unsigned)((grid + per - 1) / per);
    if (a.head_dim == 64)
      hipLaunchKernelGGL(merge_lse_wave_kernel<64>, dim3(wg), dim3(kMergeWaveThreads), 0, s, a);
    else if (a.head_dim == 128)
      hipLaunchKernelGGL(merge_lse_wave_kernel<128>, dim3(wg), dim3(kMergeWaveThreads), 0, s, a);
    else
      return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
  }
  // fewer pairs than CUs: slice the dims (32 per workgroup)
  const bool sliced = grid < 256;
  if (a.head_dim == 64) {
    if (sliced)
      hipLaunchKernelGGL((merge_lse_kernel<64, 2>), dim3((unsigned)(grid * 2)), dim3(kMergeThreads), 0, s, a);
    else
      hipLaunchKernelGGL((merge_lse_kernel<64, 1>), dim3((unsigned)grid), dim3(kMergeThreads), 0, s, a);
  } else if (a.head_dim == 128) {
    if (sliced)
      hipLaunchKernelGGL((merge_lse_kernel<128, 4>), dim3((unsigned)(grid * 4)), dim3(kMergeThreads), 0, s, a);
    else
      hipLaunchKernelGGL((merge_lse_kernel<128, 1>), dim3((unsigned)grid), dim3(kMergeThreads), 0, s, a);
  } else {
    return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

int launch_append(const AppendArgs& a, void* stream, int max_wgs) {
  hipStream_t s = (hipStream_t)stream;
  const int64_t total = (int64_t)a.n_new * a.hkv * (a.head_dim / 8);
  const int64_t blocks = (total + kThreads - 1) / kThreads;
  const int cap = max_wgs > 0 ? std::min(max_wgs, 16384) : 16384;
  const int grid = (int)(blocks < cap ? (blocks > 0 ? blocks : 1) : cap);
  hipLaunchKernelGGL(append_kernel, dim3(grid), dim3(kThreads), 0, s, a);
  return (int)hipGetLastError();
}

int launch_append_rows(const AppendArgs& a, double* table, const int32_t* plan_offsets,
                       int32_t* split_offsets, void* stream) {
  // heads per thread: at most 2, so that a few thousand rows still give
  // every CU several waves (the angles are computed once per thread)
  const int hpt = std::min(a.hkv, 2);
  const int64_t total = (int64_t)a.n_new * (a.head_dim / 8) * ((a.hkv + hpt - 1) / hpt);
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>((total + kThreads - 1) / kThreads, 16384));
  hipLaunchKernelGGL(append_rows_kernel, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream, a,
                     reinterpret_cast<double2*>(table), plan_offsets, split_offsets, hpt);
  return (int)hipGetLastError();
}

int launch_project(const ProjArgs& a, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const int ncols = 2 * a.kv_dim;
  hipLaunchKernelGGL(proj_kernel, dim3(ncols / kProjCols, a.ksplit), dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  const int64_t total = (int64_t)a.n_new * ncols;
  const int grid = (int)std::min<int64_t>((total + kThreads - 1) / kThreads, 4096);
  hipLaunchKernelGGL(proj_reduce_kernel, dim3(grid), dim3(kThreads), 0, s, a);
  return (int)hipGetLastError();
}

int launch_probe_read(const void* src, const void* src2, size_t bytes, int nwg, int mode, float* sink,
                      void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const int64_t n16 = (int64_t)(bytes / 16);
  const u32x4* p = (const u32x4*)src;
  const u32x4* p2 = (const u32x4*)src2;
  const bool nt = mode & 1;
  const int layout = (mode & 4) ? 2 : ((mode & 2) ? 1 : 0);
#define DKV_PROBE(NTV, M) hipLaunchKernelGGL((probe_read_kernel<NTV, M>), dim3(nwg), dim3(kThreads), 0, s, p, p2, n16, sink)
  if (nt) {
    if (layout == 0) DKV_PROBE(true, 0);
    else if (layout == 1) DKV_PROBE(true, 1);
    else DKV_PROBE(true, 2);
  } else {
    if (layout == 0) DKV_PROBE(false, 0);
    else if (layout == 1) DKV_PROBE(false, 1);
    else DKV_PROBE(false, 2);
  }
#undef DKV_PROBE
  return (int)hipGetLastError();
}

}  // namespace dkv
