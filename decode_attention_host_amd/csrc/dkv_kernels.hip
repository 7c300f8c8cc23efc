// dkv_kernels.hip - gfx950 kernels of the zero-copy split decode attention path.
//
//   rope_q_kernel       rotate each query head (Neox RoPE, fp64 angle) once per call
//   attn_split_kernel   stream K/V tiles of one tier into LDS, Q.K on MFMA,
//                       online softmax, P.V on the vector ALUs, write (o, lse)
//   merge_lse_kernel    combine per-split partials by log-sum-exp
//   append_kernel       Neox RoPE of new keys (fp64) + bf16 store into the cache slot
//   proj_kernel         new-token K/V projection on MFMA (split over the hidden dim)
//   probe_read_kernel   streaming-read bandwidth probe with the attention load pattern
//
// Method sources (page, section): DirectKV README, introduction (fused projection,
// Neox RoPE and attention reading KV from CPU-pinned buffers) and Attribution
// (online softmax; KV streamed from CPU memory with no GPU staging buffer);
// SplitKernel README, Overview and Key Features (direct access of the remote
// tier into on-chip memory; attention over a host/device partitioned KV cache).
//
// Design notes for CDNA4:
//   * 64-lane waves, 256-thread workgroups (4 waves).  A tile is 64 tokens of one
//     KV head: each thread moves D/32 16-byte chunks of K and of V per tile with
//     coalesced loads (host-tier loads are non-temporal), stores them into LDS,
//     and each wave then owns 16 of the 64 tokens.
//   * Q.K^T runs on v_mfma_f32_16x16x32_bf16: A = 16 keys x 32 dims from LDS,
//     B = the group's query heads; each rotated query (fp32) is split into a
//     high and a low bf16 part placed in columns h and h+8, so the product keeps
//     ~16 bits of the query and fp32 accumulation.
//   * P.V runs on the vector ALUs with one or two output dims per lane: values
//     are exact bf16, weights fp32, accumulation fp32.
//   * Host-role and HBM-role workgroups are disjoint (blockIdx below / above the
//     host workgroup count) so both tiers stream concurrently.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "dkv_internal.h"

namespace dkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (u >> 16) | ((u & 0xffffu) ? 0x40u : 0u);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// double -> bf16 bits with one rounding (nearest, ties to even).
__device__ __forceinline__ uint32_t f64_to_bf16(double x) {
  uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint32_t sign = (uint32_t)(u >> 63) << 15;
  const int e = (int)((u >> 52) & 0x7ff);
  if (e == 0x7ff) return sign | ((u << 12) ? 0x7fc0u : 0x7f80u);
  const double ax = fabs(x);
  if (ax < 0x1p-126) {
    // subnormal bf16 grid: quantum 2^-133
    const double q = rint(ax * 0x1p133);  // 0 .. 128 (128 = smallest normal)
    return sign | (uint32_t)q;
  }
  const uint64_t mant = u & ((1ull << 52) - 1);
  uint64_t keep = mant >> 45;
  const uint64_t rest = mant & ((1ull << 45) - 1);
  const uint64_t half = 1ull << 44;
  uint32_t em = (uint32_t)((e - 1023 + 127) << 7) | (uint32_t)keep;
  if (rest > half || (rest == half && (keep & 1))) em += 1;  // may carry into the exponent
  if (em >= 0x7f80u) em = 0x7f80u;                           // overflow -> inf
  return sign | em;
}

// ---------------------------------------------------------------------------
// Query rotation: q_rot[b][h][d] = scale*log2(e) * RoPE(q[b][h], q_pos[b])[d].
// Angle pos * f_i and sin/cos in fp64 (f_i from the host table).  Block 0 also
// copies the split offsets of the plan to the caller's array.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void rope_q_kernel(const uint16_t* __restrict__ q,
                                                          const int32_t* __restrict__ q_pos,
                                                          float* __restrict__ q_rot, int hq, int d,
                                                          RopeFreq freq, float scale_log2,
                                                          const int32_t* __restrict__ plan_offsets,
                                                          int32_t* __restrict__ split_offsets,
                                                          int batch) {
  const int half = d >> 1;
  if (blockIdx.x == 0 && split_offsets)
    for (int i = threadIdx.x; i <= batch; i += blockDim.x) split_offsets[i] = plan_offsets[i];
  const int64_t per_row = (int64_t)hq * half;
  const int64_t total = (int64_t)batch * per_row;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int b = (int)(idx / per_row);
    const int rem = (int)(idx - (int64_t)b * per_row);
    const int h = rem / half, i = rem - h * half;
    double s, c;
    sincos((double)q_pos[b] * freq.f[i], &s, &c);
    const uint16_t* qh = q + ((size_t)b * hq + h) * d;
    const double xl = (double)bf16_to_f32(qh[i]);
    const double xh = (double)bf16_to_f32(qh[i + half]);
    float* o = q_rot + ((size_t)b * hq + h) * d;
    o[i] = (float)(xl * c - xh * s) * scale_log2;
    o[i + half] = (float)(xh * c + xl * s) * scale_log2;
  }
}

// ---------------------------------------------------------------------------
// Split decode attention.
// ---------------------------------------------------------------------------
template <int D>
struct AttnShape {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kPitch = kRowBytes + 16;          // LDS row pitch (bytes)
  static constexpr int kChunksPerRow = D / 8;            // 16-byte chunks per row
  static constexpr int kChunksPerThread = kTile * kChunksPerRow / kThreads;  // D/32
  static constexpr int kKSteps = D / 32;                 // MFMA k-steps per key
  static constexpr int kDimsPerLane = D / 64;            // P.V output dims per lane
};

template <int D, int G, bool PAGED>
__global__ __launch_bounds__(kThreads) void attn_split_kernel(AttnArgs a, const float* __restrict__ q_rot) {
  using S = AttnShape<D>;
  constexpr int NC = S::kChunksPerThread;
  constexpr int KS = S::kKSteps;
  constexpr int DPL = S::kDimsPerLane;
  static_assert(G >= 1 && G <= 8, "group size");
  // per-wave state dump at the end of a unit must fit in the K tile buffer
  static_assert(4 * G * (D + 2) * 4 <= kTile * S::kPitch, "epilogue scratch");

  __shared__ __attribute__((aligned(16))) uint8_t k_lds[kTile * S::kPitch];
  __shared__ __attribute__((aligned(16))) uint8_t v_lds[kTile * S::kPitch];
  __shared__ __attribute__((aligned(16))) float p_lds[4][16][8];
  __shared__ float a_lds[4][8];
  __shared__ int s_next;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15;     // MFMA column / row-in-tile
  const int j4 = lane >> 4;    // 0..3

  // Role: the first host_wgs workgroups stream the host tier, the rest HBM.
  const bool host_role = (int)blockIdx.x < a.host_wgs;
  const int wg = host_role ? (int)blockIdx.x : (int)blockIdx.x - a.host_wgs;
  const int nwg = host_role ? a.host_wgs : a.dev_wgs;
  const int nunits = host_role ? a.n_host_units : a.n_dev_units;
  const PlanItem* __restrict__ items = host_role ? a.host_items : a.dev_items;
  const uint16_t* __restrict__ kpool = host_role ? a.host_k : a.dev_k;
  const uint16_t* __restrict__ vpool = host_role ? a.host_v : a.dev_v;
  const int64_t cap_rows = host_role ? a.host_rows : a.dev_rows;
  // Units [0, nwg) go to workgroups by index; each later unit goes to the
  // workgroup that finishes first (per-role counter, zeroed by the plan upload).
  int* counter = a.unit_counters + (host_role ? 1 : 0);

  const bool traced = a.wg_trace && (int)blockIdx.x < a.wg_trace_cap && tid == 0;
  const uint64_t t_start = traced ? wall_clock64() : 0;
  int units_done = 0;

  u32x4 kreg[NC], vreg[NC];
  auto load_tile = [&](const PlanItem& it, int kvh, int tile) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int chunk = tid + c * kThreads;
      const int r = chunk / S::kChunksPerRow;
      const int col = chunk - r * S::kChunksPerRow;
      const int tok = tile * kTile + r;
      bool valid = tok < it.n_tok;
      int64_t row = 0;
      if (PAGED) {
        if (valid) {
          const int lp = a.plist[it.plist + (tok >> a.page_shift)];
          const int32_t e = a.page_table[(int64_t)it.b * a.max_pages + lp];
          const int64_t phys = (int64_t)(e >> 1);
          row = (phys << a.page_shift) | (tok & ((1 << a.page_shift) - 1));
          valid = e >= 0 && ((e & 1) != 0) == host_role && row < cap_rows;
        }
      } else {
        row = it.row0 + tok;
      }
      const int64_t off = (row * a.hkv + kvh) * D + col * 8;
      if (valid) {
        const u32x4* kp = reinterpret_cast<const u32x4*>(kpool + off);
        const u32x4* vp = reinterpret_cast<const u32x4*>(vpool + off);
        // KV is read once per step: non-temporal loads on both tiers (on
        // MI355X they also stream HBM faster than ordinary loads)
        kreg[c] = __builtin_nontemporal_load(kp);
        vreg[c] = __builtin_nontemporal_load(vp);
      } else {
        kreg[c] = u32x4{0u, 0u, 0u, 0u};
        vreg[c] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  int u = wg;
  PlanItem it{};
  int kvh = 0;
  if (u < nunits) {
    it = items[u / a.hkv];
    kvh = u - (u / a.hkv) * a.hkv;
    load_tile(it, kvh, 0);
  }
  while (u < nunits) {
    ++units_done;
    const int ntiles = (it.n_tok + kTile - 1) / kTile;

    // ---- query operand: columns h (high bf16 part) and h+8 (low part)
    bf16x8_t qb[KS];
    {
      const int hsel = n & 7;
      const bool active = hsel < G;
      const float* qr = q_rot + ((size_t)it.b * a.hq + kvh * G + (active ? hsel : 0)) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int d0 = ks * 32 + j4 * 8;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = active ? qr[d0 + 2 * e] : 0.f;
          const float x1 = active ? qr[d0 + 2 * e + 1] : 0.f;
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
    float acc[G][DPL];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[h][e] = 0.f;

    int next_u = nunits;
    PlanItem nit{};
    int nkvh = 0;
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
      if (last && tid == 0) s_next = nwg + atomicAdd(counter, 1);
      __syncthreads();
      // keep one tile in flight: the next tile of this unit, or the first
      // tile of the next unit while this unit's last tile is computed
      if (!last) {
        load_tile(it, kvh, tile + 1);
      } else {
        next_u = s_next;
        if (next_u < nunits) {
          nit = items[next_u / a.hkv];
          nkvh = next_u - (next_u / a.hkv) * a.hkv;
          load_tile(nit, nkvh, 0);
        }
      }

      // ---- scores for this wave's 16 tokens: rows = tokens, columns = heads
      floatx4 sc = {0.f, 0.f, 0.f, 0.f};
      const uint8_t* krow = k_lds + (wave * 16 + n) * S::kPitch + j4 * 16;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 kv = *reinterpret_cast<const u32x4*>(krow + ks * 64);
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kv), qb[ks], sc,
                                                     0, 0, 0);
      }
      const int tok0 = tile * kTile + wave * 16 + j4 * 4;
      float s[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = sc[i] + __shfl_xor(sc[i], 8);
        s[i] = (tok0 + i < it.n_tok) ? v : -INFINITY;
      }
      float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_run - m_new);
      float p[4], ps = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = (s[i] == -INFINITY) ? 0.f : exp2f(s[i] - m_new);
        ps += p[i];
      }
      ps += __shfl_xor(ps, 16);
      ps += __shfl_xor(ps, 32);
      l_run = l_run * alpha + ps;
      m_run = m_new;
      if (n < G) {
#pragma unroll
        for (int i = 0; i < 4; ++i) p_lds[wave][j4 * 4 + i][n] = p[i];
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

    // ---- combine the four waves of this unit and write the partial
    __syncthreads();
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
      const int hq_idx = kvh * G + h;
      a.part_o[((size_t)it.slot * a.hq + hq_idx) * D + d] = o;
      if (d == 0)
        a.part_lse[(size_t)it.slot * a.hq + hq_idx] =
            (M == -INFINITY) ? -INFINITY : (M + log2f(lsum)) * 0.69314718055994530942f;
    }
    // the next unit's first tile is already in registers
    u = next_u;
    it = nit;
    kvh = nkvh;
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
// Prefill: causal attention of blocks of new query rows over the cache.
//
// A unit = (row block of QB = 64/G query rows of one sequence, run of cached
// tokens in one tier, KV head); its 64 MFMA rows are the (head, row) pairs of
// the group, 16 per wave.  Both contractions are dense here and run on
// v_mfma_f32_16x16x32_bf16:
//   S = Q.K^T   A = query rows (fp32 split into high/low bf16), B = K rows
//   O += P.V    A = probabilities (high/low bf16 from LDS), B = V transposed
//               into LDS while the tile is staged
// Causal mask: token t is visible to a row at position p iff t <= p.
// ---------------------------------------------------------------------------
template <int D, int G, bool PAGED>
__global__ __launch_bounds__(kThreads) void prefill_split_kernel(PrefillArgs a,
                                                                 const float* __restrict__ q_rot) {
  constexpr int QB = 64 / G;
  constexpr int KS = D / 32;                   // k-steps of Q.K over the head dim
  constexpr int DT = D / 16;                   // 16-wide output-dim tiles of P.V
  constexpr int KPITCH = D * 2 + 16;           // bytes per K row in LDS
  constexpr int VT_PITCH = kTile + 8;          // bf16 per transposed V row
  constexpr int P_PITCH = kTile + 8;           // bf16 per probability row
  constexpr int CPR = D / 8;                   // 16-byte chunks per KV row
  constexpr int NCK = kTile * CPR / kThreads;  // K chunks per thread
  constexpr int NPV = kTile * CPR / 2 / kThreads;  // V row pairs per thread
  static_assert(NPV >= 1, "tile shape");

  __shared__ __attribute__((aligned(16))) uint8_t k_lds[kTile * KPITCH];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[D * VT_PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t p_hi[4][16 * P_PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t p_lo[4][16 * P_PITCH];
  __shared__ int tpos_lds[kTile];
  __shared__ int s_next;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15;
  const int j4 = lane >> 4;

  const bool host_role = (int)blockIdx.x < a.host_wgs;
  const int wg = host_role ? (int)blockIdx.x : (int)blockIdx.x - a.host_wgs;
  const int nwg = host_role ? a.host_wgs : a.dev_wgs;
  const int nunits = host_role ? a.n_host_units : a.n_dev_units;
  const PrefillItem* __restrict__ items = host_role ? a.host_items : a.dev_items;
  const uint16_t* __restrict__ kpool = host_role ? a.host_k : a.dev_k;
  const uint16_t* __restrict__ vpool = host_role ? a.host_v : a.dev_v;
  const int64_t cap_rows = host_role ? a.host_rows : a.dev_rows;
  int* counter = a.unit_counters + (host_role ? 1 : 0);

  // pool row and logical position of token `tok` of an item (-1: not valid)
  auto locate = [&](const PrefillItem& it, int tok, int64_t& row) -> int {
    if (tok >= it.n_tok) return -1;
    if (PAGED) {
      const int lp = a.plist[it.plist + (tok >> a.page_shift)];
      const int32_t e = a.page_table[(int64_t)it.b * a.max_pages + lp];
      const int off = tok & ((1 << a.page_shift) - 1);
      row = ((int64_t)(e >> 1) << a.page_shift) | off;
      if (e < 0 || ((e & 1) != 0) != host_role || row >= cap_rows) return -1;
      return (lp << a.page_shift) + off;
    }
    row = it.row_pool + tok;
    return it.tok0 + tok;
  };

  u32x4 kreg[NCK], vreg[NPV][2];
  int treg = -1;
  auto load_tile = [&](const PrefillItem& it, int kvh, int tile) {
#pragma unroll
    for (int c = 0; c < NCK; ++c) {
      const int chunk = tid + c * kThreads;
      const int r = chunk / CPR, col = chunk - (chunk / CPR) * CPR;
      int64_t row = 0;
      const bool ok = locate(it, tile * kTile + r, row) >= 0;
      kreg[c] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                         kpool + (row * a.hkv + kvh) * D + col * 8))
                   : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int q = 0; q < NPV; ++q) {
      const int pr = tid + q * kThreads;
      const int rp = pr / CPR, col = pr - (pr / CPR) * CPR;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        int64_t row = 0;
        const bool ok = locate(it, tile * kTile + 2 * rp + e, row) >= 0;
        vreg[q][e] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                              vpool + (row * a.hkv + kvh) * D + col * 8))
                        : u32x4{0u, 0u, 0u, 0u};
      }
    }
    if (tid < kTile) {
      int64_t row = 0;
      treg = locate(it, tile * kTile + tid, row);
    }
  };

  int u = wg;
  PrefillItem it{};
  int kvh = 0;
  if (u < nunits) {
    it = items[u / a.hkv];
    kvh = u - (u / a.hkv) * a.hkv;
    load_tile(it, kvh, 0);
  }
  while (u < nunits) {
    const int ntiles = (it.n_tok + kTile - 1) / kTile;
    // ---- query operand (A of S = Q.K^T): MFMA row n of this wave
    bf16x8_t qa_hi[KS], qa_lo[KS];
    {
      const int rowi = wave * 16 + n;
      const int h = rowi / QB, r = rowi - (rowi / QB) * QB;
      const bool active = r < it.n_rows;
      const float* qr = q_rot + ((size_t)(it.row0 + (active ? r : 0)) * a.hq + kvh * G + h) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint32_t wh[4], wl[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int d0 = ks * 32 + j4 * 8 + 2 * e;
          const float x0 = active ? qr[d0] : 0.f, x1 = active ? qr[d0 + 1] : 0.f;
          const uint32_t h0 = f32_to_bf16(x0), h1 = f32_to_bf16(x1);
          wh[e] = h0 | (h1 << 16);
          wl[e] = f32_to_bf16(x0 - bf16_to_f32(h0)) | (f32_to_bf16(x1 - bf16_to_f32(h1)) << 16);
        }
        qa_hi[ks] = __builtin_bit_cast(bf16x8_t, (u32x4{wh[0], wh[1], wh[2], wh[3]}));
        qa_lo[ks] = __builtin_bit_cast(bf16x8_t, (u32x4{wl[0], wl[1], wl[2], wl[3]}));
      }
    }
    // C-layout rows of this lane: 4*j4 + i of the wave's 16
    int rpos[4];
    bool rvalid[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rowi = wave * 16 + j4 * 4 + i;
      const int r = rowi - (rowi / QB) * QB;
      rvalid[i] = r < it.n_rows;
      rpos[i] = it.pos0 + r;
    }
    float m_run[4], l_run[4];
    floatx4 oacc[DT];
#pragma unroll
    for (int i = 0; i < 4; ++i) { m_run[i] = -INFINITY; l_run[i] = 0.f; }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] = floatx4{0.f, 0.f, 0.f, 0.f};

    int next_u = nunits;
    PrefillItem nit{};
    int nkvh = 0;
    for (int tile = 0; tile < ntiles; ++tile) {
      __syncthreads();  // previous tile's readers are done
#pragma unroll
      for (int c = 0; c < NCK; ++c) {
        const int chunk = tid + c * kThreads;
        const int r = chunk / CPR, col = chunk - (chunk / CPR) * CPR;
        *reinterpret_cast<u32x4*>(k_lds + r * KPITCH + col * 16) = kreg[c];
      }
#pragma unroll
      for (int q = 0; q < NPV; ++q) {
        const int pr = tid + q * kThreads;
        const int rp = pr / CPR, col = pr - (pr / CPR) * CPR;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t lo = (vreg[q][0][e >> 1] >> ((e & 1) * 16)) & 0xffffu;
          const uint32_t hi = (vreg[q][1][e >> 1] >> ((e & 1) * 16)) & 0xffffu;
          *reinterpret_cast<uint32_t*>(&vt_lds[(col * 8 + e) * VT_PITCH + 2 * rp]) = lo | (hi << 16);
        }
      }
      if (tid < kTile) tpos_lds[tid] = treg;
      const bool last = tile + 1 == ntiles;
      if (last && tid == 0) s_next = nwg + atomicAdd(counter, 1);
      __syncthreads();
      if (!last) {
        load_tile(it, kvh, tile + 1);
      } else {
        next_u = s_next;
        if (next_u < nunits) {
          nit = items[next_u / a.hkv];
          nkvh = next_u - (next_u / a.hkv) * a.hkv;
          load_tile(nit, nkvh, 0);
        }
      }

      // ---- S = Q.K^T for 16 rows x 64 tokens (four 16-token column tiles)
      floatx4 sc[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        sc[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
        const uint8_t* krow = k_lds + (nt * 16 + n) * KPITCH + j4 * 16;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8_t kb = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4*>(krow + ks * 64));
          sc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa_hi[ks], kb, sc[nt], 0, 0, 0);
          sc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa_lo[ks], kb, sc[nt], 0, 0, 0);
        }
      }
      // ---- causal mask and online softmax per row (row = 4*j4 + i)
      int tp[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) tp[nt] = tpos_lds[nt * 16 + n];
      float alpha[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float mx = -INFINITY;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const bool vis = rvalid[i] && tp[nt] >= 0 && tp[nt] <= rpos[i];
          sc[nt][i] = vis ? sc[nt][i] : -INFINITY;
          mx = fmaxf(mx, sc[nt][i]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 1));
        mx = fmaxf(mx, __shfl_xor(mx, 2));
        mx = fmaxf(mx, __shfl_xor(mx, 4));
        mx = fmaxf(mx, __shfl_xor(mx, 8));
        const float m_new = fmaxf(m_run[i], mx);
        alpha[i] = (m_new == -INFINITY) ? 1.f : exp2f(m_run[i] - m_new);
        float ps = 0.f;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const float pv = (sc[nt][i] == -INFINITY) ? 0.f : exp2f(sc[nt][i] - m_new);
          ps += pv;
          const uint32_t ph = f32_to_bf16(pv);
          const int o = (j4 * 4 + i) * P_PITCH + nt * 16 + n;
          p_hi[wave][o] = (uint16_t)ph;
          p_lo[wave][o] = (uint16_t)f32_to_bf16(pv - bf16_to_f32(ph));
        }
        ps += __shfl_xor(ps, 1);
        ps += __shfl_xor(ps, 2);
        ps += __shfl_xor(ps, 4);
        ps += __shfl_xor(ps, 8);
        l_run[i] = l_run[i] * alpha[i] + ps;
        m_run[i] = m_new;
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[dt][i] *= alpha[i];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

      // ---- O += P.V: A = P rows (from LDS), B = V^T rows (from LDS)
#pragma unroll
      for (int kt = 0; kt < kTile / 32; ++kt) {
        const int ko = kt * 32 + j4 * 8;
        const bf16x8_t pa_hi = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4*>(&p_hi[wave][n * P_PITCH + ko]));
        const bf16x8_t pa_lo = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4*>(&p_lo[wave][n * P_PITCH + ko]));
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const bf16x8_t vb = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4*>(&vt_lds[(dt * 16 + n) * VT_PITCH + ko]));
          oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_hi, vb, oacc[dt], 0, 0, 0);
          oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_lo, vb, oacc[dt], 0, 0, 0);
        }
      }
      __builtin_amdgcn_wave_barrier();
    }

    // ---- write this unit's partial for every valid row
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (!rvalid[i]) continue;
      const int rowi = wave * 16 + j4 * 4 + i;
      const int h = rowi / QB, r = rowi - (rowi / QB) * QB;
      const size_t slot = (size_t)it.base + (size_t)r * it.n_splits + it.split_idx;
      const size_t head = slot * a.hq + kvh * G + h;
      const bool empty = m_run[i] == -INFINITY;
      const float inv = empty ? 0.f : 1.f / l_run[i];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) a.part_o[head * D + dt * 16 + n] = oacc[dt][i] * inv;
      if (n == 0)
        a.part_lse[head] = empty ? -INFINITY : (m_run[i] + log2f(l_run[i])) * 0.69314718055994530942f;
    }
    u = next_u;
    it = nit;
    kvh = nkvh;
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

// Workgroup = (b, h), 1024 threads: D/4 lanes each own 4 dims (one 16-byte
// load per split), 4096/D groups of lanes fold every group-th split with
// several loads in flight, then the groups combine through LDS.
constexpr int kMergeThreads = 1024;

template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_lse_kernel(MergeArgs a) {
  constexpr int LANES = D / 4;
  constexpr int NG = kMergeThreads / LANES;
  constexpr int U = 4;
  __shared__ float sm_red[kMergeThreads / 64];
  __shared__ __attribute__((aligned(16))) float sm_o[NG][D];
  const int bh = blockIdx.x;
  const int b = bh / a.hq, h = bh - b * a.hq;
  const int tid = threadIdx.x;
  const int s0 = a.split_offsets[b], s1 = a.split_offsets[b + 1];
  const float* lse = a.part_lse + h;
  float m = -INFINITY;
  for (int s = s0 + tid; s < s1; s += kMergeThreads) m = fmaxf(m, lse[(size_t)s * a.hq]);
  const float M = block_reduce_n<kMergeThreads>(m, true, sm_red);
  float* out = a.out_o + ((size_t)b * a.hq + h) * D;
  if (M == -INFINITY) {  // no finite split
    if (tid < D) out[tid] = 0.f;
    if (tid == 0 && a.out_lse) a.out_lse[(size_t)b * a.hq + h] = -INFINITY;
    return;
  }
  float l = 0.f;
  for (int s = s0 + tid; s < s1; s += kMergeThreads) {
    const float x = lse[(size_t)s * a.hq];
    l += (x == -INFINITY) ? 0.f : expf(x - M);
  }
  const float Lsum = block_reduce_n<kMergeThreads>(l, false, sm_red);
  const int g = tid / LANES, d4 = (tid - g * LANES) * 4;
  const float* po = a.part_o + (size_t)h * D + d4;
  const size_t srow = (size_t)a.hq * D;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  int s = s0 + g;
  for (; s + (U - 1) * NG < s1; s += U * NG) {
    float x[U];
    float4 o[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      x[k] = lse[(size_t)(s + k * NG) * a.hq];
      o[k] = *reinterpret_cast<const float4*>(po + (size_t)(s + k * NG) * srow);
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const float w = (x[k] == -INFINITY) ? 0.f : expf(x[k] - M);
      acc.x += w * o[k].x; acc.y += w * o[k].y; acc.z += w * o[k].z; acc.w += w * o[k].w;
    }
  }
  for (; s < s1; s += NG) {
    const float x = lse[(size_t)s * a.hq];
    const float w = (x == -INFINITY) ? 0.f : expf(x - M);
    const float4 o = *reinterpret_cast<const float4*>(po + (size_t)s * srow);
    acc.x += w * o.x; acc.y += w * o.y; acc.z += w * o.z; acc.w += w * o.w;
  }
  *reinterpret_cast<float4*>(&sm_o[g][d4]) = acc;
  __syncthreads();
  if (tid < D) {
    float o = 0.f;
#pragma unroll 8
    for (int k = 0; k < NG; ++k) o += sm_o[k][tid];
    out[tid] = o / Lsum;
    if (tid == 0 && a.out_lse) a.out_lse[(size_t)b * a.hq + h] = M + logf(Lsum);
  }
}

// ---------------------------------------------------------------------------
// Append: slot of (b, p) from the placement, K rotated in fp64 and rounded
// once to bf16, V stored as is.  Thread = (token, group of 8 rotation pairs);
// it loops over the KV heads so each angle's sin/cos is computed once.
// ---------------------------------------------------------------------------
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
    *reinterpret_cast<uint2*>(dst + p0) = make_uint2(yl[0], yl[1]);
    *reinterpret_cast<uint2*>(dst + half + p0) = make_uint2(yh[0], yh[1]);
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
      *reinterpret_cast<uint2*>(vd + p0) = make_uint2(w0[0], w0[1]);
      *reinterpret_cast<uint2*>(vd + half + p0) = make_uint2(w1[0], w1[1]);
    } else {
      const uint16_t* vs = a.v_new + (size_t)i * kvd + h * D;
      *reinterpret_cast<uint2*>(vd + p0) = *reinterpret_cast<const uint2*>(vs + p0);
      *reinterpret_cast<uint2*>(vd + half + p0) = *reinterpret_cast<const uint2*>(vs + half + p0);
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
  // ---- stage W[k0 .. k0+kProjK)[col0 .. col0+64) transposed
  for (int c = tid; c < kProjK * (kProjCols / 8); c += kThreads) {
    const int kr = c / (kProjCols / 8);
    const int cc = (c - kr * (kProjCols / 8)) * 8;
    const int gcol = col0 + cc;
    const uint16_t* src = (gcol < a.kv_dim) ? a.wk + (size_t)(k0 + kr) * a.kv_dim + gcol
                                            : a.wv + (size_t)(k0 + kr) * a.kv_dim + (gcol - a.kv_dim);
    const u32x4 w = *reinterpret_cast<const u32x4*>(src);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      wt[cc + 2 * e][kr] = (uint16_t)(w[e] & 0xffffu);
      wt[cc + 2 * e + 1][kr] = (uint16_t)(w[e] >> 16);
    }
  }
  __syncthreads();
  // ---- wave w computes columns col0 + 16w .. +16 for every 16-token tile
  const int ctile = wave * 16;
  for (int m0 = 0; m0 < a.n_new; m0 += 16) {
    floatx4 c = {0.f, 0.f, 0.f, 0.f};
    const int row = m0 + n;
    const bool rv = row < a.n_new;
    const uint16_t* xr = a.x + (size_t)(rv ? row : 0) * a.hidden + k0 + j4 * 8;
#pragma unroll 4
    for (int kk = 0; kk < kProjK; kk += 32) {
      u32x4 av = rv ? *reinterpret_cast<const u32x4*>(xr + kk) : u32x4{0u, 0u, 0u, 0u};
      const u32x4 bv = *reinterpret_cast<const u32x4*>(&wt[ctile + n][kk + j4 * 8]);
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
    for (int k = 0; k < a.ksplit; ++k) s += a.partial[((size_t)k * a.n_pad + r) * ncols + c];
    a.out[idx] = s;
  }
}

// ---------------------------------------------------------------------------
// Streaming read probe: 16 B per lane per load, coalesced, grid-stride.
// ---------------------------------------------------------------------------
template <bool NT>
__global__ __launch_bounds__(kThreads) void probe_read_kernel(const u32x4* __restrict__ src,
                                                             int64_t n16, float* sink) {
  constexpr int U = 8;  // 16-byte loads in flight per thread
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int k = 0; k < U; ++k) v[k] = NT ? __builtin_nontemporal_load(src + i + k * stride) : src[i + k * stride];
#pragma unroll
    for (int k = 0; k < U; ++k) acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = NT ? __builtin_nontemporal_load(src + i) : src[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9e3779b9u) sink[0] = (float)acc;  // keeps the loads alive
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <int D, int G>
static hipError_t launch_attn_dg(const AttnArgs& a, const float* q_rot, hipStream_t s) {
  const int grid = a.host_wgs + a.dev_wgs;
  if (a.page_shift >= 0 && a.page_table)
    hipLaunchKernelGGL((attn_split_kernel<D, G, true>), dim3(grid), dim3(kThreads), 0, s, a, q_rot);
  else
    hipLaunchKernelGGL((attn_split_kernel<D, G, false>), dim3(grid), dim3(kThreads), 0, s, a, q_rot);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_attn_d(const AttnArgs& a, const float* q_rot, hipStream_t s) {
  switch (a.hq / a.hkv) {
    case 1: return launch_attn_dg<D, 1>(a, q_rot, s);
    case 2: return launch_attn_dg<D, 2>(a, q_rot, s);
    case 4: return launch_attn_dg<D, 4>(a, q_rot, s);
    case 8: return launch_attn_dg<D, 8>(a, q_rot, s);
    default: return hipErrorInvalidValue;
  }
}

int launch_rope_q(const uint16_t* q, const int32_t* q_pos, float* q_rot, int batch, int hq, int d,
                  const RopeFreq& freq, float scale_log2, const int32_t* plan_offsets,
                  int32_t* split_offsets, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const int64_t total = (int64_t)batch * hq * (d / 2);
  const int bx = (int)std::min<int64_t>((total + kThreads - 1) / kThreads, 16384);
  hipLaunchKernelGGL(rope_q_kernel, dim3(bx), dim3(kThreads), 0, s, q, q_pos, q_rot, hq, d, freq,
                     scale_log2, plan_offsets, split_offsets, batch);
  return (int)hipGetLastError();
}

int launch_attn_with_q(const AttnArgs& a, const float* q_rot, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (a.host_wgs + a.dev_wgs <= 0) return (int)hipSuccess;
  if (a.head_dim == 64) return (int)launch_attn_d<64>(a, q_rot, s);
  if (a.head_dim == 128) return (int)launch_attn_d<128>(a, q_rot, s);
  return (int)hipErrorInvalidValue;
}

template <int D, int G>
static hipError_t launch_prefill_dg(const PrefillArgs& a, const float* q_rot, hipStream_t s) {
  const int grid = a.host_wgs + a.dev_wgs;
  if (a.page_table)
    hipLaunchKernelGGL((prefill_split_kernel<D, G, true>), dim3(grid), dim3(kThreads), 0, s, a, q_rot);
  else
    hipLaunchKernelGGL((prefill_split_kernel<D, G, false>), dim3(grid), dim3(kThreads), 0, s, a, q_rot);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_prefill_d(const PrefillArgs& a, const float* q_rot, hipStream_t s) {
  switch (a.hq / a.hkv) {
    case 1: return launch_prefill_dg<D, 1>(a, q_rot, s);
    case 2: return launch_prefill_dg<D, 2>(a, q_rot, s);
    case 4: return launch_prefill_dg<D, 4>(a, q_rot, s);
    case 8: return launch_prefill_dg<D, 8>(a, q_rot, s);
    default: return hipErrorInvalidValue;
  }
}

int launch_prefill(const PrefillArgs& a, const float* q_rot, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (a.host_wgs + a.dev_wgs <= 0) return (int)hipSuccess;
  if (a.head_dim == 64) return (int)launch_prefill_d<64>(a, q_rot, s);
  if (a.head_dim == 128) return (int)launch_prefill_d<128>(a, q_rot, s);
  return (int)hipErrorInvalidValue;
}

int launch_merge(const MergeArgs& a, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const int64_t grid = (int64_t)a.batch * a.hq;
  if (grid > 0x7fffffff) return (int)hipErrorInvalidValue;
  if (a.head_dim == 64)
    hipLaunchKernelGGL(merge_lse_kernel<64>, dim3((unsigned)grid), dim3(kMergeThreads), 0, s, a);
  else if (a.head_dim == 128)
    hipLaunchKernelGGL(merge_lse_kernel<128>, dim3((unsigned)grid), dim3(kMergeThreads), 0, s, a);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

int launch_append(const AppendArgs& a, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const int64_t total = (int64_t)a.n_new * a.hkv * (a.head_dim / 8);
  const int64_t blocks = (total + kThreads - 1) / kThreads;
  const int grid = (int)(blocks < 16384 ? (blocks > 0 ? blocks : 1) : 16384);
  hipLaunchKernelGGL(append_kernel, dim3(grid), dim3(kThreads), 0, s, a);
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

int launch_probe_read(const void* src, size_t bytes, int nwg, int nontemporal, float* sink,
                      void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const int64_t n16 = (int64_t)(bytes / 16);
  if (nontemporal)
    hipLaunchKernelGGL(probe_read_kernel<true>, dim3(nwg), dim3(kThreads), 0, s,
                       (const u32x4*)src, n16, sink);
  else
    hipLaunchKernelGGL(probe_read_kernel<false>, dim3(nwg), dim3(kThreads), 0, s,
                       (const u32x4*)src, n16, sink);
  return (int)hipGetLastError();
}

}  // namespace dkv
