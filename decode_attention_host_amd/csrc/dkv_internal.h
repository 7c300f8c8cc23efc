// dkv_internal.h - structures shared by the host runtime (C++) and the gfx950
// kernels (HIP).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "dkv.h"
#include "dkv_decomp.h"

namespace dkv {

// Rotary frequencies f_i = theta^(-2i/D), i < D/2, computed once on the host
// in fp64 and passed by value to the kernels that rotate.
struct RopeFreq {
  double f[64];
};

// Tokens staged per tile by the attention kernel (4 waves x 16 tokens).
constexpr int kTile = 64;
// Threads per attention / merge / append workgroup.
constexpr int kThreads = 256;

// Query-head rows per prefill workgroup: 4 waves x 32 rows (two 16-column
// MFMA tiles each).  A row block holds kPrefillRows / G query rows.
constexpr int kPrefillRows = 128;
// Keys per prefill tile (one LDS staging step).
constexpr int kPfTile = 128;

// Where a prefill item's tokens are read from.
// kPoolFresh: the new rows themselves, written to HBM by the fused step's
// append next to their cache slots (row = the query row's index).
enum PrefillPool : int32_t { kPoolHost = 0, kPoolDev = 1, kPoolStaged = 2, kPoolFresh = 3 };

// Prefill work item: a block of consecutive query rows of one sequence (all G
// heads of one KV head per unit) against a run of cached tokens that lie in
// one pool.  The partial of block row r for this item is split slot
// base + r * n_splits + split_idx.
struct PrefillItem {
  int32_t b;          // sequence
  int32_t row0;       // global query row of the block's first row
  int32_t n_rows;     // rows in the block (<= kPrefillRows / G)
  int32_t pos0;       // position of the block's first row
  int32_t n_tok;      // tokens in the item
  int32_t plist;      // paged: first (logical page, pool page) pair of the item
  int32_t tok0;       // contiguous: logical position of the item's first token
  int32_t split_idx;  // index of this item among its block's splits
  int32_t n_splits;   // splits of the block
  int32_t base;       // first split slot of the block
  int32_t pool;       // PrefillPool
  int32_t pad;
  int64_t row_pool;   // contiguous: pool row of the item's first token
  int64_t pad2;
};
static_assert(sizeof(PrefillItem) == 64, "PrefillItem layout");

// One copy of host-tier rows into the HBM staging pool (prefill re-reads
// them once per row block; staged, they cross the host link once).
struct StageTile {
  int64_t src_row;    // host pool row
  int64_t dst_row;    // staging pool row
  int32_t n_rows;
  int32_t pad[3];
};
static_assert(sizeof(StageTile) == 32, "StageTile layout");
constexpr int kStageTileRows = 64;

// Offloaded linear: an item is up to kLinRows output rows of one tier and a
// range [k0, k1) of the reduction dimension; slot < 0 writes y directly.
constexpr int kLinRows = 64;
constexpr int kLinMaxTokens = 64;  // tokens per launch (4 MFMA row tiles)
struct LinearItem {
  int32_t row0;
  int32_t n_rows;
  int32_t k0;
  int32_t k1;
  int32_t slot;
  int32_t pool;    // kPoolHost / kPoolDev
  int32_t pad[2];
};
static_assert(sizeof(LinearItem) == 32, "LinearItem layout");

// The items of a linear call follow from this shape alone (the kernel derives
// them; the planner lists them for introspection).  Host tier first: row block
// j of a tier covers rows r0 + 64 j .. (r0 = 0 host, n_host HBM) and is cut
// into sp K ranges of kc (the last one shorter); item i of a tier is block
// i / sp, range i % sp.  In a tier with sp > 1 item i writes partial slot i
// (host) or p_host + i (HBM; p_host = host items if the host tier is split,
// else 0), and the last range of a block to finish sums its slots in order
// into y; with sp = 1 an item writes y directly.
struct LinearShape {
  int32_t n_host = 0;         // output rows in host memory
  int32_t bh = 0, bd = 0;     // row blocks per tier
  int32_t kc_host = 0, kc_dev = 0;
  int32_t sp_host = 1, sp_dev = 1;
  int32_t host_wgs = 0, dev_wgs = 0;
  int32_t n_host_items = 0, n_dev_items = 0;
  int32_t num_splits = 0;     // partial slots (0: no K split)
  int64_t host_bytes = 0, dev_bytes = 0;
  // workspace: [4 + bh + bd] int32 counters (zero between calls), then the
  // partials [num_splits][kLinMaxTokens][kLinRows] fp32
  size_t part_off = 0;
  size_t ws_bytes = 0;
};

// Host-side result of planning; the device image is `blob` (items, then the
// page list, then split offsets), uploaded into the caller's workspace.
struct PlanLayout {
  int32_t n_host_items = 0;
  int32_t n_dev_items = 0;
  int32_t num_splits = 0;
  int32_t batch = 0;
  int32_t host_wgs = 0;
  int32_t dev_wgs = 0;
  int32_t host_chunk = 0;
  int32_t dev_chunk = 0;
  int64_t host_bytes = 0;
  int64_t dev_bytes = 0;
  size_t items_off = 0;    // byte offsets inside the blob
  size_t plist_off = 0;
  size_t offsets_off = 0;
  size_t counters_off = 0;       // two int32 counters, zero in the image
  size_t blob_bytes = 0;
  int32_t n_plist = 0;
  size_t rowpos_off = 0;         // prefill: position of every query row [T]
  int32_t n_rows = 0;            // prefill: T (query rows)
  int64_t host_reads = 0;        // prefill: K+V bytes read from each tier,
  int64_t dev_reads = 0;         //   counting re-reads by later row blocks
  size_t stage_tiles_off = 0;    // prefill: StageTile list inside the blob
  int32_t n_stage_tiles = 0;
  int64_t stage_rows = 0;        // prefill: rows of the HBM staging pool
  int64_t staged_bytes = 0;      // prefill: host K+V bytes copied once
  int32_t dev_queues = 1;        // prefill: HBM work queues (1 or 8)
  size_t rowseq_off = 0;         // prefill: sequence of every query row [T]
  size_t seqlens_off = 0;        // prefill: cached lengths [B] (device copy)
};

// Arguments of the decode kernel (dkv_decode.hip).  Every work item is
// derived in the kernel from the lengths in device memory (dkv_decomp.h).
struct DecodeArgs {
  // tiers
  uint16_t* host_k;              // mapped host-pinned pools (device addresses)
  uint16_t* host_v;
  uint16_t* dev_k;               // HBM pools
  uint16_t* dev_v;
  int64_t host_rows;
  int64_t dev_rows;
  int64_t host_stride;           // contiguous layout: rows per sequence
  int64_t dev_stride;
  const int32_t* page_table;     // paged layout: [batch][max_pages]
  int32_t max_pages;
  int32_t page_shift;            // log2(page size), -1 for the contiguous layout
  // the call
  const uint16_t* q;             // [batch][Hq][D] bf16
  const int32_t* q_pos;          // [batch]
  const int32_t* seq_lens;       // [batch] cached tokens attended (device)
  int32_t batch;
  int32_t hq;
  int32_t hkv;
  int32_t head_dim;
  double ratio;                  // contiguous: offload ratio
  float scale_log2;              // scale * log2(e)
  int32_t fused;                 // 1: merge in the kernel (last finisher per sequence and KV head)
  DecodeTemplate tmpl;
  // workspace
  int32_t* counters;             // error flags, exit count, the two tiers' unit queues (decode_queue)
  int32_t* group_cnt;            // fused: [max_slots][Hkv] units done per group of slots (at the
                                 // group's first slot), then [batch][Hkv] groups done
  const int32_t* tier_counts;    // paged: [batch][4] host pages, HBM pages, host tokens, HBM tokens
  const int32_t* tier_pages;     // paged: [2][batch][max_pages] physical pages, host tier then HBM
  // one normalised partial per (item, KV head): the caller's arrays (split
  // form) or the workspace's (fused form, where each sequence's item slots
  // are followed by one for its appended token)
  float* part_o;                 // [max_slots][Hq][D]
  float* part_lse;               // [max_slots][Hq]
  int32_t* split_offsets;        // split form: [batch + 1] (written by workgroup 0)
  int32_t max_slots;             // slots part_o and part_lse hold
  int32_t new_tokens;            // 1: each sequence first appends a token at pos_new[b]
  float* out_o;                  // [batch][Hq][D]
  float* out_lse;                // [batch][Hq] or NULL
  const int32_t* pos_new;        // [batch] position of the appended token (NULL: seq_lens[b])
  const uint16_t* k_new;         // [batch][Hkv][D] bf16, or NULL with kv_proj
  const uint16_t* v_new;
  const float* kv_proj;          // [batch][2 Hkv D] fp32 projection (K then V), or NULL
  uint64_t* wg_trace;            // optional [grid][4]: start, end, role, items (wall clock)
  int32_t wg_trace_cap;
  int32_t pad1;
  RopeFreq freq;                 // f_i = theta^(-2i/D), i < D/2
};

// Counter words of the decode workspace (int32 offsets from `counters`): the
// error flags first, at a place no other shape uses for a counter (they are
// sticky, while every counter returns to zero at the end of each call), then
// the exit count, then the unit queues (host tier, then HBM tier).
DKV_HD constexpr int decode_error_word() { return 0; }
DKV_HD constexpr int decode_exit_counter() { return 1; }
DKV_HD constexpr int decode_queue(bool host) { return host ? 2 : 3; }
DKV_HD constexpr int decode_counter_words() { return 4; }
constexpr int kDecodeErrLayout = 1;     // a contiguous sequence's rows exceed its stride or pool
constexpr int kDecodeErrPage = 2;       // a page entry is negative or beyond its tier's pool
constexpr int kDecodeErrSlot = 4;       // an appended token has no valid cache slot
constexpr int kDecodeErrCapacity = 8;   // the call needs more partial slots than it was given (nothing computed)

struct MergeArgs {
  const float* part_o;
  const float* part_lse;
  const int32_t* split_offsets;
  int32_t batch;
  int32_t hq;
  int32_t head_dim;
  int32_t pad;
  float* out_o;
  float* out_lse;
};

struct AppendArgs {
  int32_t batch;
  int32_t n_new;
  const int32_t* seq_lens;       // contiguous only
  double ratio;
  const int32_t* seq_idx;
  const int32_t* pos;
  const uint16_t* k_new;         // [n_new][Hkv][D] bf16, or NULL in projection mode
  const uint16_t* v_new;
  const float* kv_proj;          // projection mode: [n_new][2*Hkv*D] fp32 (K then V)
  uint16_t* fresh_k;             // optional second copy of token i's K/V at row i
  uint16_t* fresh_v;
  int32_t skip_slots;            // 1: write only the second copy
  uint16_t* host_k;
  uint16_t* host_v;
  uint16_t* dev_k;
  uint16_t* dev_v;
  int64_t host_rows;
  int64_t dev_rows;
  int64_t host_stride;
  int64_t dev_stride;
  const int32_t* page_table;
  int32_t max_pages;
  int32_t page_size;             // 0 = contiguous
  int32_t hkv;
  int32_t head_dim;
  RopeFreq freq;
};

struct ProjArgs {
  const uint16_t* x;     // [n_new][hidden]
  const uint16_t* wk;    // [hidden][kv_dim]
  const uint16_t* wv;
  float* partial;        // [ksplit][n_pad][2*kv_dim]
  float* out;            // [n_new][2*kv_dim] (reduced)
  int32_t n_new;
  int32_t n_pad;         // n_new rounded up to 16
  int32_t hidden;
  int32_t kv_dim;
  int32_t ksplit;
  int32_t kslice;        // hidden / ksplit
};

// Arguments of the prefill kernel.
// Prefill unit counters in the plan image: one per HBM queue, then the host's.
constexpr int kPfMaxQueues = 8;
constexpr int kPfHostCounter = kPfMaxQueues;

struct PrefillArgs {
  const PrefillItem* host_items;
  const PrefillItem* dev_items;  // HBM and staged items
  const int32_t* pages;          // paged: (logical page, pool page) pairs
  int32_t* unit_counters;        // [kPfMaxQueues + 1], zero at launch
  int32_t n_host_items;
  int32_t n_dev_items;
  int32_t host_wgs;
  int32_t dev_wgs;               // multiple of dev_queues
  int32_t dev_queues;            // 1, or 8 when Hkv % 8 == 0 (one per XCD)
  int32_t pad;
  const uint16_t* host_k;
  const uint16_t* host_v;
  const uint16_t* dev_k;
  const uint16_t* dev_v;
  const uint16_t* stage_k;
  const uint16_t* stage_v;
  const uint16_t* fresh_k;       // fused step: new rows [T][Hkv][D]
  const uint16_t* fresh_v;
  int32_t page_shift;
  int32_t hq;
  int32_t hkv;
  int32_t head_dim;
  float* part_o;                 // [S][Hq][D]
  float* part_lse;               // [S][Hq]
  int32_t writer_wgs;            // fused step: workgroups copying the new rows
  int32_t pad2;                  //   from fresh_k/v into their cache slots
  AppendArgs app;                //   (placement of new row i, as for append)
  const uint16_t* q;             // query rows [T][Hq][D] bf16 (unrotated)
  const double* rope_cs;         // [T][D/2] (cos, sin) of each row's angles
  float scale_log2;              // scale * log2(e), folded into the rotated q
  int32_t pad3;
};

struct LinearArgs {
  int32_t* counters;             // [0] HBM queue, [1] host queue, [2] exit, [3] unused, [4 + block]
                                 // ranges done per row block; zero at launch, left zero
  int32_t n_host_items;
  int32_t n_dev_items;
  int32_t host_wgs;
  int32_t dev_wgs;
  int32_t m;                     // tokens in this launch (<= kLinMaxTokens)
  int32_t n;                     // out_features
  int32_t k;                     // in_features
  int32_t n_host;                // rows of W in host memory
  int32_t bh;                    // host row blocks
  int32_t kc_host, kc_dev;       // K per item
  int32_t sp_host, sp_dev;       // items per row block
  int32_t p_host;                // partial slots of the host tier (0 when it is not split)
  const uint16_t* host_w;        // [n_host][K]
  const uint16_t* dev_w;         // [N - n_host][K]
  const uint16_t* x;             // [m][K]
  float* y;                      // [m][N]
  float* part;                   // [S][kLinMaxTokens][kLinRows]
};

// Arguments of the staging copy (host rows -> HBM staging pool).
struct StageArgs {
  const StageTile* tiles;
  int32_t n_tiles;
  int32_t row_chunks;            // 16-byte chunks per row (Hkv * D / 8)
  const uint16_t* src_k;
  const uint16_t* src_v;
  uint16_t* dst_k;
  uint16_t* dst_v;
};

// Launchers (dkv_kernels.hip).  They return hipError_t as int.
// Decode: the paged layout's per-sequence tier lists and counts, then the
// decode kernel (grid = Hkv * (team_h + team_d)).
int launch_decode_tiers(const DecodeArgs& a, int32_t* tier_counts, int32_t* tier_pages, void* stream);
int launch_decode(const DecodeArgs& a, void* stream);
// The static decode scratch of the current device (dkv_decode.hip): its
// device address (from hipGetSymbolAddress, once per device) and size.
constexpr size_t kDecodeStaticScratchBytes = DKV_STATIC_SCRATCH_BYTES;
// Its first kDecodeStaticCounterBytes hold the counters of every call and
// nothing else, so they are zero at the start of a call whatever the shape of
// the call before it (each call leaves its counters at zero).
constexpr size_t kDecodeStaticCounterBytes = 1u << 20;
constexpr int kMaxDevices = 64;
int decode_static_scratch(void** ptr, size_t* bytes);
int launch_merge(const MergeArgs& a, void* stream);
int launch_prefill(const PrefillArgs& a, void* stream);
// (cos, sin) in fp64 of the rotation angles of every prefill row:
// cs[row][i] for angle rowpos[row] * freq.f[i], i < d / 2; block 0 also copies
// plan_offsets[0 .. n_rows] to split_offsets (if not NULL).
int launch_rope_table(const int32_t* rowpos, int n_rows, int d, const RopeFreq& freq, double* cs,
                      const int32_t* plan_offsets, int32_t* split_offsets, void* stream);
int launch_stage(const StageArgs& a, int nwg, void* stream);
int launch_linear(const LinearArgs& a, void* stream);
// max_wgs > 0 caps the grid (the kernel loops over the tokens).
int launch_append(const AppendArgs& a, void* stream, int max_wgs = 0);
// Fused prefill step: the new rows' keys (rotated) and values into fresh_k /
// fresh_v (and their slots unless skip_slots), and their rotation table
// [n_new][D/2] (cos, sin) in fp64; block 0 also copies plan_offsets[0 ..
// n_new] to split_offsets.
int launch_append_rows(const AppendArgs& a, double* table, const int32_t* plan_offsets,
                       int32_t* split_offsets, void* stream);
int launch_project(const ProjArgs& a, void* stream);
// mode: bit 0 non-temporal loads, bit 1 blocked (one contiguous slice per workgroup)
// src2 (optional): a second buffer of `bytes`, read by the odd workgroups
int launch_probe_read(const void* src, const void* src2, size_t bytes, int nwg, int mode, float* sink,
                      void* stream);

// Planner (dkv_plan.cpp), no HIP calls.
struct PlanInput {
  int32_t batch;
  int32_t hq;
  int32_t hkv;
  int32_t head_dim;
  int32_t page_size;
  int32_t max_pages;
  int64_t host_stride;
  int64_t dev_stride;
  int64_t host_rows;
  int64_t dev_rows;
  const int32_t* seq_lens;        // host
  const int32_t* page_table_host; // host, paged
  double ratio;
  int32_t num_cus;
  int32_t host_wgs;               // tuning (0 = default)
  int32_t dev_wgs;
  int32_t host_chunk;
  int32_t dev_chunk;
  double host_bw;
  double dev_bw;
  int64_t stage_max_bytes;        // prefill staging budget (< 0: never stage)
  int32_t prefill_fresh;          // prefill: new rows read from the fresh pool
};

// Decode launch shape (dkv_plan.cpp): workgroups per tier and KV head and the
// item-length rules; host_tier / dev_tier say which tiers can hold tokens and
// host_frac the expected host share of them.  No sequence lengths involved.
DecodeTemplate decode_template(const PlanInput& in, bool host_tier, bool dev_tier, double host_frac);

// Host twin of decode_tiers_kernel for one sequence (plan introspection):
// the logical pages of each tier in order (the kernel lists their physical
// pages) and the tokens each tier holds among the first `attended`; false when
// an entry was left out.
bool decode_tiers_host(const PlanInput& in, int64_t b, int64_t attended, std::vector<int32_t>* host_pages,
                       std::vector<int32_t>* dev_pages, int64_t* nh, int64_t* nd);

// Every item of a call in queue order (host items, HBM items, HBM tail items)
// and the split offsets [B+1], from each sequence's tier tokens.
struct DecodeHostItem {
  int32_t host;   // 1 host tier, 0 HBM
  int32_t b;
  int32_t slot;
  int32_t n_tok;
  int64_t k0;     // first ordinal in the tier
};
void decode_enumerate(const DecodeTemplate& t, int B, const int64_t* nh, const int64_t* nd,
                      std::vector<DecodeHostItem>* items, std::vector<int32_t>* offsets, DecodeSizes* z);

// Prefill plan: query rows of sequence b are q_start[b] .. q_start[b+1]-1,
// row j of b at position q_pos0[b] + j; in.seq_lens are the cached lengths.
// Device image: host items, dev/staged items, page pairs, stage tiles, row
// positions [T], split offsets [T+1], counters.
bool build_prefill_plan(const PlanInput& in, const int32_t* q_start, const int32_t* q_pos0,
                        PlanLayout* out, std::vector<uint8_t>* blob, std::string* err);

// Offloaded-linear shape (in.ratio, tuning fields and num_cus used), and its
// items in kernel order (for introspection).
bool linear_shape(const PlanInput& in, int32_t N, int32_t K, LinearShape* out, std::string* err);
void linear_items(const LinearShape& z, int32_t N, int32_t K, std::vector<LinearItem>* items);

// Sets the calling thread's last-error message (dkv_last_error) and returns
// st; success() clears it and returns DKV_OK.
dkv_status error(dkv_status st, const char* msg);
dkv_status success();

}  // namespace dkv
