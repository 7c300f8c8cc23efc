// dkv_internal.h - structures shared by the host runtime (C++) and the gfx950
// kernels (HIP).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "dkv.h"

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

// One work item: a run of tokens of one sequence that all live in one tier.
// The attention kernel processes every item once per KV head ("unit").
struct PlanItem {
  int32_t b;      // sequence
  int32_t slot;   // split slot (row of part_o / part_lse)
  int32_t n_tok;  // tokens in the item (>= 1)
  int32_t plist;  // paged: index of the item's first entry in the page list
  int64_t row0;   // contiguous: pool row of the item's first token
  int64_t pad;
};
static_assert(sizeof(PlanItem) == 32, "PlanItem layout");

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
struct LinearBlock {  // partial slots base .. base + n_splits - 1 of rows row0 ..
  int32_t row0;
  int32_t n_rows;
  int32_t base;
  int32_t n_splits;
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

// Arguments of the split attention kernel.
struct AttnArgs {
  const PlanItem* host_items;
  const PlanItem* dev_items;
  const int32_t* plist;          // paged: logical page indices
  const int32_t* plan_offsets;   // [batch+1] split offsets (in the workspace)
  int32_t* unit_counters;        // [2] dynamic unit counters (HBM, host), zero at launch
  int32_t* split_offsets;        // [batch+1] caller copy (written by block 0), or NULL
  int32_t n_host_units;          // host items x Hkv
  int32_t n_dev_units;           // dev items x Hkv
  int32_t host_wgs;
  int32_t dev_wgs;
  const uint16_t* host_k;
  const uint16_t* host_v;
  const uint16_t* dev_k;
  const uint16_t* dev_v;
  int64_t host_rows;
  int64_t dev_rows;
  const int32_t* page_table;
  int32_t max_pages;
  int32_t page_shift;            // log2(page_size) (paged)
  const uint16_t* q;             // [batch][Hq][D]
  const int32_t* q_pos;          // [batch]
  int32_t batch;
  int32_t hq;
  int32_t hkv;
  int32_t head_dim;
  float scale_log2;              // scale * log2(e)
  float pad0;
  double theta;
  float* part_o;                 // [S][Hq][D]
  float* part_lse;               // [S][Hq]
  uint64_t* wg_trace;            // optional [grid][4]: start, end, role, units (wall clock)
  int32_t wg_trace_cap;
  int32_t pad1;
  RopeFreq freq;                 // f_i = theta^(-2i/D), i < D/2
};

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
  const LinearItem* host_items;
  const LinearItem* dev_items;
  int32_t* counters;             // [2], zero at launch
  int32_t n_host_items;
  int32_t n_dev_items;
  int32_t host_wgs;
  int32_t dev_wgs;
  int32_t m;                     // tokens in this launch (<= kLinMaxTokens)
  int32_t n;                     // out_features
  int32_t k;                     // in_features
  int32_t n_host;                // rows of W in host memory
  const uint16_t* host_w;        // [n_host][K]
  const uint16_t* dev_w;         // [N - n_host][K]
  const uint16_t* x;             // [m][K]
  float* y;                      // [m][N]
  float* part;                   // [S][kLinMaxTokens][kLinRows]
  const LinearBlock* blocks;
  int32_t n_blocks;
  int32_t pad;
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
int launch_attn(const AttnArgs& a, void* stream);
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
int launch_probe_read(const void* src, size_t bytes, int nwg, int nontemporal, float* sink,
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

// Builds the plan and its device image; on failure returns false with `err`.
bool build_plan(const PlanInput& in, PlanLayout* out, std::vector<uint8_t>* blob,
                std::string* err);

// Prefill plan: query rows of sequence b are q_start[b] .. q_start[b+1]-1,
// row j of b at position q_pos0[b] + j; in.seq_lens are the cached lengths.
// Device image: host items, dev/staged items, page pairs, stage tiles, row
// positions [T], split offsets [T+1], counters.
bool build_prefill_plan(const PlanInput& in, const int32_t* q_start, const int32_t* q_pos0,
                        PlanLayout* out, std::vector<uint8_t>* blob, std::string* err);

// Offloaded-linear plan (in.ratio, tuning fields and num_cus used).  Device
// image: host items, dev items, row blocks (n_plist of them at plist_off),
// counters.
bool build_linear_plan(const PlanInput& in, int32_t M, int32_t N, int32_t K, PlanLayout* out,
                       std::vector<uint8_t>* blob, std::string* err);

// Sets the calling thread's last-error message (dkv_last_error) and returns
// st; success() clears it and returns DKV_OK.
dkv_status error(dkv_status st, const char* msg);
dkv_status success();

}  // namespace dkv
