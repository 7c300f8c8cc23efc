/*
 * dkv.h - C ABI of libdkv: single-token decode attention over a KV cache that
 * lives mostly in host-pinned memory, read by the GPU in place (zero-copy),
 * for AMD Instinct MI355X (gfx950).
 *
 * What the operations are (page titles and sections of the method's pages):
 *   - DirectKV README, introduction: the KV cache sits in CPU-pinned memory
 *     instead of GPU HBM; one kernel fuses K/V projection, Neox RoPE and
 *     multi-head attention, loading KV straight from the pinned buffers.
 *   - DirectKV README, Attribution: FlashAttention-style online softmax,
 *     extended from GPU-resident KV to KV streamed from CPU memory with no
 *     staging copy in a GPU buffer.
 *   - SplitKernel README, Overview and Key Features: kernels read offloaded
 *     data directly from the remote tier into on-chip memory, and attention
 *     runs over a KV cache partitioned between host and device memory.
 *   - SplitKernel README, Usage: placement and offloading-ratio utilities.
 *
 * Conventions shared by every call:
 *   - Every function returns dkv_status.  On failure dkv_last_error() gives a
 *     message for the calling thread.  Nothing is launched when validation
 *     fails; no exception crosses the ABI.
 *   - "device" pointers are GPU-visible addresses: HBM allocations or the
 *     device address of a mapped host-pinned block (dkv_host_alloc).  "host"
 *     pointers are ordinary CPU memory read during the call.
 *   - bf16 tensors are raw 16-bit bfloat16 patterns.  A KV pool row is one
 *     token: [num_kv_heads][head_dim] bf16, K and V in separate pools.
 *   - Work is enqueued on `stream` (a hipStream_t, NULL = default stream) and
 *     runs asynchronously.  The caller owns every buffer and keeps it alive
 *     until the stream has passed the call.
 *   - The caller's current HIP device must be the device owning the buffers.
 */
#ifndef DKV_H
#define DKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dkv_status {
  DKV_OK = 0,
  DKV_ERR_INVALID = 1,     /* bad argument: null pointer, size, range, layout */
  DKV_ERR_UNSUPPORTED = 2, /* valid but not built: head_dim, group size, ... */
  DKV_ERR_NOMEM = 3,       /* a host-pinned or library allocation failed */
  DKV_ERR_HIP = 4          /* a HIP runtime call failed (message has the text) */
} dkv_status;

/* Message describing the last failure on this thread ("" if none). */
const char* dkv_last_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int32_t dkv_version(void);

/* ------------------------------------------------------------------------
 * KV cache description.
 *
 * Two placements (SplitKernel README, Key Features: host/device KV split):
 *
 *  page_size == 0, contiguous split.  Sequence b holds L_b tokens; its oldest
 *    n_host_b = floor(r * L_b) tokens (IEEE double product, r = offload ratio)
 *    are in the host pools at rows b*host_stride + t, the rest in the device
 *    pools at rows b*dev_stride + (t - n_host_b).  This describes a cache of
 *    fixed length; use the paged placement for caches that grow.
 *
 *  page_size > 0 (a power of two), paged.  page_table[b*max_pages + t/page]
 *    = phys << 1 | tier (tier 1 = host pools, 0 = device pools) and the row
 *    is phys*page_size + t % page_size.  page_table lives in device memory
 *    and is what every kernel reads; page_table_host, an identical host copy,
 *    is needed only by the prefill planners and by plan introspection (decode
 *    calls derive their work from the device copy).
 *
 *  host_k/host_v are device addresses of host-pinned memory (zero-copy);
 *  dev_k/dev_v are HBM.  host_rows / dev_rows are the pool capacities in rows
 *  and bound every access.  Either tier may be NULL with 0 rows when no token
 *  lives there.
 * ---------------------------------------------------------------------- */
typedef struct dkv_kv_desc {
  int32_t num_kv_heads;   /* Hkv >= 1 */
  int32_t head_dim;       /* D: 64 or 128 */
  int32_t page_size;      /* 0 = contiguous split, else power of two <= 1024 */
  int32_t max_pages;      /* paged: row stride of page_table */
  int64_t host_stride;    /* contiguous: host rows reserved per sequence */
  int64_t dev_stride;     /* contiguous: device rows reserved per sequence */
  int64_t host_rows;      /* capacity of host_k / host_v in rows */
  int64_t dev_rows;       /* capacity of dev_k / dev_v in rows */
  void* host_k;           /* device address of host-pinned K pool, bf16 */
  void* host_v;           /* device address of host-pinned V pool, bf16 */
  void* dev_k;            /* HBM K pool, bf16 */
  void* dev_v;            /* HBM V pool, bf16 */
  const int32_t* page_table;      /* device [B][max_pages] (paged only) */
  const int32_t* page_table_host; /* host [B][max_pages] copy (paged only) */
} dkv_kv_desc;

/* floor(ratio * length) in IEEE double: the number of host-resident tokens of
 * a contiguous-split sequence (SplitKernel README, Usage: offloading ratio).
 * ratio must be in [0, 1] and length >= 0. */
dkv_status dkv_split_point(double ratio, int64_t length, int64_t* n_host);

/* ------------------------------------------------------------------------
 * Fused projection + Neox RoPE + append of new tokens into the cache.
 * (DirectKV README, introduction: the fused kernel projects K/V, rotates K
 *  with Neox RoPE; Step 6 checks the new K and V after projection.)
 *
 * For each new token i (0 <= i < n_new), in sequence b = seq_idx[i] at
 * position p = pos[i]:
 *   projection mode (x != NULL):  k = x[i] . Wk, v = x[i] . Wv, accumulated
 *     in fp32; x is [n_new][hidden] bf16, Wk/Wv are [hidden][Hkv*D] bf16
 *     row-major with output column h*D + d; no bias.
 *   no-projection mode (x == NULL): k = k_new[i], v = v_new[i], both
 *     [n_new][Hkv][D] bf16.
 *   Then every head of k is rotated by rotate-half RoPE at position p,
 *   f_j = rope_theta^(-2j/D), angle and rotation in fp64, and written to the
 *   slot of (b, p) as bf16 rounded to nearest even; v is written unrotated.
 *
 * seq_idx, pos: device int32 [n_new].  Contiguous placement also needs
 * seq_lens (device int32 [batch], the lengths L_b that fix the split point
 * floor(offload_ratio * L_b)); paged placement ignores seq_lens and the ratio.
 * Tokens whose slot falls outside the layout (b outside [0,batch), p < 0,
 * page index >= max_pages, negative page entry, row beyond the pool) are
 * skipped: nothing is written for them.  Set DKV_DEBUG_VALIDATE=1 to have
 * such tokens reported as DKV_ERR_INVALID instead (synchronous host check).
 *
 * workspace: device scratch of at least dkv_append_workspace_bytes(n_new,
 * hidden, Hkv*D) bytes when x != NULL (may be NULL otherwise).  Calls that
 * share a workspace on different streams race.
 * ---------------------------------------------------------------------- */
size_t dkv_append_workspace_bytes(int32_t n_new, int32_t hidden, int32_t kv_dim);

dkv_status dkv_project_rope_append(const dkv_kv_desc* kv, int32_t batch,
                                   const int32_t* seq_lens, double offload_ratio,
                                   int32_t n_new, const int32_t* seq_idx, const int32_t* pos,
                                   const void* x, int32_t hidden, const void* wk, const void* wv,
                                   const void* k_new, const void* v_new, double rope_theta,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Split decode attention (DirectKV README, introduction and Attribution;
 * SplitKernel README, Key Features).
 *
 * One query token per sequence: q [batch][Hq][D] bf16 (device), rotated
 * in-kernel by Neox RoPE at q_pos[b] (device int32 [batch]).  Query head h
 * reads KV head h / (Hq/Hkv).  Sequence b attends to its first seq_lens[b]
 * cached tokens (device int32 [batch], each >= 0; keys already rotated by the
 * append):
 *   s_t = scale * q_rot . k_t,  o = sum_t softmax(s)_t v_t,  lse = ln sum_t e^s_t.
 *
 * No host planning per call: the kernel reads seq_lens (and, paged, the page
 * table) in device memory and cuts each sequence's tokens into work items
 * that each lie in one tier; the two tiers run at the same time on disjoint
 * sets of workgroups, each taking (item, KV head) units of its tier from a
 * queue in the workspace.  Every (item, KV head) writes a
 * normalised partial (part_o [S][Hq][D] fp32, part_lse [S][Hq] fp32, natural
 * log) in the split slots of its sequence, and split_offsets (device int32
 * [batch+1]) receives the CSR bounds: sequence b owns splits
 * [split_offsets[b], split_offsets[b+1]) (empty for seq_lens[b] = 0).
 * dkv_merge_lse turns the partials into the final output.
 *
 * dkv_decode_plan gives, for the call's shape (not its lengths), the
 * workspace size and S, the most splits any lengths that fit the pools can
 * produce: part_o / part_lse must hold num_splits_cap >= S splits.  With
 * seq_lens (host int32 [batch], optional) it also reports the items, item
 * lengths and bytes per tier those lengths give.
 *
 * Workspace (device memory, 256-byte aligned): zero-filled before its first
 * use; every call leaves its counters at zero again, so calls of the same
 * shape (descriptor, batch, heads, ratio) reuse it as is.  Where the counters
 * lie depends on the shape: zero it again before a call of another shape.
 * Calls that share a workspace must not overlap (they race).  The call
 * allocates nothing and never synchronises, so it may be captured into a HIP
 * graph: each replay reads the lengths and positions present in device
 * memory at that time, so one graph serves a cache that grows.
 *
 * Sequences whose rows fall outside the layout (contiguous: beyond host_stride,
 * dev_stride or a pool; paged: negative or out-of-pool page entries, more pages
 * than max_pages) are not read and set a flag that dkv_decode_errors reports;
 * DKV_DEBUG_VALIDATE=1 checks them on the host before launching instead
 * (synchronous).
 * ---------------------------------------------------------------------- */
typedef struct dkv_plan_info {
  int64_t workspace_bytes; /* device workspace the call needs */
  int32_t num_splits;      /* decode: split bound S (step: partial slots in the
                              workspace, S plus one per sequence); prefill: splits
                              of the plan */
  int32_t host_items;      /* work items in the host tier (per KV head) */
  int32_t dev_items;       /* work items in the HBM tier (per KV head) */
  int32_t host_wgs;        /* workgroups streaming the host tier */
  int32_t dev_wgs;         /* workgroups streaming the HBM tier */
  int32_t host_chunk;      /* tokens per host work item */
  int32_t dev_chunk;       /* tokens per HBM work item */
  int64_t host_bytes;      /* K+V bytes read from host memory per call */
  int64_t dev_bytes;       /* K+V bytes read from HBM per call */
  int64_t staged_bytes;    /* prefill: host K+V bytes copied once into HBM and
                              read from there (included in host_bytes; their
                              re-reads are in dev_bytes); 0 for decode */
} dkv_plan_info;

dkv_status dkv_decode_plan(const dkv_kv_desc* kv, int32_t batch, int32_t num_q_heads,
                           const int32_t* seq_lens, double offload_ratio, dkv_plan_info* info);

dkv_status dkv_decode_attn_split(const dkv_kv_desc* kv, int32_t batch, int32_t num_q_heads,
                                 const void* q, const int32_t* q_pos, const int32_t* seq_lens,
                                 double offload_ratio, float scale, double rope_theta,
                                 void* workspace, size_t workspace_bytes,
                                 float* part_o, float* part_lse, int32_t* split_offsets,
                                 int32_t num_splits_cap, void* stream);

/* Plan introspection with no GPU work: the items the decode kernel derives
 * for these host lengths (seq_lens host int32 [batch]) when planned for
 * `num_cus` compute units (0: tuning or current device).  items receives up
 * to items_cap rows of 5 int64 values (tier [1 host, 0 HBM], b, slot, n_tok,
 * first) in queue order (host items first) where `first` is the pool row of
 * the item's first token (contiguous) or its index into page_list (paged);
 * page_list receives up to page_cap logical page indices; split_offsets
 * receives batch+1 values.  Any output pointer may be NULL.  info as for
 * dkv_decode_plan, with num_splits the exact count. */
dkv_status dkv_plan_inspect(const dkv_kv_desc* kv, int32_t batch, int32_t num_q_heads,
                            const int32_t* seq_lens, double offload_ratio, int32_t num_cus,
                            int64_t* items, int32_t items_cap, int32_t* page_list,
                            int32_t page_cap, int32_t* split_offsets, dkv_plan_info* info);

/* ------------------------------------------------------------------------
 * Fused decode step in one launch (DirectKV README, introduction: one kernel
 * projects the new token's K/V, rotates the key with Neox RoPE, appends it to
 * the CPU-resident cache and attends; Attribution: online softmax over KV
 * streamed from CPU memory).
 *
 * Sequence b holds seq_lens[b] cached tokens (device int32 [batch]).  When a
 * new token is given (k_new/v_new [batch][Hkv][D] bf16, or x [batch][hidden]
 * bf16 with wk/wv [hidden][Hkv*D] bf16 as in dkv_project_rope_append), it is
 * appended at position pos_new[b] (device int32 [batch]; NULL: seq_lens[b])
 * into its slot of a cache of seq_lens[b] + 1 tokens (contiguous: split point
 * floor(r * (seq_lens[b] + 1)); paged: the page table entry), with its key
 * rotated at that position in fp64 and rounded once to bf16, and the query
 * attends to the seq_lens[b] cached tokens plus the new one (read from
 * registers, as stored).  With no new token (k_new = v_new = x = NULL) the
 * query attends to the cached tokens only.  Work is cut and queued as in
 * dkv_decode_attn_split; the partials of each (sequence, KV head) are merged
 * by log-sum-exp inside the same launch, in groups of up to 16 (the last
 * workgroup to finish a group merges it, the last group merges the groups):
 * out_o [batch][Hq][D] fp32, out_lse [batch][Hq] fp32 (or NULL).  A sequence
 * with nothing to attend gets out_o = 0 and out_lse = -inf.
 *
 * One kernel launch (plus the paged layout's tier lists and, with x, the
 * projection).  Workspace from dkv_decode_step_plan (hidden = 0 without
 * projection), same rules as for dkv_decode_attn_split: zero before its first
 * use, left zeroed, no allocation, capturable, valid while lengths grow.
 * ---------------------------------------------------------------------- */
dkv_status dkv_decode_step_plan(const dkv_kv_desc* kv, int32_t batch, int32_t num_q_heads,
                                double offload_ratio, int32_t hidden, dkv_plan_info* info);

dkv_status dkv_decode_step(const dkv_kv_desc* kv, int32_t batch, int32_t num_q_heads, const void* q,
                           const int32_t* q_pos, const int32_t* seq_lens, const int32_t* pos_new,
                           const void* x, int32_t hidden, const void* wk, const void* wv,
                           const void* k_new, const void* v_new, double offload_ratio, float scale,
                           double rope_theta, void* workspace, size_t workspace_bytes, float* out_o,
                           float* out_lse, void* stream);

/* ------------------------------------------------------------------------
 * The fused decode step for callers that cannot allocate device memory
 * (code under graph capture that must not allocate, serving loops and
 * harnesses that forbid hipMalloc): dkv_decode_step with the library's own
 * scratch in place of the caller's workspace.  The scratch is a static device
 * array of DKV_STATIC_SCRATCH_BYTES on every GPU the library runs on (held
 * until the process ends); a shape whose workspace (dkv_decode_step_plan)
 * exceeds it is rejected with DKV_ERR_UNSUPPORTED.  The call allocates
 * nothing.  All calls on one GPU share the array: calls that overlap in time
 * on one GPU (different streams, or threads) race and must not be issued.
 * dkv_decode_errors reads its flags with the array's address, which this
 * ABI does not expose; DKV_DEBUG_VALIDATE checks layouts on the host instead.
 * ---------------------------------------------------------------------- */
#define DKV_STATIC_SCRATCH_BYTES (64u << 20)

dkv_status dkv_decode_step_static(const dkv_kv_desc* kv, int32_t batch, int32_t num_q_heads, const void* q,
                                  const int32_t* q_pos, const int32_t* seq_lens, const int32_t* pos_new,
                                  const void* x, int32_t hidden, const void* wk, const void* wv,
                                  const void* k_new, const void* v_new, double offload_ratio, float scale,
                                  double rope_theta, float* out_o, float* out_lse, void* stream);

/* Layout errors the decode kernels flagged in this workspace since it was
 * last cleared (bit 1: contiguous rows beyond a stride or pool, 2: page entry
 * unmapped or beyond its pool, 4: appended token without a slot, 8: partial
 * slots exhausted).  Synchronises the device; clear != 0 resets the flags. */
#define DKV_DECODE_ERR_LAYOUT 1
#define DKV_DECODE_ERR_PAGE 2
#define DKV_DECODE_ERR_SLOT 4
#define DKV_DECODE_ERR_CAPACITY 8
dkv_status dkv_decode_errors(const dkv_kv_desc* kv, const void* workspace, int32_t clear, int32_t* flags);

/* ------------------------------------------------------------------------
 * Causal prefill attention over the split cache (DirectKV README,
 * introduction: one kernel projects, rotates and attends; Step 6:
 * "Prefill (all new KV)" correctness cases).
 *
 * New query rows are grouped per sequence: rows q_start[b] .. q_start[b+1]-1
 * (host int32 [batch+1], q_start[0] = 0) belong to sequence b, and row j of b
 * sits at position q_pos0[b] + j (host int32 [batch]).  Their keys and
 * values must already be in the cache (dkv_project_rope_append with the
 * same positions); seq_lens (host int32 [batch]) are the cached lengths and
 * must cover every query position.  Each row is rotated by Neox RoPE at its
 * position and attends to tokens 0 .. its position (causal):
 *   s_t = scale * q_rot . k_t (t <= p),  o = softmax(s) V,  lse = ln sum e^s.
 * q is [T][Hq][D] bf16 (device, 16-byte aligned), T = q_start[batch].
 *
 * Output is split like dkv_decode_attn_split: the rows of a block of 128/G
 * consecutive rows share runs of cached tokens, one per tier and chunk;
 * each (row, run) writes a normalised partial, and split_offsets (device
 * int32 [T+1]) gives each row's CSR range of splits.  dkv_merge_lse with
 * batch = T then yields o [T][Hq][D] and lse [T][Hq].  dkv_prefill_plan gives
 * the split count and workspace size.  Q.K^T and P.V run on MFMA.
 *
 * Host-tier rows that two or more row blocks of a sequence read are first
 * copied once into an HBM staging pool inside the workspace (one read over
 * the host link instead of one per block), within the staging budget of
 * dkv_tuning.stage_max_mib; the workspace size includes that pool.
 *
 * Plans are built on the host from the call's host arrays and cached per
 * shape (up to 64, least recently used dropped first) as images in pinned
 * host memory; each call copies its image into the workspace on its stream.
 * An image is freed when dropped and no call holds it, after a device
 * synchronisation (uploads from it may still be queued).  A plan uploaded
 * while the stream is capturing a graph is kept, whatever the cache's size,
 * because the graph's copy reads that image on every replay.
 * ---------------------------------------------------------------------- */
dkv_status dkv_prefill_plan(const dkv_kv_desc* kv, int32_t batch, int32_t num_q_heads,
                            const int32_t* q_start, const int32_t* q_pos0, const int32_t* seq_lens,
                            double offload_ratio, dkv_plan_info* info);

/* Prefill plan cache.  dkv_plan_cache_release_captured: the caller has
 * destroyed every graph that captured a prefill call, so their plans are kept
 * no longer; the cache drops entries down to its capacity (freeing their
 * images as above) and treats them like any other from now on.  Replaying a
 * graph that captured a prefill call after this call is undefined.
 * dkv_plan_cache_stats: entries in the cache, how many of them a captured
 * graph holds, and their pinned bytes (host pointers, all required). */
dkv_status dkv_plan_cache_release_captured(void);
dkv_status dkv_plan_cache_stats(int32_t* entries, int32_t* captured, int64_t* pinned_bytes);

/* Prefill planner introspection (no HIP calls; used by CPU tests): the plan
 * dkv_prefill_plan (fused = 0) or dkv_prefill_fused_plan (fused = 1) would
 * build for num_cus compute units.  Per item, 11 int64 into items: pool (0
 * host, 1 HBM, 2 HBM staging copy of host rows, 3 the fused step's new rows),
 * sequence, first query row, rows, first row's position, tokens, first
 * (contiguous layout or pool 3: pool row of the first token; paged: index of
 * the first page pair), logical position of the first token, split index,
 * splits of the block, first split slot.  pages: (logical page, pool page)
 * pairs of paged items.  tiles: 3 int64 per staging copy (host row, staging
 * row, rows).  split_offsets: [T+1].  Arrays are filled up to their caps;
 * info gives the counts (host_items + dev_items items). */
dkv_status dkv_prefill_plan_inspect(const dkv_kv_desc* kv, int32_t batch, int32_t num_q_heads,
                                    const int32_t* q_start, const int32_t* q_pos0, const int32_t* seq_lens,
                                    double offload_ratio, int32_t fused, int32_t num_cus, int64_t* items, int32_t items_cap,
                                    int32_t* pages, int32_t pages_cap, int64_t* tiles, int32_t tiles_cap,
                                    int32_t* split_offsets, int32_t offsets_cap, dkv_plan_info* info);

dkv_status dkv_prefill_attn_split(const dkv_kv_desc* kv, int32_t batch, int32_t num_q_heads,
                                  const void* q, const int32_t* q_start, const int32_t* q_pos0,
                                  const int32_t* seq_lens, double offload_ratio, float scale,
                                  double rope_theta, void* workspace, size_t workspace_bytes,
                                  float* part_o, float* part_lse, int32_t* split_offsets,
                                  int32_t num_splits_cap, void* stream);

/* ------------------------------------------------------------------------
 * Fused prefill step (DirectKV README, introduction: one kernel projects the
 * new tokens' K/V, rotates them, appends them to the CPU-resident cache and
 * attends; Step 6, "Prefill (all new KV)").
 *
 * Rows q_start[b] .. q_start[b+1]-1 of q are new tokens of sequence b at
 * positions q_pos0[b] + j (host arrays as for dkv_prefill_attn_split;
 * seq_lens are the lengths including the new tokens).  Their K/V come from
 * k_new/v_new ([T][Hkv][D] bf16) or from x [T][hidden] times wk/wv as in
 * dkv_project_rope_append.  The call appends them to their cache slots (host
 * or HBM), keeps a second copy of the new rows in the workspace, and attends
 * causally: cached tokens below q_pos0[b] come from the tiers (staged into HBM
 * when several row blocks re-read host rows), the new rows from the copy.
 * Output: out_o [T][Hq][D] fp32, out_lse [T][Hq] fp32 (or NULL).  Workspace
 * size from dkv_prefill_fused_plan (hidden = 0 without projection).  With
 * T = 0 the call does nothing (and needs no buffers).
 * ---------------------------------------------------------------------- */
dkv_status dkv_prefill_fused_plan(const dkv_kv_desc* kv, int32_t batch, int32_t num_q_heads,
                                  const int32_t* q_start, const int32_t* q_pos0, const int32_t* seq_lens,
                                  double offload_ratio, int32_t hidden, dkv_plan_info* info);

dkv_status dkv_prefill_fused(const dkv_kv_desc* kv, int32_t batch, int32_t num_q_heads, const void* q,
                             const int32_t* q_start, const int32_t* q_pos0, const int32_t* seq_lens,
                             double offload_ratio, float scale, double rope_theta, const void* x,
                             int32_t hidden, const void* wk, const void* wv, const void* k_new,
                             const void* v_new, void* workspace, size_t workspace_bytes, float* out_o,
                             float* out_lse, void* stream);

/* ------------------------------------------------------------------------
 * Offloaded linear layer read in place from both tiers (SplitKernel README,
 * Overview and Key Features: GPU kernels fetch offloaded weights directly from
 * the remote tier; an offloaded linear primitive).
 *
 *   y[i][n] = sum_k x[i][k] * W[n][k],  i < m, n < out_features, k < in_features
 *
 * W is [out_features][in_features] bf16 (a PyTorch linear weight), split by
 * output rows with the KV rule: rows [0, n_host), n_host = floor(r * N) in IEEE
 * double, are host_w (mapped host memory, its device address; row-major
 * [n_host][K]); rows [n_host, N) are dev_w (HBM, [N - n_host][K]).  Either may
 * be NULL when it holds no rows.  x [m][K] bf16 and y [m][N] fp32 are device
 * memory; no bias; fp32 accumulation on MFMA.  in_features must be a multiple
 * of 8; x and the weights 16-byte aligned.  Both tiers stream at once, each on
 * its own workgroups; tokens run in launches of up to 64.  There is no host
 * plan: the kernel derives its items (row blocks of 64 rows x K ranges) from
 * the call's shape, and when K is split the last range of a row block to
 * finish sums the block's partials in the same launch.  dkv_linear_plan gives
 * the workspace size (counters plus K-split partials).  The workspace must be
 * zero-filled before its first use; every call leaves its counters at zero,
 * so a call needs no upload and can be captured in a graph.  Calls sharing a
 * workspace must not overlap.
 * ---------------------------------------------------------------------- */
dkv_status dkv_linear_plan(int32_t m, int32_t out_features, int32_t in_features, double offload_ratio,
                           dkv_plan_info* info);

dkv_status dkv_linear_split(const void* host_w, const void* dev_w, int32_t out_features, int32_t in_features,
                            double offload_ratio, const void* x, int32_t m, float* y, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Linear planner introspection (no HIP calls; used by CPU tests): 6 int32 per
 * item: pool (0 host, 1 HBM), first output row, rows, k0, k1, partial slot
 * (-1: written to y directly).  info as for dkv_linear_plan. */
dkv_status dkv_linear_plan_inspect(int32_t out_features, int32_t in_features, double offload_ratio,
                                   int32_t num_cus, int32_t* items, int32_t items_cap, dkv_plan_info* info);

/* ------------------------------------------------------------------------
 * Staged-prefetch decode: the conventional design the zero-copy path is
 * measured against (SplitKernel README, Overview: prefetching offloaded data
 * into GPU memory costs extra HBM traffic and capacity, pipeline bubbles and
 * unused aggregate bandwidth).  For one sequence (batch 1) of seq_len tokens
 * in the contiguous-split layout, the host tier's floor(r * seq_len) tokens
 * are copied by the DMA engine (hipMemcpyAsync on a library copy stream,
 * created once per device at default priority) in chunks of chunk_tokens
 * rows into a two-slot HBM ring in the workspace; each staged chunk is
 * attended from HBM by one launch of the fused decode kernel (no new token)
 * while the next one is copied, the HBM tier alongside, and the per-chunk
 * results are merged by log-sum-exp into out_o [Hq][D] / out_lse [Hq].
 * q [Hq][D] bf16 and q_pos [1] are device memory; the keys in the cache are
 * already rotated.  dkv_decode_staged_plan gives the workspace size (the
 * per-chunk decode scratch, the ring, the partials), staged_bytes the bytes
 * copied into HBM and host_items the chunk count.  The workspace must be
 * zero-filled before its first use (left zeroed).  Calls must not overlap.
 * ---------------------------------------------------------------------- */
dkv_status dkv_decode_staged_plan(const dkv_kv_desc* kv, int32_t num_q_heads, int64_t seq_len,
                                  double offload_ratio, int32_t chunk_tokens, dkv_plan_info* info);

dkv_status dkv_decode_staged(const dkv_kv_desc* kv, int32_t num_q_heads, const void* q, const int32_t* q_pos,
                             int64_t seq_len, double offload_ratio, float scale, double rope_theta,
                             int32_t chunk_tokens, void* workspace, size_t workspace_bytes, float* out_o,
                             float* out_lse, void* stream);

/* ------------------------------------------------------------------------
 * LSE merge of partial results (the combine step implied by splitting one
 * sequence's KV over tiers and compute units: SplitKernel README, Key
 * Features; DirectKV README, Step 6, "SM-Parallel" kernel).
 *
 * For each (b, h): M = max_i lse_i over splits i in [split_offsets[b],
 * split_offsets[b+1]), w_i = exp(lse_i - M), out_o = sum w_i o_i / sum w_i,
 * out_lse = M + ln sum w_i.  Splits with lse = -inf weigh 0; a sequence with
 * no finite split gets out_o = 0, out_lse = -inf.  All device pointers;
 * out_lse may be NULL.  head_dim is 64 or 128.
 * ---------------------------------------------------------------------- */
dkv_status dkv_merge_lse(const float* part_o, const float* part_lse, const int32_t* split_offsets,
                         int32_t batch, int32_t num_q_heads, int32_t head_dim,
                         float* out_o, float* out_lse, void* stream);

/* ------------------------------------------------------------------------
 * Paged KV allocator (DirectKV README, introduction: the KV pool kept in
 * CPU-pinned memory; SplitKernel README, Overview: a cache split between
 * host and device memory by an offload ratio).
 *
 * Host-side bookkeeping for the paged layout of dkv_kv_desc: a host pool of
 * n_host_pages pages and an HBM pool of n_dev_pages pages (page_size rows
 * each, the caller allocates the pools), one LIFO free list per pool, and the
 * page table [max_seqs][max_pages] (entry phys << 1 | tier, tier 1 = host;
 * -1 = unused) that dkv_kv_desc.page_table(_host) describe.  No GPU calls:
 * the caller copies the table (dkv_pager_table) to its device copy after a
 * change and before kernels read it.
 *
 * Placement: logical page j of a sequence goes to the host pool iff
 * floor(f*(j+1)) > floor(f*j), f = host_fraction in [0, 1], so that exactly
 * floor(f*n) of its first n pages are host-resident at every length n.  If
 * the chosen pool is empty the page goes to the other pool (counted in
 * spilled_pages).
 *
 * dkv_pager_reserve(seq, n_tokens) gives sequence seq pages for tokens
 * [0, n_tokens) (never shrinks); it is all-or-nothing: with too few free
 * pages in both pools it changes nothing and returns DKV_ERR_NOMEM, and
 * n_tokens beyond max_pages*page_size returns DKV_ERR_INVALID.
 * dkv_pager_release(seq) returns all of seq's pages to their pools.  The
 * pointer from dkv_pager_table stays valid until dkv_pager_destroy.  Calls on
 * one pager must not overlap; distinct pagers are independent.
 * ---------------------------------------------------------------------- */
typedef struct dkv_pager dkv_pager;

typedef struct dkv_pager_stats {
  int32_t free_host_pages;
  int32_t free_dev_pages;
  int32_t used_host_pages;
  int32_t used_dev_pages;
  int32_t spilled_pages;  /* pages placed in the other pool since creation */
  int32_t reserved;
} dkv_pager_stats;

dkv_status dkv_pager_create(int32_t n_host_pages, int32_t n_dev_pages, int32_t page_size,
                            int32_t max_seqs, int32_t max_pages, double host_fraction, dkv_pager** out);
dkv_status dkv_pager_destroy(dkv_pager* pager);
dkv_status dkv_pager_reserve(dkv_pager* pager, int32_t seq, int64_t n_tokens);
dkv_status dkv_pager_release(dkv_pager* pager, int32_t seq);
/* *table: [max_seqs][max_pages] int32; *pages_of_seq (may be NULL): [max_seqs] */
dkv_status dkv_pager_table(const dkv_pager* pager, const int32_t** table, const int32_t** pages_of_seq);
dkv_status dkv_pager_stats_get(const dkv_pager* pager, dkv_pager_stats* stats);

/* ------------------------------------------------------------------------
 * Host-pinned memory for the host tier (DirectKV README, introduction:
 * CPU-pinned KV pool).  Allocates `bytes` of page-locked host memory mapped
 * into the GPU's address space; *host_ptr is the CPU address, *dev_ptr the
 * address kernels use.  flags: DKV_HOST_COHERENT (fine-grained, default) or
 * DKV_HOST_NONCOHERENT (coarse-grained; GPU caches may hold lines during a
 * kernel).  dkv_host_free(host_ptr) waits for all queued work on the
 * current device, then releases the block.
 * ---------------------------------------------------------------------- */
#define DKV_HOST_COHERENT 0u
#define DKV_HOST_NONCOHERENT 1u

dkv_status dkv_host_alloc(size_t bytes, uint32_t flags, void** host_ptr, void** dev_ptr);
dkv_status dkv_host_free(void* host_ptr);

/* ------------------------------------------------------------------------
 * Planner tuning (SplitKernel README, Requirements: the build fixes the SM
 * count and buffer slots; here they are run-time values).  Zero fields take
 * the library defaults; host_bw_gbs / dev_bw_gbs weigh the split of
 * workgroups between tiers.  Applies process-wide to later plans.
 * ---------------------------------------------------------------------- */
typedef struct dkv_tuning {
  int32_t num_cus;       /* compute units to plan for (0: the current device) */
  int32_t host_wgs;      /* workgroups for the host tier (0: default) */
  int32_t dev_wgs;       /* workgroups for the HBM tier (0: default) */
  int32_t host_chunk;    /* tokens per host work item, multiple of 64 (0: auto) */
  int32_t dev_chunk;     /* tokens per HBM work item, multiple of 64 (0: auto) */
  int32_t stage_max_mib;  /* prefill: HBM staging budget in MiB (0: 4096, < 0: never stage) */
  double host_bw_gbs;    /* host-link read bandwidth (0: 57) */
  double dev_bw_gbs;     /* HBM read bandwidth (0: 5300) */
  int32_t writer_wgs;    /* fused prefill: workgroups writing the new rows into
                            their cache slots (0: auto) */
  int32_t reserved;      /* must be 0 */
} dkv_tuning;

dkv_status dkv_set_tuning(const dkv_tuning* tuning); /* NULL restores defaults */
dkv_status dkv_get_tuning(dkv_tuning* tuning);

/* ------------------------------------------------------------------------
 * Bandwidth probe: reads `bytes` of memory with a streaming kernel (16 B per
 * lane, coalesced, 8 loads in flight per thread) and reports the best of
 * `iters` timed passes (1..1000), each bracketed by its own HIP events.  src
 * is a device address (HBM or mapped host memory), nwg the number of
 * workgroups (<= 65535).  src2 (optional, NULL for one buffer): a second
 * buffer of `bytes` read at the same time by the odd workgroups (as the
 * attention kernel streams the K and V pools together); the rate counts both.
 * mode: bit 0 non-temporal loads; bit 1 blocked (each workgroup streams one
 * contiguous slice, as the attention kernel streams a work item) instead of
 * grid-stride; bit 2 segments (instead of bit 1: the buffer is rows of 2 KiB,
 * and each workgroup streams one 256-byte segment of every row of its slice,
 * as the attention kernel reads one KV head of the LLaMA-3-8B row; `bytes` a
 * multiple of 2 KiB, nwg a multiple of 8 per buffer).  Also the best host->device
 * hipMemcpyAsync rate of the same block when dma_dst is non-NULL (device
 * buffer of `bytes`).  Blocks until done.  Measurement helper: it allocates a
 * 256-byte sink and its events.
 * ---------------------------------------------------------------------- */
typedef struct dkv_bw_result {
  double read_gbs;   /* kernel read rate of the best pass */
  double read_ms;    /* kernel time of the best pass */
  double dma_gbs;    /* hipMemcpyAsync rate of the best pass (0 if not measured) */
} dkv_bw_result;

dkv_status dkv_probe_read(const void* src, const void* src2, size_t bytes, int32_t nwg, int32_t mode,
                          int32_t iters, void* dma_dst, const void* dma_src_host,
                          dkv_bw_result* out, void* stream);

/* ------------------------------------------------------------------------
 * Live kernel timing for measurement.  While enabled, every launch of the
 * named kernel is bracketed by a HIP event pair recorded on the stream the
 * kernel runs on.  dkv_kernel_timing_read waits for the recorded events,
 * returns how many launches were timed and their summed duration in ms, and
 * clears the record.  kernel: DKV_KERNEL_ATTN (split attention),
 * DKV_KERNEL_ROPE_Q (the two-call prefill's rotation table; decode rotates its
 * queries inside the attention kernel), DKV_KERNEL_MERGE, DKV_KERNEL_APPEND,
 * DKV_KERNEL_PREFILL (causal prefill attention), DKV_KERNEL_STAGE (prefill's
 * copy of re-read host rows into HBM), DKV_KERNEL_LINEAR (offloaded linear),
 * DKV_KERNEL_TIERS (the paged decode's per-tier page lists).
 * ---------------------------------------------------------------------- */
#define DKV_KERNEL_ATTN 0
#define DKV_KERNEL_ROPE_Q 1
#define DKV_KERNEL_MERGE 2
#define DKV_KERNEL_APPEND 3
#define DKV_KERNEL_PREFILL 4
#define DKV_KERNEL_STAGE 5
#define DKV_KERNEL_LINEAR 6
#define DKV_KERNEL_TIERS 7

dkv_status dkv_kernel_timing(int32_t enable);

/* Per-workgroup trace of the attention kernel, for measuring how the host and
 * HBM tiers overlap.  While set, every attention launch makes workgroup i
 * (i < capacity_wgs) write 4 uint64 values at dev_buffer[4*i]: start and end
 * of its work in wall-clock ticks (100 MHz), its role (1 host tier, 0 HBM)
 * and the number of work units it processed.  dev_buffer is device memory of
 * at least 32 * capacity_wgs bytes; capacity 0 (or NULL) turns tracing off. */
dkv_status dkv_attn_trace(void* dev_buffer, int32_t capacity_wgs);
dkv_status dkv_kernel_timing_read(int32_t kernel, int32_t* count, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* DKV_H */
