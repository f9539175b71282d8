// Internal layout shared by the host library and the gfx950 kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mlv {

constexpr int kLatent = 576;          // score columns of a latent KV row (512 latent + 64 rope)
constexpr int kVdim = 512;            // value columns (leading part of the same row)
constexpr int kRowBytes = kLatent * 2;
constexpr int kChunksPerRow = kRowBytes / 16;  // 72 sixteen-byte chunks per row
constexpr int kTileKeys = 32;          // keys per LDS tile
constexpr int kTileBytes = kTileKeys * kRowBytes;  // 36864
constexpr int kRowsPerWave = 32;       // query rows (head x node) held by one wave
constexpr int kWaves = 4;
constexpr int kRowsPerBlock = kRowsPerWave * kWaves;  // 128 rows per workgroup (M tile)
constexpr int kThreads = 64 * kWaves;
constexpr int kQReg = 24;                               // Q k-steps (16 columns each) kept in VGPRs
constexpr int kMergeBlocks = 2048;                     // merge grid target: rows x column split
constexpr int kTileBufs = 3;                           // KV tiles in LDS: tile t, t+1 (in use), t+2 (landing)
constexpr int kQLdsBytes = (36 - kQReg) * 64 * 16;      // per-wave LDS slice for the other k-steps
constexpr int kMaxTree = 256;          // tree nodes per request (one thread per node builds the masks)
constexpr int kMaxTreeWords = kMaxTree / 64;  // 64-bit ancestor-mask words per node
static_assert(kMaxTree <= 64 * 4, "the mask builder has one thread per node");
static_assert(kMaxTree * kMaxTreeWords * 8 + kMaxTree * 4 <= kTileBytes, "mask scratch fits one tile buffer");
constexpr int kMaxPage = 1024;         // largest prefix page (block-table) size in slots
constexpr int kMaxBatch = 1024;        // one plan thread per request
constexpr int kTargetBlocks = 256;     // workgroups the split aims for (one per CU on MI355X)
constexpr int kMinSplit = 128;         // shortest automatic prefix split, in tokens
constexpr int kFewRequests = 32;       // split search: candidate lengths in parallel up to this batch

// Device-side error bits (mirrors MLAVERIFY_DEVERR_* in the public header).
constexpr uint32_t kErrBadParent = 0x1u;
constexpr uint32_t kErrBadIndex = 0x2u;
constexpr uint32_t kErrBadPrefix = 0x4u;
constexpr uint32_t kErrConflict = 0x8u;   // a relocation destination is out of the pool or in use
constexpr uint32_t kErrBadTreeLen = 0x10u; // a per-request tree length outside [1, T]

struct PlanHeader {
  int32_t split_len;     // prefix tokens per split unit
  int32_t total_units;   // units in use by this run
  int32_t n_mtiles;      // 128-row tiles per request
  int32_t pad0;
  uint32_t sticky_err;   // OR of every data error since the last readback
  uint32_t clk_cycles;   // shader-clock cycles of workgroup 0's first wave over its run (0: not sampled)
  uint32_t clk_ticks;    // constant-rate wall-clock ticks over the same interval
  uint32_t rescales;     // waves that raised a softmax reference, since the last plan readback
  uint32_t pad1[56];     // header is 256 bytes
};
static_assert(sizeof(PlanHeader) == 256, "header size");

struct ReqPlan {
  int32_t key_off;      // start of the request's segment in kv_indices
  int32_t prefix_len;   // P_b after validation (0 when invalid)
  int32_t first_unit;   // global index of its first split unit
  int32_t units;        // number of split units (the last one also covers the tree)
  uint32_t err;         // prefix-length / tree-length error bits of this request
  int32_t tree_nodes;   // T_b (0 when a tree length at or before this request is invalid)
  int32_t node_off;     // first row (node) of the request in q / out / lse / tree_parent
  int32_t prow;         // first partial row of its unit 0; unit u's rows start at prow + u * H * T_b
};
static_assert(sizeof(ReqPlan) == 32, "ReqPlan size");

struct PartialArgs {
  const uint16_t* q;
  const uint16_t* pool;
  const int32_t* kv_indices;
  const int32_t* prefix_lens;
  const int32_t* tree_parent;
  const int32_t* tree_lens;  // [batch] per-request tree sizes T_b <= T, or null: every request has T
  PlanHeader* hdr;       // plan published by workgroup 0 (for the merge and readback)
  ReqPlan* req;
  uint16_t* part_o;      // [rows_cap, 512] unit-normalised partial outputs (bf16 bits), H * T_b rows per unit
  float* part_lse;       // [rows_cap] log2-domain lse of each partial row (NaN: poisoned)
  int32_t* unit_fast;    // [units] 1 if the unit's prefix was read as one contiguous run
  uint32_t* sticky_err;
  int64_t pool_slots;
  int64_t row_stride_bytes;
  int32_t batch, T, H, M, n_mtiles;  // T: the call's largest tree, M = H * T rows per unit
  int32_t max_prefix, split_fixed, target_units, min_split, units_cap;  // units_cap: entries of unit_fast
  int32_t rows_cap;      // rows of part_o / part_lse
  float scale_log2;      // sm_scale * log2(e), > 0
  uint32_t flags;
  int32_t page_log2;     // prefix pages of 2^page_log2 slots (0: one slot per token)
  int32_t max_page;      // largest valid page id, (pool_slots - 1) >> page_log2
  int32_t group_xcd;     // 1: the M tiles of a unit share an XCD; 0: M tiles round-robin
};

struct MergeArgs {
  const ReqPlan* req;
  const uint16_t* part_o;  // bf16 bits
  const float* part_lse;
  uint16_t* out;
  float* lse;
  int32_t batch, H, M;   // M = H * (the call's largest T): rows of a request in out / lse
  int32_t rows_cap;      // rows of part_o / part_lse
  int32_t ragged;        // 1: a tree size per request (its partial rows are packed, H * T_b per unit)
  int32_t units_hint;              // units of one request the plan is expected to make (sizes the merge's rounds)
};

// Tier-1 relocation of prefix rows (relocate.hip).
struct RelocArgs {
  char* pool;                  // [pool_slots, row_stride_bytes]
  int32_t* kv_indices;         // the batch's index segments (prefix slots rewritten)
  const int32_t* prefix_lens;  // [batch]
  const int32_t* dst_start;    // [batch] first destination slot, < 0: request not moved
  int32_t* off;                // [batch] segment offsets (workspace)
  uint32_t* maps;              // [map_words + use_words] (workspace): claimed destinations (one bit
                               // per slot), then slots in use (one byte per slot)
  uint32_t* status;            // refusal bits of this call (workspace)
  uint32_t* sticky_err;
  int64_t pool_slots;
  int64_t row_stride_bytes;
  int64_t map_words;           // ceil(pool_slots / 32)
  int64_t use_words;           // ceil(pool_slots / 4)
  int batch, T, max_prefix;
};

// Greedy acceptance of a verified tree (accept.hip).
struct AcceptArgs {
  const float* logits;         // [batch, T + 1, vocab]
  const int32_t* draft_tokens; // [batch, T]
  const int32_t* tree_parent;  // [batch, T]
  int32_t* accept_len;         // [batch]
  int32_t* accepted;           // [batch, T]
  int32_t* bonus;              // [batch]
  uint64_t* keys;              // [rows] argmax key per logits row (workspace, zero between calls)
  uint32_t* sticky_err;
  int64_t vocab;
  int batch, T, rows, chunks;  // rows = batch * (T + 1); chunks = argmax workgroups per row
};

// Launchers (kernels.hip, relocate.hip, accept.hip).
hipError_t launch_relocate(const RelocArgs& a, hipStream_t s);
hipError_t launch_accept(const AcceptArgs& a, hipStream_t s);
int accept_chunks(int64_t vocab);
// With start/stop events (profiling), the kernel is launched so that the events take the
// begin and end timestamps of its own dispatch, not of separate markers around it.
hipError_t launch_partial(const PartialArgs& a, int grid, hipStream_t s, hipEvent_t start = nullptr,
                          hipEvent_t stop = nullptr);
hipError_t launch_merge(const MergeArgs& a, hipStream_t s, hipEvent_t start = nullptr, hipEvent_t stop = nullptr);
hipError_t launch_probe_gather(const void* pool, int64_t stride_bytes, int64_t slots, const int32_t* idx, int n,
                               int lds, int grid, uint32_t* sink, hipStream_t s);
hipError_t launch_tree_masks(const int32_t* tree_parent, int batch, int T, uint64_t* masks, uint32_t* err,
                             hipStream_t s);

}  // namespace mlv
