// Host side of the C ABI declared in include/mlaverify.h: configuration checks,
// workspace layout, grid sizing and the launch sequence of one verify pass.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

#include "mlaverify.h"
#include "mlv_internal.h"

using namespace mlv;

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int page_log2(int page_size) {
  int lg = 0;
  while ((1 << lg) < page_size) lg++;
  return lg;
}

int mtiles_for(int heads, int T) { return (int)cdiv((int64_t)heads * T, kRowsPerBlock); }

int target_units_for(int n_mtiles) { return (int)(cdiv(kTargetBlocks, n_mtiles) > 0 ? cdiv(kTargetBlocks, n_mtiles) : 1); }

// Largest number of split units a run with `batch` requests of `T` nodes can produce.
int units_for(const mlaverify_config& c, int batch, int T) {
  if (c.split_tokens > 0) return batch * (int)(c.max_prefix_len > 0 ? cdiv(c.max_prefix_len, c.split_tokens) : 1);
  return target_units_for(mtiles_for(c.num_heads, T)) + batch;
}

struct Layout {
  size_t hdr, req, unit_tab, part_lse, part_o, reloc_off, reloc_status, reloc_maps, accept_keys, total;
  int units_cap;      // entries of unit_tab
  int64_t rows_cap;   // rows of part_o / part_lse
};

Layout layout_for(const mlaverify_config& c) {
  Layout L;
  int units_cap = 0;
  int64_t rows_cap = 0;
  for (int T = 1; T <= c.max_tree_nodes; T++) {
    // a ragged call may split a request into up to n_mt times as many units, of at most one
    // M tile each (ragged_caps)
    const int u = units_for(c, c.max_batch, T);
    const int n_mt = mtiles_for(c.num_heads, T);
    if ((int64_t)u * n_mt > INT32_MAX) return Layout{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, -1, (int64_t)INT32_MAX + 1};
    if (u * n_mt > units_cap) units_cap = u * n_mt;
    const int64_t rows = std::max((int64_t)u * c.num_heads * T, (int64_t)u * n_mt * kRowsPerBlock);
    if (rows > rows_cap) rows_cap = rows;
  }
  L.units_cap = units_cap;
  L.rows_cap = rows_cap;
  size_t off = 0;
  L.hdr = off;       off = align_up(off + sizeof(PlanHeader));
  L.req = off;       off = align_up(off + sizeof(ReqPlan) * (size_t)c.max_batch);
  L.unit_tab = off;  off = align_up(off + sizeof(int32_t) * (size_t)units_cap);
  L.part_lse = off;  off = align_up(off + sizeof(float) * (size_t)rows_cap);
  L.part_o = off;    off = align_up(off + sizeof(uint16_t) * (size_t)rows_cap * kVdim);  // bf16
  // relocation: segment offsets, refusal word, a bitmap and a byte map over the pool slots
  L.reloc_off = off;    off = align_up(off + sizeof(int32_t) * (size_t)c.max_batch);
  L.reloc_status = off; off = align_up(off + sizeof(uint32_t));
  // acceptance: argmax keys, zero between calls
  L.accept_keys = off;  off = align_up(off + sizeof(uint64_t) * (size_t)c.max_batch * (c.max_tree_nodes + 1));
  L.reloc_maps = off;   off = align_up(off + sizeof(uint32_t) * (size_t)(cdiv(c.pool_slots, 32) + cdiv(c.pool_slots, 4)));
  L.total = off;
  return L;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace

struct mlaverify_handle {
  mlaverify_config cfg;
  int device;
  char* ws;
  size_t ws_bytes;
  bool owns_ws;
  Layout L;
  int last_batch;
  std::vector<hipEvent_t> prof_events;  // 4 per profiled run
  int prof_max = 0, prof_runs = 0;
};

namespace {
void release_profile(mlaverify_handle* hd) {
  for (hipEvent_t e : hd->prof_events) (void)hipEventDestroy(e);
  hd->prof_events.clear();
  hd->prof_max = hd->prof_runs = 0;
}
}  // namespace

namespace {

// Host checks shared by the entry points of the verify pass.
int check_run_args(const mlaverify_config& c, int batch, int T, const void* q, const void* kv_pool,
                   const int32_t* kv_indices, const int32_t* prefix_lens, const int32_t* tree_parent, const void* out,
                   const float* lse) {
  if (batch < 1 || batch > c.max_batch || T < 1 || T > c.max_tree_nodes) return MLAVERIFY_ERR_INVALID_ARG;
  if (!q || !kv_pool || !kv_indices || !prefix_lens || !tree_parent || !out || !lse) return MLAVERIFY_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(kv_pool, 16) || !aligned(out, 16)) return MLAVERIFY_ERR_INVALID_ARG;
  if (!aligned(kv_indices, 4) || !aligned(prefix_lens, 4) || !aligned(tree_parent, 4) || !aligned(lse, 4))
    return MLAVERIFY_ERR_INVALID_ARG;
  return MLAVERIFY_OK;
}

// The workspace areas one verify pass uses.
struct RunAreas {
  PlanHeader* hdr;
  ReqPlan* req;
  int32_t* unit_fast;
  float* part_lse;
  uint16_t* part_o;
};

// Offsets of those areas for one call of `batch` requests of T nodes; returns the bytes used.
struct RunOffsets {
  size_t hdr, req, unit_tab, part_lse, part_o;
};
size_t run_offsets(const mlaverify_config& c, int batch, int T, RunOffsets* o) {
  const int units = units_for(c, batch, T);
  const size_t rows = (size_t)units * c.num_heads * T;
  size_t off = 0;
  o->hdr = off;      off = align_up(off + sizeof(PlanHeader));
  o->req = off;      off = align_up(off + sizeof(ReqPlan) * (size_t)batch);
  o->unit_tab = off; off = align_up(off + sizeof(int32_t) * (size_t)units);
  o->part_lse = off; off = align_up(off + sizeof(float) * rows);
  o->part_o = off;   off = align_up(off + sizeof(uint16_t) * rows * kVdim);
  return off;
}

// Enqueues the two kernels of one verify pass (plan + partials, then the merge) over the
// workspace areas w; when ev is given, ev[0..1] and ev[2..3] take the begin and end
// timestamps of the two kernels' dispatches.
int enqueue_run(const mlaverify_config& c, const RunAreas& w, int batch, int T, const int32_t* tree_lens,
                const void* q, const void* kv_pool, const int32_t* kv_indices, const int32_t* prefix_lens,
                const int32_t* tree_parent, void* out, float* lse, hipStream_t s, hipEvent_t* ev) {
  const int n_mt = mtiles_for(c.num_heads, T);
  const int units_grid = units_for(c, batch, T);
  const int M = c.num_heads * T;

  PartialArgs ka;
  ka.q = static_cast<const uint16_t*>(q);
  ka.pool = static_cast<const uint16_t*>(kv_pool);
  ka.kv_indices = kv_indices;
  ka.prefix_lens = prefix_lens;
  ka.tree_parent = tree_parent;
  ka.tree_lens = tree_lens;
  ka.hdr = w.hdr;
  ka.req = w.req;
  ka.part_o = w.part_o;
  ka.part_lse = w.part_lse;
  ka.unit_fast = w.unit_fast;
  ka.sticky_err = &w.hdr->sticky_err;
  ka.pool_slots = c.pool_slots;
  ka.row_stride_bytes = c.kv_row_stride * 2;
  ka.batch = batch;
  ka.T = T;
  ka.H = c.num_heads;
  ka.M = M;
  ka.n_mtiles = n_mt;
  ka.max_prefix = c.max_prefix_len;
  ka.split_fixed = c.split_tokens;
  ka.target_units = target_units_for(n_mt);
  ka.min_split = kMinSplit;
  // Bounds of the unit table and the partial rows.  With one tree size the plan makes at
  // most units_grid units of M rows.  A ragged call weighs each unit by the M tiles its
  // request fills and keeps the weighted count within n_mt * units_grid (the grid), so it
  // makes at most that many units, each of at most kRowsPerBlock rows per M tile.
  ka.units_cap = tree_lens ? n_mt * units_grid : units_grid;
  ka.rows_cap = (int32_t)(tree_lens ? (int64_t)n_mt * units_grid * kRowsPerBlock : (int64_t)units_grid * M);
  ka.scale_log2 = c.sm_scale * 1.4426950408889634f;
  ka.flags = c.flags;
  ka.page_log2 = page_log2(c.page_size);
  ka.max_page = (int32_t)((c.pool_slots - 1) >> ka.page_log2);
  ka.group_xcd = units_grid >= 8 ? 1 : 0;  // too few units to fill 8 XCDs one unit apiece

  MergeArgs ma;
  ma.req = ka.req;
  ma.part_o = ka.part_o;
  ma.part_lse = ka.part_lse;
  ma.out = static_cast<uint16_t*>(out);
  ma.lse = lse;
  ma.batch = batch;
  ma.H = c.num_heads;
  ma.M = M;
  ma.rows_cap = ka.rows_cap;
  ma.ragged = tree_lens ? 1 : 0;
  // units of one request, as the plan is expected to make them: under an automatic split the
  // target count shared by the batch (longer requests take more of them, in more rounds)
  ma.units_hint = c.split_tokens > 0 ? (int)(c.max_prefix_len > 0 ? cdiv(c.max_prefix_len, c.split_tokens) : 1)
                                     : (int)cdiv(ka.target_units, batch);

  const int grid = n_mt * (int)(cdiv(units_grid, 8) * 8);
  if (launch_partial(ka, grid, s, ev ? ev[0] : nullptr, ev ? ev[1] : nullptr) != hipSuccess) return MLAVERIFY_ERR_HIP;
  if (launch_merge(ma, s, ev ? ev[2] : nullptr, ev ? ev[3] : nullptr) != hipSuccess) return MLAVERIFY_ERR_HIP;
  return MLAVERIFY_OK;
}

// ---- Workspace of mlaverify_run_static: a file-scope device array, one copy per GPU, held
// until the process ends.  Host code never passes `scratch` itself to a kernel or a copy (in
// host code that name is a host-side stand-in, not a device address): its address on each
// device is taken once, with that device current, and kept in g_scratch_ptr.
constexpr size_t kStaticScratchBytes = MLAVERIFY_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[kStaticScratchBytes];
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`.
int static_scratch(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MLAVERIFY_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MLAVERIFY_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MLAVERIFY_ERR_HIP;
    g_scratch_ptr[dev] = static_cast<char*>(p);
  }
  *out = g_scratch_ptr[dev];
  return MLAVERIFY_OK;
}

}  // namespace

// Launches go to the handle's device only: its workspace lives there.
static bool on_handle_device(const mlaverify_handle* hd) {
  int dev = -1;
  return hipGetDevice(&dev) == hipSuccess && dev == hd->device;
}

extern "C" {

int mlaverify_validate_config(const mlaverify_config* c) {
  if (!c) return MLAVERIFY_ERR_INVALID_ARG;
  if (c->max_tree_nodes > kMaxTree) return MLAVERIFY_ERR_UNSUPPORTED;
  if (c->num_heads < 1 || c->num_heads > 128) return MLAVERIFY_ERR_INVALID_ARG;
  if (c->max_batch < 1 || c->max_batch > kMaxBatch) return MLAVERIFY_ERR_INVALID_ARG;
  if (c->max_tree_nodes < 1) return MLAVERIFY_ERR_INVALID_ARG;
  if (c->max_prefix_len < 0 || c->max_prefix_len > (1 << 28)) return MLAVERIFY_ERR_INVALID_ARG;
  if (c->pool_slots < 1 || c->pool_slots > INT32_MAX) return MLAVERIFY_ERR_INVALID_ARG;
  if (c->kv_row_stride < kLatent || c->kv_row_stride % 8 != 0) return MLAVERIFY_ERR_INVALID_ARG;
  if (!isfinite(c->sm_scale) || !(c->sm_scale > 0.f)) return MLAVERIFY_ERR_INVALID_ARG;
  if (c->split_tokens < 0 || (c->split_tokens > 0 && c->split_tokens % kTileKeys != 0))
    return MLAVERIFY_ERR_INVALID_ARG;
  if (c->flags & ~(uint32_t)MLAVERIFY_FLAG_NO_FASTPATH) return MLAVERIFY_ERR_INVALID_ARG;
  if (c->page_size < 0 || c->page_size > kMaxPage || (c->page_size & (c->page_size - 1)) != 0)
    return MLAVERIFY_ERR_INVALID_ARG;
  // key offsets and unit indices are 32-bit on the device
  if ((int64_t)c->max_batch * ((int64_t)c->max_prefix_len + c->max_tree_nodes) > INT32_MAX)
    return MLAVERIFY_ERR_UNSUPPORTED;
  if (c->split_tokens > 0 && (int64_t)c->max_batch * cdiv(c->max_prefix_len > 0 ? c->max_prefix_len : 1, c->split_tokens) > (1 << 24))
    return MLAVERIFY_ERR_UNSUPPORTED;
  // partial rows and unit-table entries are indexed with 32-bit integers on the device
  const Layout L = layout_for(*c);
  if (L.rows_cap > INT32_MAX || L.units_cap < 0) return MLAVERIFY_ERR_UNSUPPORTED;
  return MLAVERIFY_OK;
}

size_t mlaverify_workspace_bytes(const mlaverify_config* c) {
  if (mlaverify_validate_config(c) != MLAVERIFY_OK) return 0;
  return layout_for(*c).total;
}

int mlaverify_create(const mlaverify_config* c, void* workspace, size_t workspace_bytes, mlaverify_t* out) {
  if (!out) return MLAVERIFY_ERR_INVALID_ARG;
  *out = nullptr;
  const int v = mlaverify_validate_config(c);
  if (v != MLAVERIFY_OK) return v;
  const Layout L = layout_for(*c);
  if (workspace && workspace_bytes < L.total) return MLAVERIFY_ERR_WORKSPACE;
  if (workspace && !aligned(workspace, kAlign)) return MLAVERIFY_ERR_INVALID_ARG;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLAVERIFY_ERR_HIP;
  mlaverify_handle* hd = new (std::nothrow) mlaverify_handle;
  if (!hd) return MLAVERIFY_ERR_NO_MEMORY;
  hd->cfg = *c;
  hd->device = dev;
  hd->L = L;
  hd->last_batch = 0;
  hd->owns_ws = (workspace == nullptr);
  if (hd->owns_ws) {
    void* p = nullptr;
    if (hipMalloc(&p, L.total) != hipSuccess) {
      delete hd;
      return MLAVERIFY_ERR_NO_MEMORY;
    }
    hd->ws = static_cast<char*>(p);
    hd->ws_bytes = L.total;
  } else {
    hd->ws = static_cast<char*>(workspace);
    hd->ws_bytes = workspace_bytes;
  }
  // Clear the plan header (sticky error word) and the acceptance keys once;
  // no call needs a memset afterwards (acceptance leaves its area at zero).
  if (hipMemset(hd->ws + L.hdr, 0, sizeof(PlanHeader)) != hipSuccess ||
      hipMemset(hd->ws + L.accept_keys, 0, L.reloc_maps - L.accept_keys) != hipSuccess ||
      hipDeviceSynchronize() != hipSuccess) {
    if (hd->owns_ws) (void)hipFree(hd->ws);
    delete hd;
    return MLAVERIFY_ERR_HIP;
  }
  *out = hd;
  return MLAVERIFY_OK;
}

int mlaverify_run(mlaverify_t hd, int32_t batch, int32_t T, const void* q, const void* kv_pool,
                  const int32_t* kv_indices, const int32_t* prefix_lens, const int32_t* tree_parent, void* out,
                  float* lse, void* stream) {
  if (!hd) return MLAVERIFY_ERR_INVALID_ARG;
  if (!on_handle_device(hd)) return MLAVERIFY_ERR_INVALID_ARG;
  const mlaverify_config& c = hd->cfg;
  const int v = check_run_args(c, batch, T, q, kv_pool, kv_indices, prefix_lens, tree_parent, out, lse);
  if (v != MLAVERIFY_OK) return v;
  const Layout& L = hd->L;
  const RunAreas w = {reinterpret_cast<PlanHeader*>(hd->ws + L.hdr), reinterpret_cast<ReqPlan*>(hd->ws + L.req),
                      reinterpret_cast<int32_t*>(hd->ws + L.unit_tab), reinterpret_cast<float*>(hd->ws + L.part_lse),
                      reinterpret_cast<uint16_t*>(hd->ws + L.part_o)};
  hipEvent_t* ev = nullptr;
  if (hd->prof_runs < hd->prof_max) ev = &hd->prof_events[4 * hd->prof_runs++];
  const int rc = enqueue_run(c, w, batch, T, nullptr, q, kv_pool, kv_indices, prefix_lens, tree_parent, out, lse,
                             static_cast<hipStream_t>(stream), ev);
  if (rc == MLAVERIFY_OK) hd->last_batch = batch;
  return rc;
}

int mlaverify_run_ragged(mlaverify_t hd, int32_t batch, int32_t max_T, const int32_t* tree_lens, const void* q,
                         const void* kv_pool, const int32_t* kv_indices, const int32_t* prefix_lens,
                         const int32_t* tree_parent, void* out, float* lse, void* stream) {
  if (!hd) return MLAVERIFY_ERR_INVALID_ARG;
  if (!on_handle_device(hd)) return MLAVERIFY_ERR_INVALID_ARG;
  const mlaverify_config& c = hd->cfg;
  const int v = check_run_args(c, batch, max_T, q, kv_pool, kv_indices, prefix_lens, tree_parent, out, lse);
  if (v != MLAVERIFY_OK) return v;
  if (!tree_lens || !aligned(tree_lens, 4)) return MLAVERIFY_ERR_INVALID_ARG;
  const Layout& L = hd->L;
  const RunAreas w = {reinterpret_cast<PlanHeader*>(hd->ws + L.hdr), reinterpret_cast<ReqPlan*>(hd->ws + L.req),
                      reinterpret_cast<int32_t*>(hd->ws + L.unit_tab), reinterpret_cast<float*>(hd->ws + L.part_lse),
                      reinterpret_cast<uint16_t*>(hd->ws + L.part_o)};
  hipEvent_t* ev = nullptr;
  if (hd->prof_runs < hd->prof_max) ev = &hd->prof_events[4 * hd->prof_runs++];
  const int rc = enqueue_run(c, w, batch, max_T, tree_lens, q, kv_pool, kv_indices, prefix_lens, tree_parent, out,
                             lse, static_cast<hipStream_t>(stream), ev);
  if (rc == MLAVERIFY_OK) hd->last_batch = batch;
  return rc;
}

int mlaverify_run_static(const mlaverify_config* c, int32_t batch, int32_t T, const void* q, const void* kv_pool,
                         const int32_t* kv_indices, const int32_t* prefix_lens, const int32_t* tree_parent,
                         void* out, float* lse, void* stream) {
  const int v = mlaverify_validate_config(c);
  if (v != MLAVERIFY_OK) return v;
  const int a = check_run_args(*c, batch, T, q, kv_pool, kv_indices, prefix_lens, tree_parent, out, lse);
  if (a != MLAVERIFY_OK) return a;
  RunOffsets o;
  if (run_offsets(*c, batch, T, &o) > kStaticScratchBytes) return MLAVERIFY_ERR_WORKSPACE;
  char* base = nullptr;
  const int sp = static_scratch(&base);
  if (sp != MLAVERIFY_OK) return sp;
  const RunAreas w = {reinterpret_cast<PlanHeader*>(base + o.hdr), reinterpret_cast<ReqPlan*>(base + o.req),
                      reinterpret_cast<int32_t*>(base + o.unit_tab), reinterpret_cast<float*>(base + o.part_lse),
                      reinterpret_cast<uint16_t*>(base + o.part_o)};
  return enqueue_run(*c, w, batch, T, nullptr, q, kv_pool, kv_indices, prefix_lens, tree_parent, out, lse,
                     static_cast<hipStream_t>(stream), nullptr);
}

int mlaverify_relocate(mlaverify_t hd, int32_t batch, int32_t T, void* kv_pool, int32_t* kv_indices,
                       const int32_t* prefix_lens, const int32_t* dst_start, void* stream) {
  if (!hd) return MLAVERIFY_ERR_INVALID_ARG;
  if (!on_handle_device(hd)) return MLAVERIFY_ERR_INVALID_ARG;
  const mlaverify_config& c = hd->cfg;
  if (batch < 1 || batch > c.max_batch || T < 1 || T > c.max_tree_nodes) return MLAVERIFY_ERR_INVALID_ARG;
  if (!kv_pool || !kv_indices || !prefix_lens || !dst_start) return MLAVERIFY_ERR_INVALID_ARG;
  if (c.page_size > 1) return MLAVERIFY_ERR_UNSUPPORTED;  // relocation moves single-token slots
  if (!aligned(kv_pool, 16) || !aligned(kv_indices, 4) || !aligned(prefix_lens, 4) || !aligned(dst_start, 4))
    return MLAVERIFY_ERR_INVALID_ARG;
  const Layout& L = hd->L;
  RelocArgs a;
  a.pool = static_cast<char*>(kv_pool);
  a.kv_indices = kv_indices;
  a.prefix_lens = prefix_lens;
  a.dst_start = dst_start;
  a.off = reinterpret_cast<int32_t*>(hd->ws + L.reloc_off);
  a.maps = reinterpret_cast<uint32_t*>(hd->ws + L.reloc_maps);
  a.status = reinterpret_cast<uint32_t*>(hd->ws + L.reloc_status);
  a.sticky_err = &reinterpret_cast<PlanHeader*>(hd->ws + L.hdr)->sticky_err;
  a.pool_slots = c.pool_slots;
  a.row_stride_bytes = c.kv_row_stride * 2;
  a.map_words = cdiv(c.pool_slots, 32);
  a.use_words = cdiv(c.pool_slots, 4);
  a.batch = batch;
  a.T = T;
  a.max_prefix = c.max_prefix_len;
  if (launch_relocate(a, static_cast<hipStream_t>(stream)) != hipSuccess) return MLAVERIFY_ERR_HIP;
  return MLAVERIFY_OK;
}

int mlaverify_accept(mlaverify_t hd, int32_t batch, int32_t T, int32_t vocab, const float* logits,
                     const int32_t* draft_tokens, const int32_t* tree_parent, int32_t* accept_len, int32_t* accepted,
                     int32_t* bonus, void* stream) {
  if (!hd) return MLAVERIFY_ERR_INVALID_ARG;
  if (!on_handle_device(hd)) return MLAVERIFY_ERR_INVALID_ARG;
  const mlaverify_config& c = hd->cfg;
  if (batch < 1 || batch > c.max_batch || T < 1 || T > c.max_tree_nodes || vocab < 1) return MLAVERIFY_ERR_INVALID_ARG;
  if (!logits || !draft_tokens || !tree_parent || !accept_len || !accepted || !bonus) return MLAVERIFY_ERR_INVALID_ARG;
  if (!aligned(logits, 4) || !aligned(draft_tokens, 4) || !aligned(tree_parent, 4) || !aligned(accept_len, 4) ||
      !aligned(accepted, 4) || !aligned(bonus, 4))
    return MLAVERIFY_ERR_INVALID_ARG;
  AcceptArgs a;
  a.logits = logits;
  a.draft_tokens = draft_tokens;
  a.tree_parent = tree_parent;
  a.accept_len = accept_len;
  a.accepted = accepted;
  a.bonus = bonus;
  a.keys = reinterpret_cast<uint64_t*>(hd->ws + hd->L.accept_keys);
  a.sticky_err = &reinterpret_cast<PlanHeader*>(hd->ws + hd->L.hdr)->sticky_err;
  a.vocab = vocab;
  a.batch = batch;
  a.T = T;
  a.rows = batch * (T + 1);
  a.chunks = accept_chunks(vocab);
  if ((int64_t)a.rows * a.chunks > INT32_MAX) return MLAVERIFY_ERR_UNSUPPORTED;
  if (launch_accept(a, static_cast<hipStream_t>(stream)) != hipSuccess) return MLAVERIFY_ERR_HIP;
  return MLAVERIFY_OK;
}

int mlaverify_tree_masks(const int32_t* tree_parent, int32_t batch, int32_t T, uint64_t* masks, uint32_t* err,
                         void* stream) {
  if (!tree_parent || !masks || !err || batch < 1 || T < 1) return MLAVERIFY_ERR_INVALID_ARG;
  if (T > kMaxTree) return MLAVERIFY_ERR_UNSUPPORTED;
  if (batch > (1 << 24)) return MLAVERIFY_ERR_INVALID_ARG;
  if (!aligned(tree_parent, 4) || !aligned(masks, 8) || !aligned(err, 4)) return MLAVERIFY_ERR_INVALID_ARG;
  if (launch_tree_masks(tree_parent, batch, T, masks, err, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MLAVERIFY_ERR_HIP;
  return MLAVERIFY_OK;
}

int mlaverify_probe_gather(const void* kv_pool, int64_t kv_row_stride, int64_t pool_slots, const int32_t* indices,
                           int32_t n_rows, int32_t lds_path, int32_t grid, uint32_t* sink, void* stream) {
  if (!kv_pool || !indices || !sink || n_rows < 1 || grid < 1 || grid > (1 << 20)) return MLAVERIFY_ERR_INVALID_ARG;
  if (kv_row_stride < kLatent || kv_row_stride % 8 != 0 || pool_slots < 1) return MLAVERIFY_ERR_INVALID_ARG;
  if (!aligned(kv_pool, 16) || !aligned(indices, 4) || !aligned(sink, 4)) return MLAVERIFY_ERR_INVALID_ARG;
  if (launch_probe_gather(kv_pool, kv_row_stride * 2, pool_slots, indices, n_rows, lds_path ? 1 : 0, grid, sink,
                          static_cast<hipStream_t>(stream)) != hipSuccess)
    return MLAVERIFY_ERR_HIP;
  return MLAVERIFY_OK;
}

int mlaverify_read_plan(mlaverify_t hd, int32_t batch, void* stream, int32_t* host_out, int32_t capacity) {
  if (!hd || batch < 1 || batch > hd->cfg.max_batch || (capacity > 0 && !host_out) || capacity < 0)
    return MLAVERIFY_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  constexpr int kPlanHead = 6;
  const int needed = kPlanHead + 5 * batch;
  PlanHeader hdr;
  std::vector<ReqPlan> req;
  std::vector<int32_t> fast;
  try {
    req.resize(batch);
    fast.resize(hd->L.units_cap);
  } catch (const std::bad_alloc&) {
    return MLAVERIFY_ERR_NO_MEMORY;
  }
  bool ok = hipMemcpyAsync(&hdr, hd->ws + hd->L.hdr, sizeof(hdr), hipMemcpyDeviceToHost, s) == hipSuccess &&
            hipMemcpyAsync(req.data(), hd->ws + hd->L.req, sizeof(ReqPlan) * batch, hipMemcpyDeviceToHost, s) ==
                hipSuccess &&
            hipMemcpyAsync(fast.data(), hd->ws + hd->L.unit_tab, sizeof(int32_t) * fast.size(), hipMemcpyDeviceToHost,
                           s) == hipSuccess &&
            hipStreamSynchronize(s) == hipSuccess;
  if (!ok) return MLAVERIFY_ERR_HIP;
  int32_t fast_units = 0;
  for (int u = 0; u < hdr.total_units && u < (int)fast.size(); u++) fast_units += fast[u] != 0;
  // shader clock of the partial kernel's workgroup 0, from its cycle and wall-clock samples
  int wall_khz = 0;
  int32_t sclk_khz = 0;
  if (hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, hd->device) == hipSuccess && wall_khz > 0 &&
      hdr.clk_ticks > 0)
    sclk_khz = (int32_t)((double)hdr.clk_cycles * wall_khz / hdr.clk_ticks);
  // the rescale count runs over every call since the last readback; start it again
  char* rp = hd->ws + hd->L.hdr + offsetof(PlanHeader, rescales);
  if (hipMemsetAsync(rp, 0, sizeof(uint32_t), s) != hipSuccess || hipStreamSynchronize(s) != hipSuccess)
    return MLAVERIFY_ERR_HIP;
  int32_t vals[kPlanHead] = {hdr.split_len, hdr.total_units, hdr.n_mtiles, fast_units, sclk_khz,
                             (int32_t)hdr.rescales};
  for (int i = 0; i < kPlanHead && i < capacity; i++) host_out[i] = vals[i];
  for (int b = 0; b < batch; b++) {
    const int32_t rv[5] = {req[b].key_off, req[b].prefix_len, req[b].first_unit, req[b].units, (int32_t)req[b].err};
    for (int k = 0; k < 5; k++) {
      const int pos = kPlanHead + 5 * b + k;
      if (pos < capacity) host_out[pos] = rv[k];
    }
  }
  return needed;
}

int mlaverify_read_device_errors(mlaverify_t hd, void* stream, uint32_t* flags) {
  if (!hd || !flags) return MLAVERIFY_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t v = 0;
  char* p = hd->ws + hd->L.hdr + offsetof(PlanHeader, sticky_err);
  if (hipMemcpyAsync(&v, p, sizeof(v), hipMemcpyDeviceToHost, s) != hipSuccess) return MLAVERIFY_ERR_HIP;
  if (hipMemsetAsync(p, 0, sizeof(v), s) != hipSuccess) return MLAVERIFY_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return MLAVERIFY_ERR_HIP;
  *flags = v;
  return MLAVERIFY_OK;
}

int mlaverify_profile_begin(mlaverify_t hd, int32_t max_runs) {
  if (!hd || max_runs < 1 || max_runs > (1 << 20)) return MLAVERIFY_ERR_INVALID_ARG;
  release_profile(hd);
  hd->prof_events.resize(4 * (size_t)max_runs);
  for (size_t i = 0; i < hd->prof_events.size(); i++) {
    if (hipEventCreate(&hd->prof_events[i]) != hipSuccess) {
      hd->prof_events.resize(i);
      release_profile(hd);
      return MLAVERIFY_ERR_HIP;
    }
  }
  hd->prof_max = max_runs;
  hd->prof_runs = 0;
  return MLAVERIFY_OK;
}

int mlaverify_profile_end(mlaverify_t hd, float* host_ms, int32_t capacity_runs) {
  if (!hd || capacity_runs < 0 || (capacity_runs > 0 && !host_ms)) return MLAVERIFY_ERR_INVALID_ARG;
  const int runs = hd->prof_runs;
  int rc = runs;
  if (runs > 0 && hipEventSynchronize(hd->prof_events[4 * runs - 1]) != hipSuccess) rc = MLAVERIFY_ERR_HIP;
  for (int i = 0; rc >= 0 && i < runs && i < capacity_runs; i++)
    for (int k = 0; k < 2; k++)
      if (hipEventElapsedTime(&host_ms[2 * i + k], hd->prof_events[4 * i + 2 * k], hd->prof_events[4 * i + 2 * k + 1]) !=
          hipSuccess)
        rc = MLAVERIFY_ERR_HIP;
  release_profile(hd);
  return rc;
}

int mlaverify_destroy(mlaverify_t hd) {
  if (!hd) return MLAVERIFY_ERR_INVALID_ARG;
  release_profile(hd);
  if (hd->owns_ws && hd->ws) (void)hipFree(hd->ws);
  delete hd;
  return MLAVERIFY_OK;
}

const char* mlaverify_status_string(int status) {
  switch (status) {
    case MLAVERIFY_OK: return "ok";
    case MLAVERIFY_ERR_INVALID_ARG: return "invalid argument";
    case MLAVERIFY_ERR_UNSUPPORTED: return "unsupported configuration";
    case MLAVERIFY_ERR_NO_MEMORY: return "out of memory";
    case MLAVERIFY_ERR_WORKSPACE: return "workspace too small";
    case MLAVERIFY_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

}  // extern "C"
