/*
 * mlaverify.h - C ABI of the DDTree MLA tree-verify attention library (gfx950).
 *
 * The operation (page "Chunk 66.0", magik.net llmopt segment 66, summary
 * paragraph; page "Chunk 66.1", summary paragraph):
 *   DDTree speculative decoding verifies a draft tree of T nodes per request
 *   with one attention pass of the target model.  The attention is MLA in its
 *   absorbed (latent) form: the H heads of one tensor-parallel rank (8 per rank
 *   under TP8) all score against the same 576-wide bf16 latent row per token
 *   (512 latent + 64 rope columns) and read their value from its first 512
 *   columns.  KV rows live in a shared pool with page_size=1: every token is one
 *   row, addressed through a per-request token-index table, so on a churned
 *   pool the reads are scattered.  Node i of a request attends to every prefix
 *   token of its request, to its ancestors in the tree and to itself.
 *
 *   For request b, node i, head h (sigma = sm_scale):
 *     Vis(b,i) = prefix slots of b  ++  slots of {i, parent(i), parent(parent(i)), ...}
 *     s_j      = sigma * sum_{d<576} q[b,i,h,d] * KV[j,d]
 *     lse      = ln sum_{j in Vis} exp(s_j)
 *     out      = sum_{j in Vis} exp(s_j - lse) * KV[j, 0:512]
 *
 *   The computation is split over the prefix (split-KV partials merged by their
 *   log-sum-exp, the "partial+reduce" design of the Chunk 66.0 summary) and is
 *   capture-safe in the sense of the Chunk 66.1 summary: mlaverify_run makes no
 *   host synchronisation, no host<->device copy and no allocation, and works in
 *   a caller-provided workspace, so it can be recorded into a HIP graph.
 *
 * Conventions
 *   - Every function returns MLAVERIFY_OK (0) on success or a negative status
 *     (see mlaverify_status_string).  On any host-detected error nothing is
 *     enqueued and outputs are left untouched.
 *   - All tensor pointers are DEVICE pointers on the handle's device; sizes and
 *     shapes are host integers.  The caller owns every tensor; the library keeps
 *     no pointer beyond a call except the workspace.
 *   - Calls on one handle must be ordered on one stream (they share the
 *     workspace); use one handle per concurrent stream.
 */
#ifndef MLAVERIFY_H
#define MLAVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLAVERIFY_API __attribute__((visibility("default")))

#define MLAVERIFY_LATENT_DIM 576 /* columns of a KV row used for scores */
#define MLAVERIFY_V_DIM 512      /* leading columns of a KV row used as V */
#define MLAVERIFY_MAX_TREE_NODES 256

/* Status codes. */
#define MLAVERIFY_OK 0
#define MLAVERIFY_ERR_INVALID_ARG (-1)    /* null pointer, misalignment, size out of range, or a call on a
                                             handle whose device is not the current one */
#define MLAVERIFY_ERR_UNSUPPORTED (-2)    /* a configuration the kernels do not implement */
#define MLAVERIFY_ERR_NO_MEMORY (-3)      /* library-owned workspace allocation failed */
#define MLAVERIFY_ERR_WORKSPACE (-4)      /* caller workspace smaller than mlaverify_workspace_bytes */
#define MLAVERIFY_ERR_HIP (-5)            /* a HIP runtime call or kernel launch failed */

/* Sticky device-side data-error bits (mlaverify_read_device_errors). */
#define MLAVERIFY_DEVERR_BAD_PARENT 0x1u  /* a tree_parent entry outside [-1, node) */
#define MLAVERIFY_DEVERR_BAD_INDEX 0x2u   /* a kv_indices entry outside [0, pool_slots) */
#define MLAVERIFY_DEVERR_BAD_PREFIX 0x4u  /* a prefix_lens entry outside [0, max_prefix_len]; that
                                             request and every later one of the batch are poisoned,
                                             since their index segments can no longer be located */
#define MLAVERIFY_DEVERR_RELOCATE_CONFLICT 0x8u /* mlaverify_relocate refused: a destination run leaves
                                                   the pool, overlaps another one or holds a slot in use */
#define MLAVERIFY_DEVERR_BAD_TREE_LEN 0x10u /* mlaverify_run_ragged: a tree_lens entry outside [1, max_T];
                                               that request and every later one are poisoned */

/* Flags for mlaverify_config.flags. */
#define MLAVERIFY_FLAG_NO_FASTPATH 0x1u   /* always gather row by row (A/B tests of the contiguous path) */

typedef struct mlaverify_handle* mlaverify_t;

typedef struct mlaverify_config {
  int32_t num_heads;       /* H: heads of this rank, 1..128 */
  int32_t max_batch;       /* largest batch passed to run; sizes the grid and workspace */
  int32_t max_tree_nodes;  /* largest T passed to run, 1..256 (trees over 64 nodes use a
                              kernel variant with four 64-bit mask words per node) */
  int32_t max_prefix_len;  /* largest P_b accepted; larger ones are device errors */
  int64_t pool_slots;      /* rows in kv_pool; indices outside [0, pool_slots) are device errors */
  int64_t kv_row_stride;   /* elements between consecutive pool rows, >= 576, multiple of 8 */
  float sm_scale;          /* softmax scale sigma > 0 (e.g. 1/sqrt(192)) */
  int32_t split_tokens;    /* 0: choose the prefix split length per call on the device;
                              else a fixed split length in tokens, a multiple of 32 */
  uint32_t flags;          /* MLAVERIFY_FLAG_* */
  int32_t page_size;       /* 0 or 1: one kv_indices entry (pool slot) per prefix token;
                              else a power of two up to 1024: prefixes live in pages of
                              page_size consecutive pool slots and their part of kv_indices
                              is a block table of page ids (see mlaverify_run) */
} mlaverify_config;

/* Checks a configuration without touching the GPU.  Returns MLAVERIFY_OK,
 * MLAVERIFY_ERR_INVALID_ARG or MLAVERIFY_ERR_UNSUPPORTED.  The limits it checks follow
 * from the kernels (one rank's heads, up to 256 tree nodes, 32-bit segment offsets, unit
 * counts and partial-row indices); the
 * pages fix none of them beyond page_size=1 ("Chunk 66.0" summary), which is the default. */
MLAVERIFY_API int mlaverify_validate_config(const mlaverify_config* cfg);

/* Bytes of device workspace a handle with this configuration needs (0 if the
 * configuration is invalid).  Pure host computation.  The "Chunk 66.1" summary has the
 * verify kernel run in a torch-allocated workspace with a fixed split count, so that it can
 * be captured; this is that workspace's size: the split partials (bf16 outputs and fp32
 * log-sum-exps of every unit) plus small plan, relocation and acceptance areas. */
MLAVERIFY_API size_t mlaverify_workspace_bytes(const mlaverify_config* cfg);

/* Creates a handle on the current HIP device.  workspace: a device buffer of at
 * least mlaverify_workspace_bytes(cfg) bytes, 256-byte aligned, owned by the
 * caller and kept alive until mlaverify_destroy (the caller-provided workspace of the
 * "Chunk 66.1" summary); or NULL, in which case the library allocates (and later frees)
 * it.  The workspace needs no initialisation; create clears the small error area with a
 * synchronous memset, so create itself is not for graph capture.  On success *out
 * receives the handle; on failure *out is NULL and nothing stays allocated. */
MLAVERIFY_API int mlaverify_create(const mlaverify_config* cfg, void* workspace,
                                   size_t workspace_bytes, mlaverify_t* out);

/* Enqueues one verify-attention pass on `stream` (a hipStream_t; NULL = default
 * stream).  Host arguments: batch in [1, max_batch], tree_nodes in
 * [1, max_tree_nodes].  Device arguments:
 *   q           bf16 [batch*T, H, 576], row (b*T + i)*H + h, contiguous, 16-byte aligned
 *   kv_pool     bf16 [pool_slots, kv_row_stride], 16-byte aligned; columns 0..575 are read
 *   kv_indices  int32 [sum_b (E_b + T)]: request b's prefix entries, then the T slots holding
 *               the latents of tree nodes 0..T-1; requests back to back.  With page_size
 *               <= 1, E_b = P_b and entry j is the pool slot of prefix token j.  With a page
 *               size p > 1, E_b = ceil(P_b / p) and entry e is a page id: prefix token j lives
 *               in pool slot entry[j / p] * p + j % p (a block table; tree slots stay per
 *               token).  Slots outside the pool are device errors (MLAVERIFY_DEVERR_BAD_INDEX).
 *   prefix_lens int32 [batch]: P_b, 0 <= P_b <= max_prefix_len
 *   tree_parent int32 [batch, T]: -1 for a root, else a node index smaller than the node
 *   out         bf16 [batch*T, H, 512] (written), 16-byte aligned
 *   lse         fp32 [batch*T, H] (written): natural-log sum of exp(scores)
 * Data errors found on the device (see MLAVERIFY_DEVERR_*) never cause an
 * out-of-bounds access: they set sticky bits and every output row (out and lse)
 * of the offending request becomes NaN; other requests are unaffected, except
 * that a bad prefix length also poisons the requests after it.
 * Never synchronises, copies to/from the host or allocates: graph-capturable. */
MLAVERIFY_API int mlaverify_run(mlaverify_t h, int32_t batch, int32_t tree_nodes,
                                const void* q, const void* kv_pool, const int32_t* kv_indices,
                                const int32_t* prefix_lens, const int32_t* tree_parent,
                                void* out, float* lse, void* stream);

/* The verify pass for a batch whose requests draft trees of different sizes (a budget per
 * request, as the DDTree verify step of the "Chunk 66.0" summary runs one draft tree per
 * request; the reading of the layout below is this library's).  Request b has
 * T_b = tree_lens[b] nodes, 1 <= T_b <= max_T <= max_tree_nodes; max_T (host) sizes the
 * launch, the kernels size each request's work by its own T_b, so a small tree costs no
 * padded rows, and (up to 64 requests) the prefix split is chosen over the 128-row tiles the
 * requests' rows fill, so that requests with fewer rows get shorter units.  Rows are packed request after request: node i of request b is row n_b + i
 * with n_b = T_0 + ... + T_{b-1}.  Device arguments (as for mlaverify_run otherwise):
 *   tree_lens   int32 [batch]
 *   q           bf16 [sum T_b, H, 576], row (n_b + i)*H + h
 *   kv_indices  int32 [sum_b (E_b + T_b)]: request b's prefix entries, then its T_b tree slots
 *   tree_parent int32 [sum T_b]: at n_b + i the parent of node i within its request
 *               (-1, or an earlier node of the same request)
 *   out, lse    [sum T_b, H, 512] and [sum T_b, H] (written)
 * A T_b outside [1, max_T] sets MLAVERIFY_DEVERR_BAD_TREE_LEN and poisons that request and
 * every later one: their rows' positions depend on it, so none of their rows is written.
 * With every T_b equal to T the results are those of mlaverify_run, bit for bit.  Never
 * synchronises, copies to or from the host or allocates: graph-capturable. */
MLAVERIFY_API int mlaverify_run_ragged(mlaverify_t h, int32_t batch, int32_t max_T, const int32_t* tree_lens,
                                       const void* q, const void* kv_pool, const int32_t* kv_indices,
                                       const int32_t* prefix_lens, const int32_t* tree_parent, void* out,
                                       float* lse, void* stream);

/* Bytes of the static device workspace behind mlaverify_run_static (48 MiB per GPU). */
#define MLAVERIFY_STATIC_SCRATCH_BYTES ((size_t)48 << 20)

/* For callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  The same verify pass as mlaverify_run
 * (same kernels, same results bit for bit), without a handle or a caller workspace: the
 * workspace is a static device array of MLAVERIFY_STATIC_SCRATCH_BYTES that the library
 * holds on every GPU it runs on until the process ends.  The call allocates nothing: no
 * hipMalloc, no hipFree, no allocating library routine.  Its first call on a device looks
 * up that device's copy of the array (hipGetSymbolAddress, with the device current).
 * cfg: as for mlaverify_create (validated on every call; pure host work).  The other
 * arguments are those of mlaverify_run, on the current device.  A call whose partial
 * results need more than MLAVERIFY_STATIC_SCRATCH_BYTES returns MLAVERIFY_ERR_WORKSPACE
 * and enqueues nothing: that is (H * T) rows x (units + batch) x 1028 bytes plus a few KB,
 * where units = ceil(256 / ceil(H * T / 128)) under the automatic split, about 34 MB for
 * one request of 64 nodes and 8 heads.  Every call on a GPU shares that GPU's array, so
 * calls that overlap in time on one GPU (different streams, or different host threads
 * without ordering) race and give wrong results; order them on one stream.  Data errors
 * show as NaN rows exactly as for mlaverify_run; their sticky bits are not readable here.
 * Never synchronises or copies to the host: graph-capturable. */
MLAVERIFY_API int mlaverify_run_static(const mlaverify_config* cfg, int32_t batch, int32_t tree_nodes,
                                       const void* q, const void* kv_pool, const int32_t* kv_indices,
                                       const int32_t* prefix_lens, const int32_t* tree_parent, void* out,
                                       float* lse, void* stream);

/* Tier-1 KV relocation (live defragmentation of prefix rows).  The "Chunk 66.0"
 * summary calls for K/V defragmentation of the scattered page_size=1 pool; the
 * "Chunk 66.1" summary keeps a request's KV contiguous when it is allocated (Tier 0)
 * and defers Tier 1, moving rows that are already scattered.  This call is Tier 1:
 * for every request b with dst_start[b] >= 0, prefix row j < P_b is copied (columns
 * 0..575; the rest of the row stride is left alone) from pool slot
 * kv_indices[off_b + j] to slot dst_start[b] + j, and kv_indices[off_b + j] becomes
 * dst_start[b] + j, so that the request's prefix is one contiguous run (the case the
 * verify pass reads without its index table).  Tree-node slots are never moved.
 * Host arguments: batch in [1, max_batch], tree_nodes (T) in [1, max_tree_nodes],
 * which locate the segments exactly as in mlaverify_run.  Device arguments:
 *   kv_pool     bf16 [pool_slots, kv_row_stride] (read and written), 16-byte aligned
 *   kv_indices  int32 [sum_b (P_b + T)], laid out as for mlaverify_run (read and written)
 *   prefix_lens int32 [batch]
 *   dst_start   int32 [batch]: first slot of request b's destination run, < 0 to skip b
 * The move is all or nothing and is checked on the device before any row is copied.
 * It is refused (pool and indices untouched, sticky bits set) when a prefix length is
 * outside [0, max_prefix_len] (MLAVERIFY_DEVERR_BAD_PREFIX, reported alone), when an
 * index of the batch is outside the pool (MLAVERIFY_DEVERR_BAD_INDEX), or when a
 * destination run leaves the pool, overlaps another destination run, or contains a
 * slot that any index of the batch uses (MLAVERIFY_DEVERR_RELOCATE_CONFLICT).  A row
 * already at its own destination is allowed and is not copied.  Under these rules the
 * result does not depend on the order of the copies.  Needs page_size <= 1
 * (MLAVERIFY_ERR_UNSUPPORTED otherwise).  The caller owns every buffer;
 * the call uses the handle's workspace (so it is ordered with run on one stream),
 * never synchronises, copies to the host or allocates: graph-capturable. */
MLAVERIFY_API int mlaverify_relocate(mlaverify_t h, int32_t batch, int32_t tree_nodes, void* kv_pool,
                                     int32_t* kv_indices, const int32_t* prefix_lens, const int32_t* dst_start,
                                     void* stream);

/* Greedy acceptance of a verified draft tree, the step that decides what a verify pass
 * commits (the "Chunk 66.0" summary reports the resulting commit lengths, 7-8 tokens on
 * predictable text).  Rule, per request: start at the position before the tree; take the
 * argmax g of the current logits row; move to the lowest-index child (a node with parent
 * -1 at the start) whose draft token is g, and repeat from its row; stop when no child
 * matches.  The bonus token is the argmax of the last row visited, so the step commits
 * accept_len + 1 tokens.  argmax: largest value, lowest index among equal values, NaN
 * ranked below every number (a row of NaN gives 0), -0 equal to +0.
 * Host arguments: batch in [1, max_batch], tree_nodes (T) in [1, max_tree_nodes],
 * vocab >= 1.  Device arguments:
 *   logits       fp32 [batch, T + 1, vocab]: row 0 at the position before the tree, row
 *                1 + i after tree node i (read)
 *   draft_tokens int32 [batch, T]: the token drafted at each node (read)
 *   tree_parent  int32 [batch, T], as for mlaverify_run (read)
 *   accept_len   int32 [batch] (written): nodes accepted
 *   accepted     int32 [batch, T] (written): the accepted nodes in path order, then -1
 *   bonus        int32 [batch] (written)
 * A request whose tree has a parent outside [-1, node) accepts nothing (its bonus token is
 * row 0's argmax) and sets MLAVERIFY_DEVERR_BAD_PARENT.  The caller owns every buffer; the
 * call uses the handle's workspace (ordered with run on one stream), never synchronises,
 * copies to the host or allocates: graph-capturable. */
MLAVERIFY_API int mlaverify_accept(mlaverify_t h, int32_t batch, int32_t tree_nodes, int32_t vocab,
                                   const float* logits, const int32_t* draft_tokens, const int32_t* tree_parent,
                                   int32_t* accept_len, int32_t* accepted, int32_t* bonus, void* stream);

/* Builds the tree-ancestor bitmasks alone (the mask step of run, on its own; the "Chunk
 * 66.1" summary times the CPU mask build of its serving stack at 0.18 ms per step), as
 * W = ceil(T / 64) words per node: bit j % 64 of masks[(b*T + i)*W + j / 64] is set iff
 * tree node j is node i or one of its ancestors.
 * tree_parent int32 [batch, T] and masks uint64 [batch, T, W] are device pointers;
 * err (device, uint32 [batch]) receives MLAVERIFY_DEVERR_BAD_PARENT per bad
 * request, whose masks are then 0.  1 <= T <= 256.  Enqueued on `stream`. */
MLAVERIFY_API int mlaverify_tree_masks(const int32_t* tree_parent, int32_t batch, int32_t tree_nodes,
                                       uint64_t* masks, uint32_t* err, void* stream);

/* Measurement probe, not part of the verify pass: enqueues one launch that reads the pool
 * rows kv_pool[indices[r]] (columns 0..575, 1,152 bytes each) for r < n_rows, the scattered
 * page_size=1 access pattern whose 128-bit loads the "Chunk 66.1" summary credits, through
 * one of the two 16-byte load paths the verify kernel can use: lds_path = 0 loads into
 * registers (non-temporal global_load_dwordx4), lds_path != 0 loads straight into LDS
 * (global_load_lds_dwordx4).  grid workgroups of 256 threads (1 .. 2^20); each reads tiles
 * of 32 rows, four tiles in flight.  Entries outside [0, pool_slots) read row 0.
 * sink: device uint32 [grid * 256], written with a fold of the data read (its value is of no
 * use; it keeps the loads live).  Device pointers: kv_pool (16-byte aligned), indices, sink.
 * Enqueued on `stream`; no synchronisation or allocation. */
MLAVERIFY_API int mlaverify_probe_gather(const void* kv_pool, int64_t kv_row_stride, int64_t pool_slots,
                                         const int32_t* indices, int32_t n_rows, int32_t lds_path, int32_t grid,
                                         uint32_t* sink, void* stream);

/* Copies the work partition of the most recent run into host memory (synchronises
 * `stream`; for tests and reports, not for graphs).  Writes up to `capacity`
 * int32 values: [split_len, total_units, n_mtiles, fast_units, sclk_khz, rescales, then
 * per request b: key_offset_b, prefix_len_b, first_unit_b, units_b, prefix_error_bits_b],
 * where fast_units counts the split units whose prefix slots formed one contiguous run
 * and were read without the index table (the contiguous-run fast path; a unit with no
 * prefix keys never counts), sclk_khz is the shader clock over the run of the partial
 * kernel's first workgroup (its cycle counter against the device's wall clock; 0 if it
 * was not sampled), and rescales counts the waves that raised a row's softmax reference
 * (a tile maximum more than 2^16 above it, which rescales that row's partial sums once)
 * over every call since the previous readback, which sets it back to 0.  Parent and index errors are reported by
 * mlaverify_read_device_errors only.
 * Returns the number of values available (which may exceed capacity) or a
 * negative status. */
MLAVERIFY_API int mlaverify_read_plan(mlaverify_t h, int32_t batch, void* stream, int32_t* host_out,
                                      int32_t capacity);

/* Reads and clears the sticky device-error bits (synchronises `stream`; for tests and
 * monitoring, not for graphs).  The bits are the data errors the kernels detect instead of
 * reading out of bounds (MLAVERIFY_DEVERR_*); the pages' kernel is checked for token-exact
 * agreement with a naive reference ("Chunk 66.0" summary), and these bits are how a run that
 * could not be exact says so. */
MLAVERIFY_API int mlaverify_read_device_errors(mlaverify_t h, void* stream, uint32_t* flags);

/* Kernel timing for benchmarks (not for graph capture).  The "Chunk 66.0" summary finds
 * that the reduction kernel and the tile sizing still needed work; these events time the
 * partial pass and the merge apart, on the run's own stream.  After
 * mlaverify_profile_begin(h, n) the next n calls of mlaverify_run (or _ragged) launch their two
 * kernels (partial pass, merge) with a pair of HIP events each that take the begin and end
 * timestamps of the kernel's own dispatch on the run's stream.
 * mlaverify_profile_end synchronises on the last event, writes host_ms[2*i + k] =
 * duration in milliseconds of kernel k of recorded run i for
 * i < min(runs, capacity_runs), releases the events and returns the number of runs
 * recorded (or a negative status).  begin while a session is open restarts it. */
MLAVERIFY_API int mlaverify_profile_begin(mlaverify_t h, int32_t max_runs);
MLAVERIFY_API int mlaverify_profile_end(mlaverify_t h, float* host_ms, int32_t capacity_runs);

/* Releases the handle (and the workspace if the library allocated it).  The caller must
 * have finished (synchronised) every call enqueued on it.  Returns MLAVERIFY_ERR_INVALID_ARG
 * for a NULL handle. */
MLAVERIFY_API int mlaverify_destroy(mlaverify_t h);

/* Static text for a status code (never NULL; "unknown status" for codes outside the list). */
MLAVERIFY_API const char* mlaverify_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MLAVERIFY_H */
