// gfx950 kernels of Tier-1 KV relocation: the live defragmentation that the "Chunk 66.1"
// summary defers (Tier 0 keeps a request's KV contiguous when it is allocated; Tier 1
// moves rows that are already scattered).  Each relocated request's prefix rows move to
// a caller-chosen run of pool slots and its index list is rewritten to that run, which
// is the layout the verify pass reads without its index table.
//
// Four launches on one stream, so that no row is copied before the whole batch has been
// checked (the move is all or nothing):
//   k_reloc_prepare  clear the slot maps; one workgroup checks the prefix lengths and
//                    destination ranges and writes each request's segment offset
//   k_reloc_mark     one thread per index of the batch: mark the slot it uses (a byte
//                    map: every writer stores 1, so no atomics), and for a moving prefix
//                    row claim its destination (a bitmap, claimed with atomics; a
//                    destination claimed twice is a conflict)
//   k_reloc_check    one thread per moving row: its destination must not be in use
//   k_reloc_copy     32 rows per workgroup: copy columns 0..575 of each row whose slot is
//                    not already its destination, then rewrite the row's index
// A row that already sits at its destination neither marks its slot as in use nor moves.
// Under these rules no row is overwritten before it has been read, whatever the order.
// The copy streams (non-temporal loads and stores): the moved rows are not reused soon.
#include "mlv_internal.h"

namespace mlv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRelocThreads = 256;
constexpr int kRelocRows = 32;                                         // rows per copy workgroup
constexpr int kRelocChunkIters = kRelocRows * kChunksPerRow / kRelocThreads;  // 9
static_assert(kRelocRows * kChunksPerRow % kRelocThreads == 0, "copy loop covers whole rows");
static_assert(kMaxBatch <= 4 * kRelocThreads, "prepare: at most 4 requests per thread");

__device__ __forceinline__ int valid_len(int p, int max_prefix) { return (p < 0 || p > max_prefix) ? 0 : p; }

// The destination run [dst, dst + p) of a moving request lies inside the pool.
__device__ __forceinline__ bool moving(const RelocArgs& a, int dst, int p) {
  return dst >= 0 && (int64_t)dst + p <= a.pool_slots;
}

// Byte per pool slot: 1 when some index of the batch uses the slot.
__device__ __forceinline__ uint8_t* in_use(const RelocArgs& a) {
  return reinterpret_cast<uint8_t*>(a.maps + a.map_words);
}

__device__ __forceinline__ void report(const RelocArgs& a, uint32_t err) {
  atomicOr(a.status, err);
  atomicOr(a.sticky_err, err);
}

__global__ __launch_bounds__(kRelocThreads) void k_reloc_prepare(RelocArgs a) {
  const int tid = threadIdx.x;
  const size_t words = (size_t)a.map_words + (size_t)a.use_words;
  for (size_t i = (size_t)blockIdx.x * kRelocThreads + tid; i < words; i += (size_t)gridDim.x * kRelocThreads)
    a.maps[i] = 0u;  // the destination bitmap, then the byte map of slots in use
  if (blockIdx.x != 0) return;
  __shared__ int s_sum[kRelocThreads];
  __shared__ uint32_t s_err;
  if (tid == 0) s_err = 0u;
  constexpr int kPer = kMaxBatch / kRelocThreads;  // requests per thread
  int lens[kPer], local = 0;
  uint32_t err = 0;
#pragma unroll
  for (int j = 0; j < kPer; j++) {
    const int b = tid * kPer + j;
    const int p = b < a.batch ? a.prefix_lens[b] : 0;
    if (p < 0 || p > a.max_prefix) err |= kErrBadPrefix;
    lens[j] = valid_len(p, a.max_prefix);
    local += b < a.batch ? lens[j] + a.T : 0;
  }
  s_sum[tid] = local;
  __syncthreads();
  for (int d = 1; d < kRelocThreads; d <<= 1) {  // inclusive scan of the per-thread sums
    const int v = tid >= d ? s_sum[tid - d] : 0;
    __syncthreads();
    s_sum[tid] += v;
    __syncthreads();
  }
  int off = s_sum[tid] - local;
#pragma unroll
  for (int j = 0; j < kPer; j++) {
    const int b = tid * kPer + j;
    if (b < a.batch) {
      a.off[b] = off;
      const int dst = a.dst_start[b];
      if (dst >= 0 && !moving(a, dst, lens[j])) err |= kErrConflict;  // the run leaves the pool
      off += lens[j] + a.T;
    }
  }
  if (err) atomicOr(&s_err, err);
  __syncthreads();
  if (tid == 0) {
    uint32_t e = s_err;
    if (e & kErrBadPrefix) e = kErrBadPrefix;  // reported alone: the segments cannot be located
    *a.status = e;
    if (e) atomicOr(a.sticky_err, e);
  }
}

__global__ __launch_bounds__(kRelocThreads) void k_reloc_mark(RelocArgs a) {
  if (*a.status & kErrBadPrefix) return;
  const int b = blockIdx.y;
  const int k = blockIdx.x * kRelocThreads + threadIdx.x;
  const int p = a.prefix_lens[b];
  if (k >= p + a.T) return;
  const int dst = a.dst_start[b];
  const bool mv = k < p && moving(a, dst, p);
  uint32_t err = 0;
  // Destination claims: the moving lanes of a wave are consecutive keys, hence consecutive
  // slots, so each bitmap word they touch gets one atomic with all of its bits from the
  // first moving lane in that word (32 lanes on one word would otherwise serialise).
  const uint64_t mv_lanes = __ballot(mv);
  if (mv) {
    const int d = dst + k;
    const int lane = threadIdx.x & 63;
    const int first = __builtin_ctzll(mv_lanes);
    if (lane == first || (d & 31) == 0) {
      const int rest = __popcll(mv_lanes) - (lane - first);  // moving lanes from this one on
      const int n = min(32 - (d & 31), rest);
      const uint32_t bits = (n == 32 ? ~0u : ((1u << n) - 1u)) << (d & 31);
      if (atomicOr(&a.maps[d >> 5], bits) & bits) err |= kErrConflict;  // claimed twice
    }
  }
  const int s = a.kv_indices[a.off[b] + k];
  if (s < 0 || (int64_t)s >= a.pool_slots) {
    err |= kErrBadIndex;
  } else if (!(mv && s == dst + k)) {
    in_use(a)[s] = 1;  // a row already at its destination does not count as in use
  }
  if (err) report(a, err);
}

__global__ __launch_bounds__(kRelocThreads) void k_reloc_check(RelocArgs a) {
  if (*a.status & kErrBadPrefix) return;
  const int b = blockIdx.y;
  const int k = blockIdx.x * kRelocThreads + threadIdx.x;
  const int p = a.prefix_lens[b];
  const int dst = a.dst_start[b];
  if (k >= p || !moving(a, dst, p)) return;
  const int d = dst + k;
  if (in_use(a)[d]) report(a, kErrConflict);  // the destination is in use
}

__global__ __launch_bounds__(kRelocThreads) void k_reloc_copy(RelocArgs a) {
  if (*a.status) return;  // refused: nothing moves
  const int b = blockIdx.y;
  const int dst = a.dst_start[b];
  const int p = a.prefix_lens[b];
  const int k0 = blockIdx.x * kRelocRows;
  if (dst < 0 || k0 >= p) return;
  const int nk = min(kRelocRows, p - k0);
  const int tid = threadIdx.x;
  int32_t* idx = a.kv_indices + a.off[b] + k0;
  __shared__ int s_src[kRelocRows];
  if (tid < nk) s_src[tid] = idx[tid];
  __syncthreads();
  // thread tid moves 16-byte chunks tid, tid + 256, ... of the workgroup's rows; all
  // loads are issued before the first store
  u32x4 v[kRelocChunkIters];
  bool on[kRelocChunkIters];
#pragma unroll
  for (int i = 0; i < kRelocChunkIters; i++) {
    const int c = tid + kRelocThreads * i;
    const int r = c / kChunksPerRow, ch = c - r * kChunksPerRow;
    on[i] = r < nk && s_src[r < nk ? r : 0] != dst + k0 + r;
    if (on[i])
      v[i] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(a.pool + (int64_t)s_src[r] * a.row_stride_bytes + 16 * ch));
  }
#pragma unroll
  for (int i = 0; i < kRelocChunkIters; i++) {
    const int c = tid + kRelocThreads * i;
    const int r = c / kChunksPerRow, ch = c - r * kChunksPerRow;
    if (on[i])
      __builtin_nontemporal_store(v[i],
                                  reinterpret_cast<u32x4*>(a.pool + (int64_t)(dst + k0 + r) * a.row_stride_bytes + 16 * ch));
  }
  if (tid < nk) idx[tid] = dst + k0 + tid;
}

}  // namespace

hipError_t launch_relocate(const RelocArgs& a, hipStream_t s) {
  const int64_t words = a.map_words + a.use_words;
  const int g0 = (int)(words / kRelocThreads + 1 < 1024 ? words / kRelocThreads + 1 : 1024);
  hipLaunchKernelGGL(k_reloc_prepare, dim3(g0), dim3(kRelocThreads), 0, s, a);
  const dim3 gk((a.max_prefix + a.T + kRelocThreads - 1) / kRelocThreads, a.batch);
  hipLaunchKernelGGL(k_reloc_mark, gk, dim3(kRelocThreads), 0, s, a);
  hipLaunchKernelGGL(k_reloc_check, gk, dim3(kRelocThreads), 0, s, a);
  const dim3 gc(a.max_prefix > 0 ? (a.max_prefix + kRelocRows - 1) / kRelocRows : 1, a.batch);
  hipLaunchKernelGGL(k_reloc_copy, gc, dim3(kRelocThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace mlv
