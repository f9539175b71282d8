// gfx950 kernels of greedy draft-tree acceptance, the step after the verify pass: the
// target's logits at every tree node decide which drafted tokens are committed (the
// "Chunk 66.0" summary reports the resulting commit lengths).  Rule: from the position
// before the tree, take the argmax of the current row and move to the lowest-index child
// (a first-level node at the start) whose draft token equals it; stop when none does; the
// argmax of the last row visited is the bonus token.
//
// Two launches:
//   k_accept_argmax one workgroup per (logits row, 8192-logit chunk): the chunk's best
//                   (value, index) becomes an orderable 64-bit key merged into the row's
//                   key with one atomic max; the key orders by value (NaN below every
//                   number, -0 equal to +0), then by lower index, so the atomic max of the
//                   chunk keys is the row's argmax under that order
//   k_accept_walk   one wave per request: the nodes are the lanes, each step a ballot;
//                   afterwards it zeroes the request's keys, so the workspace is clean for
//                   the next call (create clears it once) and no clearing launch is needed
// (Letting the last argmax workgroup of a request walk, found with a release/acquire
// counter, measured three times slower: the device-scope release of every workgroup
// costs more than the second launch.)
#include "mlv_internal.h"

namespace mlv {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kArgThreads = 256;
constexpr int kArgChunk = 8192;  // logits per workgroup (32 per thread)

__device__ __forceinline__ uint64_t arg_key(float v, uint32_t idx) {
  uint32_t u = __float_as_uint(v);
  uint32_t k;
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) {
    k = 0u;  // NaN: below every number
  } else {
    if (u == 0x80000000u) u = 0u;  // -0 ranks as +0
    k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  }
  return ((uint64_t)k << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)x, off, 64);
    const uint32_t hi = __shfl_xor((uint32_t)(x >> 32), off, 64);
    x = max_u64(x, ((uint64_t)hi << 32) | lo);
  }
  return x;
}

// Tree walk of request b from its argmax keys (one wave; lane l holds nodes l, l + 64, ...).
__device__ void accept_walk(const AcceptArgs& a, int b) {
  constexpr int G = kMaxTree / 64;  // node groups per lane
  const int lane = threadIdx.x, T = a.T;
  int par[G], tok[G], mine[G];
  bool bad = false;
#pragma unroll
  for (int k = 0; k < G; k++) {
    const int i = lane + 64 * k;
    par[k] = i < T ? a.tree_parent[(int64_t)b * T + i] : -2;
    tok[k] = i < T ? a.draft_tokens[(int64_t)b * T + i] : -1;
    bad |= i < T && (par[k] < -1 || par[k] >= i);
    mine[k] = -1;
  }
  bad = __any(bad);
  uint64_t* krow = a.keys + (int64_t)b * (T + 1);
  // keys were merged with atomics: read them at device scope
  auto token_of = [&](int row) -> int {
    const uint64_t k = __hip_atomic_load(krow + row, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return (int)(0xFFFFFFFFu - (uint32_t)k);
  };
  int cur = -1, row = 0, n = 0;
  if (!bad) {
    // the next node has a larger index than the current one, so at most T steps
    for (int step = 0; step < T; step++) {
      const int g = token_of(row);
      int nxt = -1;
#pragma unroll
      for (int k = G - 1; k >= 0; k--) {  // lowest matching node: the first group that has one
        const uint64_t m = __ballot(par[k] == cur && tok[k] == g);
        if (m) nxt = 64 * k + __builtin_ctzll(m);
      }
      if (nxt < 0) break;
#pragma unroll
      for (int k = 0; k < G; k++)
        if (lane + 64 * k == n) mine[k] = nxt;
      n++;
      cur = nxt;
      row = 1 + nxt;
    }
  }
  const int g = token_of(row);
#pragma unroll
  for (int k = 0; k < G; k++) {
    const int i = lane + 64 * k;
    if (i < T) a.accepted[(int64_t)b * T + i] = i < n ? mine[k] : -1;
  }
  if (lane == 0) {
    a.accept_len[b] = n;
    a.bonus[b] = g;
    if (bad) atomicOr(a.sticky_err, kErrBadParent);
  }
  // leave the request's keys at zero for the next call
  for (int r = lane; r <= T; r += 64) __hip_atomic_store(krow + r, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(64) void k_accept_walk(AcceptArgs a) { accept_walk(a, blockIdx.x); }

template <bool kVec>
__global__ __launch_bounds__(kArgThreads) void k_accept_argmax(AcceptArgs a) {
  const int row = blockIdx.x / a.chunks;
  const int64_t c0 = (int64_t)(blockIdx.x - row * a.chunks) * kArgChunk;
  const int64_t c1 = c0 + kArgChunk < a.vocab ? c0 + kArgChunk : a.vocab;
  const float* lr = a.logits + (int64_t)row * a.vocab;
  uint64_t best = 0ull;
  if (kVec) {  // vocab % 4 == 0 and 16-byte aligned rows: 4 logits per load, 8 loads in flight
    for (int64_t i = c0 + 4 * threadIdx.x; i < c1; i += 8 * 4 * kArgThreads) {
      f32x4 v[8];
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const int64_t e = i + (int64_t)j * 4 * kArgThreads;
        if (e < c1) v[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(lr + e));
      }
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const int64_t e = i + (int64_t)j * 4 * kArgThreads;
        if (e < c1) {
#pragma unroll
          for (int q = 0; q < 4; q++) best = max_u64(best, arg_key(v[j][q], (uint32_t)(e + q)));
        }
      }
    }
  } else {
    for (int64_t e = c0 + threadIdx.x; e < c1; e += kArgThreads) best = max_u64(best, arg_key(lr[e], (uint32_t)e));
  }
  best = wave_max_u64(best);
  __shared__ uint64_t s_best[kArgThreads / 64];
  if ((threadIdx.x & 63) == 0) s_best[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t m = s_best[0];
#pragma unroll
    for (int w = 1; w < kArgThreads / 64; w++) m = max_u64(m, s_best[w]);
    atomicMax(reinterpret_cast<unsigned long long*>(a.keys + row), (unsigned long long)m);
  }
}

}  // namespace

hipError_t launch_accept(const AcceptArgs& a, hipStream_t s) {
  const bool vec = (a.vocab % 4 == 0) && (((uintptr_t)a.logits & 15) == 0);
  const dim3 grid((unsigned)((int64_t)a.rows * a.chunks));
  if (vec)
    hipLaunchKernelGGL(k_accept_argmax<true>, grid, dim3(kArgThreads), 0, s, a);
  else
    hipLaunchKernelGGL(k_accept_argmax<false>, grid, dim3(kArgThreads), 0, s, a);
  hipLaunchKernelGGL(k_accept_walk, dim3(a.batch), dim3(64), 0, s, a);
  return hipGetLastError();
}

int accept_chunks(int64_t vocab) { return (int)((vocab + kArgChunk - 1) / kArgChunk); }

}  // namespace mlv
