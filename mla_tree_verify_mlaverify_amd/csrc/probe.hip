// Scattered-row read probe (measurement only, not part of the verify pass): the rate at which
// one GPU reads pool rows named by an index list, through the two 16-byte load paths the
// verify kernel can use.  The page "Chunk 66.1" (magik.net llmopt segment 66, summary
// paragraph) credits 128-bit vectorized bf16 KV loads for its kernel's gain on scattered
// page_size=1 reads; this probe measures that access pattern on its own.
//
// Every workgroup of 256 threads reads tiles of 32 rows (8 lanes per 1,152-byte row, 9
// sixteen-byte chunks per lane), kInFlight tiles per round with all their loads issued
// before any is used, tiles strided over the grid.
//   kLds = false: non-temporal global_load_dwordx4 into VGPRs, folded by XOR (one word per
//                 thread is written to `sink`, so that no load is dead);
//   kLds = true:  global_load_lds_dwordx4 straight into an LDS ring of kInFlight tiles, as the
//                 verify kernel gathers (one word of the ring per thread goes to `sink`).
// Index entries outside [0, pool_slots) read row 0.
#include "mlv_internal.h"

namespace mlv {

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kProbeInFlight = 4;  // tiles per round: 36 sixteen-byte loads per thread

__device__ __forceinline__ void probe_lds_dma(const char* gaddr, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gaddr), "s"(m0) : "memory");
}

template <bool kLds>
__global__ __launch_bounds__(256) void k_probe_gather(const char* __restrict__ pool, int64_t stride, int64_t slots,
                                                      const int32_t* __restrict__ idx, int n, uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(1024))) char ring[kLds ? kProbeInFlight * kTileBytes : 16];
  const int tid = threadIdx.x, key = tid >> 3, chunk = tid & 7;
  const int ntiles = (n + kTileKeys - 1) / kTileKeys;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int t0 = blockIdx.x * kProbeInFlight; t0 < ntiles; t0 += gridDim.x * kProbeInFlight) {
    int e[kProbeInFlight];
#pragma unroll
    for (int k = 0; k < kProbeInFlight; k++) e[k] = idx[min((t0 + k) * kTileKeys + key, n - 1)];  // tail: last row
    const char* src[kProbeInFlight];
#pragma unroll
    for (int k = 0; k < kProbeInFlight; k++) {
      const uint64_t row = (uint32_t)e[k] < (uint64_t)slots ? (uint32_t)e[k] : 0u;
      src[k] = pool + row * (uint64_t)stride + chunk * 16;
    }
    if constexpr (kLds) {
      __syncthreads();  // the ring's previous round has been read
#pragma unroll
      for (int k = 0; k < kProbeInFlight; k++) {
        const uint32_t base = (uint32_t)(uintptr_t)(ring + k * kTileBytes) + wave * 1024;
#pragma unroll
        for (int j = 0; j < 9; j++) probe_lds_dma(src[k] + j * 128, __builtin_amdgcn_readfirstlane(base + j * 4096));
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      __syncthreads();
      acc.x ^= *reinterpret_cast<const uint32_t*>(ring + (tid * 4 + t0) % (kProbeInFlight * kTileBytes));
    } else {
      u32x4 v[kProbeInFlight][9];
#pragma unroll
      for (int k = 0; k < kProbeInFlight; k++)
#pragma unroll
        for (int j = 0; j < 9; j++)
          v[k][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src[k] + j * 128));
      __builtin_amdgcn_sched_barrier(0);  // every load of the round is issued before the first fold
#pragma unroll
      for (int k = 0; k < kProbeInFlight; k++)
#pragma unroll
        for (int j = 0; j < 9; j++) acc ^= v[k][j];
    }
  }
  sink[(size_t)blockIdx.x * 256 + tid] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

hipError_t launch_probe_gather(const void* pool, int64_t stride_bytes, int64_t slots, const int32_t* idx, int n,
                               int lds, int grid, uint32_t* sink, hipStream_t s) {
  const char* p = static_cast<const char*>(pool);
  if (lds)
    hipLaunchKernelGGL(k_probe_gather<true>, dim3(grid), dim3(256), 0, s, p, stride_bytes, slots, idx, n, sink);
  else
    hipLaunchKernelGGL(k_probe_gather<false>, dim3(grid), dim3(256), 0, s, p, stride_bytes, slots, idx, n, sink);
  return hipGetLastError();
}

}  // namespace mlv
