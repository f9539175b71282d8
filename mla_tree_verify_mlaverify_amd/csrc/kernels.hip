// gfx950 kernels of DDTree MLA tree-verify attention.
//
//   k_plan        one workgroup: validates prefix lengths and tree parents, builds the
//                 ancestor-or-self bitmask of every tree node, and lays out the split-KV
//                 work units (request key offsets, split length, unit table).
//   k_partial     one workgroup per (split unit, 128-row M tile): gathers the unit's KV
//                 rows through the page_size=1 index table into LDS, computes
//                 S^T = K Q^T and O^T += V^T P^T on bf16 MFMA (32x32x16), with the
//                 online softmax kept in registers; the last unit of a request also
//                 covers the draft-tree keys under the ancestor mask.
//   k_merge       merges the unit partials of every row by their log-sum-exp.
//   k_tree_masks  the bitmask step alone (one wave per request).
//
// The split-KV partial + LSE-merge structure is the one the page "Chunk 66.0"
// (magik.net llmopt segment 66, summary paragraph) describes for its owned verify
// kernel; the tiling below is this library's own, laid out for CDNA4.
#include "mlv_internal.h"

namespace mlv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(1))) const void gmem_cvoid;
typedef __attribute__((address_space(3))) void lds_void;

// ------------------------------------------------------------------------------------------
// Ancestor-or-self bitmask of tree node i: bit j set iff j == i or j is an ancestor of i.
// Parents must satisfy -1 <= parent[j] < j; the walk stops (and reports) on the first
// violation, so it always terminates and never reads outside par[0..i].
__device__ __forceinline__ uint64_t ancestor_mask(const int32_t* __restrict__ par, int i, bool& bad) {
  uint64_t m = 0;
  int p = i;
  while (p >= 0) {
    m |= 1ull << p;
    const int pp = par[p];
    if (pp < -1 || pp >= p) {
      bad = true;
      return 0;
    }
    p = pp;
  }
  return m;
}

// Inclusive scan over the kPlanThreads threads of the block (Hillis-Steele in LDS).
__device__ int block_inclusive_scan(int v, int* s) {
  const int tid = threadIdx.x;
  s[tid] = v;
  __syncthreads();
  for (int off = 1; off < kPlanThreads; off <<= 1) {
    const int t = tid >= off ? s[tid - off] : 0;
    __syncthreads();
    s[tid] += t;
    __syncthreads();
  }
  return s[tid];
}

__global__ __launch_bounds__(kPlanThreads) void k_plan(PlanArgs a) {
  __shared__ int s_scan[kPlanThreads];
  __shared__ uint32_t s_err[kPlanThreads];
  const int tid = threadIdx.x;
  const int B = a.batch, T = a.T;
  s_err[tid] = 0;
  __syncthreads();

  // Tree-ancestor bitmasks: one node per thread.
  for (int n = tid; n < B * T; n += kPlanThreads) {
    const int b = n / T, i = n - b * T;
    bool bad = false;
    const uint64_t m = ancestor_mask(a.tree_parent + (size_t)b * T, i, bad);
    if (bad) atomicOr(&s_err[b], kErrBadParent);
    a.masks[n] = m;
  }
  int P = 0;
  if (tid < B) {
    P = a.prefix_lens[tid];
    if (P < 0 || P > a.max_prefix) {
      atomicOr(&s_err[tid], kErrBadPrefix);
      P = 0;
    }
  }
  __syncthreads();
  uint32_t err = tid < B ? s_err[tid] : 0u;
  // A prefix length outside [0, max_prefix] also hides where the later requests' index
  // segments start, so that request and every later one are poisoned (never read).
  const int bad_here = (tid < B && (err & kErrBadPrefix)) ? 1 : 0;
  const int bad_upto = block_inclusive_scan(bad_here, s_scan);
  __syncthreads();
  if (tid < B && bad_upto > 0) {
    err |= kErrBadPrefix;
    P = 0;
  }

  // Key offsets: exclusive scan of P_b + T.
  const int seg = tid < B ? P + T : 0;
  const int seg_incl = block_inclusive_scan(seg, s_scan);
  const int total_keys = s_scan[kPlanThreads - 1];
  __syncthreads();
  const int total_prefix = total_keys - B * T;

  // Split length: fixed, or the shortest multiple of 32 that spreads the batch's prefix
  // tokens over target_units units (never below min_split).
  int S = a.split_fixed;
  if (S <= 0) {
    const int per = (total_prefix + a.target_units - 1) / a.target_units;
    S = max(a.min_split, (per + kTileKeys - 1) / kTileKeys * kTileKeys);
  }
  int units = tid < B ? max(1, (P + S - 1) / S) : 0;
  const int u_incl = block_inclusive_scan(units, s_scan);
  int total_units = s_scan[kPlanThreads - 1];
  const int first = u_incl - units;
  uint32_t rerr = err;
  if (tid < B && first + units > a.units_cap) {  // cannot happen with the host's grid sizing
    rerr |= kErrBadPrefix;
    units = 0;
  }
  if (total_units > a.units_cap) total_units = a.units_cap;

  if (tid < B) {
    ReqPlan r;
    r.key_off = seg_incl - seg;
    r.prefix_len = P;
    r.first_unit = first;
    r.units = units;
    r.err = rerr;
    r.pad[0] = r.pad[1] = r.pad[2] = 0;
    a.req[tid] = r;
    for (int k = 0; k < units; k++) a.unit_tab[first + k] = tid;
    if (rerr) atomicOr(&a.hdr->sticky_err, rerr);
  }
  if (tid == 0) {
    a.hdr->split_len = S;
    a.hdr->total_units = total_units;
    a.hdr->n_mtiles = a.n_mtiles;
  }
}

__global__ __launch_bounds__(64) void k_tree_masks(const int32_t* __restrict__ par, int T,
                                                    uint64_t* __restrict__ masks, uint32_t* __restrict__ err) {
  const int b = blockIdx.x, i = threadIdx.x;
  bool bad = false;
  uint64_t m = 0;
  if (i < T) m = ancestor_mask(par + (size_t)b * T, i, bad);
  const bool any_bad = __any(bad);
  if (i < T) masks[(size_t)b * T + i] = any_bad ? 0ull : m;
  if (i == 0) err[b] = any_bad ? kErrBadParent : 0u;
}

// ------------------------------------------------------------------------------------------
// LDS tile layout (one tile = 32 keys x 576 bf16 = 36864 B): 9 groups of 8 sixteen-byte
// chunks; group j holds data chunks 8j..8j+7 of every key, key-major, 128 B per key:
//     byte(key, dc) = (dc / 8) * 4096 + key * 128 + ((dc % 8) ^ swz(key)) * 16
// The XOR swizzle (bit-reversed (key >> 1) & 7) keeps both the 16-byte K reads of the
// score MFMA (32 keys x 2 chunks per instruction) and the transposed 8-byte V reads of the
// PV MFMA (8 keys x 4 chunks) free of LDS bank conflicts on gfx950's 64 banks.
// With this layout one wave's direct-to-LDS load of 64 lanes x 16 B fills group j of 8
// keys, so each thread only ever needs the pool row of one key.
__device__ __forceinline__ int swz(int key) {
  const int t = (key >> 1) & 7;
  return ((t & 1) << 2) | (t & 2) | (t >> 2);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// bf16 MFMA 32x32x16 issued through inline asm, so that the score accumulator lives in
// VGPRs and the output accumulator in AGPRs (the compiler would put both in AGPRs and
// then shuffle the 256-register output through VGPRs every tile).  The compiler does not
// track hazards across inline asm, so each statement carries its own wait states:
// 3 before the MFMA (a VALU write of an operand needs 2), and mfma_settle() gives the
// 16+ wait states an 8-pass XDL result needs before VALU or memory instructions read it.
__device__ __forceinline__ void mfma_first_v(f32x16& acc, const u32x4& a, const u32x4& b) {
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_acc_v(f32x16& acc, const u32x4& a, const u32x4& b) {
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_settle_v(f32x16& acc) { asm volatile("s_nop 15\n\ts_nop 3" : "+v"(acc)); }

// ---- Fixed-AGPR output accumulator: block db of O^T lives in a[16db .. 16db+15].
// Only the asm statements below touch these registers, each declaring what it writes.
#define MLV_PV_MFMA_0(V, P) \
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 a[0:15], %0, %1, a[0:15]" :: "v"(V), "v"(P) : "a0", "a1", "a2", "a3", "a4", "a5", "a6", "a7", "a8", "a9", "a10", "a11", "a12", "a13", "a14", "a15")
#define MLV_PV_MFMA_1(V, P) \
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 a[16:31], %0, %1, a[16:31]" :: "v"(V), "v"(P) : "a16", "a17", "a18", "a19", "a20", "a21", "a22", "a23", "a24", "a25", "a26", "a27", "a28", "a29", "a30", "a31")
#define MLV_PV_MFMA_2(V, P) \
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 a[32:47], %0, %1, a[32:47]" :: "v"(V), "v"(P) : "a32", "a33", "a34", "a35", "a36", "a37", "a38", "a39", "a40", "a41", "a42", "a43", "a44", "a45", "a46", "a47")
#define MLV_PV_MFMA_3(V, P) \
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 a[48:63], %0, %1, a[48:63]" :: "v"(V), "v"(P) : "a48", "a49", "a50", "a51", "a52", "a53", "a54", "a55", "a56", "a57", "a58", "a59", "a60", "a61", "a62", "a63")
#define MLV_PV_MFMA_4(V, P) \
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 a[64:79], %0, %1, a[64:79]" :: "v"(V), "v"(P) : "a64", "a65", "a66", "a67", "a68", "a69", "a70", "a71", "a72", "a73", "a74", "a75", "a76", "a77", "a78", "a79")
#define MLV_PV_MFMA_5(V, P) \
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 a[80:95], %0, %1, a[80:95]" :: "v"(V), "v"(P) : "a80", "a81", "a82", "a83", "a84", "a85", "a86", "a87", "a88", "a89", "a90", "a91", "a92", "a93", "a94", "a95")
#define MLV_PV_MFMA_6(V, P) \
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 a[96:111], %0, %1, a[96:111]" :: "v"(V), "v"(P) : "a96", "a97", "a98", "a99", "a100", "a101", "a102", "a103", "a104", "a105", "a106", "a107", "a108", "a109", "a110", "a111")
#define MLV_PV_MFMA_7(V, P) \
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 a[112:127], %0, %1, a[112:127]" :: "v"(V), "v"(P) : "a112", "a113", "a114", "a115", "a116", "a117", "a118", "a119", "a120", "a121", "a122", "a123", "a124", "a125", "a126", "a127")
#define MLV_PV_MFMA_8(V, P) \
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 a[128:143], %0, %1, a[128:143]" :: "v"(V), "v"(P) : "a128", "a129", "a130", "a131", "a132", "a133", "a134", "a135", "a136", "a137", "a138", "a139", "a140", "a141", "a142", "a143")
#define MLV_PV_MFMA_9(V, P) \
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 a[144:159], %0, %1, a[144:159]" :: "v"(V), "v"(P) : "a144", "a145", "a146", "a147", "a148", "a149", "a150", "a151", "a152", "a153", "a154", "a155", "a156", "a157", "a158", "a159")
#define MLV_PV_MFMA_10(V, P) \
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 a[160:175], %0, %1, a[160:175]" :: "v"(V), "v"(P) : "a160", "a161", "a162", "a163", "a164", "a165", "a166", "a167", "a168", "a169", "a170", "a171", "a172", "a173", "a174", "a175")
#define MLV_PV_MFMA_11(V, P) \
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 a[176:191], %0, %1, a[176:191]" :: "v"(V), "v"(P) : "a176", "a177", "a178", "a179", "a180", "a181", "a182", "a183", "a184", "a185", "a186", "a187", "a188", "a189", "a190", "a191")
#define MLV_PV_MFMA_12(V, P) \
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 a[192:207], %0, %1, a[192:207]" :: "v"(V), "v"(P) : "a192", "a193", "a194", "a195", "a196", "a197", "a198", "a199", "a200", "a201", "a202", "a203", "a204", "a205", "a206", "a207")
#define MLV_PV_MFMA_13(V, P) \
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 a[208:223], %0, %1, a[208:223]" :: "v"(V), "v"(P) : "a208", "a209", "a210", "a211", "a212", "a213", "a214", "a215", "a216", "a217", "a218", "a219", "a220", "a221", "a222", "a223")
#define MLV_PV_MFMA_14(V, P) \
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 a[224:239], %0, %1, a[224:239]" :: "v"(V), "v"(P) : "a224", "a225", "a226", "a227", "a228", "a229", "a230", "a231", "a232", "a233", "a234", "a235", "a236", "a237", "a238", "a239")
#define MLV_PV_MFMA_15(V, P) \
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 a[240:255], %0, %1, a[240:255]" :: "v"(V), "v"(P) : "a240", "a241", "a242", "a243", "a244", "a245", "a246", "a247", "a248", "a249", "a250", "a251", "a252", "a253", "a254", "a255")
#define MLV_ZERO_O() \
  asm volatile("v_accvgpr_write_b32 a0, 0\n\tv_accvgpr_write_b32 a1, 0\n\tv_accvgpr_write_b32 a2, 0\n\tv_accvgpr_write_b32 a3, 0\n\tv_accvgpr_write_b32 a4, 0\n\tv_accvgpr_write_b32 a5, 0\n\tv_accvgpr_write_b32 a6, 0\n\tv_accvgpr_write_b32 a7, 0\n\tv_accvgpr_write_b32 a8, 0\n\tv_accvgpr_write_b32 a9, 0\n\tv_accvgpr_write_b32 a10, 0\n\tv_accvgpr_write_b32 a11, 0\n\tv_accvgpr_write_b32 a12, 0\n\tv_accvgpr_write_b32 a13, 0\n\tv_accvgpr_write_b32 a14, 0\n\tv_accvgpr_write_b32 a15, 0\n\tv_accvgpr_write_b32 a16, 0\n\tv_accvgpr_write_b32 a17, 0\n\tv_accvgpr_write_b32 a18, 0\n\tv_accvgpr_write_b32 a19, 0\n\tv_accvgpr_write_b32 a20, 0\n\tv_accvgpr_write_b32 a21, 0\n\tv_accvgpr_write_b32 a22, 0\n\tv_accvgpr_write_b32 a23, 0\n\tv_accvgpr_write_b32 a24, 0\n\tv_accvgpr_write_b32 a25, 0\n\tv_accvgpr_write_b32 a26, 0\n\tv_accvgpr_write_b32 a27, 0\n\tv_accvgpr_write_b32 a28, 0\n\tv_accvgpr_write_b32 a29, 0\n\tv_accvgpr_write_b32 a30, 0\n\tv_accvgpr_write_b32 a31, 0\n\tv_accvgpr_write_b32 a32, 0\n\tv_accvgpr_write_b32 a33, 0\n\tv_accvgpr_write_b32 a34, 0\n\tv_accvgpr_write_b32 a35, 0\n\tv_accvgpr_write_b32 a36, 0\n\tv_accvgpr_write_b32 a37, 0\n\tv_accvgpr_write_b32 a38, 0\n\tv_accvgpr_write_b32 a39, 0\n\tv_accvgpr_write_b32 a40, 0\n\tv_accvgpr_write_b32 a41, 0\n\tv_accvgpr_write_b32 a42, 0\n\tv_accvgpr_write_b32 a43, 0\n\tv_accvgpr_write_b32 a44, 0\n\tv_accvgpr_write_b32 a45, 0\n\tv_accvgpr_write_b32 a46, 0\n\tv_accvgpr_write_b32 a47, 0\n\tv_accvgpr_write_b32 a48, 0\n\tv_accvgpr_write_b32 a49, 0\n\tv_accvgpr_write_b32 a50, 0\n\tv_accvgpr_write_b32 a51, 0\n\tv_accvgpr_write_b32 a52, 0\n\tv_accvgpr_write_b32 a53, 0\n\tv_accvgpr_write_b32 a54, 0\n\tv_accvgpr_write_b32 a55, 0\n\tv_accvgpr_write_b32 a56, 0\n\tv_accvgpr_write_b32 a57, 0\n\tv_accvgpr_write_b32 a58, 0\n\tv_accvgpr_write_b32 a59, 0\n\tv_accvgpr_write_b32 a60, 0\n\tv_accvgpr_write_b32 a61, 0\n\tv_accvgpr_write_b32 a62, 0\n\tv_accvgpr_write_b32 a63, 0\n\tv_accvgpr_write_b32 a64, 0\n\tv_accvgpr_write_b32 a65, 0\n\tv_accvgpr_write_b32 a66, 0\n\tv_accvgpr_write_b32 a67, 0\n\tv_accvgpr_write_b32 a68, 0\n\tv_accvgpr_write_b32 a69, 0\n\tv_accvgpr_write_b32 a70, 0\n\tv_accvgpr_write_b32 a71, 0\n\tv_accvgpr_write_b32 a72, 0\n\tv_accvgpr_write_b32 a73, 0\n\tv_accvgpr_write_b32 a74, 0\n\tv_accvgpr_write_b32 a75, 0\n\tv_accvgpr_write_b32 a76, 0\n\tv_accvgpr_write_b32 a77, 0\n\tv_accvgpr_write_b32 a78, 0\n\tv_accvgpr_write_b32 a79, 0\n\tv_accvgpr_write_b32 a80, 0\n\tv_accvgpr_write_b32 a81, 0\n\tv_accvgpr_write_b32 a82, 0\n\tv_accvgpr_write_b32 a83, 0\n\tv_accvgpr_write_b32 a84, 0\n\tv_accvgpr_write_b32 a85, 0\n\tv_accvgpr_write_b32 a86, 0\n\tv_accvgpr_write_b32 a87, 0\n\tv_accvgpr_write_b32 a88, 0\n\tv_accvgpr_write_b32 a89, 0\n\tv_accvgpr_write_b32 a90, 0\n\tv_accvgpr_write_b32 a91, 0\n\tv_accvgpr_write_b32 a92, 0\n\tv_accvgpr_write_b32 a93, 0\n\tv_accvgpr_write_b32 a94, 0\n\tv_accvgpr_write_b32 a95, 0\n\tv_accvgpr_write_b32 a96, 0\n\tv_accvgpr_write_b32 a97, 0\n\tv_accvgpr_write_b32 a98, 0\n\tv_accvgpr_write_b32 a99, 0\n\tv_accvgpr_write_b32 a100, 0\n\tv_accvgpr_write_b32 a101, 0\n\tv_accvgpr_write_b32 a102, 0\n\tv_accvgpr_write_b32 a103, 0\n\tv_accvgpr_write_b32 a104, 0\n\tv_accvgpr_write_b32 a105, 0\n\tv_accvgpr_write_b32 a106, 0\n\tv_accvgpr_write_b32 a107, 0\n\tv_accvgpr_write_b32 a108, 0\n\tv_accvgpr_write_b32 a109, 0\n\tv_accvgpr_write_b32 a110, 0\n\tv_accvgpr_write_b32 a111, 0\n\tv_accvgpr_write_b32 a112, 0\n\tv_accvgpr_write_b32 a113, 0\n\tv_accvgpr_write_b32 a114, 0\n\tv_accvgpr_write_b32 a115, 0\n\tv_accvgpr_write_b32 a116, 0\n\tv_accvgpr_write_b32 a117, 0\n\tv_accvgpr_write_b32 a118, 0\n\tv_accvgpr_write_b32 a119, 0\n\tv_accvgpr_write_b32 a120, 0\n\tv_accvgpr_write_b32 a121, 0\n\tv_accvgpr_write_b32 a122, 0\n\tv_accvgpr_write_b32 a123, 0\n\tv_accvgpr_write_b32 a124, 0\n\tv_accvgpr_write_b32 a125, 0\n\tv_accvgpr_write_b32 a126, 0\n\tv_accvgpr_write_b32 a127, 0\n\tv_accvgpr_write_b32 a128, 0\n\tv_accvgpr_write_b32 a129, 0\n\tv_accvgpr_write_b32 a130, 0\n\tv_accvgpr_write_b32 a131, 0\n\tv_accvgpr_write_b32 a132, 0\n\tv_accvgpr_write_b32 a133, 0\n\tv_accvgpr_write_b32 a134, 0\n\tv_accvgpr_write_b32 a135, 0\n\tv_accvgpr_write_b32 a136, 0\n\tv_accvgpr_write_b32 a137, 0\n\tv_accvgpr_write_b32 a138, 0\n\tv_accvgpr_write_b32 a139, 0\n\tv_accvgpr_write_b32 a140, 0\n\tv_accvgpr_write_b32 a141, 0\n\tv_accvgpr_write_b32 a142, 0\n\tv_accvgpr_write_b32 a143, 0\n\tv_accvgpr_write_b32 a144, 0\n\tv_accvgpr_write_b32 a145, 0\n\tv_accvgpr_write_b32 a146, 0\n\tv_accvgpr_write_b32 a147, 0\n\tv_accvgpr_write_b32 a148, 0\n\tv_accvgpr_write_b32 a149, 0\n\tv_accvgpr_write_b32 a150, 0\n\tv_accvgpr_write_b32 a151, 0\n\tv_accvgpr_write_b32 a152, 0\n\tv_accvgpr_write_b32 a153, 0\n\tv_accvgpr_write_b32 a154, 0\n\tv_accvgpr_write_b32 a155, 0\n\tv_accvgpr_write_b32 a156, 0\n\tv_accvgpr_write_b32 a157, 0\n\tv_accvgpr_write_b32 a158, 0\n\tv_accvgpr_write_b32 a159, 0\n\tv_accvgpr_write_b32 a160, 0\n\tv_accvgpr_write_b32 a161, 0\n\tv_accvgpr_write_b32 a162, 0\n\tv_accvgpr_write_b32 a163, 0\n\tv_accvgpr_write_b32 a164, 0\n\tv_accvgpr_write_b32 a165, 0\n\tv_accvgpr_write_b32 a166, 0\n\tv_accvgpr_write_b32 a167, 0\n\tv_accvgpr_write_b32 a168, 0\n\tv_accvgpr_write_b32 a169, 0\n\tv_accvgpr_write_b32 a170, 0\n\tv_accvgpr_write_b32 a171, 0\n\tv_accvgpr_write_b32 a172, 0\n\tv_accvgpr_write_b32 a173, 0\n\tv_accvgpr_write_b32 a174, 0\n\tv_accvgpr_write_b32 a175, 0\n\tv_accvgpr_write_b32 a176, 0\n\tv_accvgpr_write_b32 a177, 0\n\tv_accvgpr_write_b32 a178, 0\n\tv_accvgpr_write_b32 a179, 0\n\tv_accvgpr_write_b32 a180, 0\n\tv_accvgpr_write_b32 a181, 0\n\tv_accvgpr_write_b32 a182, 0\n\tv_accvgpr_write_b32 a183, 0\n\tv_accvgpr_write_b32 a184, 0\n\tv_accvgpr_write_b32 a185, 0\n\tv_accvgpr_write_b32 a186, 0\n\tv_accvgpr_write_b32 a187, 0\n\tv_accvgpr_write_b32 a188, 0\n\tv_accvgpr_write_b32 a189, 0\n\tv_accvgpr_write_b32 a190, 0\n\tv_accvgpr_write_b32 a191, 0\n\tv_accvgpr_write_b32 a192, 0\n\tv_accvgpr_write_b32 a193, 0\n\tv_accvgpr_write_b32 a194, 0\n\tv_accvgpr_write_b32 a195, 0\n\tv_accvgpr_write_b32 a196, 0\n\tv_accvgpr_write_b32 a197, 0\n\tv_accvgpr_write_b32 a198, 0\n\tv_accvgpr_write_b32 a199, 0\n\tv_accvgpr_write_b32 a200, 0\n\tv_accvgpr_write_b32 a201, 0\n\tv_accvgpr_write_b32 a202, 0\n\tv_accvgpr_write_b32 a203, 0\n\tv_accvgpr_write_b32 a204, 0\n\tv_accvgpr_write_b32 a205, 0\n\tv_accvgpr_write_b32 a206, 0\n\tv_accvgpr_write_b32 a207, 0\n\tv_accvgpr_write_b32 a208, 0\n\tv_accvgpr_write_b32 a209, 0\n\tv_accvgpr_write_b32 a210, 0\n\tv_accvgpr_write_b32 a211, 0\n\tv_accvgpr_write_b32 a212, 0\n\tv_accvgpr_write_b32 a213, 0\n\tv_accvgpr_write_b32 a214, 0\n\tv_accvgpr_write_b32 a215, 0\n\tv_accvgpr_write_b32 a216, 0\n\tv_accvgpr_write_b32 a217, 0\n\tv_accvgpr_write_b32 a218, 0\n\tv_accvgpr_write_b32 a219, 0\n\tv_accvgpr_write_b32 a220, 0\n\tv_accvgpr_write_b32 a221, 0\n\tv_accvgpr_write_b32 a222, 0\n\tv_accvgpr_write_b32 a223, 0\n\tv_accvgpr_write_b32 a224, 0\n\tv_accvgpr_write_b32 a225, 0\n\tv_accvgpr_write_b32 a226, 0\n\tv_accvgpr_write_b32 a227, 0\n\tv_accvgpr_write_b32 a228, 0\n\tv_accvgpr_write_b32 a229, 0\n\tv_accvgpr_write_b32 a230, 0\n\tv_accvgpr_write_b32 a231, 0\n\tv_accvgpr_write_b32 a232, 0\n\tv_accvgpr_write_b32 a233, 0\n\tv_accvgpr_write_b32 a234, 0\n\tv_accvgpr_write_b32 a235, 0\n\tv_accvgpr_write_b32 a236, 0\n\tv_accvgpr_write_b32 a237, 0\n\tv_accvgpr_write_b32 a238, 0\n\tv_accvgpr_write_b32 a239, 0\n\tv_accvgpr_write_b32 a240, 0\n\tv_accvgpr_write_b32 a241, 0\n\tv_accvgpr_write_b32 a242, 0\n\tv_accvgpr_write_b32 a243, 0\n\tv_accvgpr_write_b32 a244, 0\n\tv_accvgpr_write_b32 a245, 0\n\tv_accvgpr_write_b32 a246, 0\n\tv_accvgpr_write_b32 a247, 0\n\tv_accvgpr_write_b32 a248, 0\n\tv_accvgpr_write_b32 a249, 0\n\tv_accvgpr_write_b32 a250, 0\n\tv_accvgpr_write_b32 a251, 0\n\tv_accvgpr_write_b32 a252, 0\n\tv_accvgpr_write_b32 a253, 0\n\tv_accvgpr_write_b32 a254, 0\n\tv_accvgpr_write_b32 a255, 0" ::: "a0", "a1", "a2", "a3", "a4", "a5", "a6", "a7", "a8", "a9", "a10", "a11", "a12", "a13", "a14", "a15", "a16", "a17", "a18", "a19", "a20", "a21", "a22", "a23", "a24", "a25", "a26", "a27", "a28", "a29", "a30", "a31", "a32", "a33", "a34", "a35", "a36", "a37", "a38", "a39", "a40", "a41", "a42", "a43", "a44", "a45", "a46", "a47", "a48", "a49", "a50", "a51", "a52", "a53", "a54", "a55", "a56", "a57", "a58", "a59", "a60", "a61", "a62", "a63", "a64", "a65", "a66", "a67", "a68", "a69", "a70", "a71", "a72", "a73", "a74", "a75", "a76", "a77", "a78", "a79", "a80", "a81", "a82", "a83", "a84", "a85", "a86", "a87", "a88", "a89", "a90", "a91", "a92", "a93", "a94", "a95", "a96", "a97", "a98", "a99", "a100", "a101", "a102", "a103", "a104", "a105", "a106", "a107", "a108", "a109", "a110", "a111", "a112", "a113", "a114", "a115", "a116", "a117", "a118", "a119", "a120", "a121", "a122", "a123", "a124", "a125", "a126", "a127", "a128", "a129", "a130", "a131", "a132", "a133", "a134", "a135", "a136", "a137", "a138", "a139", "a140", "a141", "a142", "a143", "a144", "a145", "a146", "a147", "a148", "a149", "a150", "a151", "a152", "a153", "a154", "a155", "a156", "a157", "a158", "a159", "a160", "a161", "a162", "a163", "a164", "a165", "a166", "a167", "a168", "a169", "a170", "a171", "a172", "a173", "a174", "a175", "a176", "a177", "a178", "a179", "a180", "a181", "a182", "a183", "a184", "a185", "a186", "a187", "a188", "a189", "a190", "a191", "a192", "a193", "a194", "a195", "a196", "a197", "a198", "a199", "a200", "a201", "a202", "a203", "a204", "a205", "a206", "a207", "a208", "a209", "a210", "a211", "a212", "a213", "a214", "a215", "a216", "a217", "a218", "a219", "a220", "a221", "a222", "a223", "a224", "a225", "a226", "a227", "a228", "a229", "a230", "a231", "a232", "a233", "a234", "a235", "a236", "a237", "a238", "a239", "a240", "a241", "a242", "a243", "a244", "a245", "a246", "a247", "a248", "a249", "a250", "a251", "a252", "a253", "a254", "a255")
#define MLV_READ_O_0(X) \
  asm volatile("v_accvgpr_read_b32 %0, a0\n\tv_accvgpr_read_b32 %1, a1\n\tv_accvgpr_read_b32 %2, a2\n\tv_accvgpr_read_b32 %3, a3\n\tv_accvgpr_read_b32 %4, a4\n\tv_accvgpr_read_b32 %5, a5\n\tv_accvgpr_read_b32 %6, a6\n\tv_accvgpr_read_b32 %7, a7\n\tv_accvgpr_read_b32 %8, a8\n\tv_accvgpr_read_b32 %9, a9\n\tv_accvgpr_read_b32 %10, a10\n\tv_accvgpr_read_b32 %11, a11\n\tv_accvgpr_read_b32 %12, a12\n\tv_accvgpr_read_b32 %13, a13\n\tv_accvgpr_read_b32 %14, a14\n\tv_accvgpr_read_b32 %15, a15" : "=v"(X[0]), "=v"(X[1]), "=v"(X[2]), "=v"(X[3]), "=v"(X[4]), "=v"(X[5]), "=v"(X[6]), "=v"(X[7]), "=v"(X[8]), "=v"(X[9]), "=v"(X[10]), "=v"(X[11]), "=v"(X[12]), "=v"(X[13]), "=v"(X[14]), "=v"(X[15]))
#define MLV_READ_O_1(X) \
  asm volatile("v_accvgpr_read_b32 %0, a16\n\tv_accvgpr_read_b32 %1, a17\n\tv_accvgpr_read_b32 %2, a18\n\tv_accvgpr_read_b32 %3, a19\n\tv_accvgpr_read_b32 %4, a20\n\tv_accvgpr_read_b32 %5, a21\n\tv_accvgpr_read_b32 %6, a22\n\tv_accvgpr_read_b32 %7, a23\n\tv_accvgpr_read_b32 %8, a24\n\tv_accvgpr_read_b32 %9, a25\n\tv_accvgpr_read_b32 %10, a26\n\tv_accvgpr_read_b32 %11, a27\n\tv_accvgpr_read_b32 %12, a28\n\tv_accvgpr_read_b32 %13, a29\n\tv_accvgpr_read_b32 %14, a30\n\tv_accvgpr_read_b32 %15, a31" : "=v"(X[0]), "=v"(X[1]), "=v"(X[2]), "=v"(X[3]), "=v"(X[4]), "=v"(X[5]), "=v"(X[6]), "=v"(X[7]), "=v"(X[8]), "=v"(X[9]), "=v"(X[10]), "=v"(X[11]), "=v"(X[12]), "=v"(X[13]), "=v"(X[14]), "=v"(X[15]))
#define MLV_READ_O_2(X) \
  asm volatile("v_accvgpr_read_b32 %0, a32\n\tv_accvgpr_read_b32 %1, a33\n\tv_accvgpr_read_b32 %2, a34\n\tv_accvgpr_read_b32 %3, a35\n\tv_accvgpr_read_b32 %4, a36\n\tv_accvgpr_read_b32 %5, a37\n\tv_accvgpr_read_b32 %6, a38\n\tv_accvgpr_read_b32 %7, a39\n\tv_accvgpr_read_b32 %8, a40\n\tv_accvgpr_read_b32 %9, a41\n\tv_accvgpr_read_b32 %10, a42\n\tv_accvgpr_read_b32 %11, a43\n\tv_accvgpr_read_b32 %12, a44\n\tv_accvgpr_read_b32 %13, a45\n\tv_accvgpr_read_b32 %14, a46\n\tv_accvgpr_read_b32 %15, a47" : "=v"(X[0]), "=v"(X[1]), "=v"(X[2]), "=v"(X[3]), "=v"(X[4]), "=v"(X[5]), "=v"(X[6]), "=v"(X[7]), "=v"(X[8]), "=v"(X[9]), "=v"(X[10]), "=v"(X[11]), "=v"(X[12]), "=v"(X[13]), "=v"(X[14]), "=v"(X[15]))
#define MLV_READ_O_3(X) \
  asm volatile("v_accvgpr_read_b32 %0, a48\n\tv_accvgpr_read_b32 %1, a49\n\tv_accvgpr_read_b32 %2, a50\n\tv_accvgpr_read_b32 %3, a51\n\tv_accvgpr_read_b32 %4, a52\n\tv_accvgpr_read_b32 %5, a53\n\tv_accvgpr_read_b32 %6, a54\n\tv_accvgpr_read_b32 %7, a55\n\tv_accvgpr_read_b32 %8, a56\n\tv_accvgpr_read_b32 %9, a57\n\tv_accvgpr_read_b32 %10, a58\n\tv_accvgpr_read_b32 %11, a59\n\tv_accvgpr_read_b32 %12, a60\n\tv_accvgpr_read_b32 %13, a61\n\tv_accvgpr_read_b32 %14, a62\n\tv_accvgpr_read_b32 %15, a63" : "=v"(X[0]), "=v"(X[1]), "=v"(X[2]), "=v"(X[3]), "=v"(X[4]), "=v"(X[5]), "=v"(X[6]), "=v"(X[7]), "=v"(X[8]), "=v"(X[9]), "=v"(X[10]), "=v"(X[11]), "=v"(X[12]), "=v"(X[13]), "=v"(X[14]), "=v"(X[15]))
#define MLV_READ_O_4(X) \
  asm volatile("v_accvgpr_read_b32 %0, a64\n\tv_accvgpr_read_b32 %1, a65\n\tv_accvgpr_read_b32 %2, a66\n\tv_accvgpr_read_b32 %3, a67\n\tv_accvgpr_read_b32 %4, a68\n\tv_accvgpr_read_b32 %5, a69\n\tv_accvgpr_read_b32 %6, a70\n\tv_accvgpr_read_b32 %7, a71\n\tv_accvgpr_read_b32 %8, a72\n\tv_accvgpr_read_b32 %9, a73\n\tv_accvgpr_read_b32 %10, a74\n\tv_accvgpr_read_b32 %11, a75\n\tv_accvgpr_read_b32 %12, a76\n\tv_accvgpr_read_b32 %13, a77\n\tv_accvgpr_read_b32 %14, a78\n\tv_accvgpr_read_b32 %15, a79" : "=v"(X[0]), "=v"(X[1]), "=v"(X[2]), "=v"(X[3]), "=v"(X[4]), "=v"(X[5]), "=v"(X[6]), "=v"(X[7]), "=v"(X[8]), "=v"(X[9]), "=v"(X[10]), "=v"(X[11]), "=v"(X[12]), "=v"(X[13]), "=v"(X[14]), "=v"(X[15]))
#define MLV_READ_O_5(X) \
  asm volatile("v_accvgpr_read_b32 %0, a80\n\tv_accvgpr_read_b32 %1, a81\n\tv_accvgpr_read_b32 %2, a82\n\tv_accvgpr_read_b32 %3, a83\n\tv_accvgpr_read_b32 %4, a84\n\tv_accvgpr_read_b32 %5, a85\n\tv_accvgpr_read_b32 %6, a86\n\tv_accvgpr_read_b32 %7, a87\n\tv_accvgpr_read_b32 %8, a88\n\tv_accvgpr_read_b32 %9, a89\n\tv_accvgpr_read_b32 %10, a90\n\tv_accvgpr_read_b32 %11, a91\n\tv_accvgpr_read_b32 %12, a92\n\tv_accvgpr_read_b32 %13, a93\n\tv_accvgpr_read_b32 %14, a94\n\tv_accvgpr_read_b32 %15, a95" : "=v"(X[0]), "=v"(X[1]), "=v"(X[2]), "=v"(X[3]), "=v"(X[4]), "=v"(X[5]), "=v"(X[6]), "=v"(X[7]), "=v"(X[8]), "=v"(X[9]), "=v"(X[10]), "=v"(X[11]), "=v"(X[12]), "=v"(X[13]), "=v"(X[14]), "=v"(X[15]))
#define MLV_READ_O_6(X) \
  asm volatile("v_accvgpr_read_b32 %0, a96\n\tv_accvgpr_read_b32 %1, a97\n\tv_accvgpr_read_b32 %2, a98\n\tv_accvgpr_read_b32 %3, a99\n\tv_accvgpr_read_b32 %4, a100\n\tv_accvgpr_read_b32 %5, a101\n\tv_accvgpr_read_b32 %6, a102\n\tv_accvgpr_read_b32 %7, a103\n\tv_accvgpr_read_b32 %8, a104\n\tv_accvgpr_read_b32 %9, a105\n\tv_accvgpr_read_b32 %10, a106\n\tv_accvgpr_read_b32 %11, a107\n\tv_accvgpr_read_b32 %12, a108\n\tv_accvgpr_read_b32 %13, a109\n\tv_accvgpr_read_b32 %14, a110\n\tv_accvgpr_read_b32 %15, a111" : "=v"(X[0]), "=v"(X[1]), "=v"(X[2]), "=v"(X[3]), "=v"(X[4]), "=v"(X[5]), "=v"(X[6]), "=v"(X[7]), "=v"(X[8]), "=v"(X[9]), "=v"(X[10]), "=v"(X[11]), "=v"(X[12]), "=v"(X[13]), "=v"(X[14]), "=v"(X[15]))
#define MLV_READ_O_7(X) \
  asm volatile("v_accvgpr_read_b32 %0, a112\n\tv_accvgpr_read_b32 %1, a113\n\tv_accvgpr_read_b32 %2, a114\n\tv_accvgpr_read_b32 %3, a115\n\tv_accvgpr_read_b32 %4, a116\n\tv_accvgpr_read_b32 %5, a117\n\tv_accvgpr_read_b32 %6, a118\n\tv_accvgpr_read_b32 %7, a119\n\tv_accvgpr_read_b32 %8, a120\n\tv_accvgpr_read_b32 %9, a121\n\tv_accvgpr_read_b32 %10, a122\n\tv_accvgpr_read_b32 %11, a123\n\tv_accvgpr_read_b32 %12, a124\n\tv_accvgpr_read_b32 %13, a125\n\tv_accvgpr_read_b32 %14, a126\n\tv_accvgpr_read_b32 %15, a127" : "=v"(X[0]), "=v"(X[1]), "=v"(X[2]), "=v"(X[3]), "=v"(X[4]), "=v"(X[5]), "=v"(X[6]), "=v"(X[7]), "=v"(X[8]), "=v"(X[9]), "=v"(X[10]), "=v"(X[11]), "=v"(X[12]), "=v"(X[13]), "=v"(X[14]), "=v"(X[15]))
#define MLV_READ_O_8(X) \
  asm volatile("v_accvgpr_read_b32 %0, a128\n\tv_accvgpr_read_b32 %1, a129\n\tv_accvgpr_read_b32 %2, a130\n\tv_accvgpr_read_b32 %3, a131\n\tv_accvgpr_read_b32 %4, a132\n\tv_accvgpr_read_b32 %5, a133\n\tv_accvgpr_read_b32 %6, a134\n\tv_accvgpr_read_b32 %7, a135\n\tv_accvgpr_read_b32 %8, a136\n\tv_accvgpr_read_b32 %9, a137\n\tv_accvgpr_read_b32 %10, a138\n\tv_accvgpr_read_b32 %11, a139\n\tv_accvgpr_read_b32 %12, a140\n\tv_accvgpr_read_b32 %13, a141\n\tv_accvgpr_read_b32 %14, a142\n\tv_accvgpr_read_b32 %15, a143" : "=v"(X[0]), "=v"(X[1]), "=v"(X[2]), "=v"(X[3]), "=v"(X[4]), "=v"(X[5]), "=v"(X[6]), "=v"(X[7]), "=v"(X[8]), "=v"(X[9]), "=v"(X[10]), "=v"(X[11]), "=v"(X[12]), "=v"(X[13]), "=v"(X[14]), "=v"(X[15]))
#define MLV_READ_O_9(X) \
  asm volatile("v_accvgpr_read_b32 %0, a144\n\tv_accvgpr_read_b32 %1, a145\n\tv_accvgpr_read_b32 %2, a146\n\tv_accvgpr_read_b32 %3, a147\n\tv_accvgpr_read_b32 %4, a148\n\tv_accvgpr_read_b32 %5, a149\n\tv_accvgpr_read_b32 %6, a150\n\tv_accvgpr_read_b32 %7, a151\n\tv_accvgpr_read_b32 %8, a152\n\tv_accvgpr_read_b32 %9, a153\n\tv_accvgpr_read_b32 %10, a154\n\tv_accvgpr_read_b32 %11, a155\n\tv_accvgpr_read_b32 %12, a156\n\tv_accvgpr_read_b32 %13, a157\n\tv_accvgpr_read_b32 %14, a158\n\tv_accvgpr_read_b32 %15, a159" : "=v"(X[0]), "=v"(X[1]), "=v"(X[2]), "=v"(X[3]), "=v"(X[4]), "=v"(X[5]), "=v"(X[6]), "=v"(X[7]), "=v"(X[8]), "=v"(X[9]), "=v"(X[10]), "=v"(X[11]), "=v"(X[12]), "=v"(X[13]), "=v"(X[14]), "=v"(X[15]))
#define MLV_READ_O_10(X) \
  asm volatile("v_accvgpr_read_b32 %0, a160\n\tv_accvgpr_read_b32 %1, a161\n\tv_accvgpr_read_b32 %2, a162\n\tv_accvgpr_read_b32 %3, a163\n\tv_accvgpr_read_b32 %4, a164\n\tv_accvgpr_read_b32 %5, a165\n\tv_accvgpr_read_b32 %6, a166\n\tv_accvgpr_read_b32 %7, a167\n\tv_accvgpr_read_b32 %8, a168\n\tv_accvgpr_read_b32 %9, a169\n\tv_accvgpr_read_b32 %10, a170\n\tv_accvgpr_read_b32 %11, a171\n\tv_accvgpr_read_b32 %12, a172\n\tv_accvgpr_read_b32 %13, a173\n\tv_accvgpr_read_b32 %14, a174\n\tv_accvgpr_read_b32 %15, a175" : "=v"(X[0]), "=v"(X[1]), "=v"(X[2]), "=v"(X[3]), "=v"(X[4]), "=v"(X[5]), "=v"(X[6]), "=v"(X[7]), "=v"(X[8]), "=v"(X[9]), "=v"(X[10]), "=v"(X[11]), "=v"(X[12]), "=v"(X[13]), "=v"(X[14]), "=v"(X[15]))
#define MLV_READ_O_11(X) \
  asm volatile("v_accvgpr_read_b32 %0, a176\n\tv_accvgpr_read_b32 %1, a177\n\tv_accvgpr_read_b32 %2, a178\n\tv_accvgpr_read_b32 %3, a179\n\tv_accvgpr_read_b32 %4, a180\n\tv_accvgpr_read_b32 %5, a181\n\tv_accvgpr_read_b32 %6, a182\n\tv_accvgpr_read_b32 %7, a183\n\tv_accvgpr_read_b32 %8, a184\n\tv_accvgpr_read_b32 %9, a185\n\tv_accvgpr_read_b32 %10, a186\n\tv_accvgpr_read_b32 %11, a187\n\tv_accvgpr_read_b32 %12, a188\n\tv_accvgpr_read_b32 %13, a189\n\tv_accvgpr_read_b32 %14, a190\n\tv_accvgpr_read_b32 %15, a191" : "=v"(X[0]), "=v"(X[1]), "=v"(X[2]), "=v"(X[3]), "=v"(X[4]), "=v"(X[5]), "=v"(X[6]), "=v"(X[7]), "=v"(X[8]), "=v"(X[9]), "=v"(X[10]), "=v"(X[11]), "=v"(X[12]), "=v"(X[13]), "=v"(X[14]), "=v"(X[15]))
#define MLV_READ_O_12(X) \
  asm volatile("v_accvgpr_read_b32 %0, a192\n\tv_accvgpr_read_b32 %1, a193\n\tv_accvgpr_read_b32 %2, a194\n\tv_accvgpr_read_b32 %3, a195\n\tv_accvgpr_read_b32 %4, a196\n\tv_accvgpr_read_b32 %5, a197\n\tv_accvgpr_read_b32 %6, a198\n\tv_accvgpr_read_b32 %7, a199\n\tv_accvgpr_read_b32 %8, a200\n\tv_accvgpr_read_b32 %9, a201\n\tv_accvgpr_read_b32 %10, a202\n\tv_accvgpr_read_b32 %11, a203\n\tv_accvgpr_read_b32 %12, a204\n\tv_accvgpr_read_b32 %13, a205\n\tv_accvgpr_read_b32 %14, a206\n\tv_accvgpr_read_b32 %15, a207" : "=v"(X[0]), "=v"(X[1]), "=v"(X[2]), "=v"(X[3]), "=v"(X[4]), "=v"(X[5]), "=v"(X[6]), "=v"(X[7]), "=v"(X[8]), "=v"(X[9]), "=v"(X[10]), "=v"(X[11]), "=v"(X[12]), "=v"(X[13]), "=v"(X[14]), "=v"(X[15]))
#define MLV_READ_O_13(X) \
  asm volatile("v_accvgpr_read_b32 %0, a208\n\tv_accvgpr_read_b32 %1, a209\n\tv_accvgpr_read_b32 %2, a210\n\tv_accvgpr_read_b32 %3, a211\n\tv_accvgpr_read_b32 %4, a212\n\tv_accvgpr_read_b32 %5, a213\n\tv_accvgpr_read_b32 %6, a214\n\tv_accvgpr_read_b32 %7, a215\n\tv_accvgpr_read_b32 %8, a216\n\tv_accvgpr_read_b32 %9, a217\n\tv_accvgpr_read_b32 %10, a218\n\tv_accvgpr_read_b32 %11, a219\n\tv_accvgpr_read_b32 %12, a220\n\tv_accvgpr_read_b32 %13, a221\n\tv_accvgpr_read_b32 %14, a222\n\tv_accvgpr_read_b32 %15, a223" : "=v"(X[0]), "=v"(X[1]), "=v"(X[2]), "=v"(X[3]), "=v"(X[4]), "=v"(X[5]), "=v"(X[6]), "=v"(X[7]), "=v"(X[8]), "=v"(X[9]), "=v"(X[10]), "=v"(X[11]), "=v"(X[12]), "=v"(X[13]), "=v"(X[14]), "=v"(X[15]))
#define MLV_READ_O_14(X) \
  asm volatile("v_accvgpr_read_b32 %0, a224\n\tv_accvgpr_read_b32 %1, a225\n\tv_accvgpr_read_b32 %2, a226\n\tv_accvgpr_read_b32 %3, a227\n\tv_accvgpr_read_b32 %4, a228\n\tv_accvgpr_read_b32 %5, a229\n\tv_accvgpr_read_b32 %6, a230\n\tv_accvgpr_read_b32 %7, a231\n\tv_accvgpr_read_b32 %8, a232\n\tv_accvgpr_read_b32 %9, a233\n\tv_accvgpr_read_b32 %10, a234\n\tv_accvgpr_read_b32 %11, a235\n\tv_accvgpr_read_b32 %12, a236\n\tv_accvgpr_read_b32 %13, a237\n\tv_accvgpr_read_b32 %14, a238\n\tv_accvgpr_read_b32 %15, a239" : "=v"(X[0]), "=v"(X[1]), "=v"(X[2]), "=v"(X[3]), "=v"(X[4]), "=v"(X[5]), "=v"(X[6]), "=v"(X[7]), "=v"(X[8]), "=v"(X[9]), "=v"(X[10]), "=v"(X[11]), "=v"(X[12]), "=v"(X[13]), "=v"(X[14]), "=v"(X[15]))
#define MLV_READ_O_15(X) \
  asm volatile("v_accvgpr_read_b32 %0, a240\n\tv_accvgpr_read_b32 %1, a241\n\tv_accvgpr_read_b32 %2, a242\n\tv_accvgpr_read_b32 %3, a243\n\tv_accvgpr_read_b32 %4, a244\n\tv_accvgpr_read_b32 %5, a245\n\tv_accvgpr_read_b32 %6, a246\n\tv_accvgpr_read_b32 %7, a247\n\tv_accvgpr_read_b32 %8, a248\n\tv_accvgpr_read_b32 %9, a249\n\tv_accvgpr_read_b32 %10, a250\n\tv_accvgpr_read_b32 %11, a251\n\tv_accvgpr_read_b32 %12, a252\n\tv_accvgpr_read_b32 %13, a253\n\tv_accvgpr_read_b32 %14, a254\n\tv_accvgpr_read_b32 %15, a255" : "=v"(X[0]), "=v"(X[1]), "=v"(X[2]), "=v"(X[3]), "=v"(X[4]), "=v"(X[5]), "=v"(X[6]), "=v"(X[7]), "=v"(X[8]), "=v"(X[9]), "=v"(X[10]), "=v"(X[11]), "=v"(X[12]), "=v"(X[13]), "=v"(X[14]), "=v"(X[15]))

__device__ __forceinline__ void pv_mfma(int db, const u32x4& v, const u32x4& p) {
  switch (db) {
    case 0: MLV_PV_MFMA_0(v, p); break;
    case 1: MLV_PV_MFMA_1(v, p); break;
    case 2: MLV_PV_MFMA_2(v, p); break;
    case 3: MLV_PV_MFMA_3(v, p); break;
    case 4: MLV_PV_MFMA_4(v, p); break;
    case 5: MLV_PV_MFMA_5(v, p); break;
    case 6: MLV_PV_MFMA_6(v, p); break;
    case 7: MLV_PV_MFMA_7(v, p); break;
    case 8: MLV_PV_MFMA_8(v, p); break;
    case 9: MLV_PV_MFMA_9(v, p); break;
    case 10: MLV_PV_MFMA_10(v, p); break;
    case 11: MLV_PV_MFMA_11(v, p); break;
    case 12: MLV_PV_MFMA_12(v, p); break;
    case 13: MLV_PV_MFMA_13(v, p); break;
    case 14: MLV_PV_MFMA_14(v, p); break;
    case 15: MLV_PV_MFMA_15(v, p); break;
  }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float x, float y) {
  const f32x2 v = {x, y};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));  // v_cvt_pk_bf16_f32 (RNE)
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_partial(PartialArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * kTileBytes + kWaves * kQLdsBytes];
  __shared__ int s_restart[2][kWaves];
  lds_char* lds = (lds_char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane >> 5;     // which half of the wave (k sub-block of an MFMA operand)
  const int lrow = lane & 31;  // MFMA column: query row within the wave / key within a tile

  // Workgroup -> (unit, M tile).  Consecutive workgroups go to consecutive XCDs, so the M
  // tiles of one unit are given ids that are equal mod 8: they share an XCD and its L2.
  const int bid = blockIdx.x;
  const int slot = bid >> 3;
  const int mt = slot % a.n_mtiles;
  const int g = (slot / a.n_mtiles) * 8 + (bid & 7);
  if (g >= a.hdr->total_units) return;
  const int b = a.unit_tab[g];
  const ReqPlan R = a.req[b];
  if (R.err & (kErrBadParent | kErrBadPrefix)) return;  // the merge poisons this request
  const int S = a.hdr->split_len;
  const int u = g - R.first_unit;
  const int kbeg = u * S;
  const int npk = max(0, min(S, R.prefix_len - kbeg));  // prefix keys of this unit
  const int npt = (npk + kTileKeys - 1) / kTileKeys;
  const bool last = (u == R.units - 1);
  const int ntiles = npt + (last ? (a.T + kTileKeys - 1) / kTileKeys : 0);
  const int32_t* __restrict__ pidx = a.kv_indices + R.key_off + kbeg;
  const int32_t* __restrict__ tidx = a.kv_indices + R.key_off + R.prefix_len;

  // Contiguous-run fast path: if the unit's prefix slots are one run first, first+1, ...,
  // rows are addressed from `first` without reading the index table again.
  int run_base = -1;
  if (!(a.flags & 1u) && npk > 0) {
    const int first = pidx[0];
    int ok = first >= 0 && (int64_t)first + npk <= a.pool_slots;
    for (int k0 = 0; ok && k0 < npk; k0 += kThreads) {
      const int k = k0 + tid;
      ok = __syncthreads_and(k >= npk || pidx[k] == first + k);
    }
    if (ok) run_base = first;
  }

  // Query rows of this wave: row r of the request is (node r / H, head r % H).
  const int r = mt * kRowsPerBlock + w * kRowsPerWave + lrow;
  const bool rvalid = r < a.M;
  // B operand of the score MFMA: Q[row][16kk + 8h .. +7] (bf16 pairs).  The first kQReg
  // k-steps stay in VGPRs for the whole unit; the rest are parked in this wave's LDS slice
  // (lane-major, conflict-free) to leave the register allocator headroom.
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
  lds_u32x4* qlds = (lds_u32x4*)(lds + 2 * kTileBytes + w * kQLdsBytes) + lane;
  u32x4 qf[kQReg];
  {
    // rows past M (last M tile) read the request's last row; their results are dropped
    const u32x4* qp = reinterpret_cast<const u32x4*>(a.q + ((size_t)b * a.M + (rvalid ? r : a.M - 1)) * kLatent) + h;
#pragma unroll
    for (int kk = 0; kk < kQReg; kk++) qf[kk] = qp[2 * kk];
#pragma unroll
    for (int kk = kQReg; kk < 36; kk++) qlds[(kk - kQReg) * 64] = qp[2 * kk];
  }
  uint64_t anc = ~0ull;
  if (last && rvalid) anc = a.masks[(size_t)b * a.T + r / a.H];

  // Gather geometry: thread tid loads 9 chunks of key kt of every tile.
  const int kt = tid >> 3;
  const int kxor = (tid & 7) ^ swz(kt);

  auto fetch_index = [&](int t) -> int {
    if (t < npt) {
      const int nv = min(kTileKeys, npk - t * kTileKeys);
      const int k = t * kTileKeys + (kt < nv ? kt : 0);  // tail keys re-read the tile's first key
      return run_base >= 0 ? run_base + k : pidx[k];
    }
    const int tt = t - npt;
    const int nv = min(kTileKeys, a.T - tt * kTileKeys);
    return tidx[tt * kTileKeys + (kt < nv ? kt : 0)];
  };
  auto issue_tile = [&](int t, int idx) {
    if ((uint32_t)idx >= (uint64_t)a.pool_slots) {  // never read outside the pool
      atomicOr(a.sticky_err, kErrBadIndex);
      atomicOr(&a.req_rw[b].err, kErrBadIndex);
      idx = 0;
    }
    const char* src = reinterpret_cast<const char*>(a.pool) + (size_t)idx * a.row_stride_bytes + kxor * 16;
    lds_char* dst = lds + (t & 1) * kTileBytes + w * 1024;
#pragma unroll
    for (int j = 0; j < 9; j++)
      __builtin_amdgcn_global_load_lds((gmem_cvoid*)(src + j * 128), (lds_void*)(dst + j * 4096), 16, 0, 0);
  };

  // Per-lane LDS offsets.  K operand of the score MFMA: key lrow, chunk 2kk + h.
  int koff[4];
#pragma unroll
  for (int c = 0; c < 4; c++) koff[c] = lrow * 128 + (((2 * c + h) ^ swz(lrow)) << 4);
  // V operand of the PV MFMA, read transposed (ds_read_b64_tr_b16): within each group of 16
  // lanes, lane m supplies the address of V[key0 + m/4][d0 + 4(m%4) .. +3] and receives
  // V[key0 .. key0+3][d0 + m].  Keys 16mf + 8rd + 4h + (m%16)/4, columns 32db + 16*half + 4(m%4).
  int voff[2][2];
  {
    const int half = (lane >> 4) & 1, mm = lane & 15;
    const int keyl = 4 * h + (mm >> 2);
#pragma unroll
    for (int dbp = 0; dbp < 2; dbp++)
#pragma unroll
      for (int rd = 0; rd < 2; rd++) {
        const int key = 8 * rd + keyl;  // + 16mf: same swizzle
        const int dc7 = 4 * dbp + 2 * half + ((mm & 3) >> 1);
        voff[dbp][rd] = keyl * 128 + ((dc7 ^ swz(key)) << 4) + 8 * (mm & 1);
      }
  }

  // Softmax state of row lrow (log2 domain).  mref is a fixed reference for the whole
  // pass over the unit: it is set by the first tile in which the row sees a key, and every
  // later probability 2^(s - mref) is kept <= 2^16.  A tile whose maximum exceeds mref by
  // more than 16 raises mref and restarts the unit (rare: it needs a score jump of > 11
  // nats after the first tile), so the output accumulator is never rescaled.
  float mref = -INFINITY;
  float lrun = 0.f;
  MLV_ZERO_O();  // O^T[d = 32db + ..][row] accumulates in a[0..255]

  issue_tile(0, fetch_index(0));
  int idx_next = ntiles > 1 ? fetch_index(1) : 0;
  int t = 0;
  for (;;) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's loads of tile t landed
    __syncthreads();                     // ... and everyone's; tile t-1 is no longer read
    if (t > 0) {
      const int* fl = s_restart[(t - 1) & 1];
      if (fl[0] | fl[1] | fl[2] | fl[3]) {  // some wave raised its reference: start over
        t = 0;
        MLV_ZERO_O();
        lrun = 0.f;
        issue_tile(0, fetch_index(0));
        if (ntiles > 1) idx_next = fetch_index(1);
        continue;
      }
    }
    if (t == ntiles) break;
    if (t + 1 < ntiles) {
      issue_tile(t + 1, idx_next);
      if (t + 2 < ntiles) idx_next = fetch_index(t + 2);
    }

    const lds_char* kb = lds + (t & 1) * kTileBytes;
    const bool tree = t >= npt;
    const int tt = t - npt;
    const int nv = tree ? min(kTileKeys, a.T - tt * kTileKeys) : min(kTileKeys, npk - t * kTileKeys);

    // S^T[key][row] = sum_d K[key][d] Q[row][d]
    f32x16 sacc;
#pragma unroll
    for (int kk = 0; kk < 36; kk++) {
      const u32x4 kv = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
          kb + (kk >> 2) * 4096 + koff[kk & 3]);
      const u32x4 qv = kk < kQReg ? qf[kk < kQReg ? kk : 0] : qlds[(kk < kQReg ? 0 : kk - kQReg) * 64];
      if (kk == 0)
        mfma_first_v(sacc, kv, qv);
      else
        mfma_acc_v(sacc, kv, qv);
    }
    mfma_settle_v(sacc);

    // Scores of row lrow; this lane holds keys 8(v/4) + 4h + v%4 of the tile.
    float sv[16];
    float tmax = -INFINITY;
    const uint64_t tmask = tree ? (anc >> (tt * kTileKeys)) : ~0ull;
#pragma unroll
    for (int v = 0; v < 16; v++) {
      const int key = 8 * (v >> 2) + 4 * h + (v & 3);
      const bool vis = key < nv && ((tmask >> key) & 1ull);
      sv[v] = vis ? sacc[v] * a.scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, sv[v]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const bool raise = mref != -INFINITY && tmax > mref + 16.0f;
    const bool trig = __any(raise);
    if (lane == 0) s_restart[t & 1][w] = trig ? 1 : 0;
    if (trig) {  // this pass is abandoned; keep the larger reference for the next one
      mref = fmaxf(mref, tmax);
      t++;
      continue;
    }
    if (mref == -INFINITY) mref = tmax;  // first keys this row sees (may still be -inf)

    float p[16];
#pragma unroll
    for (int v = 0; v < 16; v++) {
      p[v] = (sv[v] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sv[v] - mref);
      lrun += p[v];
    }
    u32x4 pb[2];
#pragma unroll
    for (int mf = 0; mf < 2; mf++) {
      const u32x4 pk = {pack_bf16x2(p[8 * mf + 0], p[8 * mf + 1]), pack_bf16x2(p[8 * mf + 2], p[8 * mf + 3]),
                        pack_bf16x2(p[8 * mf + 4], p[8 * mf + 5]), pack_bf16x2(p[8 * mf + 6], p[8 * mf + 7])};
      pb[mf] = pk;
    }

    // O^T[d][row] += sum_key V^T[d][key] P^T[key][row]; MFMA k index 8h + j maps to the
    // keys this lane already holds (4h + j, then 8 + 4h + j - 4; +16 for the second MFMA).
#pragma unroll
    for (int db = 0; db < 16; db++) {
#pragma unroll
      for (int mf = 0; mf < 2; mf++) {
        const lds_char* vb = kb + (db >> 1) * 4096 + mf * 16 * 128;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vb + voff[db & 1][0]));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vb + 8 * 128 + voff[db & 1][1]));
        const u32x4 vop = __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        pv_mfma(db, vop, pb[mf]);
      }
    }
    t++;
  }

  asm volatile("s_nop 15\n\ts_nop 3" ::: "memory");  // last PV MFMA results settle before reads
  const float lt = lrun + __shfl_xor(lrun, 32);
  const float inv = 1.0f / lt;
  const float lse2 = mref + __builtin_amdgcn_logf(lt);  // log2-domain lse of this unit
  if (rvalid) {
    float* po = a.part_o + ((size_t)g * a.M + r) * kVdim + 4 * h;
#pragma unroll
    for (int db = 0; db < 16; db++) {
      float X[16];
      switch (db) {
        case 0: MLV_READ_O_0(X); break;
        case 1: MLV_READ_O_1(X); break;
        case 2: MLV_READ_O_2(X); break;
        case 3: MLV_READ_O_3(X); break;
        case 4: MLV_READ_O_4(X); break;
        case 5: MLV_READ_O_5(X); break;
        case 6: MLV_READ_O_6(X); break;
        case 7: MLV_READ_O_7(X); break;
        case 8: MLV_READ_O_8(X); break;
        case 9: MLV_READ_O_9(X); break;
        case 10: MLV_READ_O_10(X); break;
        case 11: MLV_READ_O_11(X); break;
        case 12: MLV_READ_O_12(X); break;
        case 13: MLV_READ_O_13(X); break;
        case 14: MLV_READ_O_14(X); break;
        case 15: MLV_READ_O_15(X); break;
      }
#pragma unroll
      for (int q4 = 0; q4 < 4; q4++) {
        f32x4 v = {X[4 * q4] * inv, X[4 * q4 + 1] * inv, X[4 * q4 + 2] * inv, X[4 * q4 + 3] * inv};
        *reinterpret_cast<f32x4*>(po + 32 * db + 8 * q4) = v;
      }
    }
    if (h == 0) a.part_lse[(size_t)g * a.M + r] = lse2;
  }
}

// ------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (u >> 16) | 0x0040u;  // quiet NaN
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// One thread per 4 output columns; 128 threads per row, 2 rows per workgroup.
__global__ __launch_bounds__(256) void k_merge(MergeArgs a) {
  const int row = blockIdx.x * 2 + (threadIdx.x >> 7);
  if (row >= a.batch * a.M) return;
  const int c4 = threadIdx.x & 127;
  const int b = row / a.M, r = row - b * a.M;
  const ReqPlan R = a.req[b];
  uint2* po = reinterpret_cast<uint2*>(a.out + (size_t)row * kVdim) + c4;
  if (R.err) {
    *po = make_uint2(0x7FC07FC0u, 0x7FC07FC0u);
    if (c4 == 0) a.lse[row] = __uint_as_float(0x7FC00000u);
    return;
  }
  const float* pl = a.part_lse + (size_t)R.first_unit * a.M + r;
  float m = -INFINITY;
  for (int u = 0; u < R.units; u++) m = fmaxf(m, pl[(size_t)u * a.M]);
  float z = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const float* pob = a.part_o + ((size_t)R.first_unit * a.M + r) * kVdim + 4 * c4;
  for (int u = 0; u < R.units; u++) {
    const float lu = pl[(size_t)u * a.M];
    const float wu = (lu == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(lu - m);
    const f32x4 o = *reinterpret_cast<const f32x4*>(pob + (size_t)u * a.M * kVdim);
    z += wu;
    acc += wu * o;
  }
  const float inv = 1.0f / z;
  *po = make_uint2(bf16_rne_bits(acc[0] * inv) | (bf16_rne_bits(acc[1] * inv) << 16),
                   bf16_rne_bits(acc[2] * inv) | (bf16_rne_bits(acc[3] * inv) << 16));
  if (c4 == 0) a.lse[row] = (m + __builtin_amdgcn_logf(z)) * 0.69314718055994531f;
}

// ------------------------------------------------------------------------------------------
hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(kPlanThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_partial(const PartialArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL(k_partial, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  const int rows = a.batch * a.M;
  hipLaunchKernelGGL(k_merge, dim3((rows + 1) / 2), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_tree_masks(const int32_t* tree_parent, int batch, int T, uint64_t* masks, uint32_t* err,
                             hipStream_t s) {
  hipLaunchKernelGGL(k_tree_masks, dim3(batch), dim3(64), 0, s, tree_parent, T, masks, err);
  return hipGetLastError();
}

}  // namespace mlv
