// gfx950 kernels of DDTree MLA tree-verify attention.
//
//   k_partial     one workgroup per (split unit, 128-row M tile).  It first derives the work
//                 partition from the prefix lengths (every workgroup computes the same
//                 plan; workgroup 0 also publishes it), then gathers the unit's KV rows
//                 through the page_size=1 index table into LDS and computes
//                 S^T = K Q^T and O^T += V^T P^T on bf16 MFMA (32x32x16), with the softmax
//                 kept in registers; the last unit of a request also covers the draft-tree
//                 keys under the ancestor-or-self bitmask it builds in LDS.  A call with a
//                 tree size per request is planned by M tiles (plan_wave).
//   k_merge       merges the unit partials of every row by their log-sum-exp.
//   k_tree_masks  the bitmask step alone (one wave per request).
//
// The split-KV partial + LSE-merge structure is the one the page "Chunk 66.0"
// (magik.net llmopt segment 66, summary paragraph) describes for its owned verify
// kernel; the tiling below is this library's own, laid out for CDNA4.
#include "mlv_internal.h"

namespace mlv {

template <int N>
struct IntC {
  static constexpr int value = N;
};

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
// Ancestor-or-self bitmasks of the T nodes of one tree (row a.1): bit j of node i's mask
// (word j / 64 of W) is set iff j == i or j is an ancestor of i.  Pointer jumping in LDS:
// after round r, node i holds its ancestors at distance < 2^r and points at the one at
// distance 2^r, so ceil(log2 T) rounds suffice whatever the depth.  Thread i < T owns node
// i (the workgroup has at least T threads); s_m holds T x W words, s_jump T ints.  Parents
// must satisfy -1 <= parent[i] < i; the result says whether one does not (then the masks
// are not meaningful).  Called by every thread of the workgroup; thread i < T passes
// parent[i] in p.
template <int W>
__device__ bool build_masks(int p, int T, uint64_t* s_m, int* s_jump) {
  const int i = threadIdx.x;
  int jmp = -1;
  bool bad = false;
  if (i < T) {
    bad = p < -1 || p >= i;
    jmp = bad ? -1 : p;
#pragma unroll
    for (int w = 0; w < W; w++) s_m[i * W + w] = (w == (i >> 6)) ? 1ull << (i & 63) : 0ull;
    s_jump[i] = jmp;
  }
  const bool any_bad = __syncthreads_or(bad) != 0;
  for (int span = 1; span < T; span <<= 1) {
    uint64_t add[W];
    int nj = -1;
#pragma unroll
    for (int w = 0; w < W; w++) add[w] = 0ull;
    if (i < T && jmp >= 0) {
#pragma unroll
      for (int w = 0; w < W; w++) add[w] = s_m[jmp * W + w];
      nj = s_jump[jmp];
    }
    __syncthreads();
    if (i < T && jmp >= 0) {
#pragma unroll
      for (int w = 0; w < W; w++) s_m[i * W + w] |= add[w];
      s_jump[i] = nj;
      jmp = nj;
    }
    __syncthreads();
  }
  return any_bad;
}

// Standalone mask step: one workgroup per request writes masks[b][i][0 .. ceil(T/64) - 1].
__global__ __launch_bounds__(kThreads) void k_tree_masks(const int32_t* __restrict__ par, int T,
                                                         uint64_t* __restrict__ masks, uint32_t* __restrict__ err) {
  __shared__ uint64_t s_m[kMaxTree * kMaxTreeWords];
  __shared__ int s_jump[kMaxTree];
  const int b = blockIdx.x, i = threadIdx.x;
  const bool bad = build_masks<kMaxTreeWords>(i < T ? par[(size_t)b * T + i] : 0, T, s_m, s_jump);
  const int W = (T + 63) >> 6;
  for (int k = i; k < T * W; k += kThreads) {
    const int node = k / W, w = k - node * W;
    masks[(size_t)b * T * W + k] = bad ? 0ull : s_m[node * kMaxTreeWords + w];
  }
  if (i == 0) err[b] = bad ? kErrBadParent : 0u;
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

// 16-byte global -> LDS load (gfx950 global_load_lds_dwordx4): lane i's 16 bytes land at
// LDS address m0 + offset + 16 i, read from the lane's address + offset.  Piece J of a row is
// the row's 16-byte chunk J * 8 + (lane's chunk) and goes to lds_base + 4096 J: the caller
// passes the row's address, the instruction offset adds 128 J to both addresses, and M0
// (one scalar add) takes the rest of the LDS step, 4096 J - 128 J.  Issued through asm so
// that the compiler does not make every later LDS read wait for it; completion is awaited
// explicitly (vmcnt(0) + barrier) before the tile is read.  The s_nop is the wait state
// between an M0 write and its LDS-DMA use.  M0 is a reserved register that a clobber list
// cannot protect; the build instead checks that no compiler-generated instruction uses it.
template <int J>
__device__ __forceinline__ void lds_dma16(const char* gaddr, uint32_t lds_base) {
  asm volatile("s_add_u32 m0, %1, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:%3"
               ::"v"(gaddr), "s"(lds_base), "n"(J * (4096 - 128)), "n"(J * 128));
}

// Score MFMAs (bf16 32x32x16) are compiler builtins with VGPR accumulators (the library is
// built with the VGPR form of MFMA forced), so the compiler schedules them and inserts their
// hazard wait states.  The output accumulator is different: it sits in fixed AGPRs that only
// inline asm touches (below), since the compiler would otherwise move the 256-register block
// through VGPRs every tile.
__device__ __forceinline__ void mfma_first_v(f32x16& acc, const u32x4& a, const u32x4& b) {
  const f32x16 z = {};
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), z, 0, 0, 0);
}
__device__ __forceinline__ void mfma_acc_v(f32x16& acc, const u32x4& a, const u32x4& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

// ---- Fixed-AGPR output accumulator: block db of O^T lives in a[16db .. 16db+15].
// Only the asm statements below touch these registers, each declaring what it writes.
#define MLV_PV_MFMA_0(V, P) \
  asm volatile("v_mfma_f32_32x32x16_bf16 a[0:15], %0, %1, a[0:15]" :: "v"(V), "v"(P) : "a0", "a1", "a2", "a3", "a4", "a5", "a6", "a7", "a8", "a9", "a10", "a11", "a12", "a13", "a14", "a15")
#define MLV_PV_MFMA_1(V, P) \
  asm volatile("v_mfma_f32_32x32x16_bf16 a[16:31], %0, %1, a[16:31]" :: "v"(V), "v"(P) : "a16", "a17", "a18", "a19", "a20", "a21", "a22", "a23", "a24", "a25", "a26", "a27", "a28", "a29", "a30", "a31")
#define MLV_PV_MFMA_2(V, P) \
  asm volatile("v_mfma_f32_32x32x16_bf16 a[32:47], %0, %1, a[32:47]" :: "v"(V), "v"(P) : "a32", "a33", "a34", "a35", "a36", "a37", "a38", "a39", "a40", "a41", "a42", "a43", "a44", "a45", "a46", "a47")
#define MLV_PV_MFMA_3(V, P) \
  asm volatile("v_mfma_f32_32x32x16_bf16 a[48:63], %0, %1, a[48:63]" :: "v"(V), "v"(P) : "a48", "a49", "a50", "a51", "a52", "a53", "a54", "a55", "a56", "a57", "a58", "a59", "a60", "a61", "a62", "a63")
#define MLV_PV_MFMA_4(V, P) \
  asm volatile("v_mfma_f32_32x32x16_bf16 a[64:79], %0, %1, a[64:79]" :: "v"(V), "v"(P) : "a64", "a65", "a66", "a67", "a68", "a69", "a70", "a71", "a72", "a73", "a74", "a75", "a76", "a77", "a78", "a79")
#define MLV_PV_MFMA_5(V, P) \
  asm volatile("v_mfma_f32_32x32x16_bf16 a[80:95], %0, %1, a[80:95]" :: "v"(V), "v"(P) : "a80", "a81", "a82", "a83", "a84", "a85", "a86", "a87", "a88", "a89", "a90", "a91", "a92", "a93", "a94", "a95")
#define MLV_PV_MFMA_6(V, P) \
  asm volatile("v_mfma_f32_32x32x16_bf16 a[96:111], %0, %1, a[96:111]" :: "v"(V), "v"(P) : "a96", "a97", "a98", "a99", "a100", "a101", "a102", "a103", "a104", "a105", "a106", "a107", "a108", "a109", "a110", "a111")
#define MLV_PV_MFMA_7(V, P) \
  asm volatile("v_mfma_f32_32x32x16_bf16 a[112:127], %0, %1, a[112:127]" :: "v"(V), "v"(P) : "a112", "a113", "a114", "a115", "a116", "a117", "a118", "a119", "a120", "a121", "a122", "a123", "a124", "a125", "a126", "a127")
#define MLV_PV_MFMA_8(V, P) \
  asm volatile("v_mfma_f32_32x32x16_bf16 a[128:143], %0, %1, a[128:143]" :: "v"(V), "v"(P) : "a128", "a129", "a130", "a131", "a132", "a133", "a134", "a135", "a136", "a137", "a138", "a139", "a140", "a141", "a142", "a143")
#define MLV_PV_MFMA_9(V, P) \
  asm volatile("v_mfma_f32_32x32x16_bf16 a[144:159], %0, %1, a[144:159]" :: "v"(V), "v"(P) : "a144", "a145", "a146", "a147", "a148", "a149", "a150", "a151", "a152", "a153", "a154", "a155", "a156", "a157", "a158", "a159")
#define MLV_PV_MFMA_10(V, P) \
  asm volatile("v_mfma_f32_32x32x16_bf16 a[160:175], %0, %1, a[160:175]" :: "v"(V), "v"(P) : "a160", "a161", "a162", "a163", "a164", "a165", "a166", "a167", "a168", "a169", "a170", "a171", "a172", "a173", "a174", "a175")
#define MLV_PV_MFMA_11(V, P) \
  asm volatile("v_mfma_f32_32x32x16_bf16 a[176:191], %0, %1, a[176:191]" :: "v"(V), "v"(P) : "a176", "a177", "a178", "a179", "a180", "a181", "a182", "a183", "a184", "a185", "a186", "a187", "a188", "a189", "a190", "a191")
#define MLV_PV_MFMA_12(V, P) \
  asm volatile("v_mfma_f32_32x32x16_bf16 a[192:207], %0, %1, a[192:207]" :: "v"(V), "v"(P) : "a192", "a193", "a194", "a195", "a196", "a197", "a198", "a199", "a200", "a201", "a202", "a203", "a204", "a205", "a206", "a207")
#define MLV_PV_MFMA_13(V, P) \
  asm volatile("v_mfma_f32_32x32x16_bf16 a[208:223], %0, %1, a[208:223]" :: "v"(V), "v"(P) : "a208", "a209", "a210", "a211", "a212", "a213", "a214", "a215", "a216", "a217", "a218", "a219", "a220", "a221", "a222", "a223")
#define MLV_PV_MFMA_14(V, P) \
  asm volatile("v_mfma_f32_32x32x16_bf16 a[224:239], %0, %1, a[224:239]" :: "v"(V), "v"(P) : "a224", "a225", "a226", "a227", "a228", "a229", "a230", "a231", "a232", "a233", "a234", "a235", "a236", "a237", "a238", "a239")
#define MLV_PV_MFMA_15(V, P) \
  asm volatile("v_mfma_f32_32x32x16_bf16 a[240:255], %0, %1, a[240:255]" :: "v"(V), "v"(P) : "a240", "a241", "a242", "a243", "a244", "a245", "a246", "a247", "a248", "a249", "a250", "a251", "a252", "a253", "a254", "a255")
// The accumulator zeroed by the matrix core: 16 MFMAs of zero operands with a zero C input
// (128 bytes of code and 64 issue cycles, against 256 accumulator writes).
#define MLV_ZERO_O(Z) \
  asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 a[0:15], %0, %0, 0\n\tv_mfma_f32_32x32x16_bf16 a[16:31], %0, %0, 0\n\tv_mfma_f32_32x32x16_bf16 a[32:47], %0, %0, 0\n\tv_mfma_f32_32x32x16_bf16 a[48:63], %0, %0, 0\n\tv_mfma_f32_32x32x16_bf16 a[64:79], %0, %0, 0\n\tv_mfma_f32_32x32x16_bf16 a[80:95], %0, %0, 0\n\tv_mfma_f32_32x32x16_bf16 a[96:111], %0, %0, 0\n\tv_mfma_f32_32x32x16_bf16 a[112:127], %0, %0, 0\n\tv_mfma_f32_32x32x16_bf16 a[128:143], %0, %0, 0\n\tv_mfma_f32_32x32x16_bf16 a[144:159], %0, %0, 0\n\tv_mfma_f32_32x32x16_bf16 a[160:175], %0, %0, 0\n\tv_mfma_f32_32x32x16_bf16 a[176:191], %0, %0, 0\n\tv_mfma_f32_32x32x16_bf16 a[192:207], %0, %0, 0\n\tv_mfma_f32_32x32x16_bf16 a[208:223], %0, %0, 0\n\tv_mfma_f32_32x32x16_bf16 a[224:239], %0, %0, 0\n\tv_mfma_f32_32x32x16_bf16 a[240:255], %0, %0, 0" :: "v"(Z) : "a0", "a1", "a2", "a3", "a4", "a5", "a6", "a7", "a8", "a9", "a10", "a11", "a12", "a13", "a14", "a15", "a16", "a17", "a18", "a19", "a20", "a21", "a22", "a23", "a24", "a25", "a26", "a27", "a28", "a29", "a30", "a31", "a32", "a33", "a34", "a35", "a36", "a37", "a38", "a39", "a40", "a41", "a42", "a43", "a44", "a45", "a46", "a47", "a48", "a49", "a50", "a51", "a52", "a53", "a54", "a55", "a56", "a57", "a58", "a59", "a60", "a61", "a62", "a63", "a64", "a65", "a66", "a67", "a68", "a69", "a70", "a71", "a72", "a73", "a74", "a75", "a76", "a77", "a78", "a79", "a80", "a81", "a82", "a83", "a84", "a85", "a86", "a87", "a88", "a89", "a90", "a91", "a92", "a93", "a94", "a95", "a96", "a97", "a98", "a99", "a100", "a101", "a102", "a103", "a104", "a105", "a106", "a107", "a108", "a109", "a110", "a111", "a112", "a113", "a114", "a115", "a116", "a117", "a118", "a119", "a120", "a121", "a122", "a123", "a124", "a125", "a126", "a127", "a128", "a129", "a130", "a131", "a132", "a133", "a134", "a135", "a136", "a137", "a138", "a139", "a140", "a141", "a142", "a143", "a144", "a145", "a146", "a147", "a148", "a149", "a150", "a151", "a152", "a153", "a154", "a155", "a156", "a157", "a158", "a159", "a160", "a161", "a162", "a163", "a164", "a165", "a166", "a167", "a168", "a169", "a170", "a171", "a172", "a173", "a174", "a175", "a176", "a177", "a178", "a179", "a180", "a181", "a182", "a183", "a184", "a185", "a186", "a187", "a188", "a189", "a190", "a191", "a192", "a193", "a194", "a195", "a196", "a197", "a198", "a199", "a200", "a201", "a202", "a203", "a204", "a205", "a206", "a207", "a208", "a209", "a210", "a211", "a212", "a213", "a214", "a215", "a216", "a217", "a218", "a219", "a220", "a221", "a222", "a223", "a224", "a225", "a226", "a227", "a228", "a229", "a230", "a231", "a232", "a233", "a234", "a235", "a236", "a237", "a238", "a239", "a240", "a241", "a242", "a243", "a244", "a245", "a246", "a247", "a248", "a249", "a250", "a251", "a252", "a253", "a254", "a255")
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

#define MLV_WRITE_O_0(X) \
  asm volatile("v_accvgpr_write_b32 a0, %0\n\tv_accvgpr_write_b32 a1, %1\n\tv_accvgpr_write_b32 a2, %2\n\tv_accvgpr_write_b32 a3, %3\n\tv_accvgpr_write_b32 a4, %4\n\tv_accvgpr_write_b32 a5, %5\n\tv_accvgpr_write_b32 a6, %6\n\tv_accvgpr_write_b32 a7, %7\n\tv_accvgpr_write_b32 a8, %8\n\tv_accvgpr_write_b32 a9, %9\n\tv_accvgpr_write_b32 a10, %10\n\tv_accvgpr_write_b32 a11, %11\n\tv_accvgpr_write_b32 a12, %12\n\tv_accvgpr_write_b32 a13, %13\n\tv_accvgpr_write_b32 a14, %14\n\tv_accvgpr_write_b32 a15, %15" :: "v"(X[0]), "v"(X[1]), "v"(X[2]), "v"(X[3]), "v"(X[4]), "v"(X[5]), "v"(X[6]), "v"(X[7]), "v"(X[8]), "v"(X[9]), "v"(X[10]), "v"(X[11]), "v"(X[12]), "v"(X[13]), "v"(X[14]), "v"(X[15]) : "a0", "a1", "a2", "a3", "a4", "a5", "a6", "a7", "a8", "a9", "a10", "a11", "a12", "a13", "a14", "a15")
#define MLV_WRITE_O_1(X) \
  asm volatile("v_accvgpr_write_b32 a16, %0\n\tv_accvgpr_write_b32 a17, %1\n\tv_accvgpr_write_b32 a18, %2\n\tv_accvgpr_write_b32 a19, %3\n\tv_accvgpr_write_b32 a20, %4\n\tv_accvgpr_write_b32 a21, %5\n\tv_accvgpr_write_b32 a22, %6\n\tv_accvgpr_write_b32 a23, %7\n\tv_accvgpr_write_b32 a24, %8\n\tv_accvgpr_write_b32 a25, %9\n\tv_accvgpr_write_b32 a26, %10\n\tv_accvgpr_write_b32 a27, %11\n\tv_accvgpr_write_b32 a28, %12\n\tv_accvgpr_write_b32 a29, %13\n\tv_accvgpr_write_b32 a30, %14\n\tv_accvgpr_write_b32 a31, %15" :: "v"(X[0]), "v"(X[1]), "v"(X[2]), "v"(X[3]), "v"(X[4]), "v"(X[5]), "v"(X[6]), "v"(X[7]), "v"(X[8]), "v"(X[9]), "v"(X[10]), "v"(X[11]), "v"(X[12]), "v"(X[13]), "v"(X[14]), "v"(X[15]) : "a16", "a17", "a18", "a19", "a20", "a21", "a22", "a23", "a24", "a25", "a26", "a27", "a28", "a29", "a30", "a31")
#define MLV_WRITE_O_2(X) \
  asm volatile("v_accvgpr_write_b32 a32, %0\n\tv_accvgpr_write_b32 a33, %1\n\tv_accvgpr_write_b32 a34, %2\n\tv_accvgpr_write_b32 a35, %3\n\tv_accvgpr_write_b32 a36, %4\n\tv_accvgpr_write_b32 a37, %5\n\tv_accvgpr_write_b32 a38, %6\n\tv_accvgpr_write_b32 a39, %7\n\tv_accvgpr_write_b32 a40, %8\n\tv_accvgpr_write_b32 a41, %9\n\tv_accvgpr_write_b32 a42, %10\n\tv_accvgpr_write_b32 a43, %11\n\tv_accvgpr_write_b32 a44, %12\n\tv_accvgpr_write_b32 a45, %13\n\tv_accvgpr_write_b32 a46, %14\n\tv_accvgpr_write_b32 a47, %15" :: "v"(X[0]), "v"(X[1]), "v"(X[2]), "v"(X[3]), "v"(X[4]), "v"(X[5]), "v"(X[6]), "v"(X[7]), "v"(X[8]), "v"(X[9]), "v"(X[10]), "v"(X[11]), "v"(X[12]), "v"(X[13]), "v"(X[14]), "v"(X[15]) : "a32", "a33", "a34", "a35", "a36", "a37", "a38", "a39", "a40", "a41", "a42", "a43", "a44", "a45", "a46", "a47")
#define MLV_WRITE_O_3(X) \
  asm volatile("v_accvgpr_write_b32 a48, %0\n\tv_accvgpr_write_b32 a49, %1\n\tv_accvgpr_write_b32 a50, %2\n\tv_accvgpr_write_b32 a51, %3\n\tv_accvgpr_write_b32 a52, %4\n\tv_accvgpr_write_b32 a53, %5\n\tv_accvgpr_write_b32 a54, %6\n\tv_accvgpr_write_b32 a55, %7\n\tv_accvgpr_write_b32 a56, %8\n\tv_accvgpr_write_b32 a57, %9\n\tv_accvgpr_write_b32 a58, %10\n\tv_accvgpr_write_b32 a59, %11\n\tv_accvgpr_write_b32 a60, %12\n\tv_accvgpr_write_b32 a61, %13\n\tv_accvgpr_write_b32 a62, %14\n\tv_accvgpr_write_b32 a63, %15" :: "v"(X[0]), "v"(X[1]), "v"(X[2]), "v"(X[3]), "v"(X[4]), "v"(X[5]), "v"(X[6]), "v"(X[7]), "v"(X[8]), "v"(X[9]), "v"(X[10]), "v"(X[11]), "v"(X[12]), "v"(X[13]), "v"(X[14]), "v"(X[15]) : "a48", "a49", "a50", "a51", "a52", "a53", "a54", "a55", "a56", "a57", "a58", "a59", "a60", "a61", "a62", "a63")
#define MLV_WRITE_O_4(X) \
  asm volatile("v_accvgpr_write_b32 a64, %0\n\tv_accvgpr_write_b32 a65, %1\n\tv_accvgpr_write_b32 a66, %2\n\tv_accvgpr_write_b32 a67, %3\n\tv_accvgpr_write_b32 a68, %4\n\tv_accvgpr_write_b32 a69, %5\n\tv_accvgpr_write_b32 a70, %6\n\tv_accvgpr_write_b32 a71, %7\n\tv_accvgpr_write_b32 a72, %8\n\tv_accvgpr_write_b32 a73, %9\n\tv_accvgpr_write_b32 a74, %10\n\tv_accvgpr_write_b32 a75, %11\n\tv_accvgpr_write_b32 a76, %12\n\tv_accvgpr_write_b32 a77, %13\n\tv_accvgpr_write_b32 a78, %14\n\tv_accvgpr_write_b32 a79, %15" :: "v"(X[0]), "v"(X[1]), "v"(X[2]), "v"(X[3]), "v"(X[4]), "v"(X[5]), "v"(X[6]), "v"(X[7]), "v"(X[8]), "v"(X[9]), "v"(X[10]), "v"(X[11]), "v"(X[12]), "v"(X[13]), "v"(X[14]), "v"(X[15]) : "a64", "a65", "a66", "a67", "a68", "a69", "a70", "a71", "a72", "a73", "a74", "a75", "a76", "a77", "a78", "a79")
#define MLV_WRITE_O_5(X) \
  asm volatile("v_accvgpr_write_b32 a80, %0\n\tv_accvgpr_write_b32 a81, %1\n\tv_accvgpr_write_b32 a82, %2\n\tv_accvgpr_write_b32 a83, %3\n\tv_accvgpr_write_b32 a84, %4\n\tv_accvgpr_write_b32 a85, %5\n\tv_accvgpr_write_b32 a86, %6\n\tv_accvgpr_write_b32 a87, %7\n\tv_accvgpr_write_b32 a88, %8\n\tv_accvgpr_write_b32 a89, %9\n\tv_accvgpr_write_b32 a90, %10\n\tv_accvgpr_write_b32 a91, %11\n\tv_accvgpr_write_b32 a92, %12\n\tv_accvgpr_write_b32 a93, %13\n\tv_accvgpr_write_b32 a94, %14\n\tv_accvgpr_write_b32 a95, %15" :: "v"(X[0]), "v"(X[1]), "v"(X[2]), "v"(X[3]), "v"(X[4]), "v"(X[5]), "v"(X[6]), "v"(X[7]), "v"(X[8]), "v"(X[9]), "v"(X[10]), "v"(X[11]), "v"(X[12]), "v"(X[13]), "v"(X[14]), "v"(X[15]) : "a80", "a81", "a82", "a83", "a84", "a85", "a86", "a87", "a88", "a89", "a90", "a91", "a92", "a93", "a94", "a95")
#define MLV_WRITE_O_6(X) \
  asm volatile("v_accvgpr_write_b32 a96, %0\n\tv_accvgpr_write_b32 a97, %1\n\tv_accvgpr_write_b32 a98, %2\n\tv_accvgpr_write_b32 a99, %3\n\tv_accvgpr_write_b32 a100, %4\n\tv_accvgpr_write_b32 a101, %5\n\tv_accvgpr_write_b32 a102, %6\n\tv_accvgpr_write_b32 a103, %7\n\tv_accvgpr_write_b32 a104, %8\n\tv_accvgpr_write_b32 a105, %9\n\tv_accvgpr_write_b32 a106, %10\n\tv_accvgpr_write_b32 a107, %11\n\tv_accvgpr_write_b32 a108, %12\n\tv_accvgpr_write_b32 a109, %13\n\tv_accvgpr_write_b32 a110, %14\n\tv_accvgpr_write_b32 a111, %15" :: "v"(X[0]), "v"(X[1]), "v"(X[2]), "v"(X[3]), "v"(X[4]), "v"(X[5]), "v"(X[6]), "v"(X[7]), "v"(X[8]), "v"(X[9]), "v"(X[10]), "v"(X[11]), "v"(X[12]), "v"(X[13]), "v"(X[14]), "v"(X[15]) : "a96", "a97", "a98", "a99", "a100", "a101", "a102", "a103", "a104", "a105", "a106", "a107", "a108", "a109", "a110", "a111")
#define MLV_WRITE_O_7(X) \
  asm volatile("v_accvgpr_write_b32 a112, %0\n\tv_accvgpr_write_b32 a113, %1\n\tv_accvgpr_write_b32 a114, %2\n\tv_accvgpr_write_b32 a115, %3\n\tv_accvgpr_write_b32 a116, %4\n\tv_accvgpr_write_b32 a117, %5\n\tv_accvgpr_write_b32 a118, %6\n\tv_accvgpr_write_b32 a119, %7\n\tv_accvgpr_write_b32 a120, %8\n\tv_accvgpr_write_b32 a121, %9\n\tv_accvgpr_write_b32 a122, %10\n\tv_accvgpr_write_b32 a123, %11\n\tv_accvgpr_write_b32 a124, %12\n\tv_accvgpr_write_b32 a125, %13\n\tv_accvgpr_write_b32 a126, %14\n\tv_accvgpr_write_b32 a127, %15" :: "v"(X[0]), "v"(X[1]), "v"(X[2]), "v"(X[3]), "v"(X[4]), "v"(X[5]), "v"(X[6]), "v"(X[7]), "v"(X[8]), "v"(X[9]), "v"(X[10]), "v"(X[11]), "v"(X[12]), "v"(X[13]), "v"(X[14]), "v"(X[15]) : "a112", "a113", "a114", "a115", "a116", "a117", "a118", "a119", "a120", "a121", "a122", "a123", "a124", "a125", "a126", "a127")
#define MLV_WRITE_O_8(X) \
  asm volatile("v_accvgpr_write_b32 a128, %0\n\tv_accvgpr_write_b32 a129, %1\n\tv_accvgpr_write_b32 a130, %2\n\tv_accvgpr_write_b32 a131, %3\n\tv_accvgpr_write_b32 a132, %4\n\tv_accvgpr_write_b32 a133, %5\n\tv_accvgpr_write_b32 a134, %6\n\tv_accvgpr_write_b32 a135, %7\n\tv_accvgpr_write_b32 a136, %8\n\tv_accvgpr_write_b32 a137, %9\n\tv_accvgpr_write_b32 a138, %10\n\tv_accvgpr_write_b32 a139, %11\n\tv_accvgpr_write_b32 a140, %12\n\tv_accvgpr_write_b32 a141, %13\n\tv_accvgpr_write_b32 a142, %14\n\tv_accvgpr_write_b32 a143, %15" :: "v"(X[0]), "v"(X[1]), "v"(X[2]), "v"(X[3]), "v"(X[4]), "v"(X[5]), "v"(X[6]), "v"(X[7]), "v"(X[8]), "v"(X[9]), "v"(X[10]), "v"(X[11]), "v"(X[12]), "v"(X[13]), "v"(X[14]), "v"(X[15]) : "a128", "a129", "a130", "a131", "a132", "a133", "a134", "a135", "a136", "a137", "a138", "a139", "a140", "a141", "a142", "a143")
#define MLV_WRITE_O_9(X) \
  asm volatile("v_accvgpr_write_b32 a144, %0\n\tv_accvgpr_write_b32 a145, %1\n\tv_accvgpr_write_b32 a146, %2\n\tv_accvgpr_write_b32 a147, %3\n\tv_accvgpr_write_b32 a148, %4\n\tv_accvgpr_write_b32 a149, %5\n\tv_accvgpr_write_b32 a150, %6\n\tv_accvgpr_write_b32 a151, %7\n\tv_accvgpr_write_b32 a152, %8\n\tv_accvgpr_write_b32 a153, %9\n\tv_accvgpr_write_b32 a154, %10\n\tv_accvgpr_write_b32 a155, %11\n\tv_accvgpr_write_b32 a156, %12\n\tv_accvgpr_write_b32 a157, %13\n\tv_accvgpr_write_b32 a158, %14\n\tv_accvgpr_write_b32 a159, %15" :: "v"(X[0]), "v"(X[1]), "v"(X[2]), "v"(X[3]), "v"(X[4]), "v"(X[5]), "v"(X[6]), "v"(X[7]), "v"(X[8]), "v"(X[9]), "v"(X[10]), "v"(X[11]), "v"(X[12]), "v"(X[13]), "v"(X[14]), "v"(X[15]) : "a144", "a145", "a146", "a147", "a148", "a149", "a150", "a151", "a152", "a153", "a154", "a155", "a156", "a157", "a158", "a159")
#define MLV_WRITE_O_10(X) \
  asm volatile("v_accvgpr_write_b32 a160, %0\n\tv_accvgpr_write_b32 a161, %1\n\tv_accvgpr_write_b32 a162, %2\n\tv_accvgpr_write_b32 a163, %3\n\tv_accvgpr_write_b32 a164, %4\n\tv_accvgpr_write_b32 a165, %5\n\tv_accvgpr_write_b32 a166, %6\n\tv_accvgpr_write_b32 a167, %7\n\tv_accvgpr_write_b32 a168, %8\n\tv_accvgpr_write_b32 a169, %9\n\tv_accvgpr_write_b32 a170, %10\n\tv_accvgpr_write_b32 a171, %11\n\tv_accvgpr_write_b32 a172, %12\n\tv_accvgpr_write_b32 a173, %13\n\tv_accvgpr_write_b32 a174, %14\n\tv_accvgpr_write_b32 a175, %15" :: "v"(X[0]), "v"(X[1]), "v"(X[2]), "v"(X[3]), "v"(X[4]), "v"(X[5]), "v"(X[6]), "v"(X[7]), "v"(X[8]), "v"(X[9]), "v"(X[10]), "v"(X[11]), "v"(X[12]), "v"(X[13]), "v"(X[14]), "v"(X[15]) : "a160", "a161", "a162", "a163", "a164", "a165", "a166", "a167", "a168", "a169", "a170", "a171", "a172", "a173", "a174", "a175")
#define MLV_WRITE_O_11(X) \
  asm volatile("v_accvgpr_write_b32 a176, %0\n\tv_accvgpr_write_b32 a177, %1\n\tv_accvgpr_write_b32 a178, %2\n\tv_accvgpr_write_b32 a179, %3\n\tv_accvgpr_write_b32 a180, %4\n\tv_accvgpr_write_b32 a181, %5\n\tv_accvgpr_write_b32 a182, %6\n\tv_accvgpr_write_b32 a183, %7\n\tv_accvgpr_write_b32 a184, %8\n\tv_accvgpr_write_b32 a185, %9\n\tv_accvgpr_write_b32 a186, %10\n\tv_accvgpr_write_b32 a187, %11\n\tv_accvgpr_write_b32 a188, %12\n\tv_accvgpr_write_b32 a189, %13\n\tv_accvgpr_write_b32 a190, %14\n\tv_accvgpr_write_b32 a191, %15" :: "v"(X[0]), "v"(X[1]), "v"(X[2]), "v"(X[3]), "v"(X[4]), "v"(X[5]), "v"(X[6]), "v"(X[7]), "v"(X[8]), "v"(X[9]), "v"(X[10]), "v"(X[11]), "v"(X[12]), "v"(X[13]), "v"(X[14]), "v"(X[15]) : "a176", "a177", "a178", "a179", "a180", "a181", "a182", "a183", "a184", "a185", "a186", "a187", "a188", "a189", "a190", "a191")
#define MLV_WRITE_O_12(X) \
  asm volatile("v_accvgpr_write_b32 a192, %0\n\tv_accvgpr_write_b32 a193, %1\n\tv_accvgpr_write_b32 a194, %2\n\tv_accvgpr_write_b32 a195, %3\n\tv_accvgpr_write_b32 a196, %4\n\tv_accvgpr_write_b32 a197, %5\n\tv_accvgpr_write_b32 a198, %6\n\tv_accvgpr_write_b32 a199, %7\n\tv_accvgpr_write_b32 a200, %8\n\tv_accvgpr_write_b32 a201, %9\n\tv_accvgpr_write_b32 a202, %10\n\tv_accvgpr_write_b32 a203, %11\n\tv_accvgpr_write_b32 a204, %12\n\tv_accvgpr_write_b32 a205, %13\n\tv_accvgpr_write_b32 a206, %14\n\tv_accvgpr_write_b32 a207, %15" :: "v"(X[0]), "v"(X[1]), "v"(X[2]), "v"(X[3]), "v"(X[4]), "v"(X[5]), "v"(X[6]), "v"(X[7]), "v"(X[8]), "v"(X[9]), "v"(X[10]), "v"(X[11]), "v"(X[12]), "v"(X[13]), "v"(X[14]), "v"(X[15]) : "a192", "a193", "a194", "a195", "a196", "a197", "a198", "a199", "a200", "a201", "a202", "a203", "a204", "a205", "a206", "a207")
#define MLV_WRITE_O_13(X) \
  asm volatile("v_accvgpr_write_b32 a208, %0\n\tv_accvgpr_write_b32 a209, %1\n\tv_accvgpr_write_b32 a210, %2\n\tv_accvgpr_write_b32 a211, %3\n\tv_accvgpr_write_b32 a212, %4\n\tv_accvgpr_write_b32 a213, %5\n\tv_accvgpr_write_b32 a214, %6\n\tv_accvgpr_write_b32 a215, %7\n\tv_accvgpr_write_b32 a216, %8\n\tv_accvgpr_write_b32 a217, %9\n\tv_accvgpr_write_b32 a218, %10\n\tv_accvgpr_write_b32 a219, %11\n\tv_accvgpr_write_b32 a220, %12\n\tv_accvgpr_write_b32 a221, %13\n\tv_accvgpr_write_b32 a222, %14\n\tv_accvgpr_write_b32 a223, %15" :: "v"(X[0]), "v"(X[1]), "v"(X[2]), "v"(X[3]), "v"(X[4]), "v"(X[5]), "v"(X[6]), "v"(X[7]), "v"(X[8]), "v"(X[9]), "v"(X[10]), "v"(X[11]), "v"(X[12]), "v"(X[13]), "v"(X[14]), "v"(X[15]) : "a208", "a209", "a210", "a211", "a212", "a213", "a214", "a215", "a216", "a217", "a218", "a219", "a220", "a221", "a222", "a223")
#define MLV_WRITE_O_14(X) \
  asm volatile("v_accvgpr_write_b32 a224, %0\n\tv_accvgpr_write_b32 a225, %1\n\tv_accvgpr_write_b32 a226, %2\n\tv_accvgpr_write_b32 a227, %3\n\tv_accvgpr_write_b32 a228, %4\n\tv_accvgpr_write_b32 a229, %5\n\tv_accvgpr_write_b32 a230, %6\n\tv_accvgpr_write_b32 a231, %7\n\tv_accvgpr_write_b32 a232, %8\n\tv_accvgpr_write_b32 a233, %9\n\tv_accvgpr_write_b32 a234, %10\n\tv_accvgpr_write_b32 a235, %11\n\tv_accvgpr_write_b32 a236, %12\n\tv_accvgpr_write_b32 a237, %13\n\tv_accvgpr_write_b32 a238, %14\n\tv_accvgpr_write_b32 a239, %15" :: "v"(X[0]), "v"(X[1]), "v"(X[2]), "v"(X[3]), "v"(X[4]), "v"(X[5]), "v"(X[6]), "v"(X[7]), "v"(X[8]), "v"(X[9]), "v"(X[10]), "v"(X[11]), "v"(X[12]), "v"(X[13]), "v"(X[14]), "v"(X[15]) : "a224", "a225", "a226", "a227", "a228", "a229", "a230", "a231", "a232", "a233", "a234", "a235", "a236", "a237", "a238", "a239")
#define MLV_WRITE_O_15(X) \
  asm volatile("v_accvgpr_write_b32 a240, %0\n\tv_accvgpr_write_b32 a241, %1\n\tv_accvgpr_write_b32 a242, %2\n\tv_accvgpr_write_b32 a243, %3\n\tv_accvgpr_write_b32 a244, %4\n\tv_accvgpr_write_b32 a245, %5\n\tv_accvgpr_write_b32 a246, %6\n\tv_accvgpr_write_b32 a247, %7\n\tv_accvgpr_write_b32 a248, %8\n\tv_accvgpr_write_b32 a249, %9\n\tv_accvgpr_write_b32 a250, %10\n\tv_accvgpr_write_b32 a251, %11\n\tv_accvgpr_write_b32 a252, %12\n\tv_accvgpr_write_b32 a253, %13\n\tv_accvgpr_write_b32 a254, %14\n\tv_accvgpr_write_b32 a255, %15" :: "v"(X[0]), "v"(X[1]), "v"(X[2]), "v"(X[3]), "v"(X[4]), "v"(X[5]), "v"(X[6]), "v"(X[7]), "v"(X[8]), "v"(X[9]), "v"(X[10]), "v"(X[11]), "v"(X[12]), "v"(X[13]), "v"(X[14]), "v"(X[15]) : "a240", "a241", "a242", "a243", "a244", "a245", "a246", "a247", "a248", "a249", "a250", "a251", "a252", "a253", "a254", "a255")

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

// Partner value across the two 32-lane halves of a wave (rows live in lanes l and l + 32).
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Exclusive scan of one int per thread over the kThreads threads of the workgroup.
__device__ int wg_exclusive_scan(int v, int* s_tmp, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_tmp[w] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < kWaves; k++) {
    const int t = s_tmp[k];
    if (k < w) base += t;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return base + x - v;
}

// Work partition (row a.2), computed by every workgroup from the prefix lengths and, for a
// ragged batch, the per-request tree lengths:
//   * prefix lengths outside [0, max_prefix] and tree lengths outside [1, T] are errors; such a
//     request and every later one are poisoned (their index segments can no longer be
//     located) and get no keys; after a bad tree length they also get no rows, since the
//     rows' positions depend on it;
//   * node_off_b = exclusive scan of T_b (rows of request b start at node_off_b * H);
//   * key_off_b = exclusive scan of (E_b + T_b), where E_b = ceil(P_b / page) is the number
//     of prefix entries of the index segment (E_b = P_b when pages are single tokens);
//   * split length S: fixed, or the smallest multiple of 32 (at least min_split) whose
//     unit count stays within target_units (one workgroup per CU per M tile): first the
//     even spread of the batch's prefix tokens and tree keys, then, if ragged requests
//     round up past the target, a search upward from there;
//   * units_b = max(1, ceil(P_b / S)) under a fixed split; under an automatic one the tree
//     tiles count too, units_b = max(1, min(ceil((P_b + tree keys_b) / S), ceil(P_b / S) + 1));
//     first_unit_b = exclusive scan of units_b.
// Fills s_unit[] for unit g (request, key offset, P, first unit, units, error bits, S, T_b,
// node offset) and returns the number of units.  The publishing workgroup also writes the
// plan out.  (It serves batches over 64 requests; a ragged one is then planned as if every
// request had the call's largest tree, which keeps each request's partial rows apart.)
struct UnitPlan {
  int b, key_off, prefix, first, units, split, tree_nodes, node_off, total;
  int g, mt, prow;  // a ragged plan's unit and M tile for the workgroup (g < 0: no work), first partial row
  uint32_t err;
};

// Ragged calls deal their work items (unit, M tile), the M tiles of a unit consecutive, to
// the XCDs in equal contiguous ranges, so that a unit's M tiles share an XCD and its L2 and
// no XCD gets more than its share.  Workgroup bid's item, or `items` when it has none.
__device__ __forceinline__ int ragged_item(int bid, int items) {
  const int per = (items + 7) >> 3, s = bid >> 3;
  return s < per ? min((bid & 7) * per + s, items) : items;
}

// Entries of a prefix of p tokens in its index segment: one per page of 2^page_log2 slots.
__device__ __forceinline__ int seg_entries(int p, int page_log2) { return (p + (1 << page_log2) - 1) >> page_log2; }

__device__ int plan_units(const PartialArgs& a, int g, bool publish, int* s_tmp, int* s_unit, int* s_scr) {
  const int tid = threadIdx.x;
  const int B = a.batch, T = a.T;
  constexpr int kPer = kMaxBatch / kThreads;  // requests per thread
  int pv[kPer], tl[kPer], bad[kPer];
  int nbad = 0;
  // all of a thread's loads go out before the first wait (addresses clamped into the batch)
#pragma unroll
  for (int j = 0; j < kPer; j++) pv[j] = a.prefix_lens[min(kPer * tid + j, B - 1)];
#pragma unroll
  for (int j = 0; j < kPer; j++) tl[j] = a.tree_lens ? a.tree_lens[min(kPer * tid + j, B - 1)] : T;
  // bad prefix lengths count in the low 16 bits, bad tree lengths in the high ones (B <= 1024)
#pragma unroll
  for (int j = 0; j < kPer; j++) {
    const int i = kPer * tid + j;
    const int bp = (i < B && (pv[j] < 0 || pv[j] > a.max_prefix)) ? 1 : 0;
    const int bt = (i < B && (tl[j] < 1 || tl[j] > T)) ? 1 : 0;
    bad[j] = bp + (bt << 16);
    if (i >= B) pv[j] = tl[j] = 0;
    nbad += bad[j];
  }
  int tot_bad;
  int run_bad = wg_exclusive_scan(nbad, s_tmp, tot_bad);
  int segsum = 0, toksum = 0, nodesum = 0;
  uint32_t err[kPer];
#pragma unroll
  for (int j = 0; j < kPer; j++) {
    run_bad += bad[j];
    err[j] = ((run_bad & 0xFFFF) ? kErrBadPrefix : 0u) | ((run_bad >> 16) ? kErrBadTreeLen : 0u);
    if (err[j]) pv[j] = 0;
    if (err[j] & kErrBadTreeLen) tl[j] = 0;
    if (kPer * tid + j < B) segsum += seg_entries(pv[j], a.page_log2) + tl[j];
    toksum += pv[j];
    nodesum += tl[j];
  }
  int total_nodes;
  int node_off = wg_exclusive_scan(nodesum, s_tmp, total_nodes);
  int total_keys;
  int key_off = wg_exclusive_scan(segsum, s_tmp, total_keys);
  auto round_tile = [](int x) { return (x + kTileKeys - 1) / kTileKeys * kTileKeys; };
  int S = a.split_fixed;
  // Keys a request's units share: its prefix, plus its tree tiles under an automatic split,
  // so that the last unit (which also covers the tree) gets a smaller prefix share.  A
  // unit beyond the prefix units is allowed only as that last one.
  const bool fixed_split = a.split_fixed > 0;
  auto tkeys_of = [&](int t) { return fixed_split ? 0 : round_tile(t); };
  auto units_of = [&](int p, int tk, int s) { return max(1, min((p + tk + s - 1) / s, (p + s - 1) / s + 1)); };
  auto units_at = [&](int s, int* units) {  // this thread's units at split length s
    int us = 0;
#pragma unroll
    for (int j = 0; j < kPer; j++) {
      units[j] = (kPer * tid + j < B) ? units_of(pv[j], tkeys_of(tl[j]), s) : 0;
      us += units[j];
    }
    return us;
  };
  int units[kPer], total_units;
  int first = 0;
  if (S > 0) {
    first = wg_exclusive_scan(units_at(S, units), s_tmp, total_units);
  } else {
    int total_prefix = total_keys - total_nodes;  // prefix tokens (entries are tokens without pages)
    if (a.page_log2 > 0) (void)wg_exclusive_scan(toksum, s_tmp, total_prefix);
    int tksum = 0;  // the batch's tree keys, in whole tiles per request
#pragma unroll
    for (int j = 0; j < kPer; j++) tksum += tkeys_of(tl[j]);
    int total_tkeys;
    (void)wg_exclusive_scan(tksum, s_tmp, total_tkeys);
    const int U = a.target_units;
    const int work = total_prefix + total_tkeys;
    S = max(a.min_split, round_tile((work + U - 1) / U));
    first = wg_exclusive_scan(units_at(S, units), s_tmp, total_units);
    if (total_units > U && B < U) {
      // Ragged prefixes round up to more than U units, which would leave some workgroups
      // for a second round on the CUs.  Sum_b units_b <= Sum_b max(1, ceil((P_b + tkeys) / s))
      // <= work / s + B, so s = ceil(work / (U - B)) fits; search the smallest fitting
      // multiple of 32 between the two (the unit count does not grow with s).
      int lo = S + kTileKeys;
      int hi = max(lo, max(a.min_split, round_tile((work + (U - B) - 1) / (U - B))));
      // Invariant of both searches: lo - 32 does not fit, hi fits; uniform over the workgroup.
      if (B <= kFewRequests) {
        // Few requests: every thread counts the units of its own candidate length, so one
        // round tests up to kThreads lengths (spaced st apart) at once.
#pragma unroll
        for (int j = 0; j < kPer; j++)
          if (kPer * tid + j < B) {
            s_scr[kPer * tid + j] = pv[j];
            s_scr[kMaxBatch + kPer * tid + j] = tkeys_of(tl[j]);
          }
        __syncthreads();
        while (lo < hi) {
          const int n = (hi - lo) / kTileKeys;  // lengths lo, lo + 32, ..., hi - 32 are open
          const int st = kTileKeys * ((n + kThreads - 1) / kThreads);
          const int m = (hi - lo + st - 1) / st;  // candidates lo + t st, t < m, all below hi
          const int c = lo + tid * st;
          bool fits = false;
          if (tid < m) {
            int us = 0;
            for (int k = 0; k < B; k++) us += units_of(s_scr[k], s_scr[kMaxBatch + k], c);
            fits = us <= U;
          }
          if (tid == 0) s_tmp[0] = kThreads;
          __syncthreads();
          if (fits) atomicMin(&s_tmp[0], tid);
          __syncthreads();
          const int t0 = s_tmp[0];
          __syncthreads();
          if (t0 < m) {  // the smallest fitting candidate; the one before it does not fit
            hi = lo + t0 * st;
            lo = t0 == 0 ? hi : hi - st + kTileKeys;
          } else {
            lo = lo + (m - 1) * st + kTileKeys;
          }
        }
      } else {
        while (lo < hi) {
          const int mid = (lo + hi) / 2 / kTileKeys * kTileKeys;
          int tot;
          (void)wg_exclusive_scan(units_at(mid, units), s_tmp, tot);
          if (tot <= U) hi = mid; else lo = mid + kTileKeys;
        }
      }
      S = hi;
      first = wg_exclusive_scan(units_at(S, units), s_tmp, total_units);
    }
  }
#pragma unroll
  for (int j = 0; j < kPer; j++) {
    const int i = kPer * tid + j;
    if (i < B) {
      if (g >= first && g < first + units[j]) {
        s_unit[0] = i;
        s_unit[1] = key_off;
        s_unit[2] = pv[j];
        s_unit[3] = first;
        s_unit[4] = units[j];
        s_unit[5] = (int)err[j];
        s_unit[7] = tl[j];
        s_unit[8] = node_off;
      }
      if (publish) {
        ReqPlan rp;
        rp.key_off = key_off;
        rp.prefix_len = pv[j];
        rp.first_unit = first;
        rp.units = units[j];
        rp.err = err[j];
        rp.tree_nodes = tl[j];
        rp.node_off = node_off;
        rp.prow = first * a.M;
        a.req[i] = rp;
      }
      key_off += seg_entries(pv[j], a.page_log2) + tl[j];
      node_off += tl[j];
      first += units[j];
    }
  }
  if (publish && tid == 0) {
    a.hdr->split_len = S;
    a.hdr->total_units = total_units;
    a.hdr->n_mtiles = a.n_mtiles;
    if (tot_bad) atomicOr(a.sticky_err, ((tot_bad & 0xFFFF) ? kErrBadPrefix : 0u) | ((tot_bad >> 16) ? kErrBadTreeLen : 0u));
  }
  s_unit[6] = S;  // same value in every thread
  __syncthreads();
  return total_units;
}

// Inclusive scan of one int per lane over the wave (row shifts within each 16-lane row, then
// the row totals carried across rows; lanes with no source add 0).  Every lane must be active.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return x;
}

// The same partition for a batch of at most 64 requests, computed by each wave on its own
// (lane i holds request i) with wave-wide scans: no LDS and no barrier.  Returns false,
// uniformly over the workgroup, when the batch needs plan_units instead: more than 64
// requests, or ragged requests whose unit count rounds past the target (the split search).
// Fills up for unit g; a publishing wave writes the plan out.
// A ragged call (a tree size per request) is planned by M tiles: request b fills
// mt_b = ceil(H T_b / 128) of them, each unit of it takes mt_b workgroups, and the split is
// the smallest (multiple of 32, at least min_split) for which sum_b mt_b units_b stays
// within the launch's workgroup budget (target_units x M tiles), so that requests with
// fewer rows get shorter units instead of idle workgroups.  The workgroup's (unit, M tile)
// then comes from its item (ragged_item), and the partial rows of request b are packed at
// prow_b = sum_{b' < b} units_b' H T_b'.
template <bool kRagged, class Hook>
__device__ bool plan_wave(const PartialArgs& a, int bid, int g, bool publish, UnitPlan& up, Hook&& after_loads) {
  const int B = a.batch, T = a.T;
  if (B > 64) {
    after_loads();
    return false;
  }
  const int lane = threadIdx.x & 63;
  const bool in = lane < B;
  int pv = a.prefix_lens[min(lane, B - 1)];
  int tl = a.tree_lens ? a.tree_lens[min(lane, B - 1)] : T;
  __builtin_amdgcn_sched_barrier(0);
  after_loads();
  __builtin_amdgcn_sched_barrier(0);
  const int bp = (in && (pv < 0 || pv > a.max_prefix)) ? 1 : 0;
  const int bt = (in && (tl < 1 || tl > T)) ? 1 : 0;
  const int run_bad = wave_incl_scan(bp + (bt << 16));  // bad prefix lengths low, tree lengths high
  const uint32_t err = ((run_bad & 0xFFFF) ? kErrBadPrefix : 0u) | ((run_bad >> 16) ? kErrBadTreeLen : 0u);
  if (!in || err) pv = 0;
  if (!in || (err & kErrBadTreeLen)) tl = 0;
  const bool fixed_split = a.split_fixed > 0;
  const int tk = fixed_split ? 0 : (tl + kTileKeys - 1) / kTileKeys * kTileKeys;
  const int seg = in ? seg_entries(pv, a.page_log2) + tl : 0;
  const int seg_inc = wave_incl_scan(seg);
  const int node_inc = wave_incl_scan(tl);
  constexpr bool ragged = kRagged;
  // workgroups per unit of this request (a request without rows keeps one, for its bookkeeping)
  const int mtw = !in ? 0 : ragged ? max(1, (a.H * tl + kRowsPerBlock - 1) / kRowsPerBlock) : a.n_mtiles;
  auto units_at = [&](int s) { return in ? max(1, min((pv + tk + s - 1) / s, (pv + s - 1) / s + 1)) : 0; };
  int S = a.split_fixed;
  if (!fixed_split && !ragged) {
    const int work = __builtin_amdgcn_readlane(wave_incl_scan(pv + tk), 63);
    const int U = a.target_units;
    S = max(a.min_split, ((work + U - 1) / U + kTileKeys - 1) / kTileKeys * kTileKeys);
  } else if (!fixed_split) {
    // 32-bit arithmetic (64-bit division here costs the kernel registers); a weighted sum
    // that could pass 2^31 goes to plan_units instead.  With one tree size every weight is
    // the same and this is the split of a call without tree sizes.
    const int budget = a.target_units * a.n_mtiles;
    float wf = (float)(pv + tk) * (float)mtw;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) wf += __shfl_xor(wf, off, 64);
    if (__builtin_amdgcn_readfirstlane(__float_as_uint(wf)) > __float_as_uint(1.0e9f)) return false;
    const int work = __builtin_amdgcn_readlane(wave_incl_scan((pv + tk) * mtw), 63);
    const int sum_mt = __builtin_amdgcn_readlane(wave_incl_scan(mtw), 63);
    auto round_up = [](int x) { return (x + kTileKeys - 1) / kTileKeys * kTileKeys; };
    auto items_at = [&](int s) { return __builtin_amdgcn_readlane(wave_incl_scan(units_at(s) * mtw), 63); };
    S = max(a.min_split, round_up((work + budget - 1) / budget));
    if (items_at(S) > budget && sum_mt < budget) {
      // sum_b mt_b units_b <= sum_b mt_b ((P_b + tkeys_b) / s + 1), so s = ceil(work /
      // (budget - sum mt_b)) fits; bisect for the smallest fitting multiple of 32 (the count
      // does not grow with s)
      int lo = S + kTileKeys;
      int hi = max(lo, max(a.min_split, round_up((work + (budget - sum_mt) - 1) / (budget - sum_mt))));
      while (lo < hi) {
        const int mid = (lo + hi) / 2 / kTileKeys * kTileKeys;
        if (items_at(mid) <= budget) hi = mid; else lo = mid + kTileKeys;
      }
      S = hi;
    }
  }
  const int units = units_at(S);
  const int first_inc = wave_incl_scan(units);
  const int total = __builtin_amdgcn_readlane(first_inc, 63);
  if (!fixed_split && !ragged && total > a.target_units && B < a.target_units) return false;
  const int first = first_inc - units;
  int item = 0, item_inc = 0, prow_inc = 0;
  if (ragged) {
    item_inc = wave_incl_scan(units * mtw);
    item = ragged_item(bid, __builtin_amdgcn_readlane(item_inc, 63));
    prow_inc = wave_incl_scan(units * a.H * tl);
  }
  const uint64_t mine =
      __ballot(in && (ragged ? item >= item_inc - units * mtw && item < item_inc : g >= first && g < first_inc));
  up.split = S;
  up.total = total;
  if (mine) {
    const int l = __builtin_ctzll(mine);
    up.b = l;
    up.key_off = __builtin_amdgcn_readlane(seg_inc - seg, l);
    up.prefix = __builtin_amdgcn_readlane(pv, l);
    up.first = __builtin_amdgcn_readlane(first, l);
    up.units = __builtin_amdgcn_readlane(units, l);
    up.err = (uint32_t)__builtin_amdgcn_readlane((int)err, l);
    up.tree_nodes = __builtin_amdgcn_readlane(tl, l);
    up.node_off = __builtin_amdgcn_readlane(node_inc - tl, l);
  } else {
    up.b = up.key_off = up.prefix = up.first = up.units = up.tree_nodes = up.node_off = 0;
    up.err = 0;
  }
  // (assigned once: stores to the struct in both arms above get merged through a pointer
  // select, which would keep it in private memory)
  int ug = g, umt = 0, uprow = up.first * a.M;
  if (ragged) {
    const int l = mine ? __builtin_ctzll(mine) : 0;
    const int k = item - __builtin_amdgcn_readlane(item_inc - units * mtw, l);
    const int m = max(1, __builtin_amdgcn_readlane(mtw, l));
    ug = mine ? up.first + k / m : -1;
    umt = k % m;
    uprow = __builtin_amdgcn_readlane(prow_inc - units * a.H * tl, l);
  }
  up.g = ug;
  up.mt = umt;
  up.prow = uprow;
  if (publish) {
    if (in) {
      ReqPlan rp;
      rp.key_off = seg_inc - seg;
      rp.prefix_len = pv;
      rp.first_unit = first;
      rp.units = units;
      rp.err = err;
      rp.tree_nodes = tl;
      rp.node_off = node_inc - tl;
      rp.prow = ragged ? prow_inc - units * a.H * tl : first * a.M;
      a.req[lane] = rp;
    }
    if (lane == 0) {
      a.hdr->split_len = S;
      a.hdr->total_units = total;
      a.hdr->n_mtiles = a.n_mtiles;
      const int tot_bad = __builtin_amdgcn_readlane(run_bad, 63);
      if (tot_bad) atomicOr(a.sticky_err, ((tot_bad & 0xFFFF) ? kErrBadPrefix : 0u) | ((tot_bad >> 16) ? kErrBadTreeLen : 0u));
    }
  }
  return true;
}

// Gathers of a unit with at most 64 rows in one M tile, run by waves 2 and 3, which hold
// no rows, so that the compute waves issue none.  Rows pass through these waves' VGPRs
// (plain non-temporal 16-byte loads, which reach a higher rate from HBM than LDS-DMA
// gathers) on their way to LDS.  Helper thread hh covers keys hk and hk + 16 of a tile and
// chunk slot hc of each of the 9 groups.  Two register stages hold tiles t+2 and t+3: each
// tile's loads go out two iterations before it is written to LDS, so that two tiles are in
// flight; tiles 0 and 1 start them, from index entries e00 .. e11 that the kernel loaded
// with its first reads.  checks() takes part in the tree check (its barriers) and says
// whether the workgroup ends there.  The loop mirrors the compute waves' barriers one for
// one from then on: the first scores', one per iteration, and the final OR.  The function
// is inlined behind a marker that the build's register audit knows (these waves may use the
// AGPRs, the compute waves may not); it never returns, the waves end in it.  pidx / tidx
// are the prefix and tree parts of the unit's index segment, as in the kernel.
template <bool kPaged, class Checks>
[[noreturn]] __device__ __attribute__((always_inline)) inline void gather_helper(const char* pool_in, int64_t row_stride_bytes,
                                                        int64_t pool_slots, int T, int page_log2, int max_page,
                                                        const int32_t* pidx, const int32_t* tidx, int kbeg, int npk,
                                                        int npt, int ntiles, int run_base, char* smem,
                                                        int e00, int e01, int e10, int e11, Checks&& checks) {
  typedef __attribute__((address_space(1))) const char gmem_char;
  gmem_char* pool = (gmem_char*)pool_in;
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
  lds_char* lds = (lds_char*)smem;
  const int tid = threadIdx.x;
  const int hh = tid - 2 * 64, hk = hh >> 3, hc = hh & 7;
  int bad = 0;
  const int pmask = (1 << page_log2) - 1;
  auto page_slot = [&](int e, int pos) -> int {
    return (uint32_t)e <= (uint32_t)max_page ? (e << page_log2) + (pos & pmask) : -1;
  };
  auto key_of = [&](int tl, int k) -> int {
    const int nv = tl < npt ? min(kTileKeys, npk - tl * kTileKeys) : min(kTileKeys, T - (tl - npt) * kTileKeys);
    return k < nv ? k : 0;
  };
  auto index_of = [&](int tl, int k) -> int {
    if (kPaged && tl < npt)
      return ((__attribute__((address_space(1))) const int32_t*)pidx)[(kbeg + tl * kTileKeys + key_of(tl, k)) >> page_log2];
    typedef __attribute__((address_space(1))) const int32_t gmem_i32;
    gmem_i32* ip = (gmem_i32*)(tl < npt ? pidx + tl * kTileKeys : tidx + (tl - npt) * kTileKeys);
    return ip[key_of(tl, k)];
  };
  auto slot_of = [&](int tl, int e, int k) -> int {
    if (tl < npt && run_base >= 0) return run_base + tl * kTileKeys + key_of(tl, k);
    if (kPaged && tl < npt) return page_slot(e, kbeg + tl * kTileKeys + key_of(tl, k));
    return e;
  };
  auto row_of = [&](int idx) -> const char* {  // a slot outside the pool reads row 0 (and is flagged)
    const bool oob = (uint32_t)idx >= (uint64_t)pool_slots;
    bad |= oob ? 1 : 0;
    return (const char*)(pool + (uint64_t)(oob ? 0u : (uint32_t)idx) * (uint64_t)row_stride_bytes);
  };
  auto entries = [&](int (&en)[2], int tl) {
#pragma unroll
    for (int kk = 0; kk < 2; kk++) en[kk] = tl < ntiles ? index_of(tl, hk + 16 * kk) : 0;
  };
  auto rows = [&](u32x4 (&st)[18], int tl, const int (&en)[2]) {
#pragma unroll
    for (int kk = 0; kk < 2; kk++) {
      const int k = hk + 16 * kk;
      typedef __attribute__((address_space(1))) const u32x4 gmem_u32x4;
      gmem_u32x4* src = (gmem_u32x4*)row_of(tl < ntiles ? slot_of(tl, en[kk], k) : 0) + (hc ^ swz(k));
#pragma unroll
      for (int j = 0; j < 9; j++) st[9 * kk + j] = __builtin_nontemporal_load(src + 8 * j);
    }
  };
  auto write = [&](const u32x4 (&st)[18], int bufi) {
#pragma unroll
    for (int kk = 0; kk < 2; kk++) {
      const int k = hk + 16 * kk;
#pragma unroll
      for (int j = 0; j < 9; j++)
        *reinterpret_cast<lds_u32x4*>(lds + bufi * kTileBytes + j * 4096 + k * 128 + hc * 16) = st[9 * kk + j];
    }
  };
  u32x4 st0[18], st1[18];
  int en0[2], en1[2];  // index entries of the tile each stage loads next
  // Tiles 0 and 1 go out first, one per stage (their entries e00 .. e11, keys hk and hk + 16,
  // came with the kernel's first loads), each followed by the entries of the tile its stage
  // loads next (2 and 3), an order that lets each wait below leave the other stage in
  // flight, since loads complete in issue order.
  {
    const int e0[2] = {e00, e01}, e1[2] = {e10, e11};
    rows(st0, 0, e0);
    entries(en0, 2);
    rows(st1, 1, e1);
    entries(en1, 3);
  }
  if (checks()) {  // the tree check found a bad parent: the workgroup ends
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __builtin_amdgcn_endpgm();
  }
  // Tile 0 into its buffer before the compute waves' first scores, tile 1 after them (its
  // buffer is not read before the next barrier); the stages then hold tiles 2 and 3 and en0
  // and en1 the entries of tiles 4 and 5, as the loop expects.
  write(st0, 0);
  rows(st0, 2, en0);
  entries(en0, 4);
  __syncthreads();
  if (ntiles > 1) write(st1, 1);
  rows(st1, 3, en1);
  entries(en1, 5);
  // Iteration t: tile t+2 (in the stage of t's parity) goes to its buffer, which held tile
  // t-1 and is free after this iteration's barrier; the stage then loads tile t+4.
  auto step = [&](u32x4 (&st)[18], int (&en)[2], int tl) {
    if (tl + 2 < ntiles) write(st, (tl + 2) % kTileBufs);
    rows(st, tl + 4, en);
    entries(en, tl + 6);
  };
  // The loop mirrors the compute waves' barriers after their first scores': one per tile
  // until the last.  It is unrolled by two, one stage per half, so that every path into its
  // head leaves the loads in the same order (st0, en0, st1, en1) and the compiler's waits
  // stay counted.
  for (int t = 0;;) {
    __syncthreads();
    if (t == ntiles) break;
    step(st0, en0, t);
    t++;
    __syncthreads();
    if (t == ntiles) break;
    step(st1, en1, t);
    t++;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // no load in flight when the workgroup ends
  (void)__syncthreads_or(bad);         // the epilogue's
  __builtin_amdgcn_endpgm();           // the helper waves end here
}

// kPaged: the prefix is addressed through a block table of 2^page_log2-slot pages (the
// index segment holds page ids); otherwise through one slot per token.  kBigTree: T > 64,
// so a row's ancestor mask takes kMaxTreeWords 64-bit words instead of one.  kHelp: at
// most 64 rows in one M tile, so waves 2 and 3 hold no rows; they gather every tile
// (gather_helper) and the compute waves issue no gathers.  kRG: one M tile of more rows; no
// other workgroup reads the same keys, so every gather goes to HBM, and the compute waves
// stage their pieces in VGPRs (plain non-temporal 16-byte loads, which reach a higher rate
// from HBM than direct-to-LDS loads) and write them to LDS at the end of the iteration
// (tiles 0 and 1 too, except for big trees).  kRagged: the call has a tree size per request,
// planned by M tiles (plan_wave) with the workgroup's unit and M tile taken from the plan.
template <bool kPaged, bool kBigTree, bool kHelp, bool kRG, bool kRagged>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_partial(PartialArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[kTileBufs * kTileBytes + kWaves * kQLdsBytes];
  __shared__ int s_tmp[kWaves];
  __shared__ int s_unit[10];
  lds_char* lds = (lds_char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const uint32_t wu = __builtin_amdgcn_readfirstlane(w);  // wave index, known uniform
  const int h = lane >> 5;     // which half of the wave (k sub-block of an MFMA operand)
  const int lrow = lane & 31;  // MFMA column: query row within the wave / key within a tile

  // Workgroup -> (unit, M tile).  Consecutive workgroups go to consecutive XCDs, so the M
  // tiles of one unit are given ids that are equal mod 8: they share an XCD and its L2.
  // With fewer than 8 units that would leave XCDs idle; the M tiles then go round-robin.
  // A ragged call takes its (unit, M tile) from the plan instead (ragged_item).
  const int bid = blockIdx.x;
  constexpr bool ragged = kRagged;  // the call has a tree size per request
  int mt0, g0;
  if (a.group_xcd) {
    const int slot = bid >> 3;
    mt0 = slot % a.n_mtiles;
    g0 = (slot / a.n_mtiles) * 8 + (bid & 7);
  } else {
    mt0 = bid % a.n_mtiles;
    g0 = bid / a.n_mtiles;
  }
  // Workgroup 0's first wave samples the shader-cycle and wall-clock counters at its start and
  // end, for the plan readback (the shader clock under load).
  uint64_t clk0 = 0, rt0 = 0;
  if (bid == 0 && wu == 0) {
    clk0 = __builtin_amdgcn_s_memtime();
    rt0 = __builtin_amdgcn_s_memrealtime();
  }
  // Every workgroup of the launch reads the Q rows of its M tile, all at once, when its plan
  // is known.  So that those reads find Q in L2 rather than all miss together, the
  // workgroups of each XCD (consecutive ids go to consecutive XCDs) first touch one slice
  // each of the call's Q, one 4-byte load per 128-byte line, while the plan's own loads are
  // in flight.  Ragged calls (Q size known only from the plan) and large Q skip it.
  uint32_t qpf0 = 0, qpf1 = 0;
  auto prefetch_q = [&]() {
    const int64_t qbytes = kRagged ? 0 : (int64_t)a.batch * a.M * kRowBytes;
    const int xwg = ((int)gridDim.x - (bid & 7) + 7) >> 3;  // workgroups on this XCD
    const int64_t nl = (qbytes + 127) >> 7;
    const int64_t l0 = nl * (bid >> 3) / xwg, l1 = nl * ((bid >> 3) + 1) / xwg;
    if (qbytes > 0 && l1 - l0 <= 2 * kThreads) {
      const char* qc = reinterpret_cast<const char*>(a.q);
      const int64_t la = l0 + tid, lb = l0 + kThreads + tid;
      if (la < l1) qpf0 = *reinterpret_cast<const uint32_t*>(qc + min(la << 7, qbytes - 4));
      if (lb < l1) qpf1 = *reinterpret_cast<const uint32_t*>(qc + min(lb << 7, qbytes - 4));
    }
  };
  // (tile buffer 0 is the plan's scratch: no gather writes it before the plan is done)
  UnitPlan up;
  const bool pub = ragged ? bid == 0 : (g0 == 0 && mt0 == 0);  // the workgroup that publishes the plan
  const bool planned = plan_wave<kRagged>(a, bid, g0, pub && wu == 0, up, prefetch_q);
  asm volatile("" ::"v"(qpf0), "v"(qpf1));  // the touches have landed (none in flight at any return)
  if (!planned) {
    up.total = plan_units(a, g0, pub, s_tmp, s_unit, reinterpret_cast<int*>(smem));
    up.b = s_unit[0];
    up.key_off = s_unit[1];
    up.prefix = s_unit[2];
    up.first = s_unit[3];
    up.units = s_unit[4];
    up.err = (uint32_t)s_unit[5];
    up.split = s_unit[6];
    up.tree_nodes = s_unit[7];
    up.node_off = s_unit[8];
  }
  // a ragged plan by M tiles names the workgroup's unit and M tile; otherwise its id does
  const bool by_items = planned && ragged;
  const int g = by_items ? up.g : g0, mt = by_items ? up.mt : mt0;
  const int prow = planned ? up.prow : up.first * a.M;
  if (g < 0 || g >= up.total || g >= a.units_cap) return;
  const int key_off = up.key_off;
  const int prefix = up.prefix;
  const int first_unit = up.first;
  const int nunits = up.units;
  uint32_t req_err = up.err;
  const int S = up.split;
  const int Tb = up.tree_nodes;      // this request's tree nodes (the call's T unless ragged)
  const int node_off = up.node_off;  // its first row (node) in q / out / tree_parent
  const int Mb = a.H * Tb;         // its query rows
  const int u = g - first_unit;
  // The unit's partial rows: prow_u + r for its Mb query rows (never past the buffers)
  const int prow_u = prow + u * Mb;  // < rows_cap < 2^31
  if (prow < 0 || prow_u > a.rows_cap - Mb) return;
  const int kbeg = u * S;
  const int npk = max(0, min(S, prefix - kbeg));  // prefix keys of this unit
  const int npt = (npk + kTileKeys - 1) / kTileKeys;
  const bool last = (u == nunits - 1);
  const int ntiles = npt + (last ? (Tb + kTileKeys - 1) / kTileKeys : 0);
  // Prefix part of the index segment: per-token slots from this unit's first key on, or
  // the request's page ids (indexed by absolute prefix position); then the tree slots.
  const int32_t* __restrict__ pidx = a.kv_indices + key_off + (kPaged ? 0 : kbeg);
  const int32_t* __restrict__ tidx = a.kv_indices + key_off + seg_entries(prefix, a.page_log2);
  const int pmask = (1 << a.page_log2) - 1;
  // Slot of prefix position pos on page id e; a page id past the pool (which could wrap
  // when shifted) gives -1, an out-of-pool slot.
  auto page_slot = [&](int e, int pos) -> int {
    return (uint32_t)e <= (uint32_t)a.max_page ? (e << a.page_log2) + (pos & pmask) : -1;
  };

  // Tree-ancestor bitmasks of this request (row a.1), for the unit that covers the tree.
  // They are built in tile buffer 2, which no gather writes before the loop's first
  // iteration, and each row copies its own mask into registers before that.
  constexpr int kW = kBigTree ? kMaxTreeWords : 1;
  uint64_t* s_m = reinterpret_cast<uint64_t*>(smem + 2 * kTileBytes);
  const int r = mt * kRowsPerBlock + w * kRowsPerWave + lrow;
  const bool rvalid = r < Mb;

  // Gather geometry: thread tid loads 9 chunks of key kt of every tile.
  const int kt = tid >> 3;
  const int kxor = (tid & 7) ^ swz(kt);
  int bad_index = 0;
  int run_base = -1;  // first slot of the unit's prefix run, if it is one (decided below)

  // Pool slot of this thread's key of tile t (tail keys re-read the tile's first key), in two
  // steps: load_index issues the table load, slot_of turns its value into the slot once it is
  // needed (a contiguous prefix run ignores the value), so no wait follows the load.
  auto key_at = [&](int t, int k) -> int {
    const int nv = t < npt ? min(kTileKeys, npk - t * kTileKeys) : min(kTileKeys, Tb - (t - npt) * kTileKeys);
    return k < nv ? k : 0;
  };
  auto key_of = [&](int t) -> int { return key_at(t, kt); };
  auto load_index_at = [&](int t, int k) -> int {
    if (kPaged && t < npt) return pidx[(kbeg + t * kTileKeys + key_at(t, k)) >> a.page_log2];
    const int32_t* ip = t < npt ? pidx + t * kTileKeys : tidx + (t - npt) * kTileKeys;
    return ip[key_at(t, k)];
  };
  auto load_index = [&](int t) -> int { return load_index_at(t, kt); };
  auto slot_of = [&](int t, int loaded) -> int {
    if (t < npt && run_base >= 0) return run_base + t * kTileKeys + key_of(t);
    if (kPaged && t < npt) return page_slot(loaded, kbeg + t * kTileKeys + key_of(t));
    return loaded;
  };
  // Source row of this thread's key and the wave's LDS target.  A slot outside the pool is
  // never read: row 0 stands in and the error is recorded when the unit ends.
  auto tile_src = [&](int idx) -> const char* {
    const bool oob = (uint32_t)idx >= (uint64_t)a.pool_slots;
    bad_index |= oob ? 1 : 0;
    const uint32_t ic = oob ? 0u : (uint32_t)idx;
    return reinterpret_cast<const char*>(a.pool) + (uint64_t)ic * (uint64_t)a.row_stride_bytes + kxor * 16;
  };
  auto tile_dst = [&](int bi) -> uint32_t { return (uint32_t)(uintptr_t)(lds + bi * kTileBytes) + wu * 1024; };
  auto issue_piece = [&](const char* src, uint32_t dst, int j) {
    const uint32_t d = __builtin_amdgcn_readfirstlane(dst);
    switch (j) {  // j is a constant wherever this is inlined
      case 0: lds_dma16<0>(src, d); break;
      case 1: lds_dma16<1>(src, d); break;
      case 2: lds_dma16<2>(src, d); break;
      case 3: lds_dma16<3>(src, d); break;
      case 4: lds_dma16<4>(src, d); break;
      case 5: lds_dma16<5>(src, d); break;
      case 6: lds_dma16<6>(src, d); break;
      case 7: lds_dma16<7>(src, d); break;
      default: lds_dma16<8>(src, d); break;
    }
  };
  auto issue_tile = [&](int bi, const char* src) {
    const uint32_t dst = tile_dst(bi);
#pragma unroll
    for (int j = 0; j < 9; j++) issue_piece(src, dst, j);
  };

  // Contiguous-run fast path (row a.5): if the unit's prefix slots are one run first,
  // first+1, ..., rows are addressed from `first` without reading the index table again.
  auto slot_at = [&](int k) -> int {  // slot of the unit's prefix key k
    return kPaged ? page_slot(pidx[(kbeg + k) >> a.page_log2], kbeg + k) : pidx[k];
  };

  // M tiles past this request's rows (a smaller tree than the call's largest) have no work.
  // A request without rows (after a bad tree length) keeps only M tile 0's bookkeeping.
  if (mt * kRowsPerBlock >= Mb && (mt > 0 || Mb == 0)) {
    if (tid == 0 && mt == 0) a.unit_fast[g] = 0;
    if (bid == 0 && tid == 0) a.hdr->clk_cycles = 0;
    return;
  }
  // Reads that depend only on the plan go out together: the run check's first keys, the
  // index entries of tiles 0..2, the tree parents and then Q, so that Q's latency overlaps
  // the run check and the first gathers (loads complete in issue order: the waits for the
  // index entries leave Q in flight).  A poisoned request's segment offsets are unknown, so
  // nothing is read from its index segment.
  const bool plan_ok = req_err == 0;
  const bool check_run = plan_ok && !(a.flags & 1u) && npk > 0;
  int run_first = 0, run_mine = 0;
  if (check_run) {
    run_first = slot_at(0);
    if (tid < npk) run_mine = slot_at(tid);
  }
  // Index-table entries of tiles 0..2 (this thread's key); in the helper waves those of
  // tiles 0 and 1 for their two keys, kt - 16 and kt.
  int raw0 = 0, raw1 = 0, raw2 = 0, raw3 = 0;
  if (plan_ok) {
    if constexpr (kHelp) {
      if (wu >= 2) {
        raw0 = load_index_at(0, kt - 16);
        raw1 = load_index_at(0, kt);
        if (ntiles > 1) {
          raw2 = load_index_at(1, kt - 16);
          raw3 = load_index_at(1, kt);
        }
      }
    } else {
      raw0 = load_index(0);
      if (ntiles > 1) raw1 = load_index(1);
      if (ntiles > 2) raw2 = load_index(2);
    }
  }
  int par_i = 0;
  if (last && tid < Tb) par_i = a.tree_parent[(size_t)node_off + tid];
  // B operand of the score MFMA: Q[row][16kk + 8h .. +7] (bf16 pairs).  Row r of the request
  // is (node r / H, head r % H).  The first kQReg k-steps stay in VGPRs for the whole unit;
  // the rest (loaded first) are parked in this wave's LDS slice once they land.  Rows past
  // M (last M tile) read the request's last row; their results are dropped.
  u32x4 qf[kQReg], qt[36 - kQReg];
  if (plan_ok && (!kHelp || wu < 2)) {
    const u32x4* qp =
        reinterpret_cast<const u32x4*>(a.q + ((size_t)node_off * a.H + (rvalid ? r : Mb - 1)) * kLatent) + h;
#pragma unroll
    for (int kk = kQReg; kk < 36; kk++) qt[kk - kQReg] = qp[2 * kk];
#pragma unroll
    for (int kk = 0; kk < kQReg; kk++) qf[kk] = qp[2 * kk];
  }
  int* s_jump = reinterpret_cast<int*>(smem + 2 * kTileBytes + kMaxTree * kMaxTreeWords * 8);
  auto masks = [&]() {
    if (build_masks<kW>(par_i, Tb, s_m, s_jump)) {
      req_err |= kErrBadParent;
      if (tid == 0 && mt == 0) atomicOr(a.sticky_err, kErrBadParent);
    }
  };
  auto poison = [&]() {  // poisoned request: NaN partials, which the merge turns into NaN rows
    if (rvalid && h == 0) a.part_lse[prow_u + r] = __uint_as_float(0x7FC00000u);
  };
  if (!plan_ok) {
    if (last) masks();  // its parents are still checked and reported
    poison();
    if (tid == 0 && mt == 0) a.unit_fast[g] = 0;
    if (bid == 0 && tid == 0) a.hdr->clk_cycles = 0;
    return;
  }

  if (check_run) {
    int ok = run_first >= 0 && (int64_t)run_first + npk <= a.pool_slots;  // uniform
    ok = __syncthreads_and(ok && (tid >= npk || run_mine == run_first + tid));
    // longer units: kRunBatch further keys per thread in flight per round
    constexpr int kRunBatch = 8;
    for (int k0 = kThreads; ok && k0 < npk; k0 += kThreads * kRunBatch) {
      int v[kRunBatch];
#pragma unroll
      for (int j = 0; j < kRunBatch; j++) {
        const int k = k0 + j * kThreads + tid;
        v[j] = k < npk ? slot_at(k) : run_first + k;
      }
      bool mine = true;
#pragma unroll
      for (int j = 0; j < kRunBatch; j++) mine = mine && v[j] == run_first + k0 + j * kThreads + tid;
      ok = __syncthreads_and(mine);
    }
    if (ok) run_base = run_first;
  }
  if (tid == 0 && mt == 0) a.unit_fast[g] = run_base >= 0 ? 1 : 0;  // for the plan readback
  uint64_t anc[kW];  // this row's ancestor-mask words (filled before the first scores)
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
  lds_u32x4* qlds = (lds_u32x4*)(lds + kTileBufs * kTileBytes + w * kQLdsBytes) + lane;

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

  // Softmax state of row lrow (log2 domain).  mref is the row's reference: it is set by the
  // first tile in which the row sees a key, and every probability 2^(s - mref) is kept
  // <= 2^16.  A tile whose maximum exceeds mref by more than 16 raises mref to that maximum
  // and scales the row's accumulator and sum by 2^(old - new) once (rare: it needs a score
  // jump of more than 11 nats after the row's first keys), so the common path never rescales.
  const float c2 = a.scale_log2;  // > 0
  float mref = -INFINITY;
  float lrun = 0.f;

  // S^T[key][row] = sum_d K[key][d] Q[row][d] over 36 k-steps of 16 columns.  K operand of
  // k-step kk: key lrow, columns 16kk + 8h .. +7; its Q partner comes from VGPRs or LDS.
  auto load_k = [&](const lds_char* kb, int kk) -> u32x4 {
    return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(kb + (kk >> 2) * 4096 + koff[kk & 3]);
  };
  auto load_q = [&](int kk) -> u32x4 {
    return kk < kQReg ? qf[kk < kQReg ? kk : 0] : qlds[(kk < kQReg ? 0 : kk - kQReg) * 64];
  };

  // Probabilities of one tile from its scores sc (this lane: keys 8(v/4) + 4h + v%4 of
  // row lrow; invisible keys already -inf): p = 2^(s c2 - mref), packed to bf16 pairs for the
  // PV MFMA, their sum, and the row's tile maximum (log2 units) for the reference check.
  struct Soft {
    float pe;  // probability of the even key of the pair being packed
    u32x4 pb[2];
    float psum;
  };
  // Step i (0..35) of that computation; the steps are spread between the score MFMAs of the
  // next tile so that the VALU work runs while the matrix core is busy.  Each probability
  // is packed as soon as its pair is complete, so few of them are live at once.  No maximum
  // is taken here: a probability above 2^16 shows in the lane's sum, and only then (rarely)
  // is the tile's maximum computed (raise_reference).
  auto soft_step = [&](Soft& o, const f32x16& sc, float nm, int i) {
    if (i < 16) {
      const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], c2, nm));
      o.psum = i == 0 ? e : o.psum + e;
      if (i & 1)
        o.pb[i >> 3][(i >> 1) & 3] = pack_bf16x2(o.pe, e);
      else
        o.pe = e;
    }
  };

  // One chain of 36 score MFMAs over the tile at kb.  Optionally interleaves the softmax
  // steps of the previous tile (sc -> so) and this wave's 9 gather pieces of a later tile,
  // one after each of the first 9 MFMAs, so that the gathers have as much of the iteration
  // as possible to land (wc >= 0; the helper waves' tiles take none).  K fragments are read
  // kSDist k-steps ahead through a ring of registers; the caller reads the first kSDist of
  // them (s_pre) as early as the tile is known to be in LDS.
  constexpr int kSDist = 2;
  u32x4 rg[kRG ? 9 : 1];  // kRG: this thread's 9 pieces of tile t+2 on their way to LDS
  // kRGStart: tiles 0 and 1 staged the same way (big trees' masks leave too few registers)
  constexpr bool kRGStart = kRG && !kBigTree;
  u32x4 rg1[kRGStart ? 9 : 1];  // tile 1's pieces, at the start
  struct SPre {
    u32x4 k[kSDist], q[kSDist];
  };
  auto s_pre = [&](const lds_char* kb) -> SPre {
    SPre p;
#pragma unroll
    for (int i = 0; i < kSDist; i++) {
      p.k[i] = load_k(kb, i);
      p.q[i] = load_q(i);
    }
    return p;
  };
  auto s_chain = [&](auto wc, auto soft, const lds_char* kb, const char* psrc, uint32_t pdst, const f32x16& sc,
                     float nm, Soft& so, const SPre& pre) -> f32x16 {
    constexpr int W = decltype(wc)::value;  // < 0: no gather pieces
    constexpr bool kSoft = decltype(soft)::value != 0;
    f32x16 acc;
    u32x4 kr[kSDist + 1], qr[kSDist + 1];
#pragma unroll
    for (int i = 0; i < kSDist; i++) {
      kr[i] = pre.k[i];
      qr[i] = pre.q[i];
    }
#pragma unroll
    for (int i = 0; i < 36; i++) {
      if (i + kSDist < 36) {
        kr[(i + kSDist) % (kSDist + 1)] = load_k(kb, i + kSDist);
        qr[(i + kSDist) % (kSDist + 1)] = load_q(i + kSDist);
      }
      if (i == 0)
        mfma_first_v(acc, kr[0], qr[0]);
      else
        mfma_acc_v(acc, kr[i % (kSDist + 1)], qr[i % (kSDist + 1)]);
      if (W >= 0 && i < 9) {
        if constexpr (kRG)
          rg[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(psrc + 128 * i));
        else
          issue_piece(psrc, pdst, i);
      }
      if (kSoft) {
        soft_step(so, sc, nm, i);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    return acc;
  };

  // O^T[d][row] += sum_key V^T[d][key] P^T[key][row]; MFMA k index 8h + j maps to the
  // keys this lane already holds (4h + j, then 8 + 4h + j - 4; +16 for the second MFMA).
  // The caller reads the first V fragments (vc0 = load_v(kb, 0)) before its own remaining
  // work, so that their latency is hidden.
  auto load_v = [&](const lds_char* kb, int db, u32x4(&vr)[2]) {
#pragma unroll
    for (int mf = 0; mf < 2; mf++) {
      const lds_char* vb = kb + (db >> 1) * 4096 + mf * 16 * 128;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(vb + voff[db & 1][0]));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(vb + 8 * 128 + voff[db & 1][1]));
      vr[mf] = __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  // PV of a tile is split: the head runs d-blocks 0 .. 15 - kDefer and reads the V fragments
  // of the last kDefer blocks (vd); their MFMAs (pv_deferred) run after the next barrier,
  // while the first score operands of the next tile come in from LDS, so that the matrix core
  // has work across the barrier.  The fragments are read before that barrier, which is what
  // keeps them clear of the gathers that later overwrite the tile's buffer.
  // (none for big trees, whose four-word masks leave too few registers)
  constexpr int kDefer = kBigTree ? 0 : 2;
  constexpr int kDeferArr = kDefer > 0 ? kDefer : 1;
  auto pv_head = [&](const lds_char* kb, const u32x4 (&pb)[2], const u32x4 (&vc0)[2], u32x4 (&vd)[kDeferArr][2]) {
    // the asm MFMAs insert no wait states: two between the last VALU write of P and its use
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 1");
    u32x4 vc[2] = {vc0[0], vc0[1]};
#pragma unroll
    for (int db = 0; db < 16 - kDefer; db++) {
      u32x4 vn[2];
      if (db + 1 < 16) load_v(kb, db + 1, vn);
      pv_mfma(db, vc[0], pb[0]);
      pv_mfma(db, vc[1], pb[1]);
      if (db + 1 < 16) {
        vc[0] = vn[0];
        vc[1] = vn[1];
      }
    }
    if constexpr (kDefer > 0) {
      vd[0][0] = vc[0];
      vd[0][1] = vc[1];
#pragma unroll
      for (int k = 1; k < kDefer; k++) load_v(kb, 16 - kDefer + k, vd[k]);
    }
  };
  auto pv_deferred = [&](const u32x4 (&vd)[kDeferArr][2], const u32x4 (&pb)[2]) {
#pragma unroll
    for (int k = 0; k < kDefer; k++) {
      pv_mfma(16 - kDefer + k, vd[k][0], pb[0]);
      pv_mfma(16 - kDefer + k, vd[k][1], pb[1]);
    }
  };

  // Scale this lane's part of the output accumulator (256 values of its row) by f.
  auto scale_o = [&](float f) __attribute__((always_inline)) {
    asm volatile("s_nop 15\n\ts_nop 3" ::: "memory");  // every PV MFMA has written the accumulator
    float X[16];
#define MLV_SCALE_BLOCK(N)                                  \
  MLV_READ_O_##N(X);                                        \
  _Pragma("unroll") for (int k = 0; k < 16; k++) X[k] *= f; \
  MLV_WRITE_O_##N(X);
    MLV_SCALE_BLOCK(0) MLV_SCALE_BLOCK(1) MLV_SCALE_BLOCK(2) MLV_SCALE_BLOCK(3)
    MLV_SCALE_BLOCK(4) MLV_SCALE_BLOCK(5) MLV_SCALE_BLOCK(6) MLV_SCALE_BLOCK(7)
    MLV_SCALE_BLOCK(8) MLV_SCALE_BLOCK(9) MLV_SCALE_BLOCK(10) MLV_SCALE_BLOCK(11)
    MLV_SCALE_BLOCK(12) MLV_SCALE_BLOCK(13) MLV_SCALE_BLOCK(14) MLV_SCALE_BLOCK(15)
#undef MLV_SCALE_BLOCK
    asm volatile("s_nop 1" ::: "memory");  // the accumulator writes before its next MFMA use
  };
  // After the softmax of tile t (scores sc, probabilities so against mref): a lane's sum of
  // 16 probabilities exceeds 2^16 whenever one of them does, so only then (rarely) is the
  // tile's maximum taken.  Rows whose maximum exceeds mref by more than 16 raise mref to it
  // and scale their accumulator and running sum by 2^(old - new); the tile's probabilities
  // are then computed again against the new reference.
  auto raise_reference = [&](const f32x16& sc, Soft& so) {
    if (__builtin_expect(__any(so.psum > 65536.0f), 0)) {
      float m = sc[0];
#pragma unroll
      for (int v = 1; v < 16; v++) m = fmaxf(m, sc[v]);
      const float tmax = xhalf_max(m) * c2;
      const bool raise = mref != -INFINITY && tmax > mref + 16.0f;
      if (__any(raise)) {
        if (lane == 0) atomicAdd(&a.hdr->rescales, 1u);
        const float f = raise ? __builtin_amdgcn_exp2f(mref - tmax) : 1.0f;
        scale_o(f);
        lrun *= f;
        if (raise) mref = tmax;
#pragma unroll
        for (int i = 0; i < 16; i++) soft_step(so, sc, -mref, i);
      }
    }
  };

  // Software pipeline over the tiles of the unit, three LDS buffers in rotation (tile t in
  // buffer bi).  Iteration t, after the barrier that makes tile t+1 visible: the deferred PV
  // blocks of tile t-1, then S(t+1) on the matrix core with the softmax of tile t in its gaps
  // and the gathers of tile t+2 among its MFMAs, then the head of PV(t).
  int t = 0, bi = 0;
  bool need_init = true;  // some row of the wave has no reference yet
  int idx_next = 0;  // this thread's loaded index-table entry of tile t+2
  f32x16 sacc;       // S^T of tile t
  Soft dummy_soft;
  const f32x16 zero16 = {};
  // First the gathers of tiles 0 and 1.  The index entries of tiles 0..2 were loaded in the
  // prologue, and all three have landed before any gather goes out, since the compiler
  // cannot see a gather's completion and a wait for an index issued after one would also
  // wait for it.
  auto start_gathers = [&](int e0, int e1, int e2) {
    t = 0;
    bi = 0;
    const int i0 = slot_of(0, e0);
    const int i1 = ntiles > 1 ? slot_of(1, e1) : 0;
    idx_next = e2;
    const char* src0 = tile_src(i0);
    const char* src1 = tile_src(i1);
    const int i2 = idx_next;
    asm volatile("" ::"v"(i2));  // idx_next has landed too
    issue_tile(0, src0);
    if (ntiles > 1) issue_tile(1, src1);
  };
  // Then, once tile 0 has landed everywhere, its scores.
  auto start_scores = [&]() {
    if constexpr (kRGStart) {  // tile 0 from VGPRs into buffer 0
      lds_u32x4* d = reinterpret_cast<lds_u32x4*>(lds) + tid;
#pragma unroll
      for (int j = 0; j < 9; j++) d[j * 256] = rg[j];
    }
    if constexpr (!kHelp && !kRGStart) {
      if (ntiles > 1) {
        __builtin_amdgcn_s_waitcnt(0x0F79);  // vmcnt(9): tile 0 landed (tile 1 may not)
      } else {
        __builtin_amdgcn_s_waitcnt(0x0F70);
      }
    }
    __syncthreads();
    need_init = __any(mref == -INFINITY);
    sacc = s_chain(IntC<-1>{}, IntC<0>{}, lds, nullptr, 0u, zero16, 0.f, dummy_soft, s_pre(lds));
  };
  if constexpr (kHelp) {
    if (wu >= 2) {
      // From here on only the helper waves run; they hold no rows, so the build's register
      // audit lets the compiler use AGPRs past this marker.  They gather every tile of the
      // unit, tiles 0 and 1 included, and take part in the tree check.
      asm volatile("; mlv-helper-waves" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);  // keep the helper's code below the marker
      gather_helper<kPaged>(reinterpret_cast<const char*>(a.pool), a.row_stride_bytes, a.pool_slots, Tb,
                            a.page_log2, a.max_page, pidx, tidx, kbeg, npk, npt, ntiles, run_base, smem,
                            raw0, raw1, raw2, raw3, [&]() -> bool {
                              if (last) masks();
                              return req_err != 0;
                            });
    }
  } else if constexpr (kRGStart) {
    // tiles 0 and 1 through VGPRs as well: tile 0 goes to LDS before the first scores,
    // tile 1 while they run
    const char* src0 = tile_src(slot_of(0, raw0));
    const char* src1 = tile_src(ntiles > 1 ? slot_of(1, raw1) : 0);
    idx_next = raw2;
#pragma unroll
    for (int j = 0; j < 9; j++) rg[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src0 + 128 * j));
#pragma unroll
    for (int j = 0; j < 9; j++) rg1[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src1 + 128 * j));
  } else {
    start_gathers(raw0, raw1, raw2);
  }
  {  // O^T[d = 32db + ..][row] accumulates in a[0..255]: zeroed by the matrix core
    const u32x4 z4 = {0u, 0u, 0u, 0u};
    MLV_ZERO_O(z4);
  }
  if (last) masks();
  if (req_err) {  // a bad parent: the tiles' gathers must land before the workgroup ends
    __builtin_amdgcn_s_waitcnt(0x0F70);
    poison();
    return;
  }
#pragma unroll
  for (int kk = kQReg; kk < 36; kk++) qlds[(kk - kQReg) * 64] = qt[kk - kQReg];  // lane-major, conflict-free
#pragma unroll
  for (int w = 0; w < kW; w++) anc[w] = (last && rvalid) ? s_m[(r / a.H) * kW + w] : ~0ull;
  start_scores();
  if constexpr (kRGStart) {  // tile 1 into buffer 1 (read after the next barrier)
    if (ntiles > 1) {
      lds_u32x4* d = reinterpret_cast<lds_u32x4*>(lds + kTileBytes) + tid;
#pragma unroll
      for (int j = 0; j < 9; j++) d[j * 256] = rg1[j];
    }
  }
  // Deferred PV fragments and their P operand; zero before the first tile, so that the
  // deferred MFMAs at the first barrier add nothing.
  u32x4 vdef[kDeferArr][2], pdef[2];
#pragma unroll
  for (int k = 0; k < kDeferArr; k++) vdef[k][0] = vdef[k][1] = u32x4{0u, 0u, 0u, 0u};
  pdef[0] = pdef[1] = u32x4{0u, 0u, 0u, 0u};
  // Tiles t with t + 3 < nfull (all of t .. t+3 are full prefix tiles) take the steady body:
  // no tail or tree masks, no clamped keys, no first-reference step.
  const int nfull = npk / kTileKeys;
  // One iteration; returns 0 to go on, 1 at the end of the unit.
  auto iteration = [&](auto steady) -> int {
    constexpr bool kSteady = decltype(steady)::value != 0;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's loads of tile t+1 landed
    __syncthreads();                     // ... and everyone's; PV(t-1) finished everywhere
    // The first fragments of S(t+1) need only the barrier; the deferred PV MFMAs of tile t-1
    // cover their latency.
    const int b1 = bi == kTileBufs - 1 ? 0 : bi + 1;
    const int b2 = b1 == kTileBufs - 1 ? 0 : b1 + 1;
    const lds_char* kb1 = lds + b1 * kTileBytes;
    const SPre pre = s_pre(kb1);
    pv_deferred(vdef, pdef);
    // Gathers of tile t+2 go to buffer b2 (on the last tiles they re-read pool row 0 into it;
    // nothing reads that buffer before the next barrier).
    const char* pf_src = nullptr;
    uint32_t pf_dst = 0;
    if (!kHelp) {
      if (kSteady && !kPaged) {  // full tiles: no clamped keys
        pf_src = tile_src(run_base >= 0 ? run_base + (t + 2) * kTileKeys + kt : idx_next);
        idx_next = pidx[(t + 3) * kTileKeys + kt];
      } else {
        pf_src = tile_src(t + 2 < ntiles ? slot_of(t + 2, idx_next) : 0);
        if (t + 3 < ntiles) idx_next = load_index(t + 3);
      }
      pf_dst = tile_dst(b2);
    }
    if (!kSteady) {
      if (__builtin_expect(t == ntiles, 0)) return 1;
      // Tail and tree tiles: invisible keys get -inf (key of register v is 4h + 8(v/4) + v%4).
      const bool tree = t >= npt;
      const int tt = t - npt;
      const int nv = tree ? min(kTileKeys, Tb - tt * kTileKeys) : min(kTileKeys, npk - t * kTileKeys);
      if (__builtin_expect(tree || nv < kTileKeys, 0)) {
        // the word holding tree tile tt's 32 keys (masked ORs: a select chain over the array
        // is turned into an indexed private copy of it)
        uint64_t aw = 0;
#pragma unroll
        for (int w = 0; w < kW; w++) aw |= anc[w] & (0ull - (uint64_t)((tt >> 1) == w));
        const uint32_t win = tree ? (uint32_t)(aw >> ((tt & 1) * kTileKeys)) : ~0u;
        const uint32_t tm = win >> (4 * h);
        const int nvh = nv - 4 * h;
#pragma unroll
        for (int v = 0; v < 16; v++) {
          const int kv = 8 * (v >> 2) + (v & 3);
          sacc[v] = (kv < nvh && ((tm >> kv) & 1u)) ? sacc[v] : -INFINITY;
        }
      }
      // A row's first visible keys set its reference (it may stay -inf if the tile hides all).
      if (__builtin_expect(need_init, 0)) {
        float m0 = sacc[0];
#pragma unroll
        for (int v = 1; v < 16; v++) m0 = fmaxf(m0, sacc[v]);
        m0 = xhalf_max(m0) * c2;
        if (mref == -INFINITY) mref = m0;
        need_init = __any(mref == -INFINITY);
      }
    }
    const float nm = kSteady ? -mref : (mref == -INFINITY ? 0.f : -mref);  // all scores are -inf while mref is

    Soft so;
    f32x16 snext;
    if (kSteady || __builtin_expect(t + 1 < ntiles, 1)) {
      if constexpr (kHelp)  // the helper waves gather
        snext = s_chain(IntC<-1>{}, IntC<1>{}, kb1, nullptr, 0u, sacc, nm, so, pre);
      else
        snext = s_chain(IntC<1>{}, IntC<1>{}, kb1, pf_src, pf_dst, sacc, nm, so, pre);
    } else {
#pragma unroll
      for (int i = 0; i < 36; i++) soft_step(so, sacc, nm, i);
      snext = sacc;
    }
    const lds_char* kb = lds + bi * kTileBytes;
    u32x4 vc0[2];
    load_v(kb, 0, vc0);
    raise_reference(sacc, so);
    lrun += so.psum;
    pv_head(kb, so.pb, vc0, vdef);
    pdef[0] = so.pb[0];
    pdef[1] = so.pb[1];
    if constexpr (kRG) {  // tile t+2 into buffer b2 (tile t-1's, which no one reads any more)
      if (kSteady || t + 1 < ntiles) {
        lds_u32x4* d = reinterpret_cast<lds_u32x4*>(lds + b2 * kTileBytes) + tid;
#pragma unroll
        for (int j = 0; j < 9; j++) d[j * 256] = rg[j];
      }
    }
    sacc = snext;
    bi = b1;
    t++;
    return 0;
  };
  // The steady tiles run in a loop of their own: one body per loop, so that the values
  // carried from one iteration to the next stay in place (a single loop dispatching to
  // either body made the compiler copy them at every edge: 4% slower, and 24 more VGPRs).
  for (;;) {
    while (t + 3 < nfull && !need_init) (void)iteration(IntC<1>{});
    if (iteration(IntC<0>{})) break;
  }
  // (the iteration that found the end ran the last tile's deferred PV blocks at its top)

  asm volatile("s_nop 15\n\ts_nop 3" ::: "memory");  // last PV MFMA results settle before reads
  if (bid == 0 && wu == 0) {
    const uint64_t clk1 = __builtin_amdgcn_s_memtime(), rt1 = __builtin_amdgcn_s_memrealtime();
    if (lane == 0) {
      a.hdr->clk_cycles = (uint32_t)(clk1 - clk0);
      a.hdr->clk_ticks = (uint32_t)(rt1 - rt0);
    }
  }
  const int any_bad = __syncthreads_or(bad_index);
  if (any_bad && tid == 0) atomicOr(a.sticky_err, kErrBadIndex);
  const float lt = xhalf_sum(lrun);
  const float inv = 1.0f / lt;
  const float lse2 = any_bad ? __uint_as_float(0x7FC00000u) : mref + __builtin_amdgcn_logf(lt);
  if (rvalid) {
    // Partials leave as bf16 (each value rounded on its own, like the probabilities fed to
    // the PV MFMAs).  Lane pairs (lrow, h = 0/1) exchange 8-byte groups so that each lane
    // stores 8 consecutive columns.
    uint16_t* po = a.part_o + (size_t)(prow_u + r) * kVdim + 8 * h;
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
      uint32_t pk[8];
#pragma unroll
      for (int j = 0; j < 8; j++) pk[j] = pack_bf16x2(X[2 * j] * inv, X[2 * j + 1] * inv);
#pragma unroll
      for (int p = 0; p < 2; p++) {
        const auto lo = __builtin_amdgcn_permlane32_swap(pk[4 * p], pk[4 * p + 2], false, false);
        const auto hi = __builtin_amdgcn_permlane32_swap(pk[4 * p + 1], pk[4 * p + 3], false, false);
        const u32x4 v = {lo[0], hi[0], lo[1], hi[1]};
        *reinterpret_cast<u32x4*>(po + 32 * db + 16 * p) = v;
      }
    }
    if (h == 0) a.part_lse[prow_u + r] = lse2;
  }
}

// ------------------------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (u >> 16) | 0x0040u;  // quiet NaN
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Row a.6.  kSplit workgroups per output row, each over kCols = 512/kSplit of its columns,
// so that the grid fills the chip even when there are few rows.  Every lane loads kPer
// columns (16 bytes) of a unit's partial: a group of kCols/kPer lanes covers one unit, so a
// wave takes 64/(kCols/kPer) units at once and the workgroup kSlots = 4 * that many (slot s:
// units s, s + kSlots, ...).  Each slot loads up to kDepth of its units' lses and partials in
// one round, all in flight together, so that a row costs one memory round trip (rows with
// more units than kSlots * kDepth take further rounds, folded in by an online rescale).  The
// round's maximum lse, taken over the workgroup, is the reference of the weights; the slots
// add up through LDS in a fixed order.  A NaN partial lse (a poisoned unit) makes the row NaN.
// The instantiations with at most 4 column groups and 4 units per slot are held to 64 VGPRs,
// so that 8 workgroups fit on a CU and a grid of 2,048 runs in one round (at 67 VGPRs the
// last 256 waited for a second one).
template <int kSplit, int kPer, int kDepth>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu((kSplit <= 4 && kDepth <= 4) ? 8 : 1)))
void k_merge(MergeArgs a) {
  constexpr int kCols = kVdim / kSplit;   // columns of this workgroup
  constexpr int kLanes = kCols / kPer;    // lanes per unit
  constexpr int kGroups = 64 / kLanes;    // units per wave
  constexpr int kSlots = kWaves * kGroups;
  static_assert(kLanes * kGroups == 64 && kPer <= 8, "a wave covers whole units");
  typedef float fv __attribute__((ext_vector_type(kPer)));
  typedef __bf16 hv __attribute__((ext_vector_type(kPer)));
  __shared__ __attribute__((aligned(16))) float s_acc[kSlots][kCols];
  __shared__ float s_m[kWaves], s_z[kSlots];
  const int row = blockIdx.x / kSplit;
  const int c0 = (blockIdx.x % kSplit) * kCols;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int cl = lane % kLanes, slot = w * kGroups + lane / kLanes;
  const int b = row / a.M, r = row - b * a.M;
  ReqPlan R = a.req[b];
  // the request's rows, and the row stride of its partials (M unless the call is ragged)
  if (r >= R.tree_nodes * a.H) return;  // past this request's rows (ragged trees)
  const int Mb = a.ragged ? R.tree_nodes * a.H : a.M;
  const size_t orow = (size_t)R.node_off * a.H + r;  // the row in out / lse
  const int prow = min(max(R.prow, 0), a.rows_cap);  // never index past the partial buffers
  if ((int64_t)prow + (int64_t)R.units * Mb > a.rows_cap) R.units = (a.rows_cap - prow) / Mb;
  const float* pl = a.part_lse + prow + r;
  const uint16_t* pob = a.part_o + (size_t)(prow + r) * kVdim + c0 + kPer * cl;
  const size_t ustride = (size_t)Mb * kVdim;
  float m = -INFINITY, z = 0.f;
  fv acc = {};
  for (int k0 = slot; k0 - slot < R.units; k0 += kDepth * kSlots) {  // rounds (uniform over the workgroup)
    float lu[kDepth];
    hv o[kDepth];
    // every load of the round before any use; units past the last re-read it and are dropped
#pragma unroll
    for (int k = 0; k < kDepth; k++) {
      const int u = min(k0 + k * kSlots, R.units - 1);
      lu[k] = pl[(size_t)u * Mb];
      o[k] = *reinterpret_cast<const hv*>(pob + u * ustride);
    }
    float mr = -INFINITY;
#pragma unroll
    for (int k = 0; k < kDepth; k++)
      if (k0 + k * kSlots < R.units) mr = fmaxf(mr, lu[k]);
    mr = wave_max(mr);
    if (lane == 0) s_m[w] = mr;
    __syncthreads();
    mr = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
    __syncthreads();  // s_m is rewritten by the next round
    if (mr > m) {  // a larger reference: rescale what the earlier rounds summed
      const float f = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mr);
      z *= f;
      acc *= f;
      m = mr;
    }
#pragma unroll
    for (int k = 0; k < kDepth; k++) {
      const bool live = k0 + k * kSlots < R.units;
      const float wt = (!live || lu[k] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(lu[k] - m);
      z += wt;
      acc += live ? wt * __builtin_convertvector(o[k], fv) : fv{};
    }
  }
  *reinterpret_cast<fv*>(&s_acc[slot][kPer * cl]) = acc;
  if (cl == 0) s_z[slot] = z;
  __syncthreads();
  float Z = 0.f;
#pragma unroll
  for (int q = 0; q < kSlots; q++) Z += s_z[q];
  const float inv = 1.0f / Z;
  for (int c = 2 * tid; c < kCols; c += 2 * kThreads) {
    float o2[2] = {0.f, 0.f};
#pragma unroll
    for (int q = 0; q < kSlots; q++) {
      o2[0] += s_acc[q][c];
      o2[1] += s_acc[q][c + 1];
    }
    reinterpret_cast<uint32_t*>(a.out + orow * kVdim + c0 + c)[0] =
        bf16_rne_bits(o2[0] * inv) | (bf16_rne_bits(o2[1] * inv) << 16);
  }
  if (c0 == 0 && tid == 0) a.lse[orow] = (m + __builtin_amdgcn_logf(Z)) * 0.69314718055994531f;
}

// ------------------------------------------------------------------------------------------
// A launch; with events, hipExtLaunchKernelGGL has them take the dispatch's own timestamps.
template <class K, class A>
static void launch_timed(K kernel, int grid, int block, hipStream_t s, hipEvent_t start, hipEvent_t stop,
                         const A& args) {
  if (start || stop)
    hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(block), 0, s, start, stop, 0, args);
  else
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(block), 0, s, args);
}

template <bool kPaged, bool kBigTree, bool kHelp, bool kRG, bool kRagged>
static void launch_partial_t(const PartialArgs& a, int grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  launch_timed(k_partial<kPaged, kBigTree, kHelp, kRG, kRagged>, grid, kThreads, s, e0, e1, a);
}

template <bool kPaged, bool kRagged>
static void launch_partial_p(const PartialArgs& a, int grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const bool big = a.T > 64;
  const bool help = a.n_mtiles == 1 && a.M <= 2 * kRowsPerWave && !big;
  const bool rg = a.n_mtiles == 1 && !help;
  if (help)
    launch_partial_t<kPaged, false, true, false, kRagged>(a, grid, s, e0, e1);
  else if (rg && big)
    launch_partial_t<kPaged, true, false, true, kRagged>(a, grid, s, e0, e1);
  else if (rg)
    launch_partial_t<kPaged, false, false, true, kRagged>(a, grid, s, e0, e1);
  else if (big)
    launch_partial_t<kPaged, true, false, false, kRagged>(a, grid, s, e0, e1);
  else
    launch_partial_t<kPaged, false, false, false, kRagged>(a, grid, s, e0, e1);
}

// Calls with a tree size per request run their own instantiations (the plan by M tiles), so
// that the others carry none of its code.
hipError_t launch_partial(const PartialArgs& a, int grid, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  if (a.page_log2 > 0) {
    if (a.tree_lens)
      launch_partial_p<true, true>(a, grid, s, start, stop);
    else
      launch_partial_p<true, false>(a, grid, s, start, stop);
  } else {
    if (a.tree_lens)
      launch_partial_p<false, true>(a, grid, s, start, stop);
    else
      launch_partial_p<false, false>(a, grid, s, start, stop);
  }
  return hipGetLastError();
}

template <int kSplit>
static void launch_merge_split(const MergeArgs& a, int rows, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  // kDepth: the smallest of 2, 4, 8 units per slot that holds the launch's units in one round
  constexpr int kSlots = kWaves * 64 / (kVdim / kSplit / 8);
  const int depth = a.units_hint <= 2 * kSlots ? 2 : a.units_hint <= 4 * kSlots ? 4 : 8;
  if (depth == 2)
    launch_timed(k_merge<kSplit, 8, 2>, rows * kSplit, 256, s, e0, e1, a);
  else if (depth == 4)
    launch_timed(k_merge<kSplit, 8, 4>, rows * kSplit, 256, s, e0, e1, a);
  else
    launch_timed(k_merge<kSplit, 8, 8>, rows * kSplit, 256, s, e0, e1, a);
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  // about kMergeBlocks workgroups: up to 8 per row when rows are few, whole rows when many;
  // 16-byte lanes throughout
  const int rows = a.batch * a.M;
  const int split = rows * 8 <= kMergeBlocks ? 8 : rows * 4 <= kMergeBlocks ? 4 : rows * 2 <= kMergeBlocks ? 2 : 1;
  switch (split) {
    case 8: launch_merge_split<8>(a, rows, s, start, stop); break;
    case 4: launch_merge_split<4>(a, rows, s, start, stop); break;
    case 2: launch_merge_split<2>(a, rows, s, start, stop); break;
    default: launch_merge_split<1>(a, rows, s, start, stop); break;
  }
  return hipGetLastError();
}

hipError_t launch_tree_masks(const int32_t* tree_parent, int batch, int T, uint64_t* masks, uint32_t* err,
                             hipStream_t s) {
  hipLaunchKernelGGL(k_tree_masks, dim3(batch), dim3(kThreads), 0, s, tree_parent, T, masks, err);
  return hipGetLastError();
}

}  // namespace mlv
