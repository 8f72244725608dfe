// gemm_tn.hip -- TN GEMM kernels for gfx950 (MI355X) and the C ABI around them.
//
// C = A x B with A row-major M x K, B column-major K x N (K contiguous for both
// operands) and C column-major, as defined in "FP16 GEMM optimisation on AMD
// RDNA 3 and RDNA 4", section "What we compute", and the dot-product equation of
// "hello-gpu, chapter 11 (GEMM-like)", section 11.1.
//
// Kernel design.  Four kernels, each with fp16 and fp8 instantiations and an
// optional head index; a host selector picks one per problem:
//
// gemm_tn_ring_kernel / gemm_tn_kernel (K * es > 256 bytes; TN calls take the
// first, the other op-code layouts the second):
//   * 256 x 256 output tile per workgroup, 4 waves (one per SIMD), each wave owns
//     a 128 x 128 quarter as 8 x 8 MFMA tiles of 16 x 16 (256 accumulator
//     registers per lane) -- the 4-wave layout of the MI355X FP8 GEMM page,
//     section "why 4 waves", with its 16x16 matrix-core shapes
//     (v_mfma_f32_16x16x32_f16, v_mfma_f32_16x16x128_f8f6f4), which sustain a
//     higher clock under load than the 32x32 shapes.
//   * A K-step moves 128 bytes of K per row (64 fp16 or 128 fp8 elements):
//     a 256-row x 128 B strip of A and of B.  TN: three A strips and two B
//     strips in LDS (160 KiB), so A's copies are issued two steps ahead and
//     B's one; other layouts: two [A | B] stages (128 KiB).
//   * Global -> LDS copies are buffer loads that write LDS directly (no VGPR
//     staging).  The buffer resource descriptor makes out-of-range reads return
//     zero, which handles M and N tails ("FP16 GEMM optimisation ...", Step 4);
//     K-tail chunks are pointed past the descriptor's end so they read zero too
//     (the K rule of section 11.4 of the hello-gpu chapter).
//   * LDS rows are 128 B; the 16-byte chunk c of row r is stored in slot
//     c ^ ((r >> 1) & 7), the XOR swizzle of the MI355X FP8 GEMM page (section
//     "XOR swizzle"), so the 16 rows read by one ds_read_b128 phase hit 16
//     distinct 16-byte bank groups of the 256-byte bank period.
//   * One MFMA per schedule slot, with fragment reads and copies in fixed slots
//     (the prefetch interleaving of "FP16 GEMM optimisation ...", Step 7, and
//     the MFMA / ds_read interleave of the MI355X FP8 GEMM page): fragments of
//     the next sub-step are read while the current one computes, one barrier
//     per K-step; sched_barrier pins the order.  With K a multiple of the step
//     the copies' lane offsets are fixed registers and fragment reads use a
//     register plus an immediate: the K loop issues no vector ALU instruction
//     besides its MFMAs.
//   * Block ids are remapped so each XCD (workgroups are dealt round-robin over
//     the 8 XCDs) receives a contiguous range of tiles, and that range is walked
//     in the grouped order of "FP16 GEMM optimisation ...", Step 6 (groups of 8
//     tile rows), so the blocks co-resident on one XCD share A and B strips in
//     its L2 (the chiplet-aware remap of the MI355X FP8 GEMM page).
//   * Epilogue: fp32 -> fp16 (round to nearest even) or fp32 * (sa*sb) -> bf16
//     (round to nearest even), transposed through LDS into whole column runs,
//     masked column-major stores that never touch C outside its M x N logical
//     extent (section 11.4 of the hello-gpu chapter).
//
// gemm_tn_skinny_kernel (K * es <= 256 bytes, e.g. QK^T with head dim 128):
//   all of K fits one LDS row, so there is no K pipeline; blocks walk a column
//   of 128 x 128 tiles with B's strip resident, bound by writing C.
//
// gemm_tn_mid_kernel: 128 x 128 tiles, two blocks per CU with a two-stage
//   LDS ring, for grids the 256-wide tiles cannot fill; on grids of at most
//   one block per CU (and at least eight K-steps) one block per CU with a
//   four-stage ring, whose copies run three steps ahead of the products.
//   With whole K-steps (TN) both rings take a fixed-offset form like the
//   256-row kernel's, with the products accumulating in place in AGPRs.
//
// Split-K (gemm_f16_tn_splitk, gemm_f8_tn_splitk): for few output tiles and a
//   long K, the 128 x 128 kernel with SPLIT multiplies one K range per block
//   into an fp32 partial in the caller's workspace, and
//   gemm_splitk_reduce_kernel sums the partials in range order and converts.
//
// gemm_tn_pp_kernel: the 256 x 256 tile computed by 8 waves in two groups that
//   alternate between fragment reads and products (the "ping-pong" design the
//   MI355X FP8 GEMM page weighs against its 4-wave one); measured slower here,
//   so only used when forced.
//
// Plans (plan_tn): when the 256-row tiles leave a ragged last round of one
//   block per CU, a TN call may run the first columns of C in whole rounds and
//   the rest as a second launch (the selector's configuration for it, or, with
//   a caller workspace, split-K), each element computed by exactly one kernel.
//
// Other op-code layouts (gemm_f16, gemm_f8): the 256 x 256 and 128 x 128
//   kernels take template flags AMN / BMN for an M- or N-contiguous operand,
//   staged in LDS as it lies (K-rows of the tile's columns) and turned into
//   MFMA operand fragments by gfx950's transposing LDS reads (16-bit elements
//   for fp16, bytes for fp8), so data in those layouts needs no transpose pass ("FP16 GEMM optimisation on AMD RDNA 3 and RDNA 4",
//   section "What we compute", notes real data may otherwise need one).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <type_traits>

#include "dense_gemm_tn.h"

namespace dg {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t_v __attribute__((ext_vector_type(4)));
typedef int int8_t_v __attribute__((ext_vector_type(8)));
typedef int int4_t_v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(3))) uint8_t *lds_cptr;

constexpr int kTile = 256;        // rows of A / columns of B per workgroup
constexpr int kRowBytes = 128;    // bytes of K per row per K-step (full 128-byte lines)
constexpr int kStages = 2;        // LDS stages (double buffer)
constexpr int kThreads = 256;     // 4 waves of 64
constexpr int kWaveTile = 128;    // each wave owns kWaveTile x kWaveTile of C
constexpr int kXcds = 8;          // chiplets the dispatcher deals blocks over
constexpr int kGroupM = 8;        // tile rows per group in the grouped order
constexpr int kStageBytes = kTile * kRowBytes;   // 32 KiB per operand per stage
constexpr uint32_t kOob = 0x80000000u;           // an offset past every descriptor
// Word 3 of a raw (untyped, stride 0) buffer resource on gfx9-family parts:
// 32-bit data format so the hardware range-checks the byte offset.
constexpr uint32_t kRsrcWord3 = 0x00020000u;

enum Kind { kF16 = 0, kF8 = 1 };

template <int KIND> struct Traits;
template <> struct Traits<kF16> {
  static constexpr int es = 2;       // bytes per element
  static constexpr int kstep = 64;   // K elements per K-step (128 B per row)
  static constexpr int reads = 1;    // 16-byte LDS reads per lane per MFMA operand
  // 256 x 256 kernel: v_mfma_f32_16x16x32_f16, two 32-deep sub-steps per K-step.
  static constexpr int mt = 16;      // MFMA output tile edge
  static constexpr int subs = 2;     // MFMA K sub-steps per K-step
  typedef half8_t frag_t;
  typedef float4_t_v acc_t;
};
template <> struct Traits<kF8> {
  static constexpr int es = 1;
  static constexpr int kstep = 128;
  static constexpr int reads = 2;    // 32 bytes of K per lane
  // 256 x 256 kernel: v_mfma_f32_16x16x128_f8f6f4, one 128-deep sub-step per K-step.
  static constexpr int mt = 16;
  static constexpr int subs = 1;
  typedef int8_t_v frag_t;
  typedef float4_t_v acc_t;
};

__device__ __forceinline__ float4_t_v mma(const half8_t &a, const half8_t &b, float4_t_v c) {
  // v_mfma_f32_16x16x32_f16: fp16 products, fp32 accumulate.  Written as
  // inline assembly with the accumulator tied in place in AGPRs: with the
  // builtin, the register allocator rotates the 64 accumulator tiles of the
  // 256 x 256 kernel through spare registers (hundreds of v_accvgpr moves per
  // K-step).  The memory clobber keeps the LDS reads and copies in the slots
  // the schedule gives them.  Callers leave wait states before reading an
  // accumulator with anything but another MFMA (see mfma_drain).
  asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b) : "memory");
  return c;
}
__device__ __forceinline__ float4_t_v mma(const int8_t_v &a, const int8_t_v &b, float4_t_v c) {
  // v_mfma_f32_16x16x128_f8f6f4 with the default operand formats (FP8 E4M3
  // for both) and no block scales; in place in AGPRs like the fp16 form.
  asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b) : "memory");
  return c;
}

// Wait states after the last MFMA before its accumulators are read by other
// instructions (more than the 16x16x32 result latency).
__device__ __forceinline__ void mfma_drain() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}
// The products tied in place in AGPRs but with no memory clobber, so the
// compiler still places the LDS reads between them (the 128 x 128 kernel's
// fixed-offset form, where the builtin's accumulators get renamed across the
// loop's back edge).  The same wait states apply before other reads.
__device__ __forceinline__ float4_t_v mma_t(const half8_t &a, const half8_t &b, float4_t_v c) {
  asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  return c;
}
__device__ __forceinline__ float4_t_v mma_t(const int8_t_v &a, const int8_t_v &b, float4_t_v c) {
  asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  return c;
}
// The same products with the accumulators left to the compiler (the 128 x 128
// and skinny-K kernels, whose few accumulators need no pinning).
__device__ __forceinline__ float4_t_v mma_c(const half8_t &a, const half8_t &b,
                                            const float4_t_v &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float4_t_v mma_c(const int8_t_v &a, const int8_t_v &b,
                                            const float4_t_v &c) {
  // v_mfma_f32_16x16x128_f8f6f4, FP8 E4M3 operands, no block scales.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Kernel arguments (one struct, passed by value).
struct Params {
  const uint8_t *A;      // head 0, element (0,0)
  const uint8_t *B;
  uint8_t *C;
  int64_t M, N, K;
  int64_t lda_b, ldb_b;  // row strides of A and B in bytes
  int64_t ldc;           // C column stride in elements
  int64_t stride_a_b, stride_b_b, stride_c_b;  // per-head strides in bytes
  int32_t tiles_m, tiles_n;
  float scale;           // fp8 only: fp32(scale_a * scale_b)
  int32_t c_vec_ok;      // 8-byte C stores are aligned (ldc, and stride_c with heads, % 4 == 0)
  int32_t c_vec16_ok;    // 16-byte C stores are aligned (the same, % 8 == 0)
  int32_t sk_walk;       // skinny-K kernel: consecutive M tiles per block
  // Split-K partial products (128 x 128 kernel): split h covers K elements
  // [h * k_slice, min((h + 1) * k_slice, K)) and writes fp32 partial sums to
  // W + h * N * ldw, column-major with leading dimension ldw.
  int64_t k_slice;
  float *W;
  int64_t ldw;
  int32_t order;         // block -> tile order (kOrderXcd unless measuring)
  uint64_t *clk;         // per-block clock records, or null (see clock_mark)
};

// Per-block clock records (a measurement facility, off unless gemm_clock_record
// has given the library a buffer): kClockWords 64-bit words per block at
// clk[kClockWords * block] -- for each of four points (block start, K loop
// start, K loop end, block end after its first wave's last stores completed)
// the shader-clock counter (s_memtime) and the constant 100 MHz counter
// (s_memrealtime), then the XCD the block ran on and the block index.
// Counter ticks over real-time ticks give the clock the block ran at, per
// XCD; the loop points split prologue, K loop and epilogue (kernels without a
// pipelined K loop leave them zero).  Written from lane 0 of the first wave
// with ordinary vector stores; nothing is kept live across the kernel body.
enum { kClockStart = 0, kClockLoop = 1, kClockLoopEnd = 2, kClockEnd = 3, kClockWords = 10 };
// This lane's index in its wave, recomputed from the execution mask rather
// than kept from the kernel's start: an epilogue that takes the lane id from
// here does not keep the work-item id live across the main loop, which in the
// 256-register kernels would otherwise be spilled to scratch.  (Volatile, so
// the compiler cannot reuse an earlier value.)
__device__ __forceinline__ int lane_id_fresh() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// The record pointer is read from the kernel's argument segment at each mark
// (a scalar load), so the compiler need not keep it in registers across the
// K loop, where the 256-register kernels have none to spare.
template <typename P>
__device__ __forceinline__ uint64_t *clock_ptr() {
  typedef uint64_t *const __attribute__((address_space(4))) *karg_t;
  const __attribute__((address_space(4))) char *ka =
      (const __attribute__((address_space(4))) char *)__builtin_amdgcn_kernarg_segment_ptr();
  return *(volatile karg_t)(ka + offsetof(P, clk));
}

// `wave` is the caller's wave index (a uniform value); the lane index is
// recomputed, so the work-item id need not stay live for the later marks.
__device__ __forceinline__ void clock_mark(uint64_t *clk, int point, int wave) {
  if (clk == nullptr) return;
  if (point == kClockEnd) __builtin_amdgcn_s_waitcnt(0);
  const uint64_t t = __builtin_amdgcn_s_memtime();
  const uint64_t r = __builtin_amdgcn_s_memrealtime();
  if (wave != 0 || lane_id_fresh() != 0) return;
  uint64_t *rec = clk + kClockWords * (uint64_t)blockIdx.x;
  rec[2 * point] = t;
  rec[2 * point + 1] = r;
  if (point == kClockStart) {
    uint32_t xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    rec[8] = xcc & 15u;
    rec[9] = blockIdx.x;
  }
}

// Host side of the records: the buffer, its capacity in records and the next
// free record.  A launch takes one record per block if they all fit, else
// none (clk stays null).
static std::atomic<uint64_t *> g_clk_buf{nullptr};
static std::atomic<int64_t> g_clk_cap{0};
static std::atomic<int64_t> g_clk_next{0};

uint64_t *clock_slot(int64_t blocks) {
  uint64_t *buf = g_clk_buf.load(std::memory_order_acquire);
  if (buf == nullptr || blocks <= 0) return nullptr;
  const int64_t base = g_clk_next.fetch_add(blocks, std::memory_order_relaxed);
  if (base + blocks > g_clk_cap.load(std::memory_order_relaxed)) return nullptr;
  return buf + kClockWords * base;
}

// Logical tile -> (head, tile_m, tile_n): the grouped order inside a head,
// groups of kGroupM tile rows walked column by column (short last group
// allowed), heads one after another.
template <typename I>
__host__ __device__ inline void tile_coords(I logical, I tiles_m, I tiles_n, I *head, I *tm,
                                            I *tn) {
  const I per_head = tiles_m * tiles_n;
  *head = logical / per_head;
  const I t = logical - *head * per_head;
  const I span = (I)kGroupM * tiles_n;
  const I group = t / span;
  const I first_m = group * kGroupM;
  const I rows = (tiles_m - first_m) < (I)kGroupM ? (tiles_m - first_m) : (I)kGroupM;
  const I local = t - group * span;
  *tm = first_m + local % rows;
  *tn = local / rows;
}

// First logical tile of XCD x when T tiles are split into 8 contiguous ranges
// (sizes q or q + 1, q = T / 8).
template <typename I>
__host__ __device__ inline I xcd_first_tile(I x, I T) {
  const I q = T / kXcds, r = T % kXcds;
  return x * q + (x < r ? x : r);
}

// Block -> tile orders.  kOrderXcd is the one the library uses; the other two
// exist to measure what it buys (DG_TILE_ORDER in the environment selects
// them, see launch<>):
//   kOrderXcd      chiplet-aware remap, then the grouped order;
//   kOrderGrouped  the grouped order on the hardware block id (no remap);
//   kOrderRow      row order: consecutive blocks walk one row of tiles
//                  (tile_n fastest), heads one after another.
enum { kOrderXcd = 0, kOrderGrouped = 1, kOrderRow = 2 };

// Block id -> (head, tile_m, tile_n) for a grid of one block per tile.  The
// dispatcher deals block b to XCD b % 8 as that XCD's (b / 8)-th block, so XCD
// x is given the contiguous logical range starting at xcd_first_tile(x, G), a
// bijection for any G; inside it the grouped order keeps the blocks that are
// resident on one XCD at the same time on a compact patch of tiles, sharing A
// and B strips in that XCD's L2.
template <typename I>
__host__ __device__ inline void tile_of_block(I b, I G, I tiles_m, I tiles_n, I *head, I *tm,
                                              I *tn, int order = kOrderXcd) {
  if (order == kOrderRow) {
    const I per_head = tiles_m * tiles_n;
    *head = b / per_head;
    const I t = b - *head * per_head;
    *tm = t / tiles_n;
    *tn = t - *tm * tiles_n;
    return;
  }
  const I logical = order == kOrderGrouped ? b : xcd_first_tile<I>(b % kXcds, G) + b / kXcds;
  tile_coords<I>(logical, tiles_m, tiles_n, head, tm, tn);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           (int)kRsrcWord3);
}

// Copies for one K-step: a 256-row x 128-byte strip of A and of B, each as
// eight wave-wide loads per wave.  Load q of wave w fills LDS rows
// 32q + 8w .. +7 of the strip (1 KiB, lane-contiguous: lane l writes bytes
// l*16 .. l*16+15 of that KiB), so lane l lands in row 32q + 8w + (l >> 3),
// slot l & 7, and fetches the global 16-byte chunk that the swizzle stores
// there (see the kernel); eight lanes cover one full 128-byte line of a row.
// `voff` is the lane's offset for q = 0, or kOob for a K-step (or K-tail chunk)
// that must read zeros; the host guarantees kOob + 7 * q_stride < 2^32, so a
// zero-read offset stays out of range.
struct StepCopy {
  __amdgpu_buffer_rsrc_t ra, rb;
  uint32_t va, vb;                          // lane offsets for q = 0
  __attribute__((address_space(3))) uint8_t *la, *lb;  // LDS strip bases (+ wave KiB)
};

// The same copies issued from inline assembly, in the kernels with an
// M/N-contiguous operand.  The compiler's wait-count insertion makes each
// ds_read_b64_tr_b16 wait for every LDS-writing buffer load it can see
// (vmcnt(0) before each transposing read), which would drain the copy
// pipeline several times per K-step; it does not see these.  The kernels'
// barriers wait for the copies explicitly (vmcnt), as they do for the others.
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));
struct StepCopyAsm {
  v4u32 ra, rb;        // raw buffer descriptors (the words make_rsrc builds)
  uint32_t va, vb;     // lane offsets for q = 0
  uint32_t la, lb;     // LDS byte addresses of the strips (+ this wave's part)
};
__device__ __forceinline__ v4u32 rsrc_words(const void *base, uint32_t bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  return v4u32{(uint32_t)b, (uint32_t)(b >> 32) & 0xffffu, bytes, kRsrcWord3};
}
// One 16-byte-per-lane buffer load into LDS at M0 = `lds` (+ 16 * lane); one
// wait state separates the M0 write from the load.
__device__ __forceinline__ void dma16(const v4u32 &r, uint32_t voff, uint32_t lds) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voff), "s"(r), "{m0}"(lds) : "memory");
}

// One 16-byte-per-lane buffer load into LDS (64 lanes fill 1 KiB at `lds`).
__device__ __forceinline__ void lds_copy16(__amdgpu_buffer_rsrc_t r, lds_void_t *lds,
                                           uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, voff, 0, 0, 0);
}

// M/N-contiguous operands of the 256 x 256 kernel (A of an 'N' op, B of a 'T'
// op) are staged as they lie: a stage strip is T::kstep K-rows of the block's
// 256 columns (fp16: 64 K-rows of 512 B; fp8: 128 K-rows of 256 B), the
// 16-byte chunk c of K-row k in slot c ^ Mn::key(k).  Each 1 KiB load fills
// Mn::rows_per_load consecutive K-rows (lane l: row l / (64 / rows_per_load),
// slot l % (64 / rows_per_load)); load q of wave w starts at K-row
// Mn::wave_row(w) + Mn::load_row(q).  The wave supplies the row bits the key
// uses beyond the lane's own, so a lane's key is the same for all its loads.
// The key spreads the K-rows one transposing read phase touches (32 lanes)
// over distinct 16-byte bank groups.
template <int KIND> struct Mn;
template <> struct Mn<kF16> {
  static constexpr int row_bytes = 512;
  static constexpr int rows_per_load = 2;
  __host__ __device__ static constexpr int key(int k) { return 2 * (k & 3) + 8 * ((k >> 3) & 1); }
  __host__ __device__ static constexpr int wave_row(int w) { return 2 * (w & 1) + 8 * (w >> 1); }
  __host__ __device__ static constexpr int load_row(int q) {
    return 4 * (q & 1) + 16 * ((q >> 1) & 1) + 32 * (q >> 2);
  }
};
template <> struct Mn<kF8> {
  static constexpr int row_bytes = 256;
  static constexpr int rows_per_load = 4;
  __host__ __device__ static constexpr int key(int k) { return (k & 7) + 8 * ((k >> 4) & 1); }
  __host__ __device__ static constexpr int wave_row(int w) { return 4 * (w & 1) + 16 * (w >> 1); }
  __host__ __device__ static constexpr int load_row(int q) { return 8 * (q & 1) + 32 * (q >> 1); }
};
constexpr int kMnRowBytes = Mn<kF16>::row_bytes;

// Issue copy d of a step: d < 8 is load q = d of A, else load q = d - 8 of B.
// K-contiguous operands: load q is 32 rows further (q_stride = 32 rows).
// M/N-contiguous ones: load q starts Mn::load_row(q) K-rows further
// (q_stride = one K-row).
template <bool AMN, bool BMN, int KIND = kF16>
__device__ __forceinline__ void copy_one(const StepCopy &c, int d, uint32_t qs_a, uint32_t qs_b) {
  typedef Mn<KIND> G;
  if (d < 8) {
    const int lds_off = AMN ? G::load_row(d) * G::row_bytes : d * 4096;
    const uint32_t step = (uint32_t)(AMN ? G::load_row(d) : d) * qs_a;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.ra, (lds_void_t *)(c.la + lds_off), 16,
                                             c.va + step, 0, 0, 0);
  } else {
    const int q = d - 8;
    const int lds_off = BMN ? G::load_row(q) * G::row_bytes : q * 4096;
    const uint32_t step = (uint32_t)(BMN ? G::load_row(q) : q) * qs_b;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rb, (lds_void_t *)(c.lb + lds_off), 16,
                                             c.vb + step, 0, 0, 0);
  }
}

template <bool AMN, bool BMN, int KIND = kF16>
__device__ __forceinline__ void copy_one(const StepCopyAsm &c, int d, uint32_t qs_a,
                                         uint32_t qs_b) {
  typedef Mn<KIND> G;
  if (d < 8) {
    const int lds_off = AMN ? G::load_row(d) * G::row_bytes : d * 4096;
    dma16(c.ra, c.va + (uint32_t)(AMN ? G::load_row(d) : d) * qs_a, c.la + lds_off);
  } else {
    const int q = d - 8;
    const int lds_off = BMN ? G::load_row(q) * G::row_bytes : q * 4096;
    dma16(c.rb, c.vb + (uint32_t)(BMN ? G::load_row(q) : q) * qs_b, c.lb + lds_off);
  }
}

// Descriptor bytes of an M/N-contiguous operand's K-step starting at K-row k0
// (rows of ld_b bytes, `cols` elements of es bytes of the block inside the
// matrix): all `kstep` rows while the step is not the last, else up to the
// block's last element of K-row K - 1, so rows at or past K and columns past
// the matrix in that row read zero.  Other out-of-matrix columns only feed
// outputs that are never stored.
__device__ __forceinline__ uint32_t mn_records(int64_t K, int64_t k0, int64_t ld_b,
                                               int64_t cols, int kstep, int es) {
  return K - k0 > kstep ? (uint32_t)(kstep * ld_b)
                        : (uint32_t)((K - k0 - 1) * ld_b + cols * es);
}

// An fp16 MFMA operand fragment of an M/N-contiguous strip: lanes 16g .. 16g+15
// take K-rows 8g .. 8g+7 of sub-step s from two ds_read_b64_tr_b16 (rows
// 32s + 8g + 4h + (l % 16) / 4, h = 0, 1).  `off` is the lane's byte offset for
// s = 0, h = 0 (swizzle applied).
__device__ __forceinline__ half8_t mn_frag(lds_cptr strip, uint32_t off, int s) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  lds_cptr at = strip + off + s * 32 * kMnRowBytes;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)at);
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(at + 4 * kMnRowBytes));
  return __builtin_bit_cast(half8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// An fp8 MFMA operand fragment (32 bytes of K per lane) of an M/N-contiguous
// strip with rows of `row_bytes`, from four ds_read_b64_tr_b8.  Within each
// 16-lane group that read gives lane 8a + b byte e from element b of the 8
// bytes that lane 2e + a addresses (measured), so lanes 2e + a pointing at
// K-row k0 + e, columns 8a .. 8a+7 of a 16-wide tile leave lane j holding
// K-rows k0 .. k0+7 of column j.  Lanes 16g .. 16g+15 take K-rows
// 16g + {0..7, 8..15, 64..71, 72..79}, the K order of the K-contiguous fp8
// fragment (chunks g and g + 4 of a 128-byte row).  `off` is the lane's
// swizzled byte offset of its first read.
template <int ROW_BYTES>
__device__ __forceinline__ int8_t_v mn_frag8(lds_cptr strip, uint32_t off) {
  typedef int v2i32 __attribute__((ext_vector_type(2)));
  typedef __attribute__((address_space(3))) v2i32 lds_v2i32;
  lds_cptr at = strip + off;
  const v2i32 r0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i32 *)at);
  const v2i32 r1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i32 *)(at + 8 * ROW_BYTES));
  const v2i32 r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i32 *)(at + 64 * ROW_BYTES));
  const v2i32 r3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i32 *)(at + 72 * ROW_BYTES));
  return int8_t_v{r0.x, r0.y, r1.x, r1.y, r2.x, r2.y, r3.x, r3.y};
}

// One MFMA operand fragment: 32 rows x (16 fp16 or 64 fp8) of K.  Lane l reads
// row (l & 31) of the 32-row tile at `tile` and the 16-byte chunk(s) of its K
// half (l >> 5); `off[s * reads + r]` holds the lane's swizzled byte offsets
// (wave offset included) for substep s, read r.
template <int KIND>
__device__ __forceinline__ typename Traits<KIND>::frag_t read_frag(lds_cptr tile,
                                                                  const uint32_t (&off)[4],
                                                                  int sub) {
  if constexpr (Traits<KIND>::reads == 1) {
    return *(const __attribute__((address_space(3))) half8_t *)(tile + off[sub]);
  } else {
    const int4_t_v lo =
        *(const __attribute__((address_space(3))) int4_t_v *)(tile + off[2 * sub]);
    const int4_t_v hi =
        *(const __attribute__((address_space(3))) int4_t_v *)(tile + off[2 * sub + 1]);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

// s_waitcnt immediate for "at most n vector-memory operations outstanding"
// (gfx9 encoding: vmcnt bits [3:0] and [15:14]; expcnt and lgkmcnt left at max).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Accumulator layout of the 256 x 256 kernel's MFMA tiles (edge MT = 16 or 32):
// element 4*b + e of tile (i, j) in lane l is C row MT*i + 8*b + 4*(l / MT) + e,
// column MT*j + (l % MT), for b < MT*MT/256 -- runs of four consecutive rows of
// one column of the column-major C.
template <int KIND, int NTN> struct AccShape {
  static constexpr int MT = Traits<KIND>::mt;
  static constexpr int NTM = kWaveTile / MT;       // tiles per wave along M
  static constexpr int WN = MT * NTN;              // wave tile width (columns)
  static constexpr int NB = MT * MT / 256;         // runs of four per lane per tile
  typedef typename Traits<KIND>::acc_t acc_t;
};

// Four accumulator elements (one run) -> four 16-bit outputs packed in two words.
template <int KIND>
__device__ __forceinline__ void pack_run(const Params &p, const typename Traits<KIND>::acc_t &a,
                                         int first, uint32_t &w0, uint32_t &w1) {
  uint16_t h[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if constexpr (KIND == kF16) {
      h[e] = __builtin_bit_cast(uint16_t, (_Float16)a[first + e]);
    } else {
      h[e] = __builtin_bit_cast(uint16_t, (__bf16)(a[first + e] * p.scale));
    }
  }
  w0 = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
  w1 = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
}

template <int KIND, int NTN>
__device__ __forceinline__ void store_c(
    const Params &p, uint8_t *Cb,
    const typename AccShape<KIND, NTN>::acc_t (&acc)[AccShape<KIND, NTN>::NTM][NTN],
    int64_t m_base, int64_t n_base, int lane) {
  typedef AccShape<KIND, NTN> S;
  const int64_t m_lane = m_base + 4 * (lane / S::MT);
  const int64_t n_lane = n_base + (lane % S::MT);
  const bool full = (m_base + kWaveTile <= p.M) && (n_base + S::WN <= p.N) && p.c_vec_ok;
#pragma unroll
  for (int j = 0; j < NTN; ++j) {
    const int64_t n = n_lane + S::MT * j;
#pragma unroll
    for (int i = 0; i < S::NTM; ++i) {
#pragma unroll
      for (int b = 0; b < S::NB; ++b) {
        const int64_t m = m_lane + S::MT * i + 8 * b;
        uint2 w;
        pack_run<KIND>(p, acc[i][j], 4 * b, w.x, w.y);
        uint16_t *dst = (uint16_t *)Cb + (n * p.ldc + m);
        if (full) {
          *(uint2 *)dst = w;
        } else if (n < p.N) {
          if (p.c_vec_ok && m + 3 < p.M) {
            *(uint2 *)dst = w;
          } else {
            const uint16_t h[4] = {(uint16_t)w.x, (uint16_t)(w.x >> 16), (uint16_t)w.y,
                                   (uint16_t)(w.y >> 16)};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (m + e < p.M) dst[e] = h[e];
          }
        }
      }
    }
  }
}

// Epilogue through LDS: the wave's 128 x 128 tile is converted to 16-bit
// values and written column-major into the wave's own 32 KiB of LDS (column n
// at n * 256 B, its 16-byte chunk c stored in slot c ^ (n & 15), with the
// slot's two 8-byte halves swapped when n & 8), then read
// back as 16 contiguous bytes (8 rows) per lane, so each global store
// instruction writes four full 256-byte column segments of C.  The stores are
// non-temporal: C is not read again here, and keeping it out of L2 leaves the
// room to the A and B strips.  Needs 16-byte aligned columns (ldc % 8 == 0);
// rows or columns past M, N are masked.  The half swap makes the writes
// conflict-free: the 16 lanes of a write phase hold one 4-row run of 16
// columns, whose slots differ but whose half would otherwise be the same, so
// columns n and n + 8 met in the same bank (a bank period is 128 bytes).
template <int KIND, int NTN>
__device__ __forceinline__ void store_c_lds(
    const Params &p, uint8_t *Cb,
    const typename AccShape<KIND, NTN>::acc_t (&acc)[AccShape<KIND, NTN>::NTM][NTN],
    __attribute__((address_space(3))) uint8_t *buf, int64_t m_base, int64_t n_base, int lane) {
  typedef AccShape<KIND, NTN> S;
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) u32x2 lds_u2;
  typedef __attribute__((address_space(3))) u32x4 lds_u4;
#pragma unroll
  for (int j = 0; j < NTN; ++j) {
    const int n = S::MT * j + (lane % S::MT);
#pragma unroll
    for (int i = 0; i < S::NTM; ++i) {
#pragma unroll
      for (int b = 0; b < S::NB; ++b) {
        const int m = S::MT * i + 8 * b + 4 * (lane / S::MT);
        u32x2 w;
        uint32_t w0, w1;
        pack_run<KIND>(p, acc[i][j], 4 * b, w0, w1);
        w.x = w0;
        w.y = w1;
        const int chunk = (m >> 3) ^ (n & 15);
        *(lds_u2 *)(buf + n * 256 + chunk * 16 + (((m & 7) * 2) ^ (n & 8))) = w;
      }
    }
  }
  // Same wave wrote what it reads next: the LDS counter wait orders them.
  const bool full = (m_base + kWaveTile <= p.M) && (n_base + S::WN <= p.N);
#pragma unroll
  for (int r = 0; r < S::WN / 4; ++r) {
    const int n = 4 * r + (lane >> 4);
    const int mc = lane & 15;
    u32x4 v = *(lds_u4 *)(buf + n * 256 + ((mc ^ (n & 15)) * 16));
    if (r & 2) v = v.zwxy;   // n & 8: the slot's two halves are swapped
    const int64_t gm = m_base + 8 * mc, gn = n_base + n;
    uint16_t *dst = (uint16_t *)Cb + (gn * p.ldc + gm);
    if (full || (gn < p.N && gm + 7 < p.M)) {
      __builtin_nontemporal_store(v, (u32x4 *)dst);
    } else if (gn < p.N) {
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (gm + e < p.M) dst[e] = (uint16_t)(wv[e >> 1] >> (16 * (e & 1)));
    }
  }
}

// Read schedule of the 256 x 256 kernel's sub-steps (8 x NTN slots): besides
// the A fragments (slot NTN*g), item k (0 = A_7, 1 + j = B_j) is read in slot
// extra_slot(k): every other slot from NTN + 1 on, stepping over the A slots.
template <int NTN>
constexpr int extra_slot(int k) {
  return NTN == 8 ? 9 + 2 * k : 8 + 2 * k + (k >= 3) + (k >= 6);
}
static_assert(extra_slot<8>(8) == 25 && extra_slot<7>(0) == 8 && extra_slot<7>(3) == 15 &&
                  extra_slot<7>(5) == 19 && extra_slot<7>(6) == 22 && extra_slot<7>(7) == 24,
              "read slots avoid the A slots");

// NTN = 16-column MFMA tiles per wave along N: 8 (256 x 256 block tiles) or 7
// (256 x 224, which the host picks when it packs the grid into fewer rounds
// of one block per CU).  KF (TN only): K is a multiple of the K-step, so no
// step has a K tail (see the copy offsets below).
template <int KIND, int NTN, bool AMN, bool BMN, bool KF>
__global__ __launch_bounds__(kThreads, 1) void gemm_tn_kernel(Params p) {
  static_assert(!KF || (!AMN && !BMN), "whole K-steps: TN only");
  typedef Traits<KIND> T;
  typedef Mn<KIND> G;                    // M/N-contiguous staging geometry
  constexpr int kTileN = 2 * 16 * NTN;   // block tile width (columns of B / C)
  // Two stages of [A strip | B strip], 64 KiB each.
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * 2 * kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  int head, tm, tn;
  tile_of_block<int>((int)blockIdx.x, (int)gridDim.x, p.tiles_m, p.tiles_n, &head, &tm, &tn,
                     p.order);
  const int64_t m0 = (int64_t)tm * kTile, n0 = (int64_t)tn * kTileN;
  clock_mark(clock_ptr<Params>(), kClockStart, wave);

  // Block bases: K-contiguous operands at their first row, M/N-contiguous ones
  // at their first column (element m0 / n0 of K-row 0).
  const uint8_t *Ab = p.A + head * p.stride_a_b + (AMN ? m0 * T::es : m0 * p.lda_b);
  const uint8_t *Bb = p.B + head * p.stride_b_b + (BMN ? n0 * T::es : n0 * p.ldb_b);
  uint8_t *Cb = p.C + head * p.stride_c_b;
  const int64_t rows_a = (p.M - m0) < kTile ? (p.M - m0) : kTile;
  const int64_t rows_b = (p.N - n0) < kTileN ? (p.N - n0) : kTileN;
  const uint32_t kbytes = (uint32_t)(p.K * T::es);
  const uint32_t rec_a = (uint32_t)((rows_a - 1) * p.lda_b) + kbytes;
  const uint32_t rec_b = (uint32_t)((rows_b - 1) * p.ldb_b) + kbytes;

  // LDS layout: row r of a stage strip holds 128 B of K as eight 16-byte slots;
  // chunk c of row r is stored in slot c ^ ((r >> 1) & 7), the XOR swizzle of
  // the MI355X FP8 GEMM page: a ds_read_b128 phase (16 lanes, 16 consecutive
  // rows, one chunk) covers all 16 slots of the 256-byte bank period.
  // Copy geometry of this lane (same for A and B, see copy_one).
  // M/N-contiguous copies: K-row G::wave_row(w) + l / (64 / rows_per_load)
  // (+ G::load_row(q)), slot l % (64 / rows_per_load), fetching the chunk the
  // swizzle keeps there.
  const int crow = 8 * wave + (lane >> 3);            // row within a 32-row band
  const int gchunk = (lane & 7) ^ ((crow >> 1) & 7);  // global 16-B chunk of that row
  constexpr int kLanesPerRow = 64 / G::rows_per_load;
  const int mrow = G::wave_row(wave) + lane / kLanesPerRow;
  const uint32_t mchunk16 = (uint32_t)(((lane % kLanesPerRow) ^ G::key(mrow)) * 16);
  const uint32_t voff_a = AMN ? (uint32_t)(mrow * p.lda_b) + mchunk16
                              : (uint32_t)(crow * p.lda_b) + gchunk * 16;
  const uint32_t voff_b = BMN ? (uint32_t)(mrow * p.ldb_b) + mchunk16
                              : (uint32_t)(crow * p.ldb_b) + gchunk * 16;
  const uint32_t qs_a = (uint32_t)((AMN ? 1 : 32) * p.lda_b);
  const uint32_t qs_b = (uint32_t)((BMN ? 1 : 32) * p.ldb_b);
  const int kchunk = gchunk * (16 / T::es);           // K offset of the chunk in a step
  // With whole K-steps (KF) every lane's chunk is inside K in every step
  // inside the matrix, so the lane offsets of the step's copies are the same
  // in every step: they are formed once and held in registers, and the K loop
  // issues its copies with no address arithmetic (steps outside the matrix
  // get an empty descriptor instead of out-of-range lane offsets).  The empty
  // asm statements keep the compiler from re-deriving them inside the loop.
  uint32_t cva[8], cvb[8];
  if constexpr (KF) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      cva[q] = voff_a + (uint32_t)q * qs_a;
      asm volatile("" : "+v"(cva[q]));
    }
#pragma unroll
    for (int q = 0; q < NTN; ++q) {
      cvb[q] = voff_b + (uint32_t)q * qs_b;
      asm volatile("" : "+v"(cvb[q]));
    }
  }

  // Fragment geometry: an MFMA operand covers 16 rows; lane l reads row l % 16
  // of the tile and serves K group g = l / 16 of the instruction.  fp16
  // (16x16x32): the 16-byte chunk 4s + g of the 128-byte row in sub-step s.
  // fp8 (16x16x128): the chunks g and g + 4, so that, as for fp16, the 16
  // lanes of a ds_read_b128 phase read one chunk of 16 consecutive rows (with
  // chunks 2g and 2g + 1 the reads bank-conflicted).  A and B use the same
  // map, so each instruction still pairs equal K indices.
  typedef AccShape<KIND, NTN> S;
  constexpr int MT = S::MT, NTM = S::NTM;
  const int wm = wave & 1, wn = wave >> 1;
  const int rl = lane % MT, grp = lane / MT;
  uint32_t a_off[4], b_off[4];
#pragma unroll
  for (int x = 0; x < T::subs * T::reads; ++x) {
    const int chunk = (x / T::reads) * (8 / T::subs) + grp + 4 * (x % T::reads);
    const uint32_t lo = (uint32_t)(rl * kRowBytes + ((chunk ^ ((rl >> 1) & 7)) * 16));
    a_off[x] = lo + wm * kWaveTile * kRowBytes;
    b_off[x] = lo + kStageBytes + wn * S::WN * kRowBytes;
  }
  // The same offsets for each stage, held in registers: a fragment read is
  // then one register plus an immediate offset below 64 KiB (the stage base
  // alone would overflow the immediate for stage 1).
  uint32_t a_st[2][4], b_st[2][4];
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int x = 0; x < T::subs * T::reads; ++x) {
      a_st[st][x] = a_off[x] + (uint32_t)(st * 2 * kStageBytes);
      b_st[st][x] = b_off[x] + (uint32_t)(st * 2 * kStageBytes);
      if constexpr (!AMN) asm volatile("" : "+v"(a_st[st][x]));
      if constexpr (!BMN) asm volatile("" : "+v"(b_st[st][x]));
    }
  // M/N-contiguous fragments.  fp16: lane (rl, grp) reads K-row 8 grp + rl / 4
  // at elements 4 (rl % 4) .. +3 of the 16-wide tile whose first chunk is c0,
  // i.e. slot (c0 + (rl % 4) / 2) ^ key, byte 8 (rl % 2); c0 is even and the
  // key has bits 1..3 only.  fp8: K-row 16 grp + rl / 2 at bytes 8 (rl % 2) ..
  // +7 of the tile's single chunk c0 (16 columns), slot c0 ^ key.  Either way
  // the address is mn_lane ^ (16 c0): one XOR per read.
  const int mk = (KIND == kF16) ? 8 * grp + (rl >> 2) : 16 * grp + (rl >> 1);
  const uint32_t mn_lane =
      (KIND == kF16) ? (uint32_t)(mk * G::row_bytes + 16 * G::key(mk) + 16 * ((rl & 3) >> 1) +
                                  8 * (rl & 1))
                     : (uint32_t)(mk * G::row_bytes + 16 * G::key(mk) + 8 * (rl & 1));
  // First chunk of a tile (16 columns) within the strip: 2 chunks per fp16
  // tile, 1 per fp8 tile.
  constexpr int kTileChunks = 16 * T::es / 16;
  typedef typename T::frag_t frag_t;
  constexpr int kTileBytes = MT * kRowBytes;      // LDS bytes between MFMA tiles
  // Fragment g of A (16 rows at wave row 16 g) and j of B, sub-step s, from
  // stage `stg`.
  auto mn_read = [&](lds_cptr strip, int c0, int s) -> frag_t {
    const uint32_t off = mn_lane ^ (uint32_t)(16 * c0);
    if constexpr (KIND == kF16)
      return mn_frag(strip, off, s);
    else
      return mn_frag8<Mn<kF8>::row_bytes>(strip, off);
  };
  auto frag_a = [&](int stg, int g, int s) -> frag_t {
    if constexpr (AMN)
      return mn_read((lds_cptr)smem + stg * 2 * kStageBytes,
                     kTileChunks * (kWaveTile / 16 * wm + g), s);
    else
      return read_frag<KIND>((lds_cptr)smem + g * kTileBytes, a_st[stg], s);
  };
  auto frag_b = [&](int stg, int j, int s) -> frag_t {
    if constexpr (BMN)
      return mn_read((lds_cptr)smem + stg * 2 * kStageBytes + kStageBytes,
                     kTileChunks * (S::WN / 16 * wn + j), s);
    else
      return read_frag<KIND>((lds_cptr)smem + j * kTileBytes, b_st[stg], s);
  };

  typename S::acc_t acc[NTM][NTN];
#pragma unroll
  for (int i = 0; i < NTM; ++i)
#pragma unroll
    for (int j = 0; j < NTN; ++j)
#pragma unroll
      for (int e = 0; e < MT * MT / 64; ++e) acc[i][j][e] = 0.f;

  // One loop iteration runs two K-steps, stage 0 then stage 1.  An odd K-step
  // count gets one leading step whose chunks all read as zero (adding exact
  // zeros).
  // (32-bit step arithmetic: the host keeps K * es below 2^31.)
  const int nk = (int)((p.K + T::kstep - 1) / T::kstep);
  const int pad = nk & 1;
  const int nk2 = nk + pad;
  const int Ki = (int)p.K;
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  // Copy plan of step t, in three parts so the main loop can spread its
  // instructions over three MFMA slots.  Steps outside the matrix (the leading
  // pad step, and the steps past the end issued unconditionally by the last
  // iterations) read zeros and touch no memory.
  struct StepScalars {
    uint32_t kb;   // byte offset of the step's K range (K-contiguous operands)
    int left;      // K elements of the step inside the matrix (0 .. kstep)
    int stage;
    int64_t k0;    // first K index of the step (M/N-contiguous operands)
  };
  auto step_scalars = [&](int t) {
    const int k0 = (t - pad) * T::kstep;
    const bool inside = (k0 >= 0) && (t < nk2);
    const int rem = Ki - k0;
    StepScalars u;
    u.kb = inside ? (uint32_t)(k0 * T::es) : 0u;
    u.left = !inside ? 0 : (rem >= T::kstep ? T::kstep : rem);
    u.stage = (int)(t & 1);
    if constexpr (AMN || BMN) u.k0 = inside ? k0 : -1;
    return u;
  };
  typedef std::conditional_t<AMN || BMN, StepCopyAsm, StepCopy> Copy;
  auto step_rsrc = [&](const StepScalars &u, Copy &c) {
    if constexpr (AMN || BMN) {
      // M/N-contiguous: rebased on the step's first K-row; a step outside the
      // matrix gets an empty descriptor (every load reads zero).
      if constexpr (AMN)
        c.ra = u.k0 < 0 ? rsrc_words(Ab, 0u)
                        : rsrc_words(Ab + u.k0 * p.lda_b,
                                     mn_records(p.K, u.k0, p.lda_b, rows_a, T::kstep, T::es));
      else
        c.ra = rsrc_words(Ab + u.kb, rec_a - u.kb);
      if constexpr (BMN)
        c.rb = u.k0 < 0 ? rsrc_words(Bb, 0u)
                        : rsrc_words(Bb + u.k0 * p.ldb_b,
                                     mn_records(p.K, u.k0, p.ldb_b, rows_b, T::kstep, T::es));
      else
        c.rb = rsrc_words(Bb + u.kb, rec_b - u.kb);
      const uint32_t st = (uint32_t)(uintptr_t)((lds_u8 *)smem + u.stage * 2 * kStageBytes);
      c.la = st + (AMN ? G::wave_row(wave) * G::row_bytes : wave * 1024);
      c.lb = st + kStageBytes + (BMN ? G::wave_row(wave) * G::row_bytes : wave * 1024);
    } else {
      c.ra = make_rsrc(Ab + u.kb, KF && u.left == 0 ? 0u : rec_a - u.kb);
      c.rb = make_rsrc(Bb + u.kb, KF && u.left == 0 ? 0u : rec_b - u.kb);
      lds_u8 *st = (lds_u8 *)smem + u.stage * 2 * kStageBytes + wave * 1024;
      c.la = st;
      c.lb = st + kStageBytes;
    }
  };
  auto step_lanes = [&](const StepScalars &u, Copy &c) {
    if constexpr (KF) return;   // the fixed lane offsets cva / cvb
    const bool valid = kchunk < u.left;   // this lane's chunk is inside K
    c.va = (AMN || valid) ? voff_a : kOob;
    c.vb = (BMN || valid) ? voff_b : kOob;
  };
  // Issue copy d of a step (d < 8: A, else B).
  auto issue = [&](const Copy &c, int d) {
    if constexpr (KF) {
      if (d < 8)
        lds_copy16(c.ra, (lds_void_t *)(c.la + d * 4096), cva[d]);
      else
        lds_copy16(c.rb, (lds_void_t *)(c.lb + (d - 8) * 4096), cvb[d - 8]);
    } else {
      copy_one<AMN, BMN, KIND>(c, d, qs_a, qs_b);
    }
  };
  auto step_copy = [&](int t) {
    const StepScalars u = step_scalars(t);
    Copy c;
    step_rsrc(u, c);
    step_lanes(u, c);
    return c;
  };

  // The K-step barrier: step t+1's copies have landed for this wave and its
  // last reads of stage t are complete; once every wave is here, stage t+1 is
  // published and stage t may be refilled.
  auto sync = [&]() {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0) & 0xF0FF);  // vmcnt(0), lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // 8 x NTN MFMA tiles per wave; a K-step is `subs` sub-steps (fp16: two
  // 32-deep, fp8: one 128-deep) of 8 * NTN MFMA slots, MFMA (g, j) in slot
  // NTN*g + j:
  //  * A fragment g (< 7) of the next sub-step goes into the register of the
  //    current one right after its last use (slot NTN*(g+1)); A_7 alternates
  //    between two registers by sub-step parity;
  //  * B fragments are double-buffered by sub-step parity;
  //  * A_7 and the B fragments of the next sub-step are read every other slot
  //    from slot NTN + 1 on (skipping the A slots);
  //  * the last sub-step of a K-step reads nothing before slot NTN, so the
  //    K-step barrier sits there: every read of stage t was issued earlier,
  //    and the reads from slot NTN on come from stage t+1;
  //  * step t+2's 8 + NTN copies into the freed stage follow the barrier,
  //    spread evenly over a window of kWin slots (which may reach into step
  //    t+1), so the last one has most of a step to land.
  static_assert(MT == 16 && NTM == 8 && (NTN == 8 || NTN == 7), "8 x NTN tiles of 16 x 16");
  constexpr int kQ = 8 * NTN, kBarQ = NTN;
  constexpr int kBarSlot = (T::subs - 1) * kQ + kBarQ;
  constexpr int kAfter = T::subs * kQ - kBarSlot;  // window slots in the barrier's step
  constexpr int kCopies = 8 + (BMN ? 8 : NTN);     // copy instructions per wave per step
  // Copy window in slots (fp16: 64 slots of 16-cycle products, fp8: 48 of
  // 32-cycle ones), chosen by measurement (fp16 4096^3, fp8 8192^3), capped
  // by the slots before the next step's barrier.
  constexpr int kWin0 = (KIND == kF16) ? 64 : 48;
  constexpr int kWin = kWin0 < kAfter + kBarQ ? kWin0 : kAfter + kBarQ;
  static_assert(kWin >= kCopies && kWin - kAfter <= kBarQ, "copy window");
  auto first_copy = [](int x) { return (x * kCopies + kWin - 1) / kWin; };
  // Copies of step t + 1 already issued in step t - 1's window: all of them
  // when that window ends inside step t - 1 (fp8), else first_copy(kAfter).
  constexpr int kPost0 = (kAfter * kCopies + kWin - 1) / kWin;
  constexpr int kPost = kPost0 < kCopies ? kPost0 : kCopies;
  frag_t fa[8], fx, fb[2][NTN];
  if (nk2 > 0) {
    // Copies of all of step 0 and the first kPost of step 1; wait for step 0
    // only (loads complete in order) and publish it.
    const Copy c0 = step_copy(0);
#pragma unroll
    for (int d = 0; d < kCopies; ++d) issue(c0, d);
    const Copy c1 = step_copy(1);
#pragma unroll
    for (int d = 0; d < kPost; ++d) issue(c1, d);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kPost));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < NTN; ++j) fb[0][j] = frag_b(0, j, 0);
#pragma unroll
    for (int g = 0; g < 8; ++g) fa[g] = frag_a(0, g, 0);
  }
  // cn: copies of step t + 1 (its last ones are issued early in step t);
  // cnn: step t + 2's, planned in slots kPlan .. kPlan + 2 of step t.
  Copy cn = step_copy(1), cnn;
  StepScalars un;
  constexpr int kPlan = kBarSlot - 6;
  static_assert(kPlan >= 0 && kPlan >= kWin - kAfter, "plan after the last copy of step t + 1");
  clock_mark(clock_ptr<Params>(), kClockLoop, wave);
  for (int t0 = 0; t0 < nk2; t0 += 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {            // K-step t0 + h lives in stage h
      const int t = t0 + h;
#pragma unroll
      for (int s = 0; s < T::subs; ++s) {
        const bool last = (s == T::subs - 1);
        const int par = (h * T::subs + s) & 1;  // sub-step parity
        const int src = last ? 1 - h : h;      // stage of the next sub-step's data
        const int s_n = last ? 0 : s + 1;
#pragma unroll
        for (int g = 0; g < 8; ++g) {
#pragma unroll
          for (int j = 0; j < NTN; ++j) {
            const int q = NTN * g + j;
            const int slot = kQ * s + q;
            if (j == 0 && g >= 1) fa[g - 1] = frag_a(src, g - 1, s_n);
            if (q == extra_slot<NTN>(0)) {
              if (par == 0) fx = frag_a(src, 7, s_n);
              else fa[7] = frag_a(src, 7, s_n);
            }
#pragma unroll
            for (int jj = 0; jj < NTN; ++jj)
              if (q == extra_slot<NTN>(jj + 1)) fb[par ^ 1][jj] = frag_b(src, jj, s_n);
            if (slot == kPlan) un = step_scalars(t + 2);
            if (slot == kPlan + 1) step_rsrc(un, cnn);
            if (slot == kPlan + 2) step_lanes(un, cnn);
            if (slot < kWin - kAfter) {
              const int x = slot + kAfter;     // at most one copy per slot
              if (first_copy(x) < first_copy(x + 1)) issue(cn, first_copy(x));
            } else if (slot >= kBarSlot && slot - kBarSlot < kWin) {
              const int x = slot - kBarSlot;
              if (first_copy(x) < first_copy(x + 1)) issue(cnn, first_copy(x));
            }
            if (g == 7 && par == 1) acc[g][j] = mma(fx, fb[par][j], acc[g][j]);
            else acc[g][j] = mma(fa[g], fb[par][j], acc[g][j]);
            __builtin_amdgcn_sched_barrier(0);
            if (last && q == kBarQ - 1) sync();
          }
        }
      }
      cn = cnn;
    }
  }
  mfma_drain();
  // Tie every accumulator to the wait above, so the compiler cannot hoist an
  // accumulator read (it does not know the products' latency) above it.
#pragma unroll
  for (int i = 0; i < NTM; ++i)
#pragma unroll
    for (int j = 0; j < NTN; ++j) asm volatile("" : "+a"(acc[i][j]));
  clock_mark(clock_ptr<Params>(), kClockLoopEnd, wave);

  // Drain the trailing zero copies; every wave leaves the stages before the
  // epilogue reuses the LDS.
  __builtin_amdgcn_s_waitcnt(0);
  const int elane = lane_id_fresh();
  if (p.c_vec16_ok) {
    __syncthreads();
    store_c_lds<KIND, NTN>(p, Cb, acc,
                           (__attribute__((address_space(3))) uint8_t *)smem + wave * 32768,
                           m0 + wm * kWaveTile, n0 + wn * S::WN, elane);
  } else {
    store_c<KIND, NTN>(p, Cb, acc, m0 + wm * kWaveTile, n0 + wn * S::WN, elane);
  }
  clock_mark(clock_ptr<Params>(), kClockEnd, wave);
}

// ------------------------------------------------- 256-row TN kernel, 3 + 2 ring
// gemm_tn_ring_kernel: the TN form of the 256 x 256 (or 256 x 224) tile with
// the LDS split into a three-stage ring for A and a two-stage ring for B
// (5 x 32 KiB, all of the 160 KiB a gfx950 workgroup may hold).  After the
// barrier of step t a wave issues B's copies of step t + 2 and then A's of
// step t + 3: B's land within the step after their issue, A's have two steps,
// and the barrier waits only until B's copies of step t + 1 are in (the A
// copies issued after them stay in flight).  With two [A | B] stages every
// copy had to land within one step of its issue, and with operands coming
// from HBM the barrier waited for them (fp8 8192^3: a fifth of the loop).
// Tile, waves, MFMA schedule, fragment reads, swizzle, tile order and
// epilogue are those of gemm_tn_kernel.
template <int KIND, int NTN, bool KF>
__global__ __launch_bounds__(kThreads, 1) void gemm_tn_ring_kernel(Params p) {
  typedef Traits<KIND> T;
  constexpr int kTileN = 2 * 16 * NTN;
  constexpr int kHalf = kStageBytes;            // one 256-row strip of one operand
  constexpr int kBBase = 3 * kHalf;             // B stages follow A's three
  __shared__ __attribute__((aligned(1024))) uint8_t smem[5 * kHalf];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int head, tm, tn;
  tile_of_block<int>((int)blockIdx.x, (int)gridDim.x, p.tiles_m, p.tiles_n, &head, &tm, &tn,
                     p.order);
  const int64_t m0 = (int64_t)tm * kTile, n0 = (int64_t)tn * kTileN;
  clock_mark(clock_ptr<Params>(), kClockStart, wave);

  const uint8_t *Ab = p.A + head * p.stride_a_b + m0 * p.lda_b;
  const uint8_t *Bb = p.B + head * p.stride_b_b + n0 * p.ldb_b;
  uint8_t *Cb = p.C + head * p.stride_c_b;
  const int64_t rows_a = (p.M - m0) < kTile ? (p.M - m0) : kTile;
  const int64_t rows_b = (p.N - n0) < kTileN ? (p.N - n0) : kTileN;
  const uint32_t kbytes = (uint32_t)(p.K * T::es);
  const uint32_t rec_a = (uint32_t)((rows_a - 1) * p.lda_b) + kbytes;
  const uint32_t rec_b = (uint32_t)((rows_b - 1) * p.ldb_b) + kbytes;

  // Copies (as in gemm_tn_kernel): load q of wave w fills strip rows
  // 32q + 8w + (l >> 3), slot l & 7, with the global chunk the swizzle keeps
  // there; with whole K-steps the lane offsets are fixed (cva, cvb).
  const int crow = 8 * wave + (lane >> 3);
  const int gchunk = (lane & 7) ^ ((crow >> 1) & 7);
  const uint32_t voff_a = (uint32_t)(crow * p.lda_b) + gchunk * 16;
  const uint32_t voff_b = (uint32_t)(crow * p.ldb_b) + gchunk * 16;
  const uint32_t qs_a = (uint32_t)(32 * p.lda_b);
  const uint32_t qs_b = (uint32_t)(32 * p.ldb_b);
  const int kchunk = gchunk * (16 / T::es);
  uint32_t cva[8], cvb[8];
  if constexpr (KF) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      cva[q] = voff_a + (uint32_t)q * qs_a;
      asm volatile("" : "+v"(cva[q]));
    }
#pragma unroll
    for (int q = 0; q < NTN; ++q) {
      cvb[q] = voff_b + (uint32_t)q * qs_b;
      asm volatile("" : "+v"(cvb[q]));
    }
  }

  // Fragment offsets within a strip (see gemm_tn_kernel); B's per stage
  // (compile-time stage of the unrolled step pair), A's rebased each step on
  // the step's A stage (a runtime value, t mod 3).
  typedef AccShape<KIND, NTN> S;
  constexpr int MT = S::MT, NTM = S::NTM;
  constexpr int kX = T::subs * T::reads;
  const int wm = wave & 1, wn = wave >> 1;
  const int rl = lane % MT, grp = lane / MT;
  uint32_t a_off[4], b_st[2][4];   // read_frag takes four offsets (kX used)
#pragma unroll
  for (int x = 0; x < kX; ++x) {
    const int chunk = (x / T::reads) * (8 / T::subs) + grp + 4 * (x % T::reads);
    const uint32_t lo = (uint32_t)(rl * kRowBytes + ((chunk ^ ((rl >> 1) & 7)) * 16));
    a_off[x] = lo + wm * kWaveTile * kRowBytes;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      b_st[st][x] = lo + (uint32_t)(kBBase + st * kHalf) + wn * S::WN * kRowBytes;
      asm volatile("" : "+v"(b_st[st][x]));
    }
  }
  constexpr int kTileBytes = MT * kRowBytes;
  typedef typename T::frag_t frag_t;
  uint32_t a_cur[4], a_nxt[4];   // A offsets of the current and the next step
  auto a_rebase = [&](uint32_t (&dst)[4], int stage) {
#pragma unroll
    for (int x = 0; x < kX; ++x) dst[x] = a_off[x] + (uint32_t)stage * kHalf;
  };
  auto frag_a = [&](const uint32_t (&base)[4], int g, int s) -> frag_t {
    return read_frag<KIND>((lds_cptr)smem + g * kTileBytes, base, s);
  };
  auto frag_b = [&](int stg, int j, int s) -> frag_t {
    return read_frag<KIND>((lds_cptr)smem + j * kTileBytes, b_st[stg], s);
  };

  typename S::acc_t acc[NTM][NTN];
#pragma unroll
  for (int i = 0; i < NTM; ++i)
#pragma unroll
    for (int j = 0; j < NTN; ++j)
#pragma unroll
      for (int e = 0; e < MT * MT / 64; ++e) acc[i][j][e] = 0.f;

  // K-steps as in gemm_tn_kernel: two per loop iteration (B stage = step
  // parity), an odd count led by an all-zero step; steps outside the matrix
  // read zeros and touch no memory.
  const int nk = (int)((p.K + T::kstep - 1) / T::kstep);
  const int pad = nk & 1;
  const int nk2 = nk + pad;
  const int Ki = (int)p.K;
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  struct StepScalars {
    uint32_t kb;
    int left;
  };
  auto step_scalars = [&](int t) {
    const int k0 = (t - pad) * T::kstep;
    const bool inside = (k0 >= 0) && (t < nk2);
    const int rem = Ki - k0;
    StepScalars u;
    u.kb = inside ? (uint32_t)(k0 * T::es) : 0u;
    u.left = !inside ? 0 : (rem >= T::kstep ? T::kstep : rem);
    return u;
  };
  // One window's copies: B of step t + 2 and A of step t + 3.
  struct Window {
    __amdgpu_buffer_rsrc_t rb, ra;
    lds_u8 *lb, *la;
    uint32_t vb, va;     // lane offsets (unused with whole K-steps)
  };
  auto plan_b = [&](const StepScalars &u, int bstage, Window &w) {
    w.rb = make_rsrc(Bb + u.kb, KF && u.left == 0 ? 0u : rec_b - u.kb);
    w.lb = (lds_u8 *)smem + kBBase + bstage * kHalf + wave * 1024;
    if constexpr (!KF) w.vb = kchunk < u.left ? voff_b : kOob;
  };
  auto plan_a = [&](const StepScalars &u, int astage, Window &w) {
    w.ra = make_rsrc(Ab + u.kb, KF && u.left == 0 ? 0u : rec_a - u.kb);
    w.la = (lds_u8 *)smem + astage * kHalf + wave * 1024;
    if constexpr (!KF) w.va = kchunk < u.left ? voff_a : kOob;
  };
  // Copy d of a window: d < NTN is B's load d, else A's load d - NTN.
  auto issue = [&](const Window &w, int d) {
    if (d < NTN) {
      const int q = d;
      lds_copy16(w.rb, (lds_void_t *)(w.lb + q * 4096),
                 KF ? cvb[q] : w.vb + (uint32_t)q * qs_b);
    } else {
      const int q = d - NTN;
      lds_copy16(w.ra, (lds_void_t *)(w.la + q * 4096),
                 KF ? cva[q] : w.va + (uint32_t)q * qs_a);
    }
  };
  // Copies issued after the last of B's copies of step t + 1 and before step
  // t's barrier: A's copies of step t + 2 (the same window, B's first).
  constexpr int kRingVm = 8;
  auto sync = [&]() {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kRingVm) & 0xF0FF);  // + lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // Slots as in gemm_tn_kernel; the window of step t starts at its barrier
  // slot and spreads NTN + 8 copies over kWin slots, wrapping into step t + 1
  // before that step's planning slots.
  static_assert(MT == 16 && NTM == 8 && (NTN == 8 || NTN == 7), "8 x NTN tiles of 16 x 16");
  constexpr int kQ = 8 * NTN, kBarQ = NTN, kSlots = T::subs * kQ;
  constexpr int kBarSlot = (T::subs - 1) * kQ + kBarQ;
  constexpr int kAfter = kSlots - kBarSlot;
  constexpr int kCopies = NTN + 8;
  // Window in slots, chosen by measurement: fp16 (4096^3, 8192^3) 96 slots of
  // 16-cycle products against 48 / 64 / 80 / 104; fp8 (8192^3) 48 slots of
  // 32-cycle ones against 24 / 32 / 40 / 50.
  constexpr int kWin = (KIND == kF16) ? 96 : 48;
  constexpr int kPlan = kBarSlot - 6;
  static_assert(kWin >= kCopies && kWin <= kSlots && kPlan >= 0 && kWin - kAfter <= kPlan,
                "copy window");
  auto first_copy = [](int x) { return (x * kCopies + kWin - 1) / kWin; };
  constexpr int kPost0 = (kAfter * kCopies + kWin - 1) / kWin;
  constexpr int kPost = kPost0 < kCopies ? kPost0 : kCopies;  // window copies in its own step
  static_assert(kPost >= NTN, "B's copies are issued in the window's own step");

  frag_t fa[8], fx, fb[2][NTN];
  Window wc, wn_;          // the previous window (its tail) and this step's
  int sa = 0;              // A stage of the current step (t mod 3)
  a_rebase(a_cur, 0);
  if (nk2 > 0) {
    // Steps 0 and 1 of A, step 0 of B, then window -1 (B of step 1, A of
    // step 2) up to its part in its own step; wait for step 0 and publish it.
    Window w0;
    const StepScalars u0 = step_scalars(0), u1 = step_scalars(1), u2 = step_scalars(2);
    plan_a(u0, 0, w0);
    plan_b(u0, 0, w0);
#pragma unroll
    for (int d = 0; d < kCopies; ++d) issue(w0, (d + NTN) % kCopies);   // A_0, then B_0
    plan_a(u1, 1, w0);
#pragma unroll
    for (int d = 0; d < 8; ++d) issue(w0, NTN + d);                     // A_1
    plan_b(u1, 1, wc);
    plan_a(u2, 2, wc);
#pragma unroll
    for (int d = 0; d < kPost; ++d) issue(wc, d);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(8 + kPost));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < NTN; ++j) fb[0][j] = frag_b(0, j, 0);
#pragma unroll
    for (int g = 0; g < 8; ++g) fa[g] = frag_a(a_cur, g, 0);
  }
#pragma unroll
  for (int x = 0; x < kX; ++x) asm volatile("" : "+v"(a_cur[x]));
  StepScalars ub, ua;
  clock_mark(clock_ptr<Params>(), kClockLoop, wave);
  for (int t0 = 0; t0 < nk2; t0 += 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {            // step t = t0 + h: B stage h, A stage sa
      const int t = t0 + h;
      const int sa1 = sa == 2 ? 0 : sa + 1;  // A stage of step t + 1
#pragma unroll
      for (int s = 0; s < T::subs; ++s) {
        const bool last = (s == T::subs - 1);
        const int par = (h * T::subs + s) & 1;
        const int s_n = last ? 0 : s + 1;
        const int bsrc = last ? 1 - h : h;
#pragma unroll
        for (int g = 0; g < 8; ++g) {
#pragma unroll
          for (int j = 0; j < NTN; ++j) {
            const int q = NTN * g + j;
            const int slot = kQ * s + q;
            if (slot == kBarSlot) sync();
            if (j == 0 && g >= 1) fa[g - 1] = frag_a(last ? a_nxt : a_cur, g - 1, s_n);
            if (q == extra_slot<NTN>(0)) {
              if (par == 0) fx = frag_a(last ? a_nxt : a_cur, 7, s_n);
              else fa[7] = frag_a(last ? a_nxt : a_cur, 7, s_n);
            }
#pragma unroll
            for (int jj = 0; jj < NTN; ++jj)
              if (q == extra_slot<NTN>(jj + 1)) fb[par ^ 1][jj] = frag_b(bsrc, jj, s_n);
            // Plan this step's window (B of t + 2 into B stage h, A of t + 3
            // into A stage sa, both freed by this step's barrier) and the A
            // offsets of step t + 1.
            if (slot == kPlan) {
              ub = step_scalars(t + 2);
              ua = step_scalars(t + 3);
            }
            if (slot == kPlan + 1) plan_b(ub, h, wn_);
            if (slot == kPlan + 2) plan_a(ua, sa, wn_);
            if (slot == kPlan + 3) a_rebase(a_nxt, sa1);
            if (slot < kWin - kAfter) {
              const int x = slot + kAfter;
              if (first_copy(x) < first_copy(x + 1)) issue(wc, first_copy(x));
            } else if (slot >= kBarSlot && slot - kBarSlot < kWin) {
              const int x = slot - kBarSlot;
              if (first_copy(x) < first_copy(x + 1)) issue(wn_, first_copy(x));
            }
            if (g == 7 && par == 1) acc[g][j] = mma(fx, fb[par][j], acc[g][j]);
            else acc[g][j] = mma(fa[g], fb[par][j], acc[g][j]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      wc = wn_;
#pragma unroll
      for (int x = 0; x < kX; ++x) a_cur[x] = a_nxt[x];
      sa = sa1;
    }
  }
  mfma_drain();
#pragma unroll
  for (int i = 0; i < NTM; ++i)
#pragma unroll
    for (int j = 0; j < NTN; ++j) asm volatile("" : "+a"(acc[i][j]));
  clock_mark(clock_ptr<Params>(), kClockLoopEnd, wave);

  __builtin_amdgcn_s_waitcnt(0);
  const int elane = lane_id_fresh();
  if (p.c_vec16_ok) {
    __syncthreads();
    store_c_lds<KIND, NTN>(p, Cb, acc,
                           (__attribute__((address_space(3))) uint8_t *)smem + wave * 32768,
                           m0 + wm * kWaveTile, n0 + wn * S::WN, elane);
  } else {
    store_c<KIND, NTN>(p, Cb, acc, m0 + wm * kWaveTile, n0 + wn * S::WN, elane);
  }
  clock_mark(clock_ptr<Params>(), kClockEnd, wave);
}

template __global__ void gemm_tn_ring_kernel<kF16, 8, true>(Params);
template __global__ void gemm_tn_ring_kernel<kF16, 7, true>(Params);
template __global__ void gemm_tn_ring_kernel<kF8, 8, true>(Params);
template __global__ void gemm_tn_ring_kernel<kF8, 7, true>(Params);
template __global__ void gemm_tn_ring_kernel<kF16, 8, false>(Params);
template __global__ void gemm_tn_ring_kernel<kF16, 7, false>(Params);
template __global__ void gemm_tn_ring_kernel<kF8, 8, false>(Params);
template __global__ void gemm_tn_ring_kernel<kF8, 7, false>(Params);

template __global__ void gemm_tn_kernel<kF16, 8, false, false, false>(Params);
template __global__ void gemm_tn_kernel<kF16, 7, false, false, false>(Params);
template __global__ void gemm_tn_kernel<kF8, 8, false, false, false>(Params);
template __global__ void gemm_tn_kernel<kF8, 7, false, false, false>(Params);
template __global__ void gemm_tn_kernel<kF16, 8, false, false, true>(Params);
template __global__ void gemm_tn_kernel<kF16, 7, false, false, true>(Params);
template __global__ void gemm_tn_kernel<kF8, 8, false, false, true>(Params);
template __global__ void gemm_tn_kernel<kF8, 7, false, false, true>(Params);

// ----------------------------------------------------------------- skinny K
// Kernels for K * es <= 256 bytes (the QK^T shape: K = head dim 128): the whole
// K extent of a 128 x 128 tile's A and B strips fits in LDS at once (2 x 32
// KiB), so there is no K pipeline; each wave owns 64 x 64 of C (4 x 4 MFMA
// tiles of 16 x 16, 64 accumulators; the 16x16 shapes draw less power than
// the 32x32 ones, which this power-limited kernel turns into clock, measured
// 2-3 % faster on the QK^T shape).  Writing C bounds these shapes; one tile per
// block and two blocks per CU let one block's stores drain while the other
// block copies and computes.
constexpr int kSkTile = 128;       // rows of A / columns of B per block
constexpr int kSkRow = 256;        // LDS bytes per row (all of K, zero-filled)
constexpr int kSkStrip = kSkTile * kSkRow;  // 32 KiB per operand
constexpr int kSkWave = 64;        // each wave owns 64 x 64 of C
constexpr int kSkSub = 4;          // MFMA tiles of 16 x 16 per wave edge
constexpr int kSkWalkMax = 32;     // most M tiles one block walks

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// Copies of one tile's A and B strips (128 rows x 256 B each, rows of 256 B,
// chunk c of row r in slot c ^ (r & 15), so a 16-row ds_read_b128 phase hits 16
// distinct slots of the bank period) into `stage`.  Load q (0..7) of wave w
// fills rows 16q + 4w .. +3 (1 KiB): lane l lands in row 16q + 4w + (l >> 4),
// slot l & 15.  Chunks at or past K are pointed out of range and read zero.
template <int KIND>
__device__ __forceinline__ void sk_copy_strip(const Params &p, lds_u8 *strip, const uint8_t *base,
                                              int64_t ld_b, int64_t rows, int wave, int lane) {
  typedef Traits<KIND> T;
  const uint32_t kbytes = (uint32_t)(p.K * T::es);
  const int crow = 4 * wave + (lane >> 4);
  const int gchunk = (lane & 15) ^ (crow & 15);
  const bool valid = gchunk * 16 < (int)kbytes;
  const __amdgpu_buffer_rsrc_t r = make_rsrc(base, (uint32_t)((rows - 1) * ld_b) + kbytes);
  const uint32_t v = valid ? (uint32_t)(crow * ld_b) + gchunk * 16 : kOob;
  lds_u8 *l = strip + wave * 1024;
#pragma unroll
  for (int q = 0; q < 8; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)(l + q * 4096), 16,
                                             v + q * (uint32_t)(16 * ld_b), 0, 0, 0);
}

// Copies of A's strip for tile row tm and of B's strip for tile column tn
// (128 rows x 256 B each, rows of 256 B, chunk c of row r in slot c ^ (r & 15),
// so a 16-row ds_read_b128 phase hits 16 distinct slots of the bank period).
// Load q (0..7) of wave w fills rows 16q + 4w .. +3 (1 KiB): lane l lands in
// row 16q + 4w + (l >> 4), slot l & 15.  Chunks at or past K are pointed out of
// range and read zero.
template <int KIND>
__device__ __forceinline__ void sk_copy_a(const Params &p, lds_u8 *strip, int head, int tm,
                                          int wave, int lane) {
  const int64_t m0 = (int64_t)tm * kSkTile;
  const int64_t rows = (p.M - m0) < kSkTile ? (p.M - m0) : kSkTile;
  sk_copy_strip<KIND>(p, strip, p.A + head * p.stride_a_b + m0 * p.lda_b, p.lda_b, rows, wave,
                      lane);
}
template <int KIND>
__device__ __forceinline__ void sk_copy_b(const Params &p, lds_u8 *strip, int head, int tn,
                                          int wave, int lane) {
  const int64_t n0 = (int64_t)tn * kSkTile;
  const int64_t rows = (p.N - n0) < kSkTile ? (p.N - n0) : kSkTile;
  sk_copy_strip<KIND>(p, strip, p.B + head * p.stride_b_b + n0 * p.ldb_b, p.ldb_b, rows, wave,
                      lane);
}

// The wave's 64 x 64 block of A x B from a stage as 4 x 4 MFMA tiles of
// 16 x 16: lane l reads row l % 16 of a 16-row tile and K group g = l / 16 of
// each sub-step (fp16 16x16x32: chunk 4s + g; fp8 16x16x128: chunks 8s + g and
// 8s + g + 4, the K order of the 256 x 256 kernel); fragments double-buffered.
// A 16-lane read phase covers 16 consecutive rows of one chunk: 16 distinct
// slots of the bank period.
template <int KIND>
__device__ __forceinline__ void sk_compute(float4_t_v (&acc)[kSkSub][kSkSub], lds_cptr stage,
                                           int wm, int wn, int lane) {
  typedef Traits<KIND> T;
  constexpr int kSubs = (KIND == kF16) ? 4 : 2;   // sub-steps over 256 bytes of K
  const int g = lane >> 4, sw = lane & 15;
  lds_cptr la = stage + (wm * kSkWave + sw) * kSkRow;
  lds_cptr lb = stage + kSkStrip + (wn * kSkWave + sw) * kSkRow;
  auto frag = [&](lds_cptr row0, int i, int s) -> typename T::frag_t {
    lds_cptr r = row0 + i * 16 * kSkRow;
    if constexpr (KIND == kF16) {
      const int c = 4 * s + g;
      return *(const __attribute__((address_space(3))) half8_t *)(r + ((c ^ sw) * 16));
    } else {
      const int c = 8 * s + g;
      const int4_t_v lo = *(const __attribute__((address_space(3))) int4_t_v *)(r + ((c ^ sw) * 16));
      const int4_t_v hi =
          *(const __attribute__((address_space(3))) int4_t_v *)(r + (((c + 4) ^ sw) * 16));
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };
#pragma unroll
  for (int i = 0; i < kSkSub; ++i)
#pragma unroll
    for (int j = 0; j < kSkSub; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.f;
  typename T::frag_t fa[2][kSkSub], fb[2][kSkSub];
#pragma unroll
  for (int i = 0; i < kSkSub; ++i) {
    fa[0][i] = frag(la, i, 0);
    fb[0][i] = frag(lb, i, 0);
  }
#pragma unroll
  for (int s = 0; s < kSubs; ++s) {
    const int u = s & 1;
    if (s + 1 < kSubs) {
#pragma unroll
      for (int i = 0; i < kSkSub; ++i) {
        fa[u ^ 1][i] = frag(la, i, s + 1);
        fb[u ^ 1][i] = frag(lb, i, s + 1);
      }
    }
#pragma unroll
    for (int i = 0; i < kSkSub; ++i)
#pragma unroll
      for (int j = 0; j < kSkSub; ++j) acc[i][j] = mma_c(fa[u][i], fb[u][j], acc[i][j]);
  }
}

// Converted accumulators of wave (wm, wn) into the tile's 32 KiB transpose
// buffer: column n (0..127) at n * 256 B, its 16-byte chunk c (rows 8c ..
// 8c+7) in slot c ^ (n & 15), the slot's 8-byte halves swapped when n & 8
// (conflict-free writes, as in store_c_lds).  Lane (rl, grp) of tile (i, j) holds rows
// 16i + 4 grp .. +3 of column 16j + rl: one 8-byte write per tile.  A 16-lane
// read phase covers one whole column (all 16 slots of a bank period).
template <int KIND>
__device__ __forceinline__ void sk_to_lds(const Params &p, const float4_t_v (&acc)[kSkSub][kSkSub],
                                          lds_u8 *buf, int wm, int wn, int lane) {
#pragma unroll
  for (int j = 0; j < kSkSub; ++j) {
    const int n = kSkWave * wn + 16 * j + (lane & 15);
#pragma unroll
    for (int i = 0; i < kSkSub; ++i) {
      const int m = kSkWave * wm + 16 * i + 4 * (lane >> 4);
      uint32_t w0, w1;
      pack_run<KIND>(p, acc[i][j], 0, w0, w1);
      u32x2 w;
      w.x = w0;
      w.y = w1;
      *(__attribute__((address_space(3))) u32x2 *)(buf + n * 256 + (((m >> 3) ^ (n & 15)) * 16) +
                                                 (((m & 7) * 2) ^ (n & 8))) = w;
    }
  }
}

// A block walks p.sk_walk consecutive M tiles of one tile column (two blocks
// per CU).  B's strip is copied once and stays in LDS; per tile: A's strip
// lands, MFMAs, the 128 x 128 result is transposed through the A space (both
// waves' rows of a column side by side) and read back into registers, then
// the next A strip is requested and the tile's stores are issued, so the copy
// overlaps the stores.  Wave w stores columns 32w .. 32w+31, each instruction
// four whole 256-byte columns: HBM takes 256-byte column runs about 10 %
// faster than the 128-byte runs of a per-wave transpose.
template <int KIND>
__global__ __launch_bounds__(kThreads, 2) void gemm_tn_skinny_kernel(Params p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kSkStrip];  // [A strip | B strip]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int chunks_m = (p.tiles_m + p.sk_walk - 1) / p.sk_walk;
  int head, tmc, tn;
  tile_of_block<int>((int)blockIdx.x, (int)gridDim.x, chunks_m, p.tiles_n, &head, &tmc, &tn,
                     p.order);
  clock_mark(clock_ptr<Params>(), kClockStart, wave);
  const int tm0 = tmc * p.sk_walk;
  const int tm_end = (tm0 + p.sk_walk) < p.tiles_m ? (tm0 + p.sk_walk) : p.tiles_m;
  lds_u8 *const a_st = (lds_u8 *)smem;
  lds_u8 *const b_st = (lds_u8 *)smem + kSkStrip;
  // (K = 0 still copies: every chunk is then out of range and reads zero.)
  sk_copy_b<KIND>(p, b_st, head, tn, wave, lane);
  sk_copy_a<KIND>(p, a_st, head, tm0, wave, lane);
  const int wm = wave & 1, wn = wave >> 1;
  uint8_t *Cb = p.C + head * p.stride_c_b;
  const int64_t n0 = (int64_t)tn * kSkTile;
  for (int tm = tm0; tm < tm_end; ++tm) {
    // This tile's A strip (and, first time round, B's) has landed; the wait
    // also covers the previous tile's stores.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    float4_t_v acc[kSkSub][kSkSub];
    sk_compute<KIND>(acc, (lds_cptr)smem, wm, wn, lane);
    __syncthreads();  // every wave is done reading A's strip
    sk_to_lds<KIND>(p, acc, a_st, wm, wn, lane);
    __syncthreads();  // the whole tile is in the transpose buffer
    u32x4 v[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int n = 32 * wave + 4 * r + (lane >> 4);
      v[r] = *(__attribute__((address_space(3))) u32x4 *)(a_st + n * 256 + (((lane & 15) ^ (n & 15)) * 16));
      if (r & 2) v[r] = v[r].zwxy;   // n & 8: the slot's two halves are swapped
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of the A space are done
    __syncthreads();                     // everyone's are: the next A strip may land
    if (tm + 1 < tm_end) sk_copy_a<KIND>(p, a_st, head, tm + 1, wave, lane);
    const int64_t m0 = (int64_t)tm * kSkTile;
    const bool full = (m0 + kSkTile <= p.M) && (n0 + kSkTile <= p.N) && p.c_vec16_ok;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int64_t gm = m0 + 8 * (lane & 15), gn = n0 + 32 * wave + 4 * r + (lane >> 4);
      uint16_t *dst = (uint16_t *)Cb + (gn * p.ldc + gm);
      if (full || (p.c_vec16_ok && gn < p.N && gm + 7 < p.M)) {
        // Non-temporal: C is written once and never read here, and letting it
        // allocate in L2 evicts the Q and K strips that later tiles re-read.
        __builtin_nontemporal_store(v[r], (u32x4 *)dst);
      } else if (gn < p.N) {
        const uint32_t wv[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (gm + e < p.M) dst[e] = (uint16_t)(wv[e >> 1] >> (16 * (e & 1)));
      }
    }
  }
  clock_mark(clock_ptr<Params>(), kClockEnd, wave);
}

template __global__ void gemm_tn_skinny_kernel<kF16>(Params);
template __global__ void gemm_tn_skinny_kernel<kF8>(Params);

// ------------------------------------------------------------------ host side


static bool overlaps(const void *a, uint64_t abytes, const void *b, uint64_t bbytes) {
  if (abytes == 0 || bbytes == 0) return false;
  const uint64_t a0 = (uint64_t)(uintptr_t)a, b0 = (uint64_t)(uintptr_t)b;
  return a0 < b0 + bbytes && b0 < a0 + abytes;
}

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Compute units of the current device, looked up once per device (256 on
// MI355X; that value is assumed if the query fails).
static int cu_count() {
  static std::atomic<int> cached[64];  // zero-initialised; racing writers store the same value
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Bytes spanned by `rows` rows of `row_elems` elements at stride `ld` (0 if empty).
static uint64_t span_bytes(int64_t rows, int64_t row_elems, int64_t ld, int es) {
  if (rows <= 0 || row_elems <= 0) return 0;
  return (uint64_t)(((rows - 1) * ld + row_elems) * es);
}

struct Problem {
  const void *A, *B;
  void *C;
  int64_t batch, M, N, K, lda, ldb, ldc, stride_a, stride_b, stride_c;
  float scale;
};

// ---------------------------------------------------------------------------
// gemm_tn_mid_kernel<KIND>: 128 x 128 output tiles with two blocks per CU, for
// grids the 256-wide tiles cannot fill (one tile configuration is wrong for
// small or skinny products, so a set of configurations with a selector is
// needed: "FP16 GEMM optimisation on AMD RDNA 3 and RDNA 4", sections "Final
// results" and "Further tuning").
//   * 4 waves of 64 x 64 (4 x 4 MFMA tiles of 16 x 16, accumulators in VGPRs
//     and the products left to the compiler: the two co-resident blocks
//     interleave their waves on each SIMD, which hides what one wave waits on).
//   * K-steps of 128 bytes per row in two LDS stages of [A strip | B strip]
//     (128 rows x 128 B each, same XOR swizzle and fragment map as the
//     256 x 256 kernel), one barrier per K-step; the next step's copies are
//     issued right after it, so they have a whole step to land.
//   * Direct column-major stores of runs of four rows (8 bytes), masked past
//     M and N.
constexpr int kMidTile = 128;
constexpr int kMidStrip = kMidTile * kRowBytes;  // 16 KiB per operand per stage
// Relative cost per output element of the 128 x 128 kernel, in 64ths of the
// 256-row kernel's (measured; see the host selector in launch<>).
constexpr int kMidCost = 83;

// An operand of the 128 x 128 kernel in LDS.  K-major operands (K
// contiguous: A of a 'T' op, B of an 'N' op) use the 128 x 128-byte strip of
// the 256-row kernel.  M/N-major fp16 operands (A of an 'N' op: A[m + k*lda];
// B of a 'T' op: B[k*ldb + n]) keep their own layout: 64 K-rows of 128
// elements (256 B), the 16-byte chunk c of K-row k stored in slot
// c ^ (2 (k & 3) + 8 ((k >> 3) & 1)), and fragments come from gfx950's
// transposing LDS read: within each 16-lane group, ds_read_b64_tr_b16 gives
// lane 4a + b element b of the 8 bytes addressed by lane 4e + a as its value e
// (measured), so lanes 4e + a pointing at K-row k0 + e, elements 4a .. 4a + 3
// of a 16-wide tile leave lane j holding K-rows k0 .. k0 + 3 of column j --
// the MFMA operand layout.  The swizzle spreads the sixteen K-rows one such
// read touches (two 16-lane groups per LDS pass) over distinct slots.
// M/N-major fp8 operands: 128 K-rows of 128 bytes, chunk c of K-row k in slot
// c ^ mn_swz8(k), fragments from ds_read_b64_tr_b8 (see mn_frag8).
template <bool MN>
struct MidOperand {
  uint32_t off[4];     // copy offsets of loads q = 0..3 (lane constant)
  int krow[4];         // M/N-major: K-row of load q; K-major: unused
  bool cvalid[4];      // M/N-major: the load's chunk lies inside M (or N)
  uint32_t frag[4];    // fragment read offsets (see read)
};

// Swizzle key of K-row k in the 128 x 128 kernel's M/N-contiguous strips
// (fp16: 256-byte K-rows, fp8: 128-byte K-rows): distinct 16-byte bank groups
// for the K-rows one transposing read phase touches.
__device__ __forceinline__ int mn_swz(int k) { return 2 * (k & 3) + 8 * ((k >> 3) & 1); }
__device__ __forceinline__ int mn_swz8(int k) { return ((k >> 1) & 3) + 4 * ((k >> 4) & 1); }

// Copies of one operand of the 128 x 128 kernel for K-step t into this
// wave's KiB `st` of each 4 KiB quarter of the operand's LDS strip.
// ASM: issue the loads from inline assembly (kernels with an M/N-contiguous
// operand; see StepCopyAsm).
template <int KIND, bool MN, bool ASM>
__device__ __forceinline__ void mid_copy(const uint8_t *base, int64_t ld_b, int64_t K,
                                         uint32_t rec, uint32_t voff, uint32_t qs, int kchunk,
                                         const MidOperand<MN> &op, int64_t t, lds_u8 *st) {
  typedef Traits<KIND> T;
  const int64_t k0 = t * T::kstep;
  uint32_t off[4];
  const uint8_t *rbase;
  uint32_t rbytes;
  if constexpr (MN) {
    // Rebased on the step's first K-row; rows at or past K and chunks past
    // M / N read zero.  The descriptor covers the step's K-rows.
    rbase = base + k0 * ld_b;
    rbytes = (uint32_t)(T::kstep * ld_b);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool ok = op.cvalid[q] && k0 + op.krow[q] < K;
      off[q] = ok ? op.off[q] : kOob;
    }
  } else {
    const int64_t rem = K - k0;
    const int left = rem >= T::kstep ? T::kstep : (int)rem;
    const uint32_t kb = (uint32_t)(k0 * T::es);
    rbase = base + kb;
    rbytes = rec - kb;
    const uint32_t v = kchunk < left ? voff : kOob;
#pragma unroll
    for (int q = 0; q < 4; ++q) off[q] = v + q * qs;
  }
  if constexpr (ASM) {
    const v4u32 r = rsrc_words(rbase, rbytes);
#pragma unroll
    for (int q = 0; q < 4; ++q) dma16(r, off[q], (uint32_t)(uintptr_t)(st + q * 4096));
  } else {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(rbase, rbytes);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)(st + q * 4096), 16, off[q], 0,
                                               0, 0);
  }
}

// STAGES: LDS stages of the K ring.  2 (64 KiB, two blocks per CU): while one
// block waits for its next step's copies the other computes.  4 (128 KiB, one
// block per CU) for grids of at most one block per CU, where nothing else
// covers the wait: copies run three steps ahead, so a step whose operands
// come from HBM (a round trip several times the 512 MFMA cycles of a step)
// does not stall the products.
// KF (TN only): this block's K range is a whole number of K-steps, so every
// step's copies use the same lane offsets (formed once), steps past the range
// get an empty descriptor instead of out-of-range lane offsets, and every step
// issues its copies unconditionally: the loop's copy addressing and its waits
// then take no vector ALU instructions and no branches.
template <int KIND, bool AMN, bool BMN, bool SPLIT = false, int STAGES = 2, bool KF = false>
__global__ __launch_bounds__(kThreads, STAGES == 2 ? 2 : 1) void gemm_tn_mid_kernel(Params p) {
  typedef Traits<KIND> T;
  static_assert(!SPLIT || (!AMN && !BMN), "split-K partials are TN only");
  static_assert(!KF || (!AMN && !BMN), "whole K-steps: TN only");
  static_assert(STAGES == 2 || STAGES == 4, "a ring of 2 or 4 stages");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * 2 * kMidStrip];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  int head, tm, tn;
  tile_of_block<int>((int)blockIdx.x, (int)gridDim.x, p.tiles_m, p.tiles_n, &head, &tm, &tn,
                     p.order);
  const int64_t m0 = (int64_t)tm * kMidTile, n0 = (int64_t)tn * kMidTile;
  clock_mark(clock_ptr<Params>(), kClockStart, wave);
  // Split-K: the "head" index is the split; this block's K range starts at
  // k_begin (a whole number of K-steps) and the operands are read from there.
  const int64_t k_begin = SPLIT ? head * p.k_slice : 0;
  const int64_t Kx = SPLIT ? ((p.K - k_begin) < p.k_slice ? (p.K - k_begin) : p.k_slice) : p.K;
  // Block bases: K-major operands at their first row, M/N-major ones at their
  // first column (element m0 / n0 of K-row 0).
  const uint8_t *Ab = SPLIT ? p.A + m0 * p.lda_b + k_begin * T::es
                            : p.A + head * p.stride_a_b + (AMN ? m0 * T::es : m0 * p.lda_b);
  const uint8_t *Bb = SPLIT ? p.B + n0 * p.ldb_b + k_begin * T::es
                            : p.B + head * p.stride_b_b + (BMN ? n0 * T::es : n0 * p.ldb_b);
  uint8_t *Cb = p.C + head * p.stride_c_b;
  const int64_t rows_a = (p.M - m0) < kMidTile ? (p.M - m0) : kMidTile;
  const int64_t rows_b = (p.N - n0) < kMidTile ? (p.N - n0) : kMidTile;
  const uint32_t kbytes = (uint32_t)(Kx * T::es);

  // K-major copies: load q (0..3) of wave w fills strip rows 32q + 8w .. +7;
  // lane l lands in row 32q + 8w + (l >> 3), slot l & 7, and fetches the chunk
  // the swizzle keeps there.  Rows past the matrix and chunks at or past K
  // read zero.
  const int crow = 8 * wave + (lane >> 3);
  const int gchunk = (lane & 7) ^ ((crow >> 1) & 7);
  const int kchunk = gchunk * (16 / T::es);
  // M/N-major copies (load q of wave w: 1 KiB at strip byte 4096 q + 1024 w).
  // fp16 (256-byte K-rows): lane l lands in K-row 16q + 4w + (l >> 4), slot
  // l & 15.  fp8 (128-byte K-rows): K-row 32q + 16 (w >> 1) + 8 (w & 1) +
  // (l >> 3), slot l & 7.  Each fetches the chunk its slot holds under the
  // swizzle; chunks past M (N) and K-rows past K read zero.
  auto mn_operand = [&](int64_t ld_b, int64_t rows) {
    MidOperand<true> o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k = (KIND == kF16) ? 16 * q + 4 * wave + (lane >> 4)
                                   : 32 * q + 16 * (wave >> 1) + 8 * (wave & 1) + (lane >> 3);
      const int c = (KIND == kF16) ? (lane & 15) ^ mn_swz(k) : (lane & 7) ^ mn_swz8(k);
      o.krow[q] = k;
      o.off[q] = (uint32_t)(k * ld_b) + c * 16;
      o.cvalid[q] = (16 / T::es) * c < rows;
    }
    return o;
  };
  MidOperand<AMN> opa;
  MidOperand<BMN> opb;
  if constexpr (AMN) opa = mn_operand(p.lda_b, rows_a);
  if constexpr (BMN) opb = mn_operand(p.ldb_b, rows_b);
  const uint32_t voff_a = (uint32_t)(crow * p.lda_b) + gchunk * 16;
  const uint32_t voff_b = (uint32_t)(crow * p.ldb_b) + gchunk * 16;
  const uint32_t qs_a = (uint32_t)(32 * p.lda_b), qs_b = (uint32_t)(32 * p.ldb_b);
  const uint32_t rec_a = AMN ? 0u : (uint32_t)((rows_a - 1) * p.lda_b) + kbytes;
  const uint32_t rec_b = BMN ? 0u : (uint32_t)((rows_b - 1) * p.ldb_b) + kbytes;
  const int64_t nk = (Kx + T::kstep - 1) / T::kstep;

  auto copy_step = [&](int64_t t) {
    lds_u8 *st = (lds_u8 *)smem + (t & (STAGES - 1)) * 2 * kMidStrip + wave * 1024;
    mid_copy<KIND, AMN, AMN || BMN>(Ab, p.lda_b, Kx, rec_a, voff_a, qs_a, kchunk, opa, t, st);
    mid_copy<KIND, BMN, AMN || BMN>(Bb, p.ldb_b, Kx, rec_b, voff_b, qs_b, kchunk, opb, t,
                                    st + kMidStrip);
  };
  // Whole K-steps: fixed lane offsets (the empty asm statements keep them in
  // registers), one descriptor pair per step, empty past the range.
  uint32_t cva[4], cvb[4];
  if constexpr (KF) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      cva[q] = voff_a + (uint32_t)q * qs_a;
      cvb[q] = voff_b + (uint32_t)q * qs_b;
      asm volatile("" : "+v"(cva[q]));
      asm volatile("" : "+v"(cvb[q]));
    }
  }
  const int nk32 = (int)nk;
  auto copy_step_kf = [&](int t) {
    const bool inside = t < nk32;
    const uint32_t kb = inside ? (uint32_t)t * (uint32_t)(T::kstep * T::es) : 0u;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(Ab + kb, inside ? rec_a - kb : 0u);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bb + kb, inside ? rec_b - kb : 0u);
    lds_u8 *st = (lds_u8 *)smem + (t & (STAGES - 1)) * 2 * kMidStrip + wave * 1024;
#pragma unroll
    for (int q = 0; q < 4; ++q) lds_copy16(ra, (lds_void_t *)(st + q * 4096), cva[q]);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      lds_copy16(rb, (lds_void_t *)(st + kMidStrip + q * 4096), cvb[q]);
  };

  // Fragments.  K-major: lane l reads row l % 16 of a 16-row tile; fp16 takes
  // chunk 4s + g of sub-step s, fp8 chunks g and g + 4 (g = l / 16), as in the
  // 256 x 256 kernel.  M/N-major: two transposing reads per sub-step (K-rows
  // 32s + 8g + 4h + (l % 16) / 4, h = 0, 1) at elements 4 ((l % 16) % 4) of
  // the tile.
  const int wm = wave & 1, wn = wave >> 1;
  const int rl = lane & 15, grp = lane >> 4;
  uint32_t a_off[4] = {0, 0, 0, 0}, b_off[4] = {0, 0, 0, 0};
#pragma unroll
  for (int x = 0; x < T::subs * T::reads; ++x) {
    const int chunk = (x / T::reads) * (8 / T::subs) + grp + 4 * (x % T::reads);
    const uint32_t lo = (uint32_t)(rl * kRowBytes + ((chunk ^ ((rl >> 1) & 7)) * 16));
    a_off[x] = lo + wm * 64 * kRowBytes;
    b_off[x] = lo + kMidStrip + wn * 64 * kRowBytes;
  }
  // M/N-major: lane constants of the read address (see the layout above):
  // K-row 8g + (rl >> 2) (+ 32s + 4h), slot of the tile's first chunk
  // (8 w + 2i) ^ swz with swz = 2 (rl >> 2) + 8 (g & 1), plus chunk half and
  // 8-byte half from rl & 3.
  // fp8: lane (rl, grp) reads K-row 16 grp + rl / 2 (+ 8, 64, 72) at bytes
  // 8 (rl % 2) .. +7 of the tile's single 16-byte chunk 4 w + i, in slot
  // (4 w + i) ^ swz8 with swz8 = (rl >> 2) + 4 (grp & 1).
  const int mn_k = (KIND == kF16) ? 8 * grp + (rl >> 2) : 16 * grp + (rl >> 1);
  const int mn_swz_l = (KIND == kF16) ? mn_swz(mn_k) : mn_swz8(mn_k);
  auto mn_frag = [&](lds_cptr strip, int w, int i, int s) -> typename T::frag_t {
    if constexpr (KIND == kF16) {
      typedef short v4i16 __attribute__((ext_vector_type(4)));
      const int slot = ((8 * w + 2 * i) ^ mn_swz_l) + ((rl & 3) >> 1);
      const uint32_t off = (uint32_t)((32 * s + mn_k) * 256 + slot * 16 + (rl & 1) * 8);
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16 *)(strip + off));
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16 *)(strip + off + 4 * 256));
      return __builtin_bit_cast(half8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    } else {
      const int slot = (4 * w + i) ^ mn_swz_l;
      return mn_frag8<128>(strip, (uint32_t)(mn_k * 128 + slot * 16 + (rl & 1) * 8));
    }
  };

  float4_t_v acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = float4_t_v{0.f, 0.f, 0.f, 0.f};

  // Steps 0 .. STAGES - 2 ahead of the loop; step t + STAGES - 1 goes into the
  // stage step t - 1 used, right after the barrier that ends its reads.
  if constexpr (KF) {
#pragma unroll
    for (int t = 0; t < STAGES - 1; ++t) copy_step_kf(t);
  } else {
#pragma unroll
    for (int t = 0; t < STAGES - 1; ++t)
      if (t < nk) copy_step(t);
  }
  for (int64_t t = 0; t < nk; ++t) {
    // This wave's copies of step t have landed (loads complete in order; the
    // copies of the at most STAGES - 2 steps issued after it may still run,
    // eight per step: four loads of each operand) and its reads of step t - 1
    // are done; after the barrier every wave's are.  A plain barrier:
    // __syncthreads() would also wait for the later steps' copies.
    const int64_t later = nk - 1 - t;
    if constexpr (KF)   // every step issued its eight copies, past the range too
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(8 * (STAGES - 2)) & 0xF0FF);
    else if (STAGES == 2 || later <= 0)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0) & 0xF0FF);
    else if (later == 1)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(8) & 0xF0FF);
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(16) & 0xF0FF);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if constexpr (KF)
      copy_step_kf((int)t + STAGES - 1);
    else if (t + STAGES - 1 < nk)
      copy_step(t + STAGES - 1);
    lds_cptr st = (lds_cptr)smem + (t & (STAGES - 1)) * 2 * kMidStrip;
#pragma unroll
    for (int s = 0; s < T::subs; ++s) {
      typename T::frag_t fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (AMN)
          fa[i] = mn_frag(st, wm, i, s);
        else
          fa[i] = read_frag<KIND>(st + i * 16 * kRowBytes, a_off, s);
        if constexpr (BMN)
          fb[i] = mn_frag(st + kMidStrip, wn, i, s);
        else
          fb[i] = read_frag<KIND>(st + i * 16 * kRowBytes, b_off, s);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = KF ? mma_t(fa[i], fb[j], acc[i][j]) : mma_c(fa[i], fb[j], acc[i][j]);
    }
  }

  // The copies issued past the range (KF) still write the LDS: they land
  // before the block may end.  The products' wait states pass before the
  // epilogue reads the accumulators, every one tied to that wait.
  if constexpr (KF) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    mfma_drain();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) asm volatile("" : "+a"(acc[i][j]));
  }
  // Lane (rl, grp) of tile (i, j) holds C rows 16i + 4 grp .. +3 of column
  // 16j + rl of the wave's 64 x 64 block.
  const int64_t mb = m0 + wm * 64 + 4 * grp, nb = n0 + wn * 64 + rl;
  if constexpr (SPLIT) {
    // fp32 partial sums, 16 bytes per lane (ldw % 4 == 0, so aligned).
    float *Wh = p.W + head * p.N * p.ldw;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = nb + 16 * j;
      if (n >= p.N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = mb + 16 * i;
        float *dst = Wh + n * p.ldw + m;
        if (m + 3 < p.M) {
          *(float4_t_v *)dst = acc[i][j];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (m + e < p.M) dst[e] = acc[i][j][e];
        }
      }
    }
    clock_mark(clock_ptr<Params>(), kClockEnd, wave);
    return;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t n = nb + 16 * j;
    if (n >= p.N) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = mb + 16 * i;
      uint32_t w0, w1;
      pack_run<KIND>(p, acc[i][j], 0, w0, w1);
      uint16_t *dst = (uint16_t *)Cb + (n * p.ldc + m);
      if (p.c_vec_ok && m + 3 < p.M) {
        *(uint2 *)dst = uint2{w0, w1};
      } else {
        const uint16_t h[4] = {(uint16_t)w0, (uint16_t)(w0 >> 16), (uint16_t)w1,
                               (uint16_t)(w1 >> 16)};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (m + e < p.M) dst[e] = h[e];
      }
    }
  }
  clock_mark(clock_ptr<Params>(), kClockEnd, wave);
}

// Split-K reduction: C(m, n) = convert(sum over splits h = 0, 1, ... of
// W[h][n][m]) in that fixed order (deterministic), the conversion of the
// epilogue (fp16, or bf16 of the fp32 sum times the scale product).  One
// thread per four consecutive rows of a column: 16-byte partial loads.
template <int KIND>
__global__ __launch_bounds__(kThreads) void gemm_splitk_reduce_kernel(Params p, int32_t splits) {
  const int64_t quads = (p.M + 3) / 4;
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= quads * p.N) return;
  const int64_t n = idx / quads, m = 4 * (idx - n * quads);
  const float *src = p.W + n * p.ldw + m;
  const int64_t hs = p.N * p.ldw;   // floats between consecutive splits
  float4_t_v sum = *(const float4_t_v *)src;
  int32_t h = 1;
  // Four loads in flight before their (in-order) additions.
  for (; h + 3 < splits; h += 4) {
    const float4_t_v v0 = __builtin_nontemporal_load((const float4_t_v *)(src + h * hs));
    const float4_t_v v1 = __builtin_nontemporal_load((const float4_t_v *)(src + (h + 1) * hs));
    const float4_t_v v2 = __builtin_nontemporal_load((const float4_t_v *)(src + (h + 2) * hs));
    const float4_t_v v3 = __builtin_nontemporal_load((const float4_t_v *)(src + (h + 3) * hs));
    sum += v0;
    sum += v1;
    sum += v2;
    sum += v3;
  }
  for (; h < splits; ++h) sum += __builtin_nontemporal_load((const float4_t_v *)(src + h * hs));
  uint32_t w0, w1;
  pack_run<KIND>(p, sum, 0, w0, w1);
  uint16_t *dst = (uint16_t *)p.C + (n * p.ldc + m);
  if (p.c_vec_ok && m + 3 < p.M) {
    *(uint2 *)dst = uint2{w0, w1};
  } else {
    const uint16_t h4[4] = {(uint16_t)w0, (uint16_t)(w0 >> 16), (uint16_t)w1, (uint16_t)(w1 >> 16)};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (m + e < p.M) dst[e] = h4[e];
  }
}

// ---------------------------------------------------------------------------
// gemm_tn_pp_kernel<KIND>: the 8-wave "ping-pong" form of the 256 x 256 tile
// (the alternative the MI355X FP8 GEMM page weighs against its 4-wave design
// and rejects for register budget and compiler sensitivity), built here to
// measure that choice on this hardware.
//   * 512 threads = 8 waves, two per SIMD; waves 4g .. 4g+3 form group g and
//     own the 128-column half g of the tile, wave w the 64-row band w % 4:
//     4 x 8 MFMA tiles of 16 x 16 per wave (128 accumulators in AGPRs; the
//     other 128 registers of the wave's half of the register file hold one
//     K-step of fragments and addresses -- no room to double-buffer them).
//   * The two groups alternate: while one group's waves run the products of
//     a K-step, the other group's waves read their fragments of the next step
//     from LDS (and group 0 also issues the copies), so each SIMD's matrix
//     core is fed by one wave while the other waits on memory.  Phase p ends
//     with a barrier of all 8 waves; group 0 reads step t in phase 2t and
//     multiplies it in 2t + 1, group 1 one phase later.  Both groups run one
//     loop body; group 1 is delayed by one extra barrier.
//   * Group 0 issues the copies of step t + 1 in phase 2t (all 64 loads, 16
//     per wave: the 4-wave kernel's copy geometry) into the stage freed by the
//     barrier that ended phase 2t - 1, and waits for them before the barrier
//     that ends phase 2t + 1.
//   * Same LDS layout, swizzle and fragment map as the 4-wave kernel; the
//     epilogue goes through LDS (16 KiB per wave) with 16-byte stores.
constexpr int kPpThreads = 512;
constexpr int kPpWaveM = 64;     // rows per wave
constexpr int kPpWaveN = 128;    // columns per wave

// Epilogue of a 64 x 128 wave tile through the wave's 16 KiB of LDS: column n
// at n * 128 B, its 16-byte chunk c (8 rows) in slot c ^ (n & 7), the slot's
// 8-byte halves swapped when n & 8 (conflict-free writes, as in store_c_lds);
// read back as 8 rows per lane, eight 128-byte column segments per store
// instruction.
template <int KIND>
__device__ __forceinline__ void store_c_pp(const Params &p, uint8_t *Cb,
                                           const float4_t_v (&acc)[4][8],
                                           __attribute__((address_space(3))) uint8_t *buf,
                                           int64_t m_base, int64_t n_base, int lane) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) u32x2 lds_u2;
  typedef __attribute__((address_space(3))) u32x4 lds_u4;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int n = 16 * j + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 16 * i + 4 * (lane >> 4);
      uint32_t w0, w1;
      pack_run<KIND>(p, acc[i][j], 0, w0, w1);
      u32x2 w;
      w.x = w0;
      w.y = w1;
      *(lds_u2 *)(buf + n * 128 + (((m >> 3) ^ (n & 7)) * 16) + (((m & 7) * 2) ^ (n & 8))) = w;
    }
  }
  const bool full = (m_base + kPpWaveM <= p.M) && (n_base + kPpWaveN <= p.N);
#pragma unroll
  for (int r = 0; r < kPpWaveN / 8; ++r) {
    const int n = 8 * r + (lane >> 3);
    const int mc = lane & 7;
    u32x4 v = *(lds_u4 *)(buf + n * 128 + ((mc ^ (n & 7)) * 16));
    if (r & 1) v = v.zwxy;   // n & 8: the slot's two halves are swapped
    const int64_t gm = m_base + 8 * mc, gn = n_base + n;
    uint16_t *dst = (uint16_t *)Cb + (gn * p.ldc + gm);
    if (full || (gn < p.N && gm + 7 < p.M)) {
      __builtin_nontemporal_store(v, (u32x4 *)dst);
    } else if (gn < p.N) {
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (gm + e < p.M) dst[e] = (uint16_t)(wv[e >> 1] >> (16 * (e & 1)));
    }
  }
}

template <int KIND>
__global__ __launch_bounds__(kPpThreads, 1) void gemm_tn_pp_kernel(Params p) {
  typedef Traits<KIND> T;
  typedef typename T::frag_t frag_t;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * 2 * kStageBytes];
  typedef __attribute__((address_space(3))) uint8_t lds_u8;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, wm = wave & 3;

  int head, tm, tn;
  tile_of_block<int>((int)blockIdx.x, (int)gridDim.x, p.tiles_m, p.tiles_n, &head, &tm, &tn,
                     p.order);
  const int64_t m0 = (int64_t)tm * kTile, n0 = (int64_t)tn * kTile;
  clock_mark(clock_ptr<Params>(), kClockStart, wave);
  const uint8_t *Ab = p.A + head * p.stride_a_b + m0 * p.lda_b;
  const uint8_t *Bb = p.B + head * p.stride_b_b + n0 * p.ldb_b;
  uint8_t *Cb = p.C + head * p.stride_c_b;
  const int64_t rows_a = (p.M - m0) < kTile ? (p.M - m0) : kTile;
  const int64_t rows_b = (p.N - n0) < kTile ? (p.N - n0) : kTile;
  const uint32_t kbytes = (uint32_t)(p.K * T::es);
  const uint32_t rec_a = (uint32_t)((rows_a - 1) * p.lda_b) + kbytes;
  const uint32_t rec_b = (uint32_t)((rows_b - 1) * p.ldb_b) + kbytes;
  const int64_t nk = (p.K + T::kstep - 1) / T::kstep;

  // Copies (group 0 only): wave wm's share of the 4-wave kernel's geometry.
  const int crow = 8 * wm + (lane >> 3);
  const int gchunk = (lane & 7) ^ ((crow >> 1) & 7);
  const uint32_t voff_a = (uint32_t)(crow * p.lda_b) + gchunk * 16;
  const uint32_t voff_b = (uint32_t)(crow * p.ldb_b) + gchunk * 16;
  const uint32_t qs_a = (uint32_t)(32 * p.lda_b), qs_b = (uint32_t)(32 * p.ldb_b);
  const int kchunk = gchunk * (16 / T::es);
  auto copy_step = [&](int64_t t) {
    const int64_t k0 = t * T::kstep;
    const int64_t rem = p.K - k0;
    const int left = rem >= T::kstep ? T::kstep : (int)rem;
    const uint32_t kb = (uint32_t)(k0 * T::es);
    StepCopy c;
    c.ra = make_rsrc(Ab + kb, rec_a - kb);
    c.rb = make_rsrc(Bb + kb, rec_b - kb);
    lds_u8 *st = (lds_u8 *)smem + (int)(t & 1) * 2 * kStageBytes + wm * 1024;
    c.la = st;
    c.lb = st + kStageBytes;
    const bool valid = kchunk < left;
    c.va = valid ? voff_a : kOob;
    c.vb = valid ? voff_b : kOob;
#pragma unroll
    for (int d = 0; d < 16; ++d) copy_one<false, false>(c, d, qs_a, qs_b);
  };

  // Fragments: lane l reads row l % 16 of a 16-row tile (as in the 4-wave
  // kernel); A tiles of the wave's 64-row band, B tiles of its 128 columns.
  const int rl = lane & 15, kg = lane >> 4;
  uint32_t a_off[4], b_off[4];
#pragma unroll
  for (int x = 0; x < T::subs * T::reads; ++x) {
    const int chunk = (x / T::reads) * (8 / T::subs) + kg + 4 * (x % T::reads);
    const uint32_t lo = (uint32_t)(rl * kRowBytes + ((chunk ^ ((rl >> 1) & 7)) * 16));
    a_off[x] = lo + wm * kPpWaveM * kRowBytes;
    b_off[x] = lo + kStageBytes + grp * kPpWaveN * kRowBytes;
  }
  constexpr int kTileBytes = 16 * kRowBytes;

  float4_t_v acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = float4_t_v{0.f, 0.f, 0.f, 0.f};
  frag_t fa[T::subs][4], fb[T::subs][8];

  auto barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // Read all fragments of step t; they are complete (lgkmcnt 0) before the
  // phase's barrier, so the stage may be refilled right after the next one.
  auto mem_phase = [&](int64_t t) {
    lds_cptr st = (lds_cptr)smem + (int)(t & 1) * 2 * kStageBytes;
#pragma unroll
    for (int s = 0; s < T::subs; ++s) {
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[s][i] = read_frag<KIND>(st + i * kTileBytes, a_off, s);
#pragma unroll
      for (int j = 0; j < 8; ++j) fb[s][j] = read_frag<KIND>(st + j * kTileBytes, b_off, s);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(63) & 0xC0FF);  // lgkmcnt(0)
  };
  auto compute_phase = [&]() {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int s = 0; s < T::subs; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = mma(fa[s][i], fb[s][j], acc[i][j]);
    __builtin_amdgcn_s_setprio(0);
  };

  // Prologue: step 0's copies, landed and published.  Then both groups run
  // the same loop -- read step t, barrier, multiply step t, barrier -- group 1
  // one barrier behind group 0 (an extra barrier before its loop, matched by
  // one after group 0's), so one group's reads overlap the other's products.
  if (grp == 0 && nk > 0) copy_step(0);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();
  if (grp == 1) barrier();
  for (int64_t t = 0; t < nk; ++t) {
    if (grp == 0 && t + 1 < nk) copy_step(t + 1);
    mem_phase(t);
    __builtin_amdgcn_sched_barrier(0);
    barrier();
    compute_phase();
    // Group 0's copies of step t + 1 have landed before the barrier that lets
    // either group read them.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __builtin_amdgcn_sched_barrier(0);
    barrier();
  }
  if (grp == 0) barrier();
  mfma_drain();
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) asm volatile("" : "+a"(acc[i][j]));
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const int64_t mb = m0 + wm * kPpWaveM, nb = n0 + grp * kPpWaveN;
  const int elane = lane_id_fresh();   // not kept live across the loop (see lane_id_fresh)
  if (p.c_vec16_ok) {
    store_c_pp<KIND>(p, Cb, acc, (lds_u8 *)smem + wave * 16384, mb, nb, elane);
  } else {
    // Runs of four rows, 8-byte or 2-byte stores.
    const int erl = elane & 15, ekg = elane >> 4;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t n = nb + 16 * j + erl;
      if (n >= p.N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = mb + 16 * i + 4 * ekg;
        uint32_t w0, w1;
        pack_run<KIND>(p, acc[i][j], 0, w0, w1);
        uint16_t *dst = (uint16_t *)Cb + (n * p.ldc + m);
        if (p.c_vec_ok && m + 3 < p.M) {
          *(uint2 *)dst = uint2{w0, w1};
        } else {
          const uint16_t h[4] = {(uint16_t)w0, (uint16_t)(w0 >> 16), (uint16_t)w1,
                                 (uint16_t)(w1 >> 16)};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (m + e < p.M) dst[e] = h[e];
        }
      }
    }
  }
  clock_mark(clock_ptr<Params>(), kClockEnd, wave);
}

// Kernel configuration of a problem (the codes are the C ABI's
// gemm_tn_config values).
enum { kCfg256 = 0, kCfg224 = 1, kCfgMid = 2, kCfgSkinny = 3, kCfgPingPong = 4 };
// DG_GEMM_RING = 0 in the environment makes TN calls take gemm_tn_kernel's two
// [A | B] stages instead of gemm_tn_ring_kernel (measurement only).
static bool ring_env() {
  const char *r = getenv("DG_GEMM_RING");
  return !(r && r[0] == '0');
}
struct Config {
  int kind;
};
// Skinny contractions (all of K fits one 256-byte LDS row) take the skinny-K
// kernel.  Otherwise the 256-row pipeline takes 256- or 224-column tiles
// (NTN = 8 or 7 MFMA tiles per wave): with one block per CU its time is about
// (rounds of CU-count blocks) x (tile width), so the narrower tile wins when
// it packs the grid into enough fewer rounds (1920 x 13900: 440 wide tiles are
// two rounds of 256 CUs, 504 narrow ones also two, each 7/8 as long).  Grids
// that leave CUs idle that way take the 128 x 128 kernel instead: modelled
// time = (blocks per CU, rounded up) x tile area, the small tile's area
// weighted by kMidCost / 64.  DG_GEMM_TILE = 256, 224 or 128 in the
// environment forces the tile of a non-skinny problem (measurement and tests).
// tn = false: a layout with an M/N-contiguous operand, which has neither the
// skinny-K kernel (its problems take the 128 x 128 tiles) nor the 224-wide
// tiles.
static Config choose_config(int es, int64_t M, int64_t N, int64_t K, int64_t batch,
                            bool tn = true) {
  if (K * es <= kSkRow) return Config{tn ? kCfgSkinny : kCfgMid};
  if (const char *force = getenv("DG_GEMM_TILE")) {
    if (!strcmp(force, "256")) return Config{kCfg256};
    if (!strcmp(force, "224")) return Config{tn ? kCfg224 : kCfg256};
    if (!strcmp(force, "128")) return Config{kCfgMid};
    if (!strcmp(force, "pingpong") && tn) return Config{kCfgPingPong};
  }
  const int64_t cus = cu_count();
  const int64_t tm = (M + kTile - 1) / kTile;
  auto cost = [&](int64_t w) {
    const int64_t blocks = tm * ((N + 32 * w - 1) / (32 * w)) * batch;
    return ((blocks + cus - 1) / cus) * w;
  };
  const int64_t ntn = tn && cost(7) < cost(8) ? 7 : 8;
  const int64_t mid_blocks = ((M + kMidTile - 1) / kMidTile) * ((N + kMidTile - 1) / kMidTile) * batch;
  const int64_t t_big = cost(ntn) * kTile * 32 * 64;  // x 64: the scale of kMidCost
  const int64_t t_mid = ((mid_blocks + cus - 1) / cus) * kMidTile * kMidTile * kMidCost;
  if (t_mid < t_big) return Config{kCfgMid};
  return Config{ntn == 7 ? kCfg224 : kCfg256};
}

// DG_TILE_ORDER = row | grouped selects a measurement order for the TN
// calls (see tile_of_block); anything else, or nothing, the library's own.
static int tile_order_env() {
  const char *o = getenv("DG_TILE_ORDER");
  if (!o) return kOrderXcd;
  if (!strcmp(o, "row")) return kOrderRow;
  if (!strcmp(o, "grouped")) return kOrderGrouped;
  return kOrderXcd;
}

// Host-side validation of a TN call (the rules the header states); -1 for a
// valid call with nothing to do (M, N or batch 0).
static int check_tn(const Problem &pr, int es) {
  if (pr.batch < 0 || pr.M < 0 || pr.N < 0 || pr.K < 0) return DG_ERR_INVALID_ARGUMENT;
  if (pr.lda < pr.K || pr.ldb < pr.K || pr.ldc < pr.M) return DG_ERR_INVALID_ARGUMENT;
  if (pr.batch == 0 || pr.M == 0 || pr.N == 0) return -1;  // a valid no-op
  if (!pr.A || !pr.B || !pr.C) return DG_ERR_INVALID_ARGUMENT;
  if (pr.batch > 1 && (pr.stride_a < 0 || pr.stride_b < 0 || pr.stride_c < 0))
    return DG_ERR_INVALID_ARGUMENT;
  // Heads of C must not overlap each other.
  const uint64_t c_head = span_bytes(pr.N, pr.M, pr.ldc, 2);
  if (pr.batch > 1 && (uint64_t)pr.stride_c * 2 < c_head) return DG_ERR_INVALID_ARGUMENT;
  // C must not overlap A or B (whole strided ranges, conservatively).
  const uint64_t a_all = span_bytes(pr.M, pr.K, pr.lda, es) + (uint64_t)(pr.batch - 1) * pr.stride_a * es;
  const uint64_t b_all = span_bytes(pr.N, pr.K, pr.ldb, es) + (uint64_t)(pr.batch - 1) * pr.stride_b * es;
  const uint64_t c_all = c_head + (uint64_t)(pr.batch - 1) * pr.stride_c * 2;
  if (overlaps(pr.C, c_all, pr.A, a_all) || overlaps(pr.C, c_all, pr.B, b_all))
    return DG_ERR_INVALID_ARGUMENT;

  const int64_t vec = 16 / es;  // elements per 16-byte chunk
  if (pr.K % vec || pr.lda % vec || pr.ldb % vec) return DG_ERR_UNSUPPORTED;
  if (!aligned16(pr.A) || !aligned16(pr.B) || !aligned16(pr.C)) return DG_ERR_UNSUPPORTED;
  if (pr.batch > 1 && ((pr.stride_a * es) % 16 || (pr.stride_b * es) % 16))
    return DG_ERR_UNSUPPORTED;
  // Per-block descriptors span at most 256 rows; offsets must stay below kOob.
  const int64_t strip_a = (int64_t)span_bytes(pr.M < kTile ? pr.M : kTile, pr.K, pr.lda, es);
  const int64_t strip_b = (int64_t)span_bytes(pr.N < kTile ? pr.N : kTile, pr.K, pr.ldb, es);
  // Lanes of rows past the matrix still form offsets up to 256 row strides.
  const int64_t reach_a = kTile * pr.lda * es + kRowBytes;
  const int64_t reach_b = kTile * pr.ldb * es + kRowBytes;
  if (strip_a >= (int64_t)kOob || strip_b >= (int64_t)kOob || reach_a >= (int64_t)kOob ||
      reach_b >= (int64_t)kOob)
    return DG_ERR_UNSUPPORTED;
  return DG_OK;
}

// The 128 x 128 kernel's four-stage ring for grids of at most one block per
// CU and at least eight K-steps per block (shorter loops cannot fill it).
// Measured against the two-stage ring on such grids: 15-32 % faster with the
// operands in HBM (each step's copies wait for a DRAM round trip), between 4 %
// faster and 4 % slower with them already in the last-level cache.
static bool mid_deep_ring(int64_t blocks, int64_t ksteps) {
  return blocks <= cu_count() && ksteps >= 8;
}

// One launch of a validated TN problem in configuration `cfg`.
template <int KIND>
static int launch_cfg(const Problem &pr, Config cfg, hipStream_t stream) {
  typedef Traits<KIND> T;
  const int es = T::es;
  const bool skinny = cfg.kind == kCfgSkinny, mid = cfg.kind == kCfgMid;
  const bool pp = cfg.kind == kCfgPingPong;
  const int ntn = cfg.kind == kCfg224 ? 7 : 8;
  const int64_t tile_m = skinny ? kSkTile : mid ? kMidTile : kTile;
  const int64_t tile_n = skinny ? kSkTile : mid ? kMidTile : 32 * ntn;
  const int64_t tiles_m = (pr.M + tile_m - 1) / tile_m;
  const int64_t tiles_n = (pr.N + tile_n - 1) / tile_n;
  // Skinny-K blocks walk up to kSkWalkMax M tiles of one column (each walk
  // step saves a copy of B's strip), halved while that would leave fewer than
  // eight blocks per CU.
  int64_t walk = 1;
  if (skinny) {
    const int64_t want = 8 * (int64_t)cu_count();
    walk = tiles_m < kSkWalkMax ? tiles_m : kSkWalkMax;
    while (walk > 1 && ((tiles_m + walk - 1) / walk) * tiles_n * pr.batch < want) walk = (walk + 1) / 2;
  }
  const int64_t blocks = ((tiles_m + walk - 1) / walk) * tiles_n * pr.batch;
  if (blocks > 0x7fffffffLL) return DG_ERR_UNSUPPORTED;

  Params p = {};
  p.A = (const uint8_t *)pr.A;
  p.B = (const uint8_t *)pr.B;
  p.C = (uint8_t *)pr.C;
  p.M = pr.M; p.N = pr.N; p.K = pr.K;
  p.lda_b = pr.lda * es; p.ldb_b = pr.ldb * es; p.ldc = pr.ldc;
  p.stride_a_b = pr.stride_a * es; p.stride_b_b = pr.stride_b * es; p.stride_c_b = pr.stride_c * 2;
  p.tiles_m = (int32_t)tiles_m; p.tiles_n = (int32_t)tiles_n;
  p.scale = pr.scale;
  // Store widths: a column start (and, with several heads, a head start) is
  // 8-byte aligned when ldc (stride_c) is a multiple of 4 elements, 16-byte
  // aligned when it is a multiple of 8 (C itself is 16-byte aligned).
  const bool heads = pr.batch > 1;
  p.c_vec_ok = (pr.ldc % 4 == 0 && (!heads || pr.stride_c % 4 == 0)) ? 1 : 0;
  p.c_vec16_ok = (pr.ldc % 8 == 0 && (!heads || pr.stride_c % 8 == 0)) ? 1 : 0;
  p.sk_walk = (int32_t)walk;
  p.order = tile_order_env();
  p.clk = clock_slot(blocks);

  if (skinny)
    hipLaunchKernelGGL(gemm_tn_skinny_kernel<KIND>, dim3((unsigned)blocks), dim3(kThreads), 0,
                       stream, p);
  else if (pp)
    hipLaunchKernelGGL(gemm_tn_pp_kernel<KIND>, dim3((unsigned)blocks), dim3(kPpThreads), 0,
                       stream, p);
  else if (mid) {
    // Whole K-steps take the form with fixed copy offsets.
    typedef void (*kernel_t)(Params);
    const bool kf = pr.K % T::kstep == 0;
    const kernel_t k =
        mid_deep_ring(blocks, (pr.K + T::kstep - 1) / T::kstep)
            ? (kf ? gemm_tn_mid_kernel<KIND, false, false, false, 4, true>
                  : gemm_tn_mid_kernel<KIND, false, false, false, 4, false>)
            : (kf ? gemm_tn_mid_kernel<KIND, false, false, false, 2, true>
                  : gemm_tn_mid_kernel<KIND, false, false, false, 2, false>);
    hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
  }
  else {
    // The 3 + 2 ring; whole K-steps take the form with fixed copy offsets.
    const bool kf = pr.K % T::kstep == 0;
    typedef void (*kernel_t)(Params);
    const kernel_t k =
        ring_env() ? (ntn == 8 ? (kf ? gemm_tn_ring_kernel<KIND, 8, true>
                                     : gemm_tn_ring_kernel<KIND, 8, false>)
                               : (kf ? gemm_tn_ring_kernel<KIND, 7, true>
                                     : gemm_tn_ring_kernel<KIND, 7, false>))
                   : ntn == 8 ? (kf ? gemm_tn_kernel<KIND, 8, false, false, true>
                                    : gemm_tn_kernel<KIND, 8, false, false, false>)
                              : (kf ? gemm_tn_kernel<KIND, 7, false, false, true>
                                    : gemm_tn_kernel<KIND, 7, false, false, false>);
    hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError() == hipSuccess ? DG_OK : DG_ERR_HIP;
}

// The planned TN launch (defined with the planner below).
template <int KIND>
static int launch(const Problem &pr, hipStream_t stream);

// Products in any of the four op-code layouts (fp16 in and out, or fp8 E4M3FN
// in and bf16 out with per-tensor scales).  TN goes through launch<> and its
// configurations; for the others each M- or N-contiguous operand (A of an 'N'
// op, B of a 'T' op) is staged as it lies in memory and turned by the
// fragment reads -- no transpose pass -- in the 256-row kernel or the
// 128 x 128 one, picked by the same selector (the skinny-K kernel is TN-only;
// its problems take the 128 x 128 tiles).
template <int KIND>
static int launch_layout(char ta, char tb, const Problem &pr, hipStream_t stream) {
  typedef Traits<KIND> T;
  const int es = T::es;
  const int64_t vec = 16 / es;  // elements per 16-byte chunk
  const bool a_t = ta == 'T' || ta == 't', a_n = ta == 'N' || ta == 'n';
  const bool b_t = tb == 'T' || tb == 't', b_n = tb == 'N' || tb == 'n';
  if (!(a_t || a_n) || !(b_t || b_n)) return DG_ERR_INVALID_ARGUMENT;
  if (a_t && b_n) return launch<KIND>(pr, stream);
  const bool amn = a_n, bmn = b_t;
  if (pr.M < 0 || pr.N < 0 || pr.K < 0) return DG_ERR_INVALID_ARGUMENT;
  if (pr.lda < (amn ? pr.M : pr.K) || pr.ldb < (bmn ? pr.N : pr.K) || pr.ldc < pr.M)
    return DG_ERR_INVALID_ARGUMENT;
  if (pr.M == 0 || pr.N == 0) return DG_OK;
  if (!pr.A || !pr.B || !pr.C) return DG_ERR_INVALID_ARGUMENT;
  const uint64_t a_all = amn ? span_bytes(pr.K, pr.M, pr.lda, es) : span_bytes(pr.M, pr.K, pr.lda, es);
  const uint64_t b_all = bmn ? span_bytes(pr.K, pr.N, pr.ldb, es) : span_bytes(pr.N, pr.K, pr.ldb, es);
  const uint64_t c_all = span_bytes(pr.N, pr.M, pr.ldc, 2);
  if (overlaps(pr.C, c_all, pr.A, a_all) || overlaps(pr.C, c_all, pr.B, b_all))
    return DG_ERR_INVALID_ARGUMENT;

  // 16-byte chunks along each operand's contiguous dimension; K only has to be
  // a multiple of the chunk when an operand is K-contiguous.
  if (pr.lda % vec || pr.ldb % vec) return DG_ERR_UNSUPPORTED;
  if ((!amn || !bmn) && pr.K % vec) return DG_ERR_UNSUPPORTED;
  if ((amn && pr.M % vec) || (bmn && pr.N % vec)) return DG_ERR_UNSUPPORTED;
  if (!aligned16(pr.A) || !aligned16(pr.B) || !aligned16(pr.C)) return DG_ERR_UNSUPPORTED;
  // Offsets inside one block's descriptors stay below kOob: 256 rows of a
  // K-contiguous operand (and its strip), one K-step of an M/N-contiguous one
  // (plus a 256-column row).
  auto fits = [&](bool mn, int64_t ld, int64_t rows) {
    if (mn) return T::kstep * ld * es + 2 * Mn<KIND>::row_bytes < (int64_t)kOob;
    const int64_t strip = (int64_t)span_bytes(rows < kTile ? rows : kTile, pr.K, ld, es);
    return kTile * ld * es + kRowBytes < (int64_t)kOob && strip < (int64_t)kOob;
  };
  if (!fits(amn, pr.lda, pr.M) || !fits(bmn, pr.ldb, pr.N)) return DG_ERR_UNSUPPORTED;

  const bool mid = choose_config(es, pr.M, pr.N, pr.K, 1, false).kind == kCfgMid;
  const int64_t tile_m = mid ? kMidTile : kTile;
  const int64_t tile_n = mid ? kMidTile : kTile;
  const int64_t tiles_m = (pr.M + tile_m - 1) / tile_m;
  const int64_t tiles_n = (pr.N + tile_n - 1) / tile_n;
  const int64_t blocks = tiles_m * tiles_n;
  if (blocks > 0x7fffffffLL) return DG_ERR_UNSUPPORTED;

  Params p = {};
  p.A = (const uint8_t *)pr.A;
  p.B = (const uint8_t *)pr.B;
  p.C = (uint8_t *)pr.C;
  p.M = pr.M; p.N = pr.N; p.K = pr.K;
  p.lda_b = pr.lda * es; p.ldb_b = pr.ldb * es; p.ldc = pr.ldc;
  p.stride_a_b = 0; p.stride_b_b = 0; p.stride_c_b = 0;
  p.tiles_m = (int32_t)tiles_m; p.tiles_n = (int32_t)tiles_n;
  p.scale = pr.scale;
  p.c_vec_ok = (pr.ldc % 4 == 0) ? 1 : 0;
  p.c_vec16_ok = (pr.ldc % 8 == 0) ? 1 : 0;
  p.sk_walk = 1;
  p.clk = clock_slot(blocks);
  const dim3 grid((unsigned)blocks), block(kThreads);
  // One kernel per (layout, configuration).
  typedef void (*kernel_t)(Params);
  static const kernel_t mids[3] = {gemm_tn_mid_kernel<KIND, true, false>,
                                   gemm_tn_mid_kernel<KIND, false, true>,
                                   gemm_tn_mid_kernel<KIND, true, true>};
  static const kernel_t mids4[3] = {gemm_tn_mid_kernel<KIND, true, false, false, 4>,
                                    gemm_tn_mid_kernel<KIND, false, true, false, 4>,
                                    gemm_tn_mid_kernel<KIND, true, true, false, 4>};
  static const kernel_t bigs[3] = {gemm_tn_kernel<KIND, 8, true, false, false>,
                                   gemm_tn_kernel<KIND, 8, false, true, false>,
                                   gemm_tn_kernel<KIND, 8, true, true, false>};
  const int li = amn && bmn ? 2 : amn ? 0 : 1;
  const bool deep = mid && mid_deep_ring(blocks, (pr.K + T::kstep - 1) / T::kstep);
  const kernel_t k = deep ? mids4[li] : mid ? mids[li] : bigs[li];
  hipLaunchKernelGGL(k, grid, block, 0, stream, p);
  return hipGetLastError() == hipSuccess ? DG_OK : DG_ERR_HIP;
}

// Split-K for grids of few output tiles with a long K (128 x 128 tiles): split
// h of S multiplies the K range [h * k_slice, (h + 1) * k_slice) of every tile
// into an fp32 partial in the caller's workspace, and one reduction kernel sums
// the S partials in split order and converts.  k_slice is a whole number of
// K-steps, so every split starts on a step boundary; S = ceil(K-steps /
// steps per split) <= the requested count.
constexpr int64_t kSplitMax = 64;

static int64_t splitk_ldw(int64_t M) { return (M + 3) / 4 * 4; }

template <int KIND>
static int launch_splitk(const Problem &pr, int64_t splits, void *ws, int64_t ws_bytes,
                         hipStream_t stream) {
  typedef Traits<KIND> T;
  const int es = T::es;
  if (splits < 1 || splits > kSplitMax || ws_bytes < 0) return DG_ERR_INVALID_ARGUMENT;
  const int chk = check_tn(pr, es);
  if (chk < 0) return DG_OK;
  if (chk != DG_OK) return chk;
  const int64_t nk = (pr.K + T::kstep - 1) / T::kstep;
  const int64_t per = nk > 0 ? (nk + splits - 1) / splits : 0;   // K-steps per split
  const int64_t S = per > 0 ? (nk + per - 1) / per : 0;
  if (S <= 1) return launch<KIND>(pr, stream);
  const int64_t ldw = splitk_ldw(pr.M);
  const uint64_t need = (uint64_t)splits * (uint64_t)pr.N * (uint64_t)ldw * 4u;
  if (!ws || (uint64_t)ws_bytes < need) return DG_ERR_INVALID_ARGUMENT;
  const uint64_t used = (uint64_t)S * (uint64_t)pr.N * (uint64_t)ldw * 4u;
  if (overlaps(ws, used, pr.A, span_bytes(pr.M, pr.K, pr.lda, es)) ||
      overlaps(ws, used, pr.B, span_bytes(pr.N, pr.K, pr.ldb, es)) ||
      overlaps(ws, used, pr.C, span_bytes(pr.N, pr.M, pr.ldc, 2)))
    return DG_ERR_INVALID_ARGUMENT;
  if (!aligned16(ws)) return DG_ERR_UNSUPPORTED;
  const int64_t tiles_m = (pr.M + kMidTile - 1) / kMidTile;
  const int64_t tiles_n = (pr.N + kMidTile - 1) / kMidTile;
  const int64_t blocks = tiles_m * tiles_n * S;
  const int64_t quads = ldw / 4 * pr.N;
  const int64_t rblocks = (quads + kThreads - 1) / kThreads;
  if (blocks > 0x7fffffffLL || rblocks > 0x7fffffffLL) return DG_ERR_UNSUPPORTED;

  Params p = {};
  p.A = (const uint8_t *)pr.A;
  p.B = (const uint8_t *)pr.B;
  p.C = (uint8_t *)pr.C;
  p.M = pr.M; p.N = pr.N; p.K = pr.K;
  p.lda_b = pr.lda * es; p.ldb_b = pr.ldb * es; p.ldc = pr.ldc;
  p.tiles_m = (int32_t)tiles_m; p.tiles_n = (int32_t)tiles_n;
  p.scale = pr.scale;
  p.c_vec_ok = (pr.ldc % 4 == 0) ? 1 : 0;
  p.c_vec16_ok = (pr.ldc % 8 == 0) ? 1 : 0;
  p.sk_walk = 1;
  p.k_slice = per * T::kstep;
  p.W = (float *)ws;
  p.ldw = ldw;
  p.clk = clock_slot(blocks);
  {
    // Whole K-steps in every range (K a multiple of the step) take the form
    // with fixed copy offsets.
    typedef void (*kernel_t)(Params);
    const bool kf = pr.K % T::kstep == 0;
    const kernel_t k = mid_deep_ring(blocks, per)
                           ? (kf ? gemm_tn_mid_kernel<KIND, false, false, true, 4, true>
                                 : gemm_tn_mid_kernel<KIND, false, false, true, 4, false>)
                           : (kf ? gemm_tn_mid_kernel<KIND, false, false, true, 2, true>
                                 : gemm_tn_mid_kernel<KIND, false, false, true, 2, false>);
    hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
  }
  if (hipGetLastError() != hipSuccess) return DG_ERR_HIP;
  p.clk = nullptr;
  hipLaunchKernelGGL(gemm_splitk_reduce_kernel<KIND>, dim3((unsigned)rblocks), dim3(kThreads), 0,
                     stream, p, (int32_t)S);
  return hipGetLastError() == hipSuccess ? DG_OK : DG_ERR_HIP;
}

// The no-allocation split-K entry point keeps its fp32 partials in this
// file-scope device array instead of a caller workspace: 32 MiB per device,
// which the runtime places on each GPU the library runs on and keeps until
// the process ends.  Host code never passes `scratch` itself to a kernel (on
// the host that name is only a stand-in for the symbol): scratch_ptr() looks
// the device address up once per device with hipGetSymbolAddress and every
// launch takes that address.  Nothing in the array has to start at zero:
// each launch writes every partial it later reads (the reduction's reads of
// the row padding between M and the rounded-up M only feed rows that are not
// stored).  All calls on one device share the array, so calls that overlap
// in time on that device (concurrent streams) race.
constexpr int64_t kScratchBytes = 32ll << 20;
static __device__ __align__(256) float scratch[kScratchBytes / 4];

static std::mutex g_scratch_mu;
static void *g_scratch_dev[64];   // device address of `scratch` per device, once looked up

// Device address of `scratch` on the current device (nullptr if the lookup fails).
static void *scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return nullptr;
    g_scratch_dev[dev] = ptr;
  }
  return g_scratch_dev[dev];
}

// Suggested split count: as many splits of the 128 x 128 tiles as fit one
// block per CU (never a second round), doubled to two blocks per CU when the
// one-block-per-CU ranges are 4 * kSplitMinSteps K-steps or longer (so the
// doubled ranges keep at least 2 * kSplitMinSteps; the second block hides the
// first one's waits), each split keeping at least kSplitMinSteps K-steps.
// (Measured on 512^2 x 32768, 256^2 x 65536, 1024^2 x 16384, 1024 x 512 x
// 16384 and 768^2 x 8192: within 3 % of the best count of a sweep.)  Grids of
// more than half and fewer than all CUs' worth of tiles leave CUs idle
// unsplit, and no split count spreads them evenly: they take the count that
// fits two blocks per CU in one round when the busiest CU's block-steps drop
// to at most 0.8 of the unsplit K-steps, else 1 (measured: 1536^2 x 4096,
// 144 tiles, S = 3 33.4 vs 37.5 us; 1536^2 x 8192 53.4 vs 74.7; 1792^2 x 4096,
// 196 tiles, stays unsplit: S = 2 40.1 vs 37.8).  1 for a full grid or a
// short K.
constexpr int64_t kSplitMinSteps = 16;
static int64_t choose_splits(int es, int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return 1;
  const int64_t kstep = 128 / es;
  const int64_t nk = (K + kstep - 1) / kstep;
  const int64_t tiles = ((M + kMidTile - 1) / kMidTile) * ((N + kMidTile - 1) / kMidTile);
  const int64_t cus = cu_count();
  if (tiles >= cus) return 1;
  if (2 * tiles > cus) {
    int64_t s2 = 2 * cus / tiles;
    if (s2 > nk / kSplitMinSteps) s2 = nk / kSplitMinSteps;
    if (s2 < 2) return 1;
    const int64_t busiest = ((tiles * s2 + cus - 1) / cus) * ((nk + s2 - 1) / s2);
    return 5 * busiest <= 4 * nk ? s2 : 1;
  }
  int64_t s = cus / tiles;
  if (s >= 1 && nk / s >= 4 * kSplitMinSteps) s *= 2;
  const int64_t by_k = nk / kSplitMinSteps;
  if (s > by_k) s = by_k;
  if (s > kSplitMax) s = kSplitMax;
  return s < 1 ? 1 : s;
}

// ---------------------------------------------------------------------------
// Plans for grids with a ragged last round.  With one block per CU, a grid of
// T tiles of the 256-row kernel takes ceil(T / CUs) rounds however few tiles
// the last one holds (4096 x 4608 in 256 x 256 tiles: 288 tiles, a second
// round of 32), and the selector's fallback, the 128 x 128 kernel, pays its
// own per-element cost on the whole product.  A plan may instead run the
// first dp_cols columns of C as whole rounds of the 256-row kernel and the
// remaining columns as a second launch: the selector's configuration for that
// narrower product or, given a caller workspace, the split-K kernels with the
// tail's K range cut into `splits` ranges, so the few tail tiles spread over
// every CU (the data-parallel + split-tail hybrid that stream-K scheduling
// generalises; here the split points are K-step boundaries).  A plan that
// splits nothing computes every element exactly as the single launch does
// (same products, same K order).  Plans are compared with a time model fitted
// to MI355X measurements, and a split is taken only when it models at least
// kPlanGain faster than the single launch.
//
// Time model, microseconds:
//   * 256-row kernel: a round of one block per CU takes nk K-steps of
//     kStepUs (x kNarrow for 256 x 224 tiles) plus kRoundUs of prologue and
//     epilogue;
//   * 128 x 128 kernel: kMidRel of that K-step per block-step, counted per CU
//     in blocks -- two co-resident blocks take two units, a lone block
//     kMidLone (no second block hides its waits);
//   * split-K: its partial products plus the fp32 partials written and read
//     back (and C written) at kHbmBytesPerUs;
//   * kLaunchUs per launch.
struct TnPlan {
  int whole;         // configuration of the single launch (dp_cols == 0, splits == 1)
  int64_t dp_cols;   // columns of C run in whole rounds first (0: no column split)
  int dp_cfg;        // kCfg256 or kCfg224 for those columns
  int64_t splits;    // K ranges of the tail (of the whole product when dp_cols == 0)
  int64_t ws_bytes;  // workspace bytes the plan uses
  double us;         // modelled time
};
constexpr double kStepUsF16 = 1.5, kStepUsF8 = 1.25;
constexpr double kNarrow = 0.8;
constexpr double kRoundUs = 7.0;
constexpr double kMidRel = kMidCost / 64.0 / 4.0;
constexpr double kMidLone = 1.35;
constexpr double kHbmBytesPerUs = 5.0e6;
constexpr double kLaunchUs = 2.0;
constexpr double kPlanGain = 0.05;

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
static double step_us(int es) { return es == 1 ? kStepUsF8 : kStepUsF16; }
static double mid_units(int64_t blocks, int64_t cus) {
  return blocks <= cus ? kMidLone : (double)cdiv(blocks, cus);
}
static double model_big(int es, int64_t tiles, int ntn, int64_t nk, int64_t cus) {
  return cdiv(tiles, cus) * (nk * step_us(es) * (ntn == 8 ? 1.0 : kNarrow) + kRoundUs) +
         kLaunchUs;
}
static double model_splitk(int es, int64_t M, int64_t N, int64_t nk, int64_t S, int64_t cus) {
  const int64_t tiles = cdiv(M, kMidTile) * cdiv(N, kMidTile);
  const double bytes = (double)M * (double)N * (8.0 * S + 2.0);
  return mid_units(tiles * S, cus) * cdiv(nk, S) * step_us(es) * kMidRel +
         bytes / kHbmBytesPerUs + 2 * kLaunchUs;
}
static double model_cfg(int es, int kind, int64_t M, int64_t N, int64_t nk, int64_t batch,
                        int64_t cus) {
  if (kind == kCfgMid)
    return mid_units(cdiv(M, kMidTile) * cdiv(N, kMidTile) * batch, cus) * nk * step_us(es) *
               kMidRel + kLaunchUs;
  const int ntn = kind == kCfg224 ? 7 : 8;
  return model_big(es, cdiv(M, kTile) * cdiv(N, 32 * ntn) * batch, ntn, nk, cus);
}

// The plan for a TN problem given `ws_avail` bytes of workspace (0: none).
static TnPlan plan_tn(int es, int64_t M, int64_t N, int64_t K, int64_t batch, int64_t ws_avail) {
  const int whole = choose_config(es, M, N, K, batch).kind;
  TnPlan best{whole, 0, kCfg256, 1, 0, 0.0};
  // Forced tiles, skinny-K problems and empty ones run as one launch.
  if (getenv("DG_GEMM_TILE") || whole == kCfgSkinny || M <= 0 || N <= 0 || K <= 0 || batch <= 0)
    return best;
  const int64_t cus = cu_count();
  const int64_t nk = cdiv(K, 128 / es);
  best.us = model_cfg(es, whole, M, N, nk, batch, cus);
  const double bar = best.us * (1.0 - kPlanGain);
  auto consider = [&](const TnPlan &c) {
    if (c.us < bar && c.us < best.us) best = c;
  };
  const int64_t ldw = splitk_ldw(M);
  // Split-K of the whole product (few tiles, long K).
  if (batch == 1) {
    const int64_t s = choose_splits(es, M, N, K);
    const int64_t need = s * N * ldw * 4;
    if (s > 1 && need <= ws_avail)
      consider(TnPlan{whole, 0, kCfg256, s, need, model_splitk(es, M, N, nk, s, cus)});
  }
  // Whole rounds of 256 x 256 or 256 x 224 tiles, then the remaining columns.
  const int64_t tm = cdiv(M, kTile) * batch;  // tiles per tile column, all heads
  for (const int ntn : {8, 7}) {
    const int64_t w = 32 * ntn;
    const int64_t rounds = cdiv(tm * cdiv(N, w), cus);
    if (rounds < 2) continue;
    const int64_t kcols = (rounds - 1) * cus / tm;
    const int64_t dp = kcols * w;
    if (kcols < 1 || dp >= N) continue;
    const int64_t nt = N - dp;
    const int dp_cfg = ntn == 8 ? kCfg256 : kCfg224;
    const double t_dp = model_big(es, tm * kcols, ntn, nk, cus);
    const int tail = choose_config(es, M, nt, K, batch).kind;
    consider(TnPlan{whole, dp, dp_cfg, 1, 0, t_dp + model_cfg(es, tail, M, nt, nk, batch, cus)});
    if (batch != 1) continue;
    for (const int64_t S : {2, 4, 8}) {
      const int64_t need = S * nt * ldw * 4;
      if (S > nk || need > ws_avail) continue;
      consider(TnPlan{whole, dp, dp_cfg, S, need, t_dp + model_splitk(es, M, nt, nk, S, cus)});
    }
  }
  return best;
}

// A TN problem by its plan: one launch, split-K, or whole rounds of columns
// followed by the rest (as one launch or split-K).  `ws` may be null (no
// workspace: plans that need none).
template <int KIND>
static int launch_ws(const Problem &pr, void *ws, int64_t ws_bytes, hipStream_t stream) {
  const int es = Traits<KIND>::es;
  if (ws_bytes < 0 || (ws == nullptr && ws_bytes != 0)) return DG_ERR_INVALID_ARGUMENT;
  const int chk = check_tn(pr, es);
  if (chk < 0) return DG_OK;
  if (chk != DG_OK) return chk;
  const TnPlan plan = plan_tn(es, pr.M, pr.N, pr.K, pr.batch, ws != nullptr ? ws_bytes : 0);
  if (plan.ws_bytes > 0) {
    // The bytes the plan uses must not overlap an operand (a larger arena
    // around them may).
    const uint64_t used = (uint64_t)plan.ws_bytes;
    const uint64_t a_all = span_bytes(pr.M, pr.K, pr.lda, es) + (uint64_t)(pr.batch - 1) * pr.stride_a * es;
    const uint64_t b_all = span_bytes(pr.N, pr.K, pr.ldb, es) + (uint64_t)(pr.batch - 1) * pr.stride_b * es;
    const uint64_t c_all = span_bytes(pr.N, pr.M, pr.ldc, 2) + (uint64_t)(pr.batch - 1) * pr.stride_c * 2;
    if (overlaps(ws, used, pr.A, a_all) || overlaps(ws, used, pr.B, b_all) ||
        overlaps(ws, used, pr.C, c_all))
      return DG_ERR_INVALID_ARGUMENT;
    if (!aligned16(ws)) return DG_ERR_UNSUPPORTED;
  }
  if (plan.dp_cols == 0) {
    if (plan.splits > 1) return launch_splitk<KIND>(pr, plan.splits, ws, ws_bytes, stream);
    return launch_cfg<KIND>(pr, Config{plan.whole}, stream);
  }
  Problem dp = pr, tail = pr;
  dp.N = plan.dp_cols;
  tail.N = pr.N - plan.dp_cols;
  tail.B = (const uint8_t *)pr.B + plan.dp_cols * pr.ldb * es;
  tail.C = (uint8_t *)pr.C + plan.dp_cols * pr.ldc * 2;
  const int st = launch_cfg<KIND>(dp, Config{plan.dp_cfg}, stream);
  if (st != DG_OK) return st;
  if (plan.splits > 1) return launch_splitk<KIND>(tail, plan.splits, ws, ws_bytes, stream);
  return launch_cfg<KIND>(tail, choose_config(es, tail.M, tail.N, tail.K, tail.batch), stream);
}

template <int KIND>
static int launch(const Problem &pr, hipStream_t stream) {
  return launch_ws<KIND>(pr, nullptr, 0, stream);
}

}  // namespace dg

extern "C" {

int gemm_f16(char transa, char transb, const void *A, const void *B, void *C, int64_t M,
             int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, void *stream) {
  dg::Problem pr{A, B, C, 1, M, N, K, lda, ldb, ldc, 0, 0, 0, 1.0f};
  return dg::launch_layout<dg::kF16>(transa, transb, pr, (hipStream_t)stream);
}

int gemm_f8(char transa, char transb, const void *A, const void *B, void *C, int64_t M,
            int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, float scale_a,
            float scale_b, void *stream) {
  dg::Problem pr{A, B, C, 1, M, N, K, lda, ldb, ldc, 0, 0, 0, scale_a * scale_b};
  return dg::launch_layout<dg::kF8>(transa, transb, pr, (hipStream_t)stream);
}

int gemm_f16_tn(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K,
                int64_t lda, int64_t ldb, int64_t ldc, void *stream) {
  dg::Problem pr{A, B, C, 1, M, N, K, lda, ldb, ldc, 0, 0, 0, 1.0f};
  return dg::launch<dg::kF16>(pr, (hipStream_t)stream);
}

int gemm_f8_tn(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K,
               int64_t lda, int64_t ldb, int64_t ldc, float scale_a, float scale_b,
               void *stream) {
  // The epilogue multiplies by one fp32 factor: the fp32 product of the scales.
  const float s = scale_a * scale_b;
  dg::Problem pr{A, B, C, 1, M, N, K, lda, ldb, ldc, 0, 0, 0, s};
  return dg::launch<dg::kF8>(pr, (hipStream_t)stream);
}

int gemm_batched_qkt(const void *Q, const void *Kmat, void *S, int64_t batch, int64_t M,
                     int64_t N, int64_t D, int64_t ldq, int64_t ldk, int64_t lds,
                     int64_t stride_q, int64_t stride_k, int64_t stride_s, void *stream) {
  dg::Problem pr{Q, Kmat, S, batch, M, N, D, ldq, ldk, lds, stride_q, stride_k, stride_s, 1.0f};
  return dg::launch<dg::kF16>(pr, (hipStream_t)stream);
}

const char *gemm_status_string(int status) {
  switch (status) {
  case DG_OK: return "ok";
  case DG_ERR_INVALID_ARGUMENT: return "invalid argument";
  case DG_ERR_UNSUPPORTED: return "unsupported argument";
  case DG_ERR_HIP: return "HIP launch error";
  default: return "unknown status";
  }
}

int gemm_tile_order(int64_t tiles_m, int64_t tiles_n, int64_t batch, int64_t *out) {
  if (!out || tiles_m <= 0 || tiles_n <= 0 || batch <= 0) return DG_ERR_INVALID_ARGUMENT;
  const int64_t G = tiles_m * tiles_n * batch;
  for (int64_t b = 0; b < G; ++b) {
    int64_t h, tm, tn;
    dg::tile_of_block<int64_t>(b, G, tiles_m, tiles_n, &h, &tm, &tn);
    out[3 * b] = h;
    out[3 * b + 1] = tm;
    out[3 * b + 2] = tn;
  }
  return DG_OK;
}

int gemm_block_tile(void) { return dg::kTile; }

static int layout_config(int es, char transa, char transb, int64_t M, int64_t N, int64_t K) {
  const bool a_t = transa == 'T' || transa == 't', a_n = transa == 'N' || transa == 'n';
  const bool b_t = transb == 'T' || transb == 't', b_n = transb == 'N' || transb == 'n';
  if (!(a_t || a_n) || !(b_t || b_n) || M < 0 || N < 0 || K < 0) return -1;
  return dg::choose_config(es, M, N, K, 1, a_t && b_n).kind;
}

int gemm_f16_config(char transa, char transb, int64_t M, int64_t N, int64_t K) {
  return layout_config(2, transa, transb, M, N, K);
}

int gemm_f8_config(char transa, char transb, int64_t M, int64_t N, int64_t K) {
  return layout_config(1, transa, transb, M, N, K);
}

int gemm_tn_config(int fp8, int64_t M, int64_t N, int64_t K, int64_t batch) {
  if (M < 0 || N < 0 || K < 0 || batch < 0) return -1;
  return dg::choose_config(fp8 ? 1 : 2, M, N, K, batch).kind;
}

int gemm_mid_stages(int64_t blocks, int64_t ksteps) {
  if (blocks < 0 || ksteps < 0) return -1;
  return dg::mid_deep_ring(blocks, ksteps) ? 4 : 2;
}

int gemm_clock_record(void *buf, int64_t records) {
  if (records < 0 || (buf == nullptr && records != 0) || (buf != nullptr && records == 0))
    return DG_ERR_INVALID_ARGUMENT;
  if (((uintptr_t)buf & 7u) != 0) return DG_ERR_UNSUPPORTED;
  dg::g_clk_buf.store(nullptr, std::memory_order_release);
  dg::g_clk_cap.store(records, std::memory_order_relaxed);
  dg::g_clk_next.store(0, std::memory_order_relaxed);
  dg::g_clk_buf.store((uint64_t *)buf, std::memory_order_release);
  return DG_OK;
}

int64_t gemm_clock_records_used(void) { return dg::g_clk_next.load(std::memory_order_relaxed); }

int64_t gemm_splitk_workspace_bytes(int64_t M, int64_t N, int64_t splits) {
  if (M < 0 || N < 0 || splits < 1 || splits > dg::kSplitMax) return -1;
  return splits * N * dg::splitk_ldw(M) * 4;
}

int64_t gemm_splitk_choose(int fp8, int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0) return -1;
  return dg::choose_splits(fp8 ? 1 : 2, M, N, K);
}

int gemm_f16_tn_splitk(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K,
                       int64_t lda, int64_t ldb, int64_t ldc, int64_t splits, void *workspace,
                       int64_t workspace_bytes, void *stream) {
  dg::Problem pr{A, B, C, 1, M, N, K, lda, ldb, ldc, 0, 0, 0, 1.0f};
  return dg::launch_splitk<dg::kF16>(pr, splits, workspace, workspace_bytes, (hipStream_t)stream);
}

int gemm_f16_tn_splitk_noalloc(const void *A, const void *B, void *C, int64_t M, int64_t N,
                               int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int64_t splits,
                               void *stream) {
  // The size rule first, on the host: at most kScratchBytes of partials.
  if (M < 0 || N < 0 || splits < 1 || splits > dg::kSplitMax) return DG_ERR_INVALID_ARGUMENT;
  const uint64_t need = (uint64_t)splits * (uint64_t)N * (uint64_t)dg::splitk_ldw(M) * 4u;
  if (need > (uint64_t)dg::kScratchBytes) return DG_ERR_UNSUPPORTED;
  dg::Problem pr{A, B, C, 1, M, N, K, lda, ldb, ldc, 0, 0, 0, 1.0f};
  // Argument errors are reported before the device array is looked up.
  const int chk = dg::check_tn(pr, 2);
  if (chk < 0) return DG_OK;
  if (chk != DG_OK) return chk;
  void *ws = dg::scratch_ptr();
  if (ws == nullptr) return DG_ERR_HIP;
  return dg::launch_splitk<dg::kF16>(pr, splits, ws, dg::kScratchBytes, (hipStream_t)stream);
}

int gemm_f8_tn_splitk(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K,
                      int64_t lda, int64_t ldb, int64_t ldc, float scale_a, float scale_b,
                      int64_t splits, void *workspace, int64_t workspace_bytes, void *stream) {
  const float s = scale_a * scale_b;
  dg::Problem pr{A, B, C, 1, M, N, K, lda, ldb, ldc, 0, 0, 0, s};
  return dg::launch_splitk<dg::kF8>(pr, splits, workspace, workspace_bytes, (hipStream_t)stream);
}

int gemm_f16_tn_ws(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K,
                   int64_t lda, int64_t ldb, int64_t ldc, void *workspace,
                   int64_t workspace_bytes, void *stream) {
  dg::Problem pr{A, B, C, 1, M, N, K, lda, ldb, ldc, 0, 0, 0, 1.0f};
  return dg::launch_ws<dg::kF16>(pr, workspace, workspace_bytes, (hipStream_t)stream);
}

int gemm_f8_tn_ws(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K,
                  int64_t lda, int64_t ldb, int64_t ldc, float scale_a, float scale_b,
                  void *workspace, int64_t workspace_bytes, void *stream) {
  dg::Problem pr{A, B, C, 1, M, N, K, lda, ldb, ldc, 0, 0, 0, scale_a * scale_b};
  return dg::launch_ws<dg::kF8>(pr, workspace, workspace_bytes, (hipStream_t)stream);
}

int64_t gemm_tn_workspace_bytes(int fp8, int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0) return -1;
  return dg::plan_tn(fp8 ? 1 : 2, M, N, K, 1, INT64_MAX).ws_bytes;
}

int gemm_tn_plan(int fp8, int64_t M, int64_t N, int64_t K, int64_t batch,
                 int64_t workspace_bytes, int64_t *out) {
  if (!out || M < 0 || N < 0 || K < 0 || batch < 0 || workspace_bytes < 0)
    return DG_ERR_INVALID_ARGUMENT;
  const dg::TnPlan p = dg::plan_tn(fp8 ? 1 : 2, M, N, K, batch, workspace_bytes);
  out[0] = p.whole;
  out[1] = p.dp_cols;
  out[2] = p.dp_cols > 0 ? p.dp_cfg : -1;
  out[3] = p.splits;
  out[4] = p.ws_bytes;
  return DG_OK;
}

}  // extern "C"
