// attention.hip -- fused softmax attention forward for gfx950 (MI355X).
//
// O_h = softmax(scale * Q_h K_h^T) V_h for every head h, without writing the
// score matrix: the step that the chapter summary of "hello-gpu, chapter 11
// (GEMM-like)" names after the GEMM (joining the product with softmax so the
// intermediate result stays on chip), and the fused attention that the mlqm.cn
// TileLang attention page motivates for QK^T.  Both products are TN products
// in the sense of "FP16 GEMM optimisation on AMD RDNA 3 and RDNA 4", section
// "What we compute": Q and K are row-major with the head dim contiguous, and V
// is passed transposed (Vt, keys contiguous), so each operand is contiguous
// along the dimension its product sums over.
//
// Kernel design (head dim 128, fp16 in, fp32 accumulate, fp16 out):
//   * One workgroup = 4 waves = 256 queries of one head; wave w owns 64
//     queries as two halves of 32 (each two 16-query MFMA column tiles), whose
//     schedules run half a key block apart so one half's softmax arithmetic
//     issues beside the other half's products.  One workgroup per CU.
//   * The wave's Q rows live in AGPRs for the whole kernel as B operands of
//     v_mfma_f32_16x16x32_f16 (the 16x16 shapes of the MI355X FP8 GEMM page),
//     and so do the output accumulators O^T.
//   * Keys are processed 64 at a time.  A key block of K (64 x 256 B) and of Vt
//     (128 x 128 B) is copied global -> LDS by buffer loads that write LDS
//     directly into three K slots and two Vt slots (80 KiB), one barrier per
//     key block.
//   * S^T = K Q^T is computed tile by tile, so each accumulator lane holds one
//     query (column) and four keys.  The K rows given to MFMA tile t are chosen
//     so that the keys a lane ends up holding from tiles 2j and 2j+1 are eight
//     consecutive keys: the probabilities then feed O^T += Vt P^T as the B
//     operand straight from the lane's registers (no shuffle), and the Vt
//     operand is one 16-byte LDS read.
//   * Online softmax in base 2 (exp2 of scale*log2(e)*s minus the running
//     reference maximum), the maximum reduced across the four lanes of a query
//     by two lane-swap instructions; the running sum stays per lane until the
//     end.  The reference maximum moves only when a block's maximum exceeds it
//     by more than 2^8 in probability, so O is rarely rescaled.
//   * LDS swizzles: K rows (256 B) store chunk c of row r in slot
//     c ^ ((r & 3) | ((r >> 1) & 12)), which is the lane's row index in its
//     MFMA tile, so a 16-lane read phase touches 16 distinct 16-byte slots;
//     Vt rows (128 B) use c ^ ((r >> 1) & 7), the XOR swizzle of the MI355X FP8
//     GEMM page.
//   * Block ids are remapped so each XCD receives a contiguous range of query
//     tiles, i.e. mostly the tiles of one or two heads, whose K and V then stay
//     in that XCD's L2.
//   * Tails: query rows past M read zeros and are not stored; key rows past N
//     read zeros and are masked out of the softmax; an 8-key Vt chunk that N
//     cuts is copied as zeros and its valid keys are then written into LDS
//     one by one, so no element past N is read.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "dense_gemm_tn.h"

namespace dga {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef int int4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int kD = 128;                 // head dim
constexpr int kWaveQ = 64;              // queries per wave
constexpr int kBM = 4 * kWaveQ;         // queries per workgroup
constexpr int kBN = 64;                 // keys per block
constexpr int kThreads = 256;           // 4 waves
constexpr int kKRow = kD * 2;           // bytes per K row in LDS
constexpr int kVRow = kBN * 2;          // bytes per Vt row in LDS
constexpr int kKBytes = kBN * kKRow;    // 16 KiB
constexpr int kVBytes = kD * kVRow;     // 16 KiB
constexpr int kLdsBytes = 3 * kKBytes + 2 * kVBytes;  // three K slots, two Vt slots
constexpr int kXcds = 8;
constexpr uint32_t kOob = 0x80000000u;  // an offset past every descriptor
// Word 3 of a raw buffer resource (32-bit data format: byte range checking).
constexpr uint32_t kRsrcWord3 = 0x00020000u;

struct AttnParams {
  const uint8_t *Q, *K, *V;
  uint8_t *O;
  int64_t M, N;
  int64_t ldq_b, ldk_b, ldv_b;   // row strides of Q, K, Vt in bytes
  int64_t ldo;                   // row stride of O in elements
  int64_t sq_b, sk_b, sv_b;      // head strides of Q, K, Vt in bytes
  int64_t so;                    // head stride of O in elements
  uint32_t q_bytes, k_bytes, v_bytes;  // descriptor extents of one head
  int32_t tiles_m;               // query tiles per head
  int32_t blocks;                // grid size
  int32_t n_blocks;              // key blocks: ceil(N / 64)
  float c;                       // scale * log2(e)
  uint64_t *clk;                 // per-block clock records, or null (see clock_mark)
};

// Per-block clock record (measurement only; the layout of the GEMM kernels'
// records in gemm_tn.hip): s_memtime and s_memrealtime at the block's start
// (words 0-1) and after its first wave's last stores have completed (words
// 6-7), the XCD (word 8) and the block index (word 9); words 2-5 stay zero.
enum { kClockStart = 0, kClockEnd = 3, kClockWords = 10 };
__device__ __forceinline__ void clock_mark(uint64_t *clk, int point) {
  if (clk == nullptr) return;
  if (point == kClockEnd) __builtin_amdgcn_s_waitcnt(0);
  const uint64_t t = __builtin_amdgcn_s_memtime();
  const uint64_t r = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x != 0) return;
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

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           (int)kRsrcWord3);
}

// s_waitcnt immediate for "no vector-memory operation outstanding" (vmcnt 0,
// expcnt and lgkmcnt left at their maxima).
constexpr int kVmcnt0 = (7 << 4) | (15 << 8);

// Exchanges between the four lanes l, l ^ 16, l ^ 32, l ^ 48 that hold one
// query column, with the gfx950 lane-swap instructions (no trip through LDS).
// v_permlane32_swap exchanges the upper 32 lanes of its first operand with
// the lower 32 lanes of its second, v_permlane16_swap the odd 16-lane rows of
// the first with the even rows of the second; starting from two copies of x,
// each pair of results then holds x and its partner lane's x in every lane.
// Written as inline assembly because the compiler folds the builtins' two
// results into one when both inputs are the same value.  The s_nop gives the
// wait states a lane-swap needs after a VALU write of its operands.
__device__ __forceinline__ void swap32(float &a, float &b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32_e32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap16(float &a, float &b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32_e32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float max_over_column(float x) {
  float a = x, b = x;
  swap32(a, b);
  float c = fmaxf(a, b), d = c;
  swap16(c, d);
  return fmaxf(c, d);
}
// max(a, b, c) without the quieting the compiler adds to fmaxf in IEEE mode
// (the operands here are finite scores or -inf).
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm volatile("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float sum_over_column(float x) {
  float a = x, b = x;
  swap32(a, b);
  float c = a + b, d = c;
  swap16(c, d);
  return c + d;
}

// Matrix-core products, all v_mfma_f32_16x16x32_f16 written as inline
// assembly so each operand stays in the register file chosen for it:
//   * score products S^T = K Q^T accumulate in VGPRs (the softmax reads
//     them) and take the wave's resident Q fragments from AGPRs;
//   * output products O^T += Vt P^T accumulate in place in AGPRs.  While an
//     MFMA with AGPR accumulators runs, the SIMD still issues about two
//     independent VALU instructions of the same wave (measured on MI355X; with
//     VGPR accumulators about one), which is what hides the softmax.
// The compiler knows no latency for these, so every VALU read of an MFMA
// result is placed behind a scheduling barrier far enough after the product
// (or behind mfma_drain), and a product whose B operand was just written by
// the VALU starts with the two wait states that hazard needs.
__device__ __forceinline__ void mma_s0(const half8_t &a, const half8_t &b, float4_t &c) {
  asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mma_s(const half8_t &a, const half8_t &b, float4_t &c) {
  asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mma_o(const half8_t &a, const half8_t &b, float4_t &c) {
  asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mma_o_fresh_b(const half8_t &a, const half8_t &b, float4_t &c) {
  asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
// fp32 16x16x4 products that rewrite an output tile (see the rescale below).
// The first one overwrites the tile in place ("+a" keeps the tile in its
// registers, so no copies appear where the rare path rejoins).
__device__ __forceinline__ void mma_f32_0(float a, float b, float4_t &c) {
  asm volatile("s_nop 1\n\tv_mfma_f32_16x16x4_f32 %0, %1, %2, 0" : "+a"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mma_f32(float a, float b, float4_t &c) {
  asm volatile("s_nop 1\n\tv_mfma_f32_16x16x4_f32 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
// Wait states after the last MFMA before other instructions read its result.
__device__ __forceinline__ void mfma_drain() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// Empty statements that "modify" a value in place: placed after mfma_drain,
// they keep reads of an MFMA result from being hoisted above the wait.
__device__ __forceinline__ void tie_agpr(float4_t &v) { asm volatile("" : "+a"(v)); }
__device__ __forceinline__ void tie_vgpr(float4_t &v) { asm volatile("" : "+v"(v)); }

// mfma_drain for accumulators that other instructions read next: the empty
// statements tie each tile to the wait, so no read is hoisted above it.
template <int R, int C>
__device__ __forceinline__ void drain_agprs(float4_t (&acc)[R][C]) {
  mfma_drain();
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int c = 0; c < C; ++c) tie_agpr(acc[r][c]);
}

// f(std::integral_constant<int, k>) for k = B .. E-1, in order: compile-time
// slot indices, so every register-array index below is a constant.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Schedule of one key block kb ("body"), per wave.  The wave's 64 queries are
// two halves of 32 (query tiles u = 2H, 2H + 1), each with its own scores,
// softmax state and output tiles, run half a block apart so one half's
// matrix-core products always overlap the other half's softmax arithmetic:
//
//   slots   MFMA (one per slot)                VALU (about two per slot)
//   0..31   scores of half 1, block kb         probabilities of half 0, block kb
//   32..63  output of half 0, block kb         ... and maxima of half 1, block kb
//   64..95  scores of half 0, block kb + 1     probabilities of half 1, block kb
//   96..127 output of half 1, block kb         ... and maxima of half 0, block kb + 1
//
// Each group of two slots shares one operand fragment (K rows for scores, Vt
// rows for outputs).  Every fragment is read from LDS once, three groups
// ahead of its first use, and kept in registers for its second: the 16 Vt
// fragments of block kb from half 0's output products (slots 32..63) to half
// 1's (96..127), the 16 K fragments of block kb + 1 from half 0's score
// products (64..95) to half 1's, which open the next body (0..31).  A half's
// reference maximum is checked (and, rarely, moved) right after its maxima.
constexpr int kSlots = 128;
constexpr int kGroups = kSlots / 2;   // one fragment per group of two MFMAs
constexpr int kAhead = 3;             // fragment lookahead in groups

__global__ __launch_bounds__(kThreads, 1) void attention_fwd_kernel(const AttnParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kLdsBytes];
  // The wave index as a uniform value, so LDS destinations of the copies and
  // other per-wave addresses are computed in scalar registers.
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 15, g = lane >> 4;

  // Hardware block b runs on XCD b % 8 as its (b / 8)-th block; XCD x takes the
  // contiguous logical range that starts at x * q + min(x, r).
  const int b = blockIdx.x;
  const int x = b % kXcds, q8 = p.blocks / kXcds, r8 = p.blocks % kXcds;
  const int logical = x * q8 + (x < r8 ? x : r8) + b / kXcds;
  const int head = logical / p.tiles_m;
  const int64_t q0 = (int64_t)(logical - head * p.tiles_m) * kBM + kWaveQ * w;
  clock_mark(p.clk, kClockStart);

  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.Q + head * p.sq_b, p.q_bytes);

  // Q fragments (AGPRs): query tile u, K-step s (32 dims): lane (i, g) holds
  // query q0 + 16u + i, dims 32s + 8g .. +7.
  half8_t qf[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t row = q0 + 16 * u + i;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t off =
          row < p.M ? (uint32_t)(row * p.ldq_b) + (uint32_t)((32 * s + 8 * g) * 2) : kOob;
      qf[u][s] = __builtin_bit_cast(half8_t, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
    }
  }

  // LDS: three K slots (block b in slot b % 3) and two Vt slots (b & 1).
  // K: wave load q fills LDS rows 16q + 4w .. +3 (1 KiB); lane l lands in row
  // 16q + 4w + (l >> 4), slot l & 15, and fetches the chunk the swizzle keeps
  // there.  Vt: wave load q fills rows 32q + 8w .. +7; lane l lands in row
  // 32q + 8w + (l >> 3), slot l & 7.
  uint32_t koff[4], voff[4];
  int vkey[4];  // first key (block-relative) of the lane's Vt chunk
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 16 * q + 4 * w + (lane >> 4);
    const int cc = (lane & 15) ^ ((r & 3) | ((r >> 1) & 12));
    koff[q] = (uint32_t)(r * p.ldk_b) + (uint32_t)(cc * 16);
    const int rv_ = 32 * q + 8 * w + (lane >> 3);
    const int cv = (lane & 7) ^ ((rv_ >> 1) & 7);
    voff[q] = (uint32_t)(rv_ * p.ldv_b) + (uint32_t)(cv * 16);
    vkey[q] = 8 * cv;
  }
  lds_u8 *const lds = (lds_u8 *)smem;
  auto kslot = [&](int kb) { return lds + (kb % 3) * kKBytes; };
  auto vslot = [&](int kb) { return lds + 3 * kKBytes + (kb & 1) * kVBytes; };

  // Load q (0..3) of this wave's share of K block kb / Vt block kb.  Each
  // block's loads go through a descriptor rebased on the block's first key
  // (scalar arithmetic), so the lanes' offsets need no per-block add; the
  // descriptor's end stays the head's, so rows past N still read zero.
  const uint8_t *kh = p.K + head * p.sk_b, *vh = p.V + head * p.sv_b;
  auto copy_k1 = [&](int kb, int q) {
    lds_u8 *kd = kslot(kb) + (4 * w) * kKRow;
    const uint32_t kbase = (uint32_t)((int64_t)kb * kBN * p.ldk_b);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(kh + kbase, p.k_bytes - kbase),
                                             (lds_void_t *)(kd + q * 16 * kKRow), 16, koff[q], 0,
                                             0, 0);
  };
  // masked: block kb may be cut by N.  Only whole 8-key chunks are copied; a
  // chunk that straddles N is filled by finish_v, so nothing past a row's N
  // keys is ever read.
  auto copy_v1 = [&](int kb, int q, auto masked) {
    lds_u8 *vd = vslot(kb) + (8 * w) * kVRow;
    const uint32_t vbase = (uint32_t)(kb * kVRow);
    uint32_t off = voff[q];
    if constexpr (decltype(masked)::value)
      if ((int64_t)kb * kBN + vkey[q] + 8 > p.N) off = kOob;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(vh + vbase, p.v_bytes - vbase),
                                             (lds_void_t *)(vd + q * 32 * kVRow), 16, off, 0, 0,
                                             0);
  };
  auto copy_k = [&](int kb) {
#pragma unroll
    for (int q = 0; q < 4; ++q) copy_k1(kb, q);
  };
  auto copy_v = [&](int kb) {
#pragma unroll
    for (int q = 0; q < 4; ++q) copy_v1(kb, q, std::true_type{});
  };
  // After this wave's copies have landed: if N cuts an 8-key chunk of Vt
  // block kb, the lane that owns the chunk's LDS slot (its copy read zeros)
  // fills the valid keys with 2-byte loads and leaves the rest zero; the slot
  // is the lane's own, so no other wave is involved.
  auto finish_v = [&](int kb) {
    const int64_t tail = p.N - (int64_t)kb * kBN;  // valid keys in this block
    if (tail < kBN && (tail & 7)) {
      lds_u8 *vd = vslot(kb) + (8 * w) * kVRow;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (vkey[q] == (int)(tail & ~7)) {
          const int r = 32 * q + 8 * w + (lane >> 3);
          const _Float16 *src = (const _Float16 *)(p.V + head * p.sv_b + r * p.ldv_b) +
                                (int64_t)kb * kBN + vkey[q];
          _Float16 *slot = (_Float16 *)(vd + q * 32 * kVRow + lane * 16);
          for (int h = 0; h < (int)(tail & 7); ++h) slot[h] = src[h];
        }
      }
    }
  };

  // Fragment addresses.  K row read by lane i of score tile t (block-relative
  // key): 32 (t >> 1) + 8 (i >> 2) + 4 (t & 1) + (i & 3); the lane then holds
  // keys 32 (t >> 1) + 8 g + 4 (t & 1) + e of its query column, e < 4, and
  // the keys of tiles 2j, 2j + 1 are the eight consecutive keys 32j + 8g ..
  // of the Vt fragment of K-step j.
  const uint32_t kread0 = (uint32_t)((8 * (i >> 2) + (i & 3)) * kKRow);
  uint32_t ksw[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) ksw[s] = kread0 + (uint32_t)((((4 * s + g) ^ i) << 4));
  uint32_t vsw[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) vsw[j] = (uint32_t)(i * kVRow + (((4 * j + g) ^ ((i >> 1) & 7)) << 4));
  // Fragment of group f (0..63) of the body over key block kb: groups 0..15
  // and 32..47 are K fragments (t, s) of blocks kb and kb + 1, the others Vt
  // fragments (j, dt) of block kb.
  auto frag = [&](int kb, auto fc) -> half8_t {
    constexpr int f = decltype(fc)::value, ph = f >> 4, y = f & 15;
    if constexpr (ph == 0 || ph == 2) {
      constexpr int t = y >> 2, s = y & 3;
      const lds_u8 *Ks = kslot(ph == 0 ? kb : kb + 1);
      return *(const __attribute__((address_space(3))) half8_t *)(
          Ks + ksw[s] + (32 * (t >> 1) + 4 * (t & 1)) * kKRow);
    } else {
      constexpr int j = y >> 3, dt = y & 7;
      return *(const __attribute__((address_space(3))) half8_t *)(vslot(kb) + vsw[j] +
                                                                 dt * 16 * kVRow);
    }
  };

  const int n = p.n_blocks;
  const float c = p.c;
  typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
  const half2_t ones = {(_Float16)1.0f, (_Float16)1.0f};
  float4_t o[8][4];  // O^T tiles [dt][u], AGPRs
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int u = 0; u < 4; ++u) o[dt][u] = float4_t{0.f, 0.f, 0.f, 0.f};
  // Per query tile u: reference maximum (log2 units) and this lane's part of
  // the sum of the fp16-rounded probabilities.
  float m_run[4], l_run[4] = {0.f, 0.f, 0.f, 0.f};
  float4_t sc[2][4][2];  // scores [half][t][uu] of the half's current block
  half8_t pf[2][2][2];   // probabilities [half][j][uu] as output-product operands
  float mloc[2][2], mx[2][2];
  float pv8[8];
  half8_t vsave[16];  // Vt fragments of block kb, read once for both halves
  half8_t ksave[16];  // K fragments of block kb + 1, read once for both halves

  auto fence_accumulators = [&]() {
    mfma_drain();
    static_for<0, 32>([&](auto tc) {
      tie_agpr(o[decltype(tc)::value >> 2][decltype(tc)::value & 3]);
    });
    static_for<0, 16>([&](auto tc) {
      constexpr int v = decltype(tc)::value;
      tie_vgpr(sc[v >> 3][(v >> 1) & 3][v & 1]);
    });
  };

  // The reference maximum moves only when a block's maximum exceeds it by
  // more than 2^kTau in probability: probabilities stay <= 2^kTau, far inside
  // fp16 range, and O and l are rescaled (exact in real arithmetic: the factor
  // cancels in O / l) only on those rare blocks.  The decision is per wave.
  constexpr float kTau = 8.0f;
  // Moves half H's reference maxima to cover mx[H] (rare).  O's tiles are
  // rewritten by v_mfma_f32_16x16x4_f32 with A (lane l: row l & 15, k = l >> 4)
  // = [row == 4k + kk] and B (lane l: k-row l >> 4, column l & 15) = element kk
  // of the lane's scaled tile, which gives back the scaled tile: the rewrite
  // stays in the AGPRs and O is never written by anything but MFMAs.
  auto check_half = [&](auto hc) {
    constexpr int H = decltype(hc)::value;
    if (__builtin_amdgcn_ballot_w64(mx[H][0] > m_run[2 * H] + kTau ||
                                    mx[H][1] > m_run[2 * H + 1] + kTau)) {
      // Column maxima across the four lanes of each query.
#pragma unroll
      for (int uu = 0; uu < 2; ++uu) mx[H][uu] = max_over_column(mloc[H][uu]) * c;
      mfma_drain();
      static_for<0, 8>([&](auto dc) {
        constexpr int dt = decltype(dc)::value;
        tie_agpr(o[dt][2 * H]);
        tie_agpr(o[dt][2 * H + 1]);
      });
      float alpha[2];
#pragma unroll
      for (int uu = 0; uu < 2; ++uu) {
        const int u = 2 * H + uu;
        const float mnew = fmaxf(m_run[u], mx[H][uu]);
        alpha[uu] = __builtin_amdgcn_exp2f(m_run[u] - mnew);
        m_run[u] = mnew;
        l_run[u] *= alpha[uu];
      }
      float sel[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) sel[kk] = (i == 4 * g + kk) ? 1.0f : 0.0f;
      static_for<0, 16>([&](auto tc) {
        constexpr int dt = decltype(tc)::value >> 1, uu = decltype(tc)::value & 1;
        const float4_t v = o[dt][2 * H + uu] * alpha[uu];
        mma_f32_0(sel[0], v[0], o[dt][2 * H + uu]);
#pragma unroll
        for (int kk = 1; kk < 4; ++kk) mma_f32(sel[kk], v[kk], o[dt][2 * H + uu]);
        __builtin_amdgcn_sched_barrier(0);
      });
      mfma_drain();
    }
  };

  // VALU share of the probabilities of half H (item 0..47): items 12 (2j + uu)
  // .. +11 make pf[H][j][uu]: eight exp2 items, then four pack-and-sum items.
  auto prob_item = [&](auto hc, auto ic, int valid, auto mask) {
    constexpr int H = decltype(hc)::value, it = decltype(ic)::value;
    constexpr int j = it / 24, uu = (it % 24) / 12, r = it % 12, u = 2 * H + uu;
    if constexpr (r < 8) {
      constexpr int t = 2 * j + (r >> 2), e = r & 3;
      float pv = __builtin_amdgcn_exp2f(fmaf(sc[H][t][uu][e], c, -m_run[u]));
      if (decltype(mask)::value && 32 * j + 8 * g + 4 * (t & 1) + e >= valid) pv = 0.f;
      pv8[r] = pv;
    } else {
      constexpr int h = r - 8;
      pf[H][j][uu][2 * h] = (_Float16)pv8[2 * h];
      pf[H][j][uu][2 * h + 1] = (_Float16)pv8[2 * h + 1];
      l_run[u] = __builtin_amdgcn_fdot2(half2_t{pf[H][j][uu][2 * h], pf[H][j][uu][2 * h + 1]},
                                        ones, l_run[u], false);
    }
  };
  // VALU share of the maxima of half H (item 0..11): per uu, four items fold
  // one score tile each into the lane's running maximum, then it is scaled to
  // log2 units.  Only the lane's own keys are covered: the reference is
  // checked lane by lane (any lane over it moves the whole column, and the
  // column maximum is reduced across lanes only then).
  auto max_item = [&](auto hc, auto ic, int valid, auto mask) {
    constexpr int H = decltype(hc)::value, it = decltype(ic)::value;
    constexpr int uu = it / 6, r = it % 6;
    if constexpr (r < 4) {
      constexpr int t = r;
      if constexpr (decltype(mask)::value) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (32 * (t >> 1) + 8 * g + 4 * (t & 1) + e >= valid) sc[H][t][uu][e] = -INFINITY;
      }
      const float4_t &v = sc[H][t][uu];
      if constexpr (r == 0) {
        mloc[H][uu] = max3(max3(v[0], v[1], v[2]), v[3], v[3]);
      } else {
        mloc[H][uu] = max3(max3(mloc[H][uu], v[0], v[1]), v[2], v[3]);
      }
    } else if constexpr (r == 4) {
      mx[H][uu] = mloc[H][uu] * c;
    }
  };
  // The MFMA of group slot (phase ph, group y, member uu).
  auto slot_mfma = [&](auto fc, auto uc, const half8_t &a) {
    constexpr int f = decltype(fc)::value, uu = decltype(uc)::value;
    constexpr int ph = f >> 4, y = f & 15;
    if constexpr (ph == 0 || ph == 2) {
      constexpr int H = ph == 0 ? 1 : 0, t = y >> 2, s = y & 3;
      if constexpr (s == 0)
        mma_s0(a, qf[2 * H + uu][s], sc[H][t][uu]);
      else
        mma_s(a, qf[2 * H + uu][s], sc[H][t][uu]);
    } else {
      constexpr int H = ph == 1 ? 0 : 1, j = y >> 3, dt = y & 7;
      if constexpr (dt == 0)
        mma_o_fresh_b(a, pf[H][j][uu], o[dt][2 * H + uu]);
      else
        mma_o(a, pf[H][j][uu], o[dt][2 * H + uu]);
    }
  };

  // One body.  kNext: block kb + 1 exists (its half-0 scores and maxima are
  // part of this body).  mask_cur: block kb may be cut by N; mask_next: block
  // kb + 1 may be.  The K fragments of this body's first 16 groups were read
  // by the previous body (or the prologue).
  auto body = [&](int kb, auto has_next, auto mask_cur, auto mask_next) {
    constexpr bool kNext = decltype(has_next)::value;
    const int64_t rest = p.N - (int64_t)kb * kBN;
    const int valid = decltype(mask_cur)::value && rest < kBN ? (int)rest : kBN;
    const int64_t rest1 = rest - kBN;
    const int valid1 = decltype(mask_next)::value && rest1 < kBN ? (int)rest1 : kBN;
    const bool more_k = kb + 2 < n;
    auto run_slots = [&](auto lo, auto hi) {
      static_for<decltype(lo)::value, decltype(hi)::value>([&](auto kc) {
        constexpr int k = decltype(kc)::value, f = k >> 1, uu = k & 1, ph = f >> 4;
        // Fragment read kAhead groups ahead of its first use.
        if constexpr (uu == 0) {
          constexpr int fn = f + kAhead;
          if constexpr (fn < kGroups) {
            if constexpr (fn >= 16 && fn < 32)
              vsave[fn - 16] = frag(kb, std::integral_constant<int, fn>{});
            else if constexpr (fn >= 32 && fn < 48) {
              if constexpr (kNext) ksave[fn - 32] = frag(kb, std::integral_constant<int, fn>{});
            }
            // groups 0 .. 15 use the K fragments kept from the previous body
            // (or the prologue), groups 48 .. 63 the Vt fragments of 16 .. 31
          }
        }
        // Copies of K block kb + 2 and Vt block kb + 1, one every other slot
        // from the start of the body (the most time to land before its end).
        if constexpr (kNext && (k & 1) == 1 && k < 16) {
          if constexpr ((k >> 1) < 4) {
            if (more_k) copy_k1(kb + 2, k >> 1);
          } else {
            copy_v1(kb + 1, (k >> 1) - 4, mask_next);
          }
        }
        // VALU share.
        if constexpr (k < 48) {
          prob_item(std::integral_constant<int, 0>{}, std::integral_constant<int, k>{}, valid,
                    mask_cur);
        } else if constexpr (k >= 50 && k < 62) {
          max_item(std::integral_constant<int, 1>{}, std::integral_constant<int, k - 50>{},
                   valid, mask_cur);
        } else if constexpr (k >= 64 && k < 112) {
          prob_item(std::integral_constant<int, 1>{}, std::integral_constant<int, k - 64>{},
                    valid, mask_cur);
        } else if constexpr (kNext && k >= 114 && k < 126) {
          max_item(std::integral_constant<int, 0>{}, std::integral_constant<int, k - 114>{},
                   valid1, mask_next);
        }
        // The MFMA.
        if constexpr (kNext || ph != 2)
          slot_mfma(std::integral_constant<int, f>{}, std::integral_constant<int, uu>{},
                    (ph & 1) ? vsave[f & 15] : ksave[f & 15]);
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    // Each run of slots ends a basic block; the compiler may place register
    // copies at block boundaries, so the products still in flight are drained
    // and every accumulator is tied to that point first.
    run_slots(std::integral_constant<int, 0>{}, std::integral_constant<int, 64>{});
    fence_accumulators();
    check_half(std::integral_constant<int, 1>{});
    run_slots(std::integral_constant<int, 64>{}, std::integral_constant<int, 128>{});
    fence_accumulators();
    if constexpr (kNext) {
      check_half(std::integral_constant<int, 0>{});
      __builtin_amdgcn_s_waitcnt(kVmcnt0);
      finish_v(kb + 1);
      __syncthreads();
    }
  };

  // Prologue: K blocks 0 and 1, Vt block 0; half-0 scores and maxima of block
  // 0 set half 0's first reference maximum (half 1's is set by the first
  // check, which always moves it from -inf).
  copy_k(0);
  if (n > 1) copy_k(1);
  copy_v(0);
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
  finish_v(0);
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 4; ++u) m_run[u] = -1e30f;
  {
    // Scores of half 0, block 0 (K slot 0).
    static_for<0, 16>([&](auto yc) {
      constexpr int y = decltype(yc)::value, t = y >> 2, s = y & 3;
      const half8_t a = *(const __attribute__((address_space(3))) half8_t *)(
          kslot(0) + ksw[s] + (32 * (t >> 1) + 4 * (t & 1)) * kKRow);
      ksave[y] = a;
      if constexpr (s == 0) {
        mma_s0(a, qf[0][s], sc[0][t][0]);
        mma_s0(a, qf[1][s], sc[0][t][1]);
      } else {
        mma_s(a, qf[0][s], sc[0][t][0]);
        mma_s(a, qf[1][s], sc[0][t][1]);
      }
    });
    mfma_drain();
    static_for<0, 4>([&](auto tc) {
      constexpr int t = decltype(tc)::value;
      tie_vgpr(sc[0][t][0]);
      tie_vgpr(sc[0][t][1]);
    });
    const int64_t rest = p.N;
    const int valid0 = rest < kBN ? (int)rest : kBN;
    static_for<0, 12>([&](auto ic) {
      max_item(std::integral_constant<int, 0>{}, ic, valid0, std::true_type{});
    });
#pragma unroll
    for (int uu = 0; uu < 2; ++uu) m_run[uu] = max_over_column(mloc[0][uu]) * c;
  }

  const std::true_type T;
  const std::false_type F;
  int kb = 0;
  for (; kb + 2 < n; ++kb) body(kb, T, F, F);
  if (kb + 1 < n) {
    body(kb, T, F, T);
    ++kb;
  }
  body(kb, F, T, F);

  drain_agprs(o);
  // Normalise and store: lane (i, g) holds O[q][16 dt + 4 g + e] of query
  // q = q0 + 16u + i.
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const float inv = 1.0f / sum_over_column(l_run[u]);
    const int64_t q = q0 + 16 * u + i;
    if (q < p.M) {
      _Float16 *orow = (_Float16 *)p.O + head * p.so + q * p.ldo + 4 * g;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
        half4_t h;
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = (_Float16)(o[dt][u][e] * inv);
        *(half4_t *)(orow + 16 * dt) = h;
      }
    }
  }
  clock_mark(p.clk, kClockEnd);
}

}  // namespace dga

using dga::AttnParams;

namespace dg {
uint64_t *clock_slot(int64_t blocks);  // gemm_tn.hip: the per-block clock records
}

namespace {

bool overlaps(const void *a, int64_t a_bytes, const void *b, int64_t b_bytes) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)b_bytes && b0 < a0 + (uintptr_t)a_bytes;
}

}  // namespace

extern "C" int attention_fwd_f16(const void *Q, const void *K, const void *Vt, void *O,
                                 int64_t batch, int64_t M, int64_t N, int64_t D, int64_t ldq,
                                 int64_t ldk, int64_t ldv, int64_t ldo, int64_t stride_q,
                                 int64_t stride_k, int64_t stride_v, int64_t stride_o,
                                 float scale, void *stream) {
  if (batch < 0 || M < 0 || N < 0 || D < 0) return DG_ERR_INVALID_ARGUMENT;
  if (stride_q < 0 || stride_k < 0 || stride_v < 0 || stride_o < 0)
    return DG_ERR_INVALID_ARGUMENT;
  if (!(scale >= 0.0f) || !isfinite(scale)) return DG_ERR_INVALID_ARGUMENT;
  if (batch == 0 || M == 0) return DG_OK;
  if (N < 1 || D < 1) return DG_ERR_INVALID_ARGUMENT;
  if (!Q || !K || !Vt || !O) return DG_ERR_INVALID_ARGUMENT;
  if (ldq < D || ldk < D || ldo < D || ldv < N) return DG_ERR_INVALID_ARGUMENT;
  // Heads of O must not overlap; inputs may be shared (stride 0 broadcasts).
  if (batch > 1 && stride_o < (M - 1) * ldo + D) return DG_ERR_INVALID_ARGUMENT;
  if (D != dga::kD) return DG_ERR_UNSUPPORTED;
  // Extents in elements; every product below stays far from 2^63 once the
  // 2^31-byte per-head limits further down hold.
  const double ext_q = (double)(batch - 1) * stride_q + (double)(M - 1) * ldq + D;
  const double ext_k = (double)(batch - 1) * stride_k + (double)(N - 1) * ldk + D;
  const double ext_v = (double)(batch - 1) * stride_v + (double)(D - 1) * ldv + N;
  const double ext_o = (double)(batch - 1) * stride_o + (double)(M - 1) * ldo + D;
  if (ext_q > 4e18 || ext_k > 4e18 || ext_v > 4e18 || ext_o > 4e18)
    return DG_ERR_UNSUPPORTED;
  const int64_t bo = 2 * ((batch - 1) * stride_o + (M - 1) * ldo + D);
  if (overlaps(O, bo, Q, 2 * ((batch - 1) * stride_q + (M - 1) * ldq + D)) ||
      overlaps(O, bo, K, 2 * ((batch - 1) * stride_k + (N - 1) * ldk + D)) ||
      overlaps(O, bo, Vt, 2 * ((batch - 1) * stride_v + (D - 1) * ldv + N)))
    return DG_ERR_INVALID_ARGUMENT;
  // 16-byte vectors: aligned bases, row and head strides in whole vectors.
  if (((uintptr_t)Q | (uintptr_t)K | (uintptr_t)Vt | (uintptr_t)O) & 15)
    return DG_ERR_UNSUPPORTED;
  if ((ldq | ldk | ldv | ldo | stride_q | stride_k | stride_v | stride_o) & 7)
    return DG_ERR_UNSUPPORTED;
  // Per-head buffer offsets, including the rows and columns of the last
  // (partly out-of-range) key block, must stay below 2^31.
  const int64_t lim = (int64_t)1 << 31;
  const int64_t q_bytes = 2 * ((M - 1) * ldq + D);
  const int64_t k_bytes = 2 * ((N - 1) * ldk + D);
  const int64_t v_bytes = 2 * ((D - 1) * ldv + N);
  if (q_bytes >= lim || 2 * (N + dga::kBN) * ldk >= lim ||
      2 * ((D - 1) * ldv + N + dga::kBN) >= lim)
    return DG_ERR_UNSUPPORTED;
  const int64_t tiles_m = (M + dga::kBM - 1) / dga::kBM;
  if (batch * tiles_m >= lim) return DG_ERR_UNSUPPORTED;

  AttnParams p;
  p.Q = (const uint8_t *)Q;
  p.K = (const uint8_t *)K;
  p.V = (const uint8_t *)Vt;
  p.O = (uint8_t *)O;
  p.M = M;
  p.N = N;
  p.ldq_b = 2 * ldq;
  p.ldk_b = 2 * ldk;
  p.ldv_b = 2 * ldv;
  p.ldo = ldo;
  p.sq_b = 2 * stride_q;
  p.sk_b = 2 * stride_k;
  p.sv_b = 2 * stride_v;
  p.so = stride_o;
  p.q_bytes = (uint32_t)q_bytes;
  p.k_bytes = (uint32_t)k_bytes;
  p.v_bytes = (uint32_t)v_bytes;
  p.tiles_m = (int32_t)tiles_m;
  p.blocks = (int32_t)(batch * tiles_m);
  p.n_blocks = (int32_t)((N + dga::kBN - 1) / dga::kBN);
  p.c = (float)((double)scale * 1.4426950408889634);  // scale * log2(e)
  p.clk = dg::clock_slot(p.blocks);
  hipLaunchKernelGGL(dga::attention_fwd_kernel, dim3((unsigned)p.blocks), dim3(dga::kThreads), 0,
                     (hipStream_t)stream, p);
  return hipGetLastError() == hipSuccess ? DG_OK : DG_ERR_HIP;
}
