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
//   * One workgroup = 4 waves = 128 queries of one head; wave w owns 32 queries
//     (two 16-query MFMA column tiles).  Two workgroups per CU.
//   * The wave's Q rows live in registers for the whole kernel as B operands of
//     v_mfma_f32_16x16x32_f16 (the 16x16 shapes of the MI355X FP8 GEMM page).
//   * Keys are processed 64 at a time.  A key block of K (64 x 256 B) and of Vt
//     (128 x 128 B) is copied global -> LDS by buffer loads that write LDS
//     directly, double-buffered (2 x 32 KiB), one barrier per key block.
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
constexpr int kBM = 128;                // queries per workgroup
constexpr int kBN = 64;                 // keys per block
constexpr int kThreads = 256;           // 4 waves
constexpr int kKRow = kD * 2;           // bytes per K row in LDS
constexpr int kVRow = kBN * 2;          // bytes per Vt row in LDS
constexpr int kKBytes = kBN * kKRow;    // 16 KiB
constexpr int kVBytes = kD * kVRow;     // 16 KiB
constexpr int kStage = kKBytes + kVBytes;
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
};

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
__device__ __forceinline__ float sum_over_column(float x) {
  float a = x, b = x;
  swap32(a, b);
  float c = a + b, d = c;
  swap16(c, d);
  return c + d;
}

__device__ __forceinline__ float4_t mma(const half8_t &a, const half8_t &b, const float4_t &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(kThreads, 2) void attention_fwd_kernel(const AttnParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kStage];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i = lane & 15, g = lane >> 4;

  // Hardware block b runs on XCD b % 8 as its (b / 8)-th block; XCD x takes the
  // contiguous logical range that starts at x * q + min(x, r).
  const int b = blockIdx.x;
  const int x = b % kXcds, q8 = p.blocks / kXcds, r8 = p.blocks % kXcds;
  const int logical = x * q8 + (x < r8 ? x : r8) + b / kXcds;
  const int head = logical / p.tiles_m;
  const int64_t q0 = (int64_t)(logical - head * p.tiles_m) * kBM + 32 * w;

  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.Q + head * p.sq_b, p.q_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.K + head * p.sk_b, p.k_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.V + head * p.sv_b, p.v_bytes);

  // Q fragments: column tile u, K-step s (32 dims): lane (i, g) holds query
  // q0 + 16u + i, dims 32s + 8g .. +7.
  half8_t qf[2][4];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int64_t row = q0 + 16 * u + i;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t off =
          row < p.M ? (uint32_t)(row * p.ldq_b) + (uint32_t)((32 * s + 8 * g) * 2) : kOob;
      qf[u][s] = __builtin_bit_cast(half8_t, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
    }
  }

  // Copy plan.  K: wave load q fills LDS rows 16q + 4w .. +3 (1 KiB); lane l
  // lands in row 16q + 4w + (l >> 4), slot l & 15, and fetches the chunk the
  // swizzle keeps there.  Vt: wave load q fills rows 32q + 8w .. +7; lane l
  // lands in row 32q + 8w + (l >> 3), slot l & 7.
  uint32_t koff[4], voff[4];
  int vkey[4];  // first key (block-relative) of the lane's Vt chunk
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 16 * q + 4 * w + (lane >> 4);
    const int c = (lane & 15) ^ ((r & 3) | ((r >> 1) & 12));
    koff[q] = (uint32_t)(r * p.ldk_b) + (uint32_t)(c * 16);
    const int rv_ = 32 * q + 8 * w + (lane >> 3);
    const int cv = (lane & 7) ^ ((rv_ >> 1) & 7);
    voff[q] = (uint32_t)(rv_ * p.ldv_b) + (uint32_t)(cv * 16);
    vkey[q] = 8 * cv;
  }
  lds_u8 *const lds = (lds_u8 *)smem;

  auto issue_copies = [&](int kb, int st) {
    lds_u8 *kd = lds + st * kStage + (4 * w) * kKRow;
    lds_u8 *vd = lds + st * kStage + kKBytes + (8 * w) * kVRow;
    const uint32_t kbase = (uint32_t)((int64_t)kb * kBN * p.ldk_b);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t *)(kd + q * 16 * kKRow), 16,
                                               kbase + koff[q], 0, 0, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // Only whole 8-key chunks are copied; a chunk that straddles N is filled
      // by finish_copies, so nothing past a row's N keys is ever read.
      const uint32_t off =
          (int64_t)kb * kBN + vkey[q] + 8 <= p.N ? voff[q] + (uint32_t)(kb * kVRow) : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t *)(vd + q * 32 * kVRow), 16, off,
                                               0, 0, 0);
    }
  };
  // Wait for this wave's copies of key block kb (in stage st).  If N cuts an
  // 8-key chunk of that block, the lane that owns the chunk's LDS slot (its
  // copy read zeros) fills the valid keys with 2-byte loads and leaves the
  // rest zero; the slot is the lane's own, so no other wave is involved.
  auto finish_copies = [&](int kb, int st) {
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    const int64_t tail = p.N - (int64_t)kb * kBN;  // valid keys in this block
    if (tail < kBN && (tail & 7)) {
      lds_u8 *vd = lds + st * kStage + kKBytes + (8 * w) * kVRow;
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

  issue_copies(0, 0);
  finish_copies(0, 0);
  __syncthreads();

  // K row read by lane i of S^T tile t (block-relative key):
  // 32 (t >> 1) + 8 (i >> 2) + 4 (t & 1) + (i & 3).  The lane then holds keys
  // 32 (t >> 1) + 8 g + 4 (t & 1) + e of its query column, e < 4.
  uint32_t kread[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
    kread[t] = (uint32_t)((32 * (t >> 1) + 8 * (i >> 2) + 4 * (t & 1) + (i & 3)) * kKRow);
  const uint32_t vread = (uint32_t)(i * kVRow);
  const int vsw = (i >> 1) & 7;

  float4_t o[8][2];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt][0] = o[dt][1] = float4_t{0.f, 0.f, 0.f, 0.f};
  // Running reference maximum (log2 units) and this lane's part of the sum of
  // the fp16-rounded probabilities, per query column u.
  float m_run[2] = {-1e30f, -1e30f}, l_run[2] = {0.f, 0.f};
  const float c = p.c;
  typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
  const half2_t ones = {(_Float16)1.0f, (_Float16)1.0f};

  // One key block.  kMasked: the block is the last one and N cuts it, so keys
  // past N get score -inf and probability 0 (only that block pays for it).
  auto block = [&](int kb, auto masked_tag) {
    constexpr bool kMasked = decltype(masked_tag)::value;
    const int st = kb & 1;
    if (kb + 1 < p.n_blocks) issue_copies(kb + 1, st ^ 1);
    const lds_u8 *Ks = lds + st * kStage;
    const lds_u8 *Vs = Ks + kKBytes;

    float4_t sacc[4][2];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const half8_t a =
            *(const __attribute__((address_space(3))) half8_t *)(Ks + kread[t] +
                                                                 (((4 * s + g) ^ i) << 4));
#pragma unroll
        for (int u = 0; u < 2; ++u)
          sacc[t][u] = mma(a, qf[u][s], s == 0 ? float4_t{0.f, 0.f, 0.f, 0.f} : sacc[t][u]);
      }
    }

    const int valid = kMasked ? (int)(p.N - (int64_t)kb * kBN) : kBN;
    float mx[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float m = -INFINITY;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (kMasked && 32 * (t >> 1) + 8 * g + 4 * (t & 1) + e >= valid)
            sacc[t][u][e] = -INFINITY;
          m = fmaxf(m, sacc[t][u][e]);
        }
      mx[u] = max_over_column(m) * c;
    }
    // The reference maximum moves only when a block's maximum exceeds it by
    // more than 2^kTau in probability (or on the first block): probabilities
    // then stay <= 2^kTau, far inside fp16 range, and the rescaling of O and l
    // (exact in real arithmetic: it cancels in O / l) is skipped for most
    // blocks.  The branch is taken per wave.
    constexpr float kTau = 8.0f;
    if (__builtin_amdgcn_ballot_w64(mx[0] > m_run[0] + kTau || mx[1] > m_run[1] + kTau)) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float mnew = fmaxf(m_run[u], mx[u]);
        const float alpha = __builtin_amdgcn_exp2f(m_run[u] - mnew);
        m_run[u] = mnew;
        l_run[u] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[dt][u] *= alpha;
      }
    }

    half8_t pf[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float pv = __builtin_amdgcn_exp2f(fmaf(sacc[t][u][e], c, -m_run[u]));
          if (kMasked && 32 * (t >> 1) + 8 * g + 4 * (t & 1) + e >= valid) pv = 0.f;
          pf[t >> 1][u][4 * (t & 1) + e] = (_Float16)pv;
        }
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int h = 0; h < 4; ++h)
          l_run[u] = __builtin_amdgcn_fdot2(
              half2_t{pf[j][u][2 * h], pf[j][u][2 * h + 1]}, ones, l_run[u], false);
    }

#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const half8_t a = *(const __attribute__((address_space(3))) half8_t *)(
            Vs + dt * 16 * kVRow + vread + (((4 * j + g) ^ vsw) << 4));
#pragma unroll
        for (int u = 0; u < 2; ++u) o[dt][u] = mma(a, pf[j][u], o[dt][u]);
      }
    }

    if (kb + 1 < p.n_blocks) finish_copies(kb + 1, st ^ 1);
    __syncthreads();
  };

  const int full_blocks = (int)(p.N / kBN);
  for (int kb = 0; kb < full_blocks; ++kb) block(kb, std::false_type{});
  if (full_blocks < p.n_blocks) block(full_blocks, std::true_type{});

  // Normalise and store: lane (i, g) holds O[q][16 dt + 4 g + e] of query
  // q = q0 + 16u + i.
#pragma unroll
  for (int u = 0; u < 2; ++u) {
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
}

}  // namespace dga

using dga::AttnParams;

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
  hipLaunchKernelGGL(dga::attention_fwd_kernel, dim3((unsigned)p.blocks), dim3(dga::kThreads), 0,
                     (hipStream_t)stream, p);
  return hipGetLastError() == hipSuccess ? DG_OK : DG_ERR_HIP;
}
