// gemm_tn.hip -- TN GEMM kernels for gfx950 (MI355X) and the C ABI around them.
//
// C = A x B with A row-major M x K, B column-major K x N (K contiguous for both
// operands) and C column-major, as defined in "FP16 GEMM optimisation on AMD
// RDNA 3 and RDNA 4", section "What we compute", and the dot-product equation of
// "hello-gpu, chapter 11 (GEMM-like)", section 11.1.
//
// Kernel design (one family, fp16 and fp8 instantiations, optional head index):
//   * 256 x 256 output tile per workgroup, 4 waves (one per SIMD), each wave owns
//     a 128 x 128 quarter held as 8 x 8 MFMA 16x16 accumulator tiles -- the
//     4-wave layout of the MI355X FP8 GEMM page, section "why 4 waves".
//   * A K-step moves 128 bytes of K per row (64 fp16 or 128 fp8 elements):
//     256 rows x 128 B of A and of B per stage, two stages in LDS (128 KiB).
//   * Global -> LDS copies are buffer loads that write LDS directly (no VGPR
//     staging).  The buffer resource descriptor makes out-of-range reads return
//     zero, which handles M and N tails ("FP16 GEMM optimisation ...", Step 4);
//     K-tail chunks are pointed past the descriptor's end so they read zero too
//     (the K rule of section 11.4 of the hello-gpu chapter).
//   * LDS rows are 128 B; the 16-byte chunk c of row r is stored in slot
//     c ^ ((r >> 1) & 7), the XOR swizzle of the MI355X FP8 GEMM page (section
//     "XOR swizzle"), so the 16 rows read by one ds_read_b128 phase hit 16
//     distinct 16-byte bank groups of the 256-byte bank period.
//   * Block ids are remapped so each XCD (workgroups are dealt round-robin over
//     the 8 XCDs) receives a contiguous range of tiles, and that range is walked
//     in the grouped order of "FP16 GEMM optimisation ...", Step 6 (groups of 8
//     tile rows), so the blocks co-resident on one XCD share A and B strips in
//     its L2 (the chiplet-aware remap of the MI355X FP8 GEMM page).
//   * Epilogue: fp32 -> fp16 (round to nearest even) or fp32 * (sa*sb) -> bf16
//     (round to nearest even), masked column-major stores that never touch C
//     outside its M x N logical extent (section 11.4 of the hello-gpu chapter).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dense_gemm_tn.h"

namespace dg {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef int int8_t_v __attribute__((ext_vector_type(8)));
typedef int int4_t_v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kTile = 256;        // rows of A / columns of B per workgroup
constexpr int kRowBytes = 128;    // bytes of K per row per K-step
constexpr int kThreads = 256;     // 4 waves of 64
constexpr int kWaveTile = 128;    // each wave owns kWaveTile x kWaveTile of C
constexpr int kSub = 8;           // 16x16 MFMA tiles per wave edge (128 / 16)
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
  static constexpr int subs = 2;     // MFMA K sub-steps per K-step (32 each)
  typedef half8_t frag_t;
};
template <> struct Traits<kF8> {
  static constexpr int es = 1;
  static constexpr int kstep = 128;
  static constexpr int reads = 2;    // 32 bytes of K per lane
  static constexpr int subs = 1;     // one 16x16x128 MFMA covers the K-step
  typedef int8_t_v frag_t;
};

__device__ __forceinline__ float4_t mma(const half8_t &a, const half8_t &b, float4_t c) {
  // v_mfma_f32_16x16x32_f16: fp16 products, fp32 accumulate.
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float4_t mma(const int8_t_v &a, const int8_t_v &b, float4_t c) {
  // v_mfma_f32_16x16x128_f8f6f4 with both operand formats = 0 (FP8 E4M3) and
  // no block scales; the per-tensor scales are applied in the epilogue.
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
  int32_t c_vec_ok;      // 8-byte C stores are aligned (ldc % 4 == 0)
};

// Block id -> (head, tile_m, tile_n).  First the chiplet remap: block b runs on
// XCD b % 8 and is the (b / 8)-th block there; XCD x gets the contiguous logical
// range starting at x*q + min(x, r) (q = G / 8, r = G % 8), a bijection for any
// G.  Then the grouped order inside a head: groups of kGroupM tile rows, walked
// column by column (short last group allowed).
template <typename I>
__host__ __device__ inline void tile_of_block(I b, I G, I tiles_m, I tiles_n, I *head, I *tm,
                                              I *tn) {
  const I q = G / kXcds, r = G % kXcds;
  const I x = b % kXcds, idx = b / kXcds;
  const I logical = x * q + (x < r ? x : r) + idx;
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

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           (int)kRsrcWord3);
}

// One K-step's copy of a 256-row operand strip into one LDS stage.  Load q of
// wave w fills LDS rows 32q + 8w .. +7 (1 KiB, lane-contiguous: lane l writes
// bytes l*16 .. l*16+15 of that KiB).  Lane l therefore lands in row
// 32q + 8w + (l >> 3), slot l & 7, and fetches the global chunk that the
// swizzle stores there.
template <int ES>
__device__ __forceinline__ void copy_stage(lds_void_t *stage, __amdgpu_buffer_rsrc_t rsrc,
                                           uint32_t voff, uint32_t q_stride, bool chunk_valid,
                                           int wave) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint32_t off = chunk_valid ? voff + q * q_stride : kOob;
    lds_void_t *dst = (lds_void_t *)((__attribute__((address_space(3))) uint8_t *)stage +
                                     q * 4096 + wave * 1024);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, off, 0, 0, 0);
  }
}

template <int KIND>
__device__ __forceinline__ void load_frags(typename Traits<KIND>::frag_t (&f)[kSub],
                                           const __attribute__((address_space(3))) uint8_t *base,
                                           const uint32_t (&lane_off)[2], int s) {
  typedef Traits<KIND> T;
#pragma unroll
  for (int i = 0; i < kSub; ++i) {
    if constexpr (T::reads == 1) {
      f[i] = *(const __attribute__((address_space(3))) half8_t *)(base + i * 16 * kRowBytes +
                                                                  lane_off[s]);
    } else {
      int4_t_v lo = *(const __attribute__((address_space(3))) int4_t_v *)(base + i * 16 * kRowBytes +
                                                                          lane_off[0]);
      int4_t_v hi = *(const __attribute__((address_space(3))) int4_t_v *)(base + i * 16 * kRowBytes +
                                                                          lane_off[1]);
      f[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }
}

template <int KIND>
__device__ __forceinline__ void compute_stage(float4_t (&acc)[kSub][kSub],
                                              const __attribute__((address_space(3))) uint8_t *sa,
                                              const __attribute__((address_space(3))) uint8_t *sb,
                                              const uint32_t (&lane_off)[2]) {
  typedef Traits<KIND> T;
#pragma unroll
  for (int s = 0; s < T::subs; ++s) {
    typename T::frag_t a[kSub], b[kSub];
    load_frags<KIND>(a, sa, lane_off, s);
    load_frags<KIND>(b, sb, lane_off, s);
#pragma unroll
    for (int i = 0; i < kSub; ++i)
#pragma unroll
      for (int j = 0; j < kSub; ++j) acc[i][j] = mma(a[i], b[j], acc[i][j]);
  }
}

template <int KIND>
__device__ __forceinline__ void store_c(const Params &p, uint8_t *Cb, const float4_t (&acc)[kSub][kSub],
                                        int64_t m_base, int64_t n_base, int lane) {
  // Accumulator tile (i, j): lane l holds rows 4*(l >> 4) .. +3 of column (l & 15),
  // i.e. four consecutive elements of one column of the column-major C.
  const int64_t m_lane = m_base + 4 * (lane >> 4);
  const int64_t n_lane = n_base + (lane & 15);
  const bool full = (m_base + kWaveTile <= p.M) && (n_base + kWaveTile <= p.N) && p.c_vec_ok;
#pragma unroll
  for (int j = 0; j < kSub; ++j) {
    const int64_t n = n_lane + 16 * j;
#pragma unroll
    for (int i = 0; i < kSub; ++i) {
      const int64_t m = m_lane + 16 * i;
      uint16_t h[4];
      if constexpr (KIND == kF16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          _Float16 v = (_Float16)acc[i][j][e];
          h[e] = __builtin_bit_cast(uint16_t, v);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          __bf16 v = (__bf16)(acc[i][j][e] * p.scale);
          h[e] = __builtin_bit_cast(uint16_t, v);
        }
      }
      uint16_t *dst = (uint16_t *)Cb + (n * p.ldc + m);
      if (full) {
        uint2 w;
        w.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
        w.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
        *(uint2 *)dst = w;
      } else if (n < p.N) {
        if (p.c_vec_ok && m + 3 < p.M) {
          uint2 w;
          w.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
          w.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
          *(uint2 *)dst = w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (m + e < p.M) dst[e] = h[e];
        }
      }
    }
  }
}

template <int KIND>
__global__ __launch_bounds__(kThreads, 1) void gemm_tn_kernel(Params p) {
  typedef Traits<KIND> T;
  // Two stages of [A strip | B strip], 64 KiB each.
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * 2 * kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  int head, tm, tn;
  tile_of_block<int>((int)blockIdx.x, (int)gridDim.x, p.tiles_m, p.tiles_n, &head, &tm, &tn);
  const int64_t m0 = (int64_t)tm * kTile, n0 = (int64_t)tn * kTile;

  const uint8_t *Ab = p.A + head * p.stride_a_b + m0 * p.lda_b;
  const uint8_t *Bb = p.B + head * p.stride_b_b + n0 * p.ldb_b;
  uint8_t *Cb = p.C + head * p.stride_c_b;
  const int64_t rows_a = (p.M - m0) < kTile ? (p.M - m0) : kTile;
  const int64_t rows_b = (p.N - n0) < kTile ? (p.N - n0) : kTile;
  const uint32_t kbytes = (uint32_t)(p.K * T::es);
  const uint32_t rec_a = (uint32_t)((rows_a - 1) * p.lda_b) + kbytes;
  const uint32_t rec_b = (uint32_t)((rows_b - 1) * p.ldb_b) + kbytes;

  // Copy geometry of this lane (same for A and B, see copy_stage).
  const int crow = 8 * wave + (lane >> 3);           // row within a 32-row band
  const int gchunk = (lane & 7) ^ ((crow >> 1) & 7);  // global 16-B chunk of that row
  const uint32_t voff_a = (uint32_t)(crow * p.lda_b) + gchunk * 16;
  const uint32_t voff_b = (uint32_t)(crow * p.ldb_b) + gchunk * 16;
  const uint32_t qs_a = (uint32_t)(32 * p.lda_b), qs_b = (uint32_t)(32 * p.ldb_b);
  const int kchunk = gchunk * (16 / T::es);          // K offset of the chunk in a step

  // Fragment geometry: lane l reads row (l & 15) of each 16-row MFMA tile and the
  // 16-byte chunk(s) of its K group (l >> 4); slots are swizzled by row.
  const int wm = wave & 1, wn = wave >> 1;
  uint32_t lane_off[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int chunk = (T::reads == 1) ? (j * 4 + (lane >> 4)) : ((lane >> 4) * 2 + j);
    lane_off[j] = (uint32_t)((lane & 15) * kRowBytes + ((chunk ^ ((lane & 15) >> 1)) * 16));
  }
  const int a_wave_off = wm * kWaveTile * kRowBytes;
  const int b_wave_off = wn * kWaveTile * kRowBytes;

  float4_t acc[kSub][kSub];
#pragma unroll
  for (int i = 0; i < kSub; ++i)
#pragma unroll
    for (int j = 0; j < kSub; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};

  const int64_t nk = (p.K + T::kstep - 1) / T::kstep;
  auto issue = [&](int64_t ks, lds_void_t *da, lds_void_t *db) {
    const int64_t k0 = ks * T::kstep;
    const uint32_t kb = (uint32_t)(k0 * T::es);
    const bool valid = kchunk < p.K - k0;
    copy_stage<T::es>(da, make_rsrc(Ab + kb, rec_a - kb), voff_a, qs_a, valid, wave);
    copy_stage<T::es>(db, make_rsrc(Bb + kb, rec_b - kb), voff_b, qs_b, valid, wave);
  };
  typedef const __attribute__((address_space(3))) uint8_t *lds_cptr;

  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  lds_u8 *const lds = (lds_u8 *)smem;
  if (nk > 0) issue(0, (lds_void_t *)lds, (lds_void_t *)(lds + kStageBytes));
  for (int64_t ks = 0; ks < nk; ++ks) {
    // Stage ks&1 has landed and every wave is done reading the other stage.
    __syncthreads();
    const int cur = (int)(ks & 1) * 2 * kStageBytes;
    const int nxt = 2 * kStageBytes - cur;
    if (ks + 1 < nk)
      issue(ks + 1, (lds_void_t *)(lds + nxt), (lds_void_t *)(lds + nxt + kStageBytes));
    compute_stage<KIND>(acc, (lds_cptr)(lds + cur + a_wave_off),
                        (lds_cptr)(lds + cur + kStageBytes + b_wave_off), lane_off);
  }

  store_c<KIND>(p, Cb, acc, m0 + wm * kWaveTile, n0 + wn * kWaveTile, lane);
}

template __global__ void gemm_tn_kernel<kF16>(Params);
template __global__ void gemm_tn_kernel<kF8>(Params);

// ------------------------------------------------------------------ host side

static bool overlaps(const void *a, uint64_t abytes, const void *b, uint64_t bbytes) {
  if (abytes == 0 || bbytes == 0) return false;
  const uint64_t a0 = (uint64_t)(uintptr_t)a, b0 = (uint64_t)(uintptr_t)b;
  return a0 < b0 + bbytes && b0 < a0 + abytes;
}

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

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

template <int KIND>
static int launch(const Problem &pr, hipStream_t stream) {
  typedef Traits<KIND> T;
  const int es = T::es;
  if (pr.batch < 0 || pr.M < 0 || pr.N < 0 || pr.K < 0) return DG_ERR_INVALID_ARGUMENT;
  if (pr.lda < pr.K || pr.ldb < pr.K || pr.ldc < pr.M) return DG_ERR_INVALID_ARGUMENT;
  if (pr.batch == 0 || pr.M == 0 || pr.N == 0) return DG_OK;
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

  const int64_t tiles_m = (pr.M + kTile - 1) / kTile;
  const int64_t tiles_n = (pr.N + kTile - 1) / kTile;
  const int64_t blocks = tiles_m * tiles_n * pr.batch;
  if (blocks > 0x7fffffffLL) return DG_ERR_UNSUPPORTED;

  Params p;
  p.A = (const uint8_t *)pr.A;
  p.B = (const uint8_t *)pr.B;
  p.C = (uint8_t *)pr.C;
  p.M = pr.M; p.N = pr.N; p.K = pr.K;
  p.lda_b = pr.lda * es; p.ldb_b = pr.ldb * es; p.ldc = pr.ldc;
  p.stride_a_b = pr.stride_a * es; p.stride_b_b = pr.stride_b * es; p.stride_c_b = pr.stride_c * 2;
  p.tiles_m = (int32_t)tiles_m; p.tiles_n = (int32_t)tiles_n;
  p.scale = pr.scale;
  p.c_vec_ok = (pr.ldc % 4 == 0) ? 1 : 0;

  hipLaunchKernelGGL(gemm_tn_kernel<KIND>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError() == hipSuccess ? DG_OK : DG_ERR_HIP;
}

}  // namespace dg

extern "C" {

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

}  // extern "C"
