// Internal definitions shared by the HIP kernels and the runtime of libpsgd.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace psgd {

// ------------------------------------------------------------------------------------------
// vector types for the gfx950 MFMA builtins
// ------------------------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum GradType : int { G_F16 = 1, G_BF16 = 2, G_F32 = 3 };

// Pointers read out of the descriptor table are generic; accesses through them would compile
// to FLAT instructions (which wait on both the vector-memory and the LDS counters). Every
// kernel casts them to the global address space first so the compiler emits global_load /
// global_store.
#define GLOBAL __attribute__((address_space(1)))
template <typename T> __device__ __forceinline__ GLOBAL T* gbl(T* p) { return (GLOBAL T*)p; }
template <typename T> __device__ __forceinline__ const GLOBAL T* gbl(const T* p) { return (const GLOBAL T*)p; }
template <typename T, typename U> __device__ __forceinline__ const GLOBAL T* gcast(const GLOBAL U* p) {
  return reinterpret_cast<const GLOBAL T*>(p);
}
template <typename T, typename U> __device__ __forceinline__ GLOBAL T* gcast(GLOBAL U* p) {
  return reinterpret_cast<GLOBAL T*>(p);
}

// Buffer resources. The streamed gradient, error and output matrices are accessed through a
// per-matrix buffer descriptor whose range is the matrix's byte span. A lane whose element is
// out of range uses the offset kOOB: the hardware returns zero for such loads and drops such
// stores, so ragged edges need no branches and the compiler keeps every load in flight.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOOB = 0x80000000u;          // beyond every range (spans are < 2^31 bytes)
constexpr int kRsrcWord3 = 0x00020000;          // raw 32-bit data format (gfx9 family)
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}
// Cache policy bits of the streamed G/E/D accesses: 0 (default) or kNonTemporal (the "nt"
// bit: evict first). The decompression streams G, E and D non-temporally, which keeps its
// factor tiles in L2 (4.52 -> 3.96 ms). The two product kernels use the default: with
// non-temporal loads they measured 9% and 6% slower.
constexpr int kNonTemporal = 2;
#ifndef PSGD_STREAM_POLICY
#define PSGD_STREAM_POLICY 0
#endif
constexpr int kStream = PSGD_STREAM_POLICY;
template <int POL = kStream>
__device__ __forceinline__ u32x4 bload16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POL));
}
template <int POL = kStream>
__device__ __forceinline__ u32x2 bload8(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, POL));
}
template <int POL = kStream>
__device__ __forceinline__ uint32_t bload4(rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, POL);
}

// N consecutive gradient elements of dtype GT (N * size bytes, 4..16), loaded through a
// buffer descriptor and widened to fp32.
template <int GT, int N> struct GradVec {
  static constexpr int kBytes = N * (GT == G_F32 ? 4 : 2);
  typedef uint32_t raw_t __attribute__((ext_vector_type(kBytes / 4)));
  raw_t v;
  template <int POL = kStream>
  __device__ __forceinline__ void load(rsrc_t r, uint32_t off) {
    if constexpr (kBytes == 4) v = raw_t{bload4<POL>(r, off)};
    else if constexpr (kBytes == 8) v = __builtin_bit_cast(raw_t, bload8<POL>(r, off));
    else v = __builtin_bit_cast(raw_t, bload16<POL>(r, off));
  }
  typedef float fN __attribute__((ext_vector_type(N)));
  __device__ __forceinline__ fN f32() const {
    if constexpr (GT == G_F16) {
      typedef _Float16 hN __attribute__((ext_vector_type(N)));
      return __builtin_convertvector(__builtin_bit_cast(hN, v), fN);
    } else if constexpr (GT == G_BF16) {
      typedef __bf16 bN __attribute__((ext_vector_type(N)));
      return __builtin_convertvector(__builtin_bit_cast(bN, v), fN);
    } else {
      return __builtin_bit_cast(fN, v);
    }
  }
};

template <int POL = kStream>
__device__ __forceinline__ void bstore16(u32x4 v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b128(r, 0, 0, 0)), v), r, off, 0, POL);
}

constexpr int kWave = 64;
constexpr int kMaxRankTiles = 8;          // 16-column rank tiles one product pass carries (128)
constexpr int kMaxRank = 1024;            // largest compression rank
constexpr int kBlk = 128;                 // column block of the blocked orthonormalisation (r > 128)
constexpr int kXcds = 8;                  // MI355X: 8 XCDs, 32 CUs each
constexpr int kGramRows = 256;            // rows per Gram partial, r <= 128
constexpr int kGramRowsBig = 1024;        // rows per Gram partial, r > 128
// A column of M q whose squared norm after projecting out the earlier columns is at most
// 2^-40 of its squared norm before is dependent (its direction is lost to rounding).
constexpr double kDegenerate = 9.094947017729282e-13;   // 2^-40
// The Gram (Cholesky) form loses orthogonality as eps_64 times the squared condition number of
// M q. When a kept column's squared residual ratio falls below 2^-20 the orthonormalisation is
// repeated on its own result (a second pass restores orthogonality to rounding level).
constexpr double kReorth = 9.5367431640625e-07;         // 2^-20

// ------------------------------------------------------------------------------------------
// device-side description of one gradient matrix and its plan workspace
// ------------------------------------------------------------------------------------------
struct DevMat {
  const void* grad;  int64_t ld_grad;
  float* err;        int64_t ld_err;
  float* q;          float* q_next;    float* p;
  float* out;        int64_t ld_out;
  int32_t m, n, block, r;
  int32_t rpad;      // r rounded up to 16 (MFMA tile)
  int32_t kpad3;     // r rounded up to 32 (K of the fp16 decompression MFMA)
  int32_t pad1_;
  int32_t mpad;      // m rounded up to a whole stage of the M^T P kernel
  int32_t gram_parts;
  int32_t gram_rows;   // rows per Gram partial (multiple of 16)
  uint32_t g_bytes, e_bytes, o_bytes;   // byte spans of G, E and out (buffer ranges, < 2^31)
  uint32_t pad2_;
  // workspace (library owned)
  float* p_raw;                        // m x rpad fp32: M q before orthonormalisation
  uint16_t* pt_hi; uint16_t* pt_lo;    // rpad x mpad bf16: P^T split into hi + lo
  int32_t* p3_exp;                     // m3 (m rounded up to a decompression tile; zero rows):
                                       // row exponent of P for the decompression's fp16 split
  int32_t* q3_exp;                     // n3 likewise for q_next
  uint16_t* p3h;                       // r > 128 (else NULL): m3 rows of kpad3 ranks, P_hat scaled
                                       // by its row exponent and split into fp16 hi + lo, as
                                       // 16-byte pairs per 8 ranks (hi, then lo); zero rows past m
  uint16_t* q3h;                       // n3 rows likewise for q_next
  double* gram;                        // gram_parts x rpad x rpad fp64 partial Gram matrices
  double* tmat;                        // rpad x rpad fp64 upper-triangular T, P = (M q) T
  double* wsum;                        // rpad x rpad fp64 summed Gram matrix, updated in place by
                                       // the blocked factorisation (r > 128 only; else unused)
  double* wdiag;                       // rpad fp64: its diagonal before the factorisation (r > 128)
  float* p2;                           // m x rpad fp32: first-pass orthonormal factor, the input
                                       // of the second pass when one is needed
  int32_t* reorth;                     // 1: this step's factor needs a second pass
  // r > 128: M split once per step into bf16 halves for the two factor GEMMs
  uint16_t* mh; uint16_t* ml;          // mpad x npad_b: M (zero beyond m x n)
  uint16_t* qth; uint16_t* qtl;        // rpad_b x npad_b: q^T (zero beyond r x n)
  int32_t npad_b;                      // n rounded up to 64
  int32_t rpad_b;                      // rpad rounded up to a whole GEMM tile (128)
  // optimizer state (psgd_adam_attach; NULL until attached)
  void* param;       int64_t ld_param; // m x n parameter, type of the attachment
  uint16_t* m1;      uint16_t* m2;     // m x n 16-bit moments (leading dimension n)
  uint32_t p_bytes, mo_bytes;          // byte spans of param and of each moment (< 2^31)
};

// One item of the global-norm reduction: a contiguous fp32 range of a gradient (q_next of a
// compressed matrix, or a pass-through gradient), at most kNormItem elements.
struct NormItem {
  const float* ptr;
  int64_t n;
};
constexpr int64_t kNormItem = 65536;
// An fp32 tensor updated by the pass-through Adam kernel.
struct AdamTensor {
  float* param; float* m1; float* m2; const float* grad; int64_t n;
};
constexpr int kAdamTensors = 16;          // tensors per launch (kernel argument)
struct AdamTensorArgs {
  AdamTensor t[kAdamTensors];
  int count;
};

// Scalars of one Adam step for the fused decompression (hyperparameters by value; the step
// count and the clipping factor stay on the device).
struct AdamArgs {
  float lr, beta1, beta2, eps, weight_decay;
  const int32_t* step;     // t after this step's increment
  const float* clip;       // clipping factor c
};

// One unit of grouped work: a matrix and a block of it. Unused slots have mat = -1.
struct Work {
  int32_t mat;
  int32_t a;   // first row (K1, Gram, apply, decompress) or first column (K2)
  int32_t b;   // rank chunk (K1, K2) / first column (decompress) / Gram part
  int32_t c;
};

// ------------------------------------------------------------------------------------------
// helpers
// ------------------------------------------------------------------------------------------
// Workgroups are dispatched round-robin over the 8 XCDs. Remap so that each XCD walks one
// contiguous range of the work list (neighbouring blocks of one matrix share its factor in L2).
// `grid` is a multiple of 8.
__device__ __forceinline__ int xcd_remap(int bid, int grid) {
  const int per = grid >> 3;
  return (bid & (kXcds - 1)) * per + (bid >> 3);
}

// class mask: signalling NaN | quiet NaN | -inf | +inf
__device__ __forceinline__ bool nonfinite(float x) { return __builtin_amdgcn_classf(x, 1 | 2 | 4 | 512); }

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f64x4 mfma_f64(double a, double b, f64x4 c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

// x = hi + lo with hi, lo bfloat16 (round to nearest even); |x - hi - lo| <= 2^-17 |x|.
__device__ __forceinline__ void split_bf16(const f32x8& x, bf16x8& hi, bf16x8& lo) {
  hi = __builtin_convertvector(x, bf16x8);
  const f32x8 rest = x - __builtin_convertvector(hi, f32x8);
  lo = __builtin_convertvector(rest, bf16x8);
}

// Power-of-two exponent e with |x| * 2^e in [2^13, 2^14) for the largest |x| of a row; 0 for
// rows that are all zero or not finite.
__device__ __forceinline__ int fp16_row_exponent(float amax) {
  if (!(amax > 0.0f) || nonfinite(amax)) return 0;
  int ex;
  (void)frexpf(amax, &ex);           // amax = f * 2^ex, f in [0.5, 1)
  return 14 - ex;
}

// 16-bit patterns of float values
__device__ __forceinline__ uint16_t bf16_bits(__bf16 v) { return __builtin_bit_cast(uint16_t, v); }
__device__ __forceinline__ uint16_t f16_bits(_Float16 v) { return __builtin_bit_cast(uint16_t, v); }

// Load 8 gradient elements as fp32 (16-byte aligned source of the gradient dtype).
template <int GT> struct GradIO;
template <> struct GradIO<G_F16> {
  static constexpr int kBytes = 2;
  __device__ __forceinline__ static f32x8 load8(const GLOBAL char* base) {
    const u32x4 raw = *gcast<u32x4>(base);
    return __builtin_convertvector(__builtin_bit_cast(f16x8, raw), f32x8);
  }
  __device__ __forceinline__ static f32x4 load4(const GLOBAL char* base) {
    const u32x2 raw = *gcast<u32x2>(base);
    return __builtin_convertvector(__builtin_bit_cast(f16x4, raw), f32x4);
  }
};
template <> struct GradIO<G_BF16> {
  static constexpr int kBytes = 2;
  __device__ __forceinline__ static f32x8 load8(const GLOBAL char* base) {
    const u32x4 raw = *gcast<u32x4>(base);
    return __builtin_convertvector(__builtin_bit_cast(bf16x8, raw), f32x8);
  }
  __device__ __forceinline__ static f32x4 load4(const GLOBAL char* base) {
    const u32x2 raw = *gcast<u32x2>(base);
    return __builtin_convertvector(__builtin_bit_cast(bf16x4, raw), f32x4);
  }
};
template <> struct GradIO<G_F32> {
  static constexpr int kBytes = 4;
  __device__ __forceinline__ static f32x8 load8(const GLOBAL char* base) {
    const f32x4 a = gcast<f32x4>(base)[0];
    const f32x4 b = gcast<f32x4>(base)[1];
    return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
  __device__ __forceinline__ static f32x4 load4(const GLOBAL char* base) {
    return *gcast<f32x4>(base);
  }
};

__device__ __forceinline__ f32x8 load_f32x8(const GLOBAL float* p) {
  const f32x4 a = gcast<f32x4>(p)[0];
  const f32x4 b = gcast<f32x4>(p)[1];
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

}  // namespace psgd

// ------------------------------------------------------------------------------------------
// host-side launchers (one translation unit per kernel family)
// ------------------------------------------------------------------------------------------
namespace psgd {
hipError_t launch_zero_u8(uint8_t* p, int n, hipStream_t s);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);          // bytes % 16 == 0
hipError_t launch_upload(void* dst, const void* src, size_t bytes, hipStream_t s);  // bytes % 4 == 0
hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t s);
hipError_t launch_ef_mq(int gt, int rtc, const DevMat* mats, const Work* work, int n_work,
                        const float* scale, uint8_t* flags, hipStream_t s);
hipError_t launch_gs_gram(int rt, bool big, int pass, const DevMat* mats, const Work* work, int n_work, hipStream_t s);
hipError_t launch_gs_reduce(int pass, const DevMat* mats, const Work* work, int n_work, hipStream_t s);
hipError_t launch_gs_factor(int pass, const DevMat* mats, const Work* work, int n_work, hipStream_t s);
hipError_t launch_gs_fdiag(int pass, int kb, const DevMat* mats, const Work* work, int n_work, hipStream_t s);
hipError_t launch_gs_bgemm(int pass, int kb, int phase, const DevMat* mats, const Work* work, int n_work,
                           hipStream_t s);
hipError_t launch_gs_apply(int rt, bool big, int pass, const DevMat* mats, const Work* work, int n_work, hipStream_t s);
hipError_t launch_split3(const DevMat* mats, const Work* work, int n_work, hipStream_t s);
hipError_t launch_mtp(int gt, int rtc, const DevMat* mats, const Work* work, int n_work,
                      const float* scale, hipStream_t s);
hipError_t launch_decompress(int gt, bool presplit, const DevMat* mats, const Work* work, int n_work,
                             const float* scale, const int32_t* skip, int64_t* counters, hipStream_t s);
hipError_t launch_sqnorm(const NormItem* items, int n_items, double* partial, hipStream_t s);
hipError_t launch_adam_finalize(const double* partial, int n, float max_norm, const int32_t* skip,
                                int32_t* step, float* norm_out, hipStream_t s);
hipError_t launch_adam_f32(const AdamTensor* ts, int n, const AdamArgs& aa, const int32_t* skip,
                           hipStream_t s);
hipError_t launch_decompress_adam(int gt, int pt, bool presplit, const DevMat* mats, const Work* work, int n_work,
                                  const float* scale, const int32_t* skip, const AdamArgs& aa,
                                  int64_t* counters, hipStream_t s);
struct PassList;
int big_split_tile();
int big_gemm_tile_m();
int big_gemm_tile_n();
hipError_t launch_split_m(int gt, const DevMat* mats, const Work* work, int n_work, const float* scale,
                          uint8_t* flags, hipStream_t s);
hipError_t launch_split_qt(const DevMat* mats, const Work* work, int n_work, hipStream_t s);
hipError_t launch_gemm_nt(const DevMat* mats, const Work* work, int n_work, bool a_k_outer, hipStream_t s);
hipError_t launch_block_enter(int dt, const float* dx, int64_t n, const float* scale, uint16_t* out,
                              hipStream_t s);
hipError_t launch_block_exit(int dt, float* dx, const uint16_t* g, int64_t n, const float* scale,
                             uint8_t* flag, hipStream_t s);
hipError_t launch_block_exit_enter(int dt, float* dx, const uint16_t* g, int64_t n, const float* scale_exit,
                                   const float* scale_enter, uint16_t* out, uint8_t* flag, hipStream_t s);
hipError_t launch_check_finite(const uint8_t* flags, int n_flags, const float* scale, int n_scale,
                               const float* const* pass_ptr, const int64_t* pass_n, int n_pass,
                               int32_t* skip, hipStream_t s);
}  // namespace psgd
