// K2: Q' = M^T P, the next warm start, with M = s_b G + E recomputed from G and E.
//
// The factor product comes from the P·Q decomposition of the Korean summary of the DALL·E
// paper (section "Distributed Optimization"). The contraction runs over the m rows of M, so an
// MFMA B-fragment needs 8 consecutive rows of one column. Reading that directly would
// stride through memory. Instead every lane loads an 8-row x 4-column block of M: each load
// is 4 consecutive columns of one row, and a wave instruction covers 4 rows x 64 columns,
// contiguous along the row. The lane then holds the B-fragments of 4 column tiles at once.
// Column tile t of a wave holds columns {4j + t : j = 0..15} of its 64-column strip.
// The shared operand P^T, split into bf16 hi/lo by the orthonormalisation kernel, is staged
// in LDS 32 rows of m at a time and double-buffered. Products use the same three-term bf16
// split as K1.
//
// Epilogue: Q' is written in fp32 (the caller's q_next). When the whole rank fits one chunk
// the kernel also writes the decompression operand: each row of Q' scaled by a power of two
// (so its largest entry lies in [2^13, 2^14)) and split into fp16 hi + lo.
#include "psgd_internal.h"

namespace psgd {
namespace {

constexpr int K2_W = 4;       // waves per workgroup, 64 columns each
constexpr int LDS_K = 40;

template <int GT> struct Raw4;
template <> struct Raw4<G_F16> {
  u32x2 v;
  __device__ __forceinline__ void load(const void* p) { v = *reinterpret_cast<const u32x2*>(p); }
  __device__ __forceinline__ void zero() { v = u32x2{0, 0}; }
  __device__ __forceinline__ f32x4 f32() const { return __builtin_convertvector(__builtin_bit_cast(f16x4, v), f32x4); }
};
template <> struct Raw4<G_BF16> {
  u32x2 v;
  __device__ __forceinline__ void load(const void* p) { v = *reinterpret_cast<const u32x2*>(p); }
  __device__ __forceinline__ void zero() { v = u32x2{0, 0}; }
  __device__ __forceinline__ f32x4 f32() const { return __builtin_convertvector(__builtin_bit_cast(bf16x4, v), f32x4); }
};
template <> struct Raw4<G_F32> {
  f32x4 v;
  __device__ __forceinline__ void load(const void* p) { v = *reinterpret_cast<const f32x4*>(p); }
  __device__ __forceinline__ void zero() { v = f32x4{0, 0, 0, 0}; }
  __device__ __forceinline__ f32x4 f32() const { return v; }
};

template <int GT, int RTC>
__global__ __launch_bounds__(K2_W * kWave)
void k_mtp(const DevMat* __restrict__ mats, const Work* __restrict__ work,
           const float* __restrict__ scale)
{
  const Work wi = work[xcd_remap(blockIdx.x, gridDim.x)];
  if (wi.mat < 0) return;
  const DevMat& d = mats[wi.mat];
  const int m = d.m, n = d.n, mpad = d.mpad, r = d.r, rpad = d.rpad;
  const char* __restrict__ G = reinterpret_cast<const char*>(d.grad);
  const float* __restrict__ E = d.err;
  const int64_t ldg = d.ld_grad, lde = d.ld_err;
  const uint16_t* __restrict__ pth = d.pt_hi;
  const uint16_t* __restrict__ ptl = d.pt_lo;
  const float s = scale[d.block];

  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int c = lane & 15, g = lane >> 4;
  const int colbase = wi.a + wv * 64 + 4 * c;
  const bool colok = colbase < n;              // n % 8 == 0: 4-column groups are all in or out
  const int rc0 = wi.b * RTC * 16;

  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][RTC * 16][LDS_K];

  constexpr int UNITS = RTC * 16 * 4 * 2;
  constexpr int THREADS = K2_W * kWave;
  constexpr int UPT = (UNITS + THREADS - 1) / THREADS;
  u32x4 stage[UPT];
  auto load_stage = [&](int k0) {
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      const int u = threadIdx.x + j * THREADS;
      if (UNITS % THREADS == 0 || u < UNITS) {
        const int arr = u / (RTC * 64);
        const int rem = u - arr * (RTC * 64);
        const int rr = rem >> 2, q4 = rem & 3;
        const uint16_t* src = (arr ? ptl : pth) + (int64_t)(rc0 + rr) * mpad + k0 + 8 * q4;
        stage[j] = *reinterpret_cast<const u32x4*>(src);
      }
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      const int u = threadIdx.x + j * THREADS;
      if (UNITS % THREADS == 0 || u < UNITS) {
        const int arr = u / (RTC * 64);
        const int rem = u - arr * (RTC * 64);
        const int rr = rem >> 2, q4 = rem & 3;
        *reinterpret_cast<u32x4*>(&lds[buf][arr][rr][8 * q4]) = stage[j];
      }
    }
  };

  Raw4<GT> gcur[8];
  f32x4 ecur[8];
  auto load_m = [&](int k0, Raw4<GT>* gq, f32x4* eq) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int row = k0 + 8 * g + kk;
      if (colok && row < m) {
        gq[kk].load(G + ((int64_t)row * ldg + colbase) * GradIO<GT>::kBytes);
        eq[kk] = *reinterpret_cast<const f32x4*>(E + (int64_t)row * lde + colbase);
      } else {
        gq[kk].zero();
        eq[kk] = f32x4{0, 0, 0, 0};
      }
    }
  };

  f32x4 acc[RTC][4];
#pragma unroll
  for (int i = 0; i < RTC; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[i][t] = f32x4{0, 0, 0, 0};

  const int nsteps = mpad / 32;
  load_stage(0);
  store_stage(0);
  load_m(0, gcur, ecur);
  __syncthreads();

  for (int ks = 0; ks < nsteps; ++ks) {
    const int buf = ks & 1;
    const bool more = ks + 1 < nsteps;
    Raw4<GT> gnxt[8];
    f32x4 enxt[8];
    if (more) {
      load_stage((ks + 1) * 32);
      load_m((ks + 1) * 32, gnxt, enxt);
    }

    // B-fragments: tile t takes column t of every loaded row (k = 8g + kk).
    f32x8 mt[4];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const f32x4 gf = gcur[kk].f32();
#pragma unroll
      for (int t = 0; t < 4; ++t) mt[t][kk] = __builtin_fmaf(s, gf[t], ecur[kk][t]);
    }
    bf16x8 bh[4], bl[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) split_bf16(mt[t], bh[t], bl[t]);

#pragma unroll
    for (int i = 0; i < RTC; ++i) {
      const bf16x8 ah = *reinterpret_cast<const bf16x8*>(&lds[buf][0][i * 16 + c][8 * g]);
      const bf16x8 al = *reinterpret_cast<const bf16x8*>(&lds[buf][1][i * 16 + c][8 * g]);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        acc[i][t] = mfma_bf16(ah, bh[t], acc[i][t]);
        acc[i][t] = mfma_bf16(ah, bl[t], acc[i][t]);
        acc[i][t] = mfma_bf16(al, bh[t], acc[i][t]);
      }
    }

    if (more) {
      store_stage(buf ^ 1);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) { gcur[kk] = gnxt[kk]; ecur[kk] = enxt[kk]; }
    }
    __syncthreads();
  }

  // Output tile (i, t): lane holds Q'^T rows rc0 + 16i + 4g + {0..3}, i.e. Q'[colbase + t][..].
  if (!colok) return;
  float* __restrict__ qn = d.q_next;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int ncol = colbase + t;
#pragma unroll
    for (int i = 0; i < RTC; ++i) {
      const int rr = rc0 + i * 16 + 4 * g;
      float* dst = qn + (int64_t)ncol * r + rr;
      if (rr + 3 < r && (r & 3) == 0) {
        *reinterpret_cast<f32x4*>(dst) = acc[i][t];
      } else {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
          if (rr + ii < r) dst[ii] = acc[i][t][ii];
      }
    }
  }

  // Decompression operand (only when this chunk covers the whole padded rank).
  if (RTC * 16 != rpad) return;
  const int kpad3 = d.kpad3;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < RTC; ++i)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) amax = fmaxf(amax, fabsf(acc[i][t][ii]));
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    const int ex = fp16_row_exponent(amax);
    const int ncol = colbase + t;
    uint16_t* hi = d.q3_hi + (int64_t)ncol * kpad3;
    uint16_t* lo = d.q3_lo + (int64_t)ncol * kpad3;
#pragma unroll
    for (int i = 0; i < RTC; ++i) {
      const int rr = i * 16 + 4 * g;
      uint16_t h4[4], l4[4];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const float x = ldexpf(acc[i][t][ii], ex);
        const _Float16 h = (_Float16)x;
        h4[ii] = f16_bits(h);
        l4[ii] = f16_bits((_Float16)(x - (float)h));
      }
      *reinterpret_cast<u32x2*>(hi + rr) = u32x2{h4[0] | ((uint32_t)h4[1] << 16), h4[2] | ((uint32_t)h4[3] << 16)};
      *reinterpret_cast<u32x2*>(lo + rr) = u32x2{l4[0] | ((uint32_t)l4[1] << 16), l4[2] | ((uint32_t)l4[3] << 16)};
    }
    if (g == 0) d.q3_exp[ncol] = ex;
  }
}

template <int GT>
hipError_t launch_gt(int rtc, dim3 grid, dim3 block, hipStream_t s, const DevMat* mats,
                     const Work* work, const float* scale) {
  switch (rtc) {
#define CASE(R) case R: k_mtp<GT, R><<<grid, block, 0, s>>>(mats, work, scale); break;
    CASE(1) CASE(2) CASE(3) CASE(4) CASE(5) CASE(6) CASE(7) CASE(8)
#undef CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int mtp_cols_per_block() { return K2_W * 64; }

hipError_t launch_mtp(int gt, int rtc, const DevMat* mats, const Work* work, int n_work,
                      const float* scale, hipStream_t s) {
  if (n_work <= 0) return hipSuccess;
  const dim3 grid(n_work), block(K2_W * kWave);
  switch (gt) {
    case G_F16: return launch_gt<G_F16>(rtc, grid, block, s, mats, work, scale);
    case G_BF16: return launch_gt<G_BF16>(rtc, grid, block, s, mats, work, scale);
    case G_F32: return launch_gt<G_F32>(rtc, grid, block, s, mats, work, scale);
  }
  return hipErrorInvalidValue;
}

}  // namespace psgd
