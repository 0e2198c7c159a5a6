// K1: fused error-feedback accumulate, P = M Q and the per-matrix non-finite flag.
//
// M = s_b * G + E is formed in fp32 registers and never stored. The error buffer and its
// finite checks come from "Zero-Shot Text-to-Image Generation — 中文验证版" (section 证据);
// the per-resblock multiplier s_b reflects per-resblock gradient scaling (same card, section
// 方法适配). The product is a tall-skinny GEMM on gfx950 MFMA (v_mfma_f32_16x16x32_bf16)
// with fp32 accumulation. Each operand is split into two bfloat16 halves, x = hi + lo, and
// three products hi*hi + hi*lo + lo*hi keep the result within about 2^-16 of fp32 products
// while the kernel stays bound by HBM bandwidth.
//
// Data flow per workgroup (a block of rows of one matrix, one rank chunk):
//   * every lane streams its own MFMA A-fragments straight from HBM: 8 consecutive columns of
//     one row of G (16 B of fp16) and of E (32 B), so no LDS round trip is needed for M;
//   * the shared operand, Q^T split into bf16 hi/lo (prepared once per step), is staged in LDS
//     32 columns of k at a time and double-buffered;
//   * the flag test runs on M (one class test per element); only when M is non-finite are the
//     inputs G and E themselves examined, so the flag is exactly "G or E holds inf/NaN".
#include "psgd_internal.h"

namespace psgd {
namespace {

constexpr int K1_RA = 2;     // 16-row tiles per wave
constexpr int K1_W = 4;      // waves per workgroup
constexpr int K1_ROWS = K1_RA * 16 * K1_W;
constexpr int LDS_K = 40;    // 32 k values + 8 padding (bf16 elements per LDS row)

template <int GT> struct Raw8;
template <> struct Raw8<G_F16> {
  u32x4 v;
  __device__ __forceinline__ void load(const void* p) { v = *reinterpret_cast<const u32x4*>(p); }
  __device__ __forceinline__ void zero() { v = u32x4{0, 0, 0, 0}; }
  __device__ __forceinline__ f32x8 f32() const { return __builtin_convertvector(__builtin_bit_cast(f16x8, v), f32x8); }
};
template <> struct Raw8<G_BF16> {
  u32x4 v;
  __device__ __forceinline__ void load(const void* p) { v = *reinterpret_cast<const u32x4*>(p); }
  __device__ __forceinline__ void zero() { v = u32x4{0, 0, 0, 0}; }
  __device__ __forceinline__ f32x8 f32() const { return __builtin_convertvector(__builtin_bit_cast(bf16x8, v), f32x8); }
};
template <> struct Raw8<G_F32> {
  f32x8 v;
  __device__ __forceinline__ void load(const void* p) { v = load_f32x8(reinterpret_cast<const float*>(p)); }
  __device__ __forceinline__ void zero() { v = f32x8{0, 0, 0, 0, 0, 0, 0, 0}; }
  __device__ __forceinline__ f32x8 f32() const { return v; }
};

template <int GT, int RTC>
__global__ __launch_bounds__(K1_W * kWave)
void k_ef_mq(const DevMat* __restrict__ mats, const Work* __restrict__ work,
             const float* __restrict__ scale, uint8_t* __restrict__ flags)
{
  const Work wi = work[xcd_remap(blockIdx.x, gridDim.x)];
  if (wi.mat < 0) return;
  const DevMat& d = mats[wi.mat];
  const int m = d.m, n = d.n, npad = d.npad, rpad = d.rpad;
  const char* __restrict__ G = reinterpret_cast<const char*>(d.grad);
  const float* __restrict__ E = d.err;
  const int64_t ldg = d.ld_grad, lde = d.ld_err;
  const uint16_t* __restrict__ qth = d.qt_hi;
  const uint16_t* __restrict__ qtl = d.qt_lo;
  const float s = scale[d.block];

  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int c = lane & 15, g = lane >> 4;
  const int row0 = wi.a + wv * (K1_RA * 16);
  const int rc0 = wi.b * RTC * 16;

  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][RTC * 16][LDS_K];

  // Q^T chunk staging: RTC*16 rank rows x 32 k x {hi, lo}, in 16-byte units.
  constexpr int UNITS = RTC * 16 * 4 * 2;
  constexpr int THREADS = K1_W * kWave;
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
        const uint16_t* src = (arr ? qtl : qth) + (int64_t)(rc0 + rr) * npad + k0 + 8 * q4;
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

  Raw8<GT> gcur[K1_RA];
  f32x8 ecur[K1_RA];
  auto load_m = [&](int k0, Raw8<GT>* gq, f32x8* eq) {
    const int col = k0 + 8 * g;
#pragma unroll
    for (int a = 0; a < K1_RA; ++a) {
      const int row = row0 + a * 16 + c;
      if (row < m && col < n) {
        gq[a].load(G + ((int64_t)row * ldg + col) * GradIO<GT>::kBytes);
        eq[a] = load_f32x8(E + (int64_t)row * lde + col);
      } else {
        gq[a].zero();
        eq[a] = f32x8{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
  };

  f32x4 acc[K1_RA][RTC];
#pragma unroll
  for (int a = 0; a < K1_RA; ++a)
#pragma unroll
    for (int cc = 0; cc < RTC; ++cc) acc[a][cc] = f32x4{0, 0, 0, 0};
  bool bad = false;

  const int nsteps = npad / 32;
  load_stage(0);
  store_stage(0);
  load_m(0, gcur, ecur);
  __syncthreads();

  for (int ks = 0; ks < nsteps; ++ks) {
    const int buf = ks & 1;
    const bool more = ks + 1 < nsteps;
    Raw8<GT> gnxt[K1_RA];
    f32x8 enxt[K1_RA];
    if (more) {
      load_stage((ks + 1) * 32);
      load_m((ks + 1) * 32, gnxt, enxt);
    }

    bf16x8 ah[K1_RA], al[K1_RA];
#pragma unroll
    for (int a = 0; a < K1_RA; ++a) {
      const f32x8 gf = gcur[a].f32();
      f32x8 mv;
      bool mb = false;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        mv[e] = __builtin_fmaf(s, gf[e], ecur[a][e]);
        mb |= nonfinite(mv[e]);
      }
      if (mb) {
        // rare: decide on the inputs, not on M (M may also be inf through s or overflow)
#pragma unroll
        for (int e = 0; e < 8; ++e) bad |= nonfinite(gf[e]) || nonfinite(ecur[a][e]);
      }
      split_bf16(mv, ah[a], al[a]);
    }

#pragma unroll
    for (int cc = 0; cc < RTC; ++cc) {
      const bf16x8 bh = *reinterpret_cast<const bf16x8*>(&lds[buf][0][cc * 16 + c][8 * g]);
      const bf16x8 bl = *reinterpret_cast<const bf16x8*>(&lds[buf][1][cc * 16 + c][8 * g]);
#pragma unroll
      for (int a = 0; a < K1_RA; ++a) {
        acc[a][cc] = mfma_bf16(ah[a], bh, acc[a][cc]);
        acc[a][cc] = mfma_bf16(ah[a], bl, acc[a][cc]);
        acc[a][cc] = mfma_bf16(al[a], bh, acc[a][cc]);
      }
    }

    if (more) {
      store_stage(buf ^ 1);
#pragma unroll
      for (int a = 0; a < K1_RA; ++a) { gcur[a] = gnxt[a]; ecur[a] = enxt[a]; }
    }
    __syncthreads();
  }

  // C layout of v_mfma_f32_16x16x32: lane holds rows 4g..4g+3, column c of the 16x16 tile.
  float* __restrict__ praw = d.p_raw;
#pragma unroll
  for (int a = 0; a < K1_RA; ++a)
#pragma unroll
    for (int cc = 0; cc < RTC; ++cc)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = row0 + a * 16 + 4 * g + i;
        if (row < m) praw[(int64_t)row * rpad + rc0 + cc * 16 + c] = acc[a][cc][i];
      }
  if (bad) flags[wi.mat] = 1;
}

template <int GT>
hipError_t launch_gt(int rtc, dim3 grid, dim3 block, hipStream_t s, const DevMat* mats,
                     const Work* work, const float* scale, uint8_t* flags) {
  switch (rtc) {
#define CASE(R) case R: k_ef_mq<GT, R><<<grid, block, 0, s>>>(mats, work, scale, flags); break;
    CASE(1) CASE(2) CASE(3) CASE(4) CASE(5) CASE(6) CASE(7) CASE(8)
#undef CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int ef_mq_rows_per_block() { return K1_ROWS; }

hipError_t launch_ef_mq(int gt, int rtc, const DevMat* mats, const Work* work, int n_work,
                        const float* scale, uint8_t* flags, hipStream_t s) {
  if (n_work <= 0) return hipSuccess;
  const dim3 grid(n_work), block(K1_W * kWave);
  switch (gt) {
    case G_F16: return launch_gt<G_F16>(rtc, grid, block, s, mats, work, scale, flags);
    case G_BF16: return launch_gt<G_BF16>(rtc, grid, block, s, mats, work, scale, flags);
    case G_F32: return launch_gt<G_F32>(rtc, grid, block, s, mats, work, scale, flags);
  }
  return hipErrorInvalidValue;
}

}  // namespace psgd
