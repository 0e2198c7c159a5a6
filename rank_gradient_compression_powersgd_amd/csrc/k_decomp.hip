// K3: decompression D = P Q'^T with fp32-accurate products, and the error-feedback write-back
// E = M - D with M = s_b G + E recomputed; optional D output.
//
// "Zero-Shot Text-to-Image Generation — 中文验证版" (section 证据) asks for 32-bit products in
// the decompressed gradient. Both factors were stored as fp16 hi + lo pairs of rows scaled by
// powers of two (|x - hi - lo| <= 2^-22 |x|), and three fp16 MFMA products (hi*hi + hi*lo +
// lo*hi) with fp32 accumulation reproduce fp32 products to about 2^-21. The power-of-two row
// scales are removed exactly with ldexp.
//
// The tile is computed transposed, D^T = Q' P^T. In that form the MFMA C layout gives every
// lane 4 consecutive columns of one row of D, so the G/E/out traffic is 8- and 16-byte vector
// accesses along rows.
//
// Skip: the device-side skip word is read first. A skipped step zeroes the error buffer over
// the tile and writes nothing else (the error buffer is zeroed on non-finite values: Korean
// summary of the paper, section "Distributed Optimization").
#include "psgd_internal.h"

namespace psgd {
namespace {

constexpr int K3_WM = 2, K3_WN = 2;      // waves along m and n; wave tile 64 x 64
constexpr int K3_TM = K3_WM * 64, K3_TN = K3_WN * 64;
constexpr int K3_THREADS = K3_WM * K3_WN * kWave;
constexpr int LDS_K = 40;                // fp16 elements per LDS row (32 + 8 padding)

template <int GT>
__global__ __launch_bounds__(K3_THREADS)
void k_decomp(const DevMat* __restrict__ mats, const Work* __restrict__ work,
              const float* __restrict__ scale, const int32_t* __restrict__ skip)
{
  const Work wi = work[xcd_remap(blockIdx.x, gridDim.x)];
  if (wi.mat < 0) return;
  const DevMat& d = mats[wi.mat];
  const int m = d.m, n = d.n, kpad3 = d.kpad3;
  const int m0 = wi.a, n0 = wi.b;
  float* __restrict__ E = d.err;
  const int64_t lde = d.ld_err;

  if (*skip != 0) {
    // zero E over the tile: 2 threads per row, 64 columns each
    const int row = m0 + threadIdx.x / 2;
    if (row < m) {
      const int cb = n0 + (threadIdx.x & 1) * 64;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int col = cb + 4 * j;
        if (col < n) *reinterpret_cast<f32x4*>(E + (int64_t)row * lde + col) = f32x4{0, 0, 0, 0};
      }
    }
    return;
  }

  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int wm = wv % K3_WM, wn = wv / K3_WM;
  const int c = lane & 15, g = lane >> 4;

  __shared__ __attribute__((aligned(16))) uint16_t ldq[2][2][K3_TN][LDS_K];
  __shared__ __attribute__((aligned(16))) uint16_t ldp[2][2][K3_TM][LDS_K];

  // staging: (K3_TN + K3_TM) rows x 32 k x {hi, lo} in 16-byte units
  constexpr int UNITS = (K3_TN + K3_TM) * 4 * 2;
  constexpr int UPT = UNITS / K3_THREADS;
  static_assert(UNITS % K3_THREADS == 0, "staging units");
  u32x4 stage[UPT];
  auto load_stage = [&](int k0) {
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      const int u = threadIdx.x + j * K3_THREADS;
      const bool isq = u < K3_TN * 8;
      const int v = isq ? u : u - K3_TN * 8;
      const int arr = v & 1, q4 = (v >> 1) & 3, rr = v >> 3;
      const int row = (isq ? n0 : m0) + rr;
      const int lim = isq ? n : m;
      const uint16_t* base = isq ? (arr ? d.q3_lo : d.q3_hi) : (arr ? d.p3_lo : d.p3_hi);
      stage[j] = row < lim ? *reinterpret_cast<const u32x4*>(base + (int64_t)row * kpad3 + k0 + 8 * q4)
                           : u32x4{0, 0, 0, 0};
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      const int u = threadIdx.x + j * K3_THREADS;
      const bool isq = u < K3_TN * 8;
      const int v = isq ? u : u - K3_TN * 8;
      const int arr = v & 1, q4 = (v >> 1) & 3, rr = v >> 3;
      uint16_t* dst = isq ? &ldq[buf][arr][rr][8 * q4] : &ldp[buf][arr][rr][8 * q4];
      *reinterpret_cast<u32x4*>(dst) = stage[j];
    }
  };

  f32x4 acc[4][4];     // [n-tile][m-tile]
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0, 0, 0, 0};

  const int nsteps = kpad3 / 32;
  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int ks = 0; ks < nsteps; ++ks) {
    const int buf = ks & 1;
    const bool more = ks + 1 < nsteps;
    if (more) load_stage((ks + 1) * 32);
    f16x8 bh[4], bl[4];
#pragma unroll
    for (int im = 0; im < 4; ++im) {
      bh[im] = *reinterpret_cast<const f16x8*>(&ldp[buf][0][wm * 64 + im * 16 + c][8 * g]);
      bl[im] = *reinterpret_cast<const f16x8*>(&ldp[buf][1][wm * 64 + im * 16 + c][8 * g]);
    }
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) {
      const f16x8 ah = *reinterpret_cast<const f16x8*>(&ldq[buf][0][wn * 64 + jn * 16 + c][8 * g]);
      const f16x8 al = *reinterpret_cast<const f16x8*>(&ldq[buf][1][wn * 64 + jn * 16 + c][8 * g]);
#pragma unroll
      for (int im = 0; im < 4; ++im) {
        acc[jn][im] = mfma_f16(ah, bh[im], acc[jn][im]);
        acc[jn][im] = mfma_f16(ah, bl[im], acc[jn][im]);
        acc[jn][im] = mfma_f16(al, bh[im], acc[jn][im]);
      }
    }
    if (more) store_stage(buf ^ 1);
    __syncthreads();
  }

  // acc[jn][im]: lane holds D[m = m0 + wm*64 + im*16 + c][n = n0 + wn*64 + jn*16 + 4g + {0..3}]
  const char* __restrict__ G = reinterpret_cast<const char*>(d.grad);
  const int64_t ldg = d.ld_grad, ldo = d.ld_out;
  float* __restrict__ out = d.out;
  const float s = scale[d.block];
#pragma unroll
  for (int im = 0; im < 4; ++im) {
    const int row = m0 + wm * 64 + im * 16 + c;
    if (row >= m) continue;
    const int ep = d.p3_exp[row];
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) {
      const int col = n0 + wn * 64 + jn * 16 + 4 * g;
      if (col >= n) continue;
      const f32x4 gf = GradIO<GT>::load4(G + ((int64_t)row * ldg + col) * GradIO<GT>::kBytes);
      float* ep4 = E + (int64_t)row * lde + col;
      const f32x4 ev = *reinterpret_cast<const f32x4*>(ep4);
      f32x4 dv, en;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dv[i] = ldexpf(acc[jn][im][i], -(ep + d.q3_exp[col + i]));
        en[i] = __builtin_fmaf(s, gf[i], ev[i]) - dv[i];
      }
      *reinterpret_cast<f32x4*>(ep4) = en;
      if (out) *reinterpret_cast<f32x4*>(out + (int64_t)row * ldo + col) = dv;
    }
  }
}

// q <- q_next when the step is not skipped
__global__ __launch_bounds__(256)
void k_commit_q(const DevMat* __restrict__ mats, const Work* __restrict__ work,
                const int32_t* __restrict__ skip)
{
  const Work wi = work[blockIdx.x];
  if (wi.mat < 0 || *skip != 0) return;
  const DevMat& d = mats[wi.mat];
  const int64_t total = (int64_t)d.n * d.r;
  const int64_t beg = (int64_t)wi.a * 4096;
  const int64_t end = beg + 4096 < total ? beg + 4096 : total;
  for (int64_t i = beg + threadIdx.x; i < end; i += 256) d.q[i] = d.q_next[i];
}

template <int GT>
hipError_t launch_gt(dim3 grid, hipStream_t s, const DevMat* mats, const Work* work,
                     const float* scale, const int32_t* skip) {
  k_decomp<GT><<<grid, dim3(K3_THREADS), 0, s>>>(mats, work, scale, skip);
  return hipGetLastError();
}

}  // namespace

int decomp_tile_m() { return K3_TM; }
int decomp_tile_n() { return K3_TN; }

hipError_t launch_decompress(int gt, const DevMat* mats, const Work* work, int n_work,
                             const float* scale, const int32_t* skip, hipStream_t s) {
  if (n_work <= 0) return hipSuccess;
  const dim3 grid(n_work);
  switch (gt) {
    case G_F16: return launch_gt<G_F16>(grid, s, mats, work, scale, skip);
    case G_BF16: return launch_gt<G_BF16>(grid, s, mats, work, scale, skip);
    case G_F32: return launch_gt<G_F32>(grid, s, mats, work, scale, skip);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_commit_q(const DevMat* mats, const Work* work, int n_work, const int32_t* skip,
                           hipStream_t s) {
  if (n_work <= 0) return hipSuccess;
  k_commit_q<<<dim3(n_work), dim3(256), 0, s>>>(mats, work, skip);
  return hipGetLastError();
}

}  // namespace psgd
