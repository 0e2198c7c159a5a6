// Orthonormalisation of P = M Q: Gram-Schmidt in Gram-matrix form, batched over matrices.
//
// The pages only say that low-rank factors replace the gradient matrices; the factor P must be
// orthonormalised between the two products, and the plain reading is Gram-Schmidt, whose
// result is the thin-QR factor with a positive R diagonal. A column-by-column Gram-Schmidt
// over an m x r panel needs r dependent reductions over m rows. That is a long latency chain
// per matrix that one CU cannot hide, and it does not spread over CUs. Here the m-long
// reductions are done once, as the Gram matrix W = P^T P, and the Gram-Schmidt recurrence runs
// on the small r x r side:
//
//   gs_gram    W = P^T P per 256-row block, v_mfma_f64_16x16x4 (products of fp32 values are
//              exact in fp64); partial sums are added later in a fixed order (deterministic).
//   gs_factor  modified Gram-Schmidt carried out on coefficient vectors. Column j of the
//              result is P t_j. The inner products <q_i, v_j> and the norms ||v_j|| are read
//              from the running Gram matrix, which is updated as columns are projected out.
//              This gives the upper-triangular T with P T orthonormal, T = R^-1 of the thin
//              QR. fp64, one workgroup per matrix, W and T resident in LDS.
//              A column whose remaining squared norm is at most 2^-40 of its original squared
//              norm (or zero, or not finite) is dependent: its column of T is set to zero.
//   gs_apply   P_hat = P T with fp64 MFMA accumulation, then the stores the products need:
//              P_hat in fp32 (caller's p), P_hat^T split bf16 hi/lo for K2, and P_hat rows
//              scaled by a power of two and split fp16 hi/lo for the decompression kernel.
#include "psgd_internal.h"

namespace psgd {
namespace {

constexpr int GS_THREADS = 256;

// ------------------------------------------------------------------------------------------
// Gram partials
// ------------------------------------------------------------------------------------------
template <int RT>
__global__ __launch_bounds__(GS_THREADS)
void k_gs_gram(const DevMat* __restrict__ mats, const Work* __restrict__ work)
{
  const Work wi = work[xcd_remap(blockIdx.x, gridDim.x)];
  if (wi.mat < 0) return;
  const DevMat& d = mats[wi.mat];
  const int m = d.m, rpad = d.rpad;
  const GLOBAL float* __restrict__ P = gbl(d.p_raw);
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int c = lane & 15, g = lane >> 4;
  constexpr int NP = RT * (RT + 1) / 2;
  constexpr int NW = GS_THREADS / kWave;
  constexpr int PPW = (NP + NW - 1) / NW;

  f64x4 acc[PPW];
#pragma unroll
  for (int j = 0; j < PPW; ++j) acc[j] = f64x4{0, 0, 0, 0};

  const int row0 = wi.a;
  constexpr int KB = 4;                      // k steps (of 4 rows) whose loads are batched
  for (int ks = 0; ks < kGramRows / 4; ks += KB) {
    float v[KB][RT];
#pragma unroll
    for (int b = 0; b < KB; ++b) {
      const int row = row0 + 4 * (ks + b) + g;
      const int rr = row < m ? row : 0;
#pragma unroll
      for (int t = 0; t < RT; ++t) v[b][t] = P[(int64_t)rr * rpad + t * 16 + c];
      if (row >= m) {
#pragma unroll
        for (int t = 0; t < RT; ++t) v[b][t] = 0.0f;
      }
    }
    // lane supplies A[c][g] = P[row][ti*16 + c] and B[g][c] = P[row][tj*16 + c]
#pragma unroll
    for (int b = 0; b < KB; ++b) {
      int p = 0;
#pragma unroll
      for (int ti = 0; ti < RT; ++ti)
#pragma unroll
        for (int tj = ti; tj < RT; ++tj, ++p)
          if (p % NW == wv) acc[p / NW] = mfma_f64((double)v[b][ti], (double)v[b][tj], acc[p / NW]);
    }
  }

  // C layout of v_mfma_f64_16x16x4f64: lane 16g + c, register i holds C[g + 4i][c].
  GLOBAL double* __restrict__ out = gbl(d.gram) + (int64_t)wi.b * rpad * rpad;
  int p = 0;
#pragma unroll
  for (int ti = 0; ti < RT; ++ti)
#pragma unroll
    for (int tj = ti; tj < RT; ++tj, ++p)
      if (p % NW == wv) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          out[(int64_t)(ti * 16 + g + 4 * i) * rpad + tj * 16 + c] = acc[p / NW][i];
      }
}

// ------------------------------------------------------------------------------------------
// Gram-Schmidt on the Gram matrix (rpad <= 128)
// ------------------------------------------------------------------------------------------
constexpr int kPackMax = 128 * 129 / 2;

__device__ __forceinline__ int pidx(int i, int j, int rp) {   // packed upper, i <= j
  return i * rp - (i * (i - 1)) / 2 + (j - i);
}

constexpr int GSF_THREADS = 1024;     // 32 x 32 thread grid over the r x r problem

__global__ __launch_bounds__(GSF_THREADS)
void k_gs_factor(const DevMat* __restrict__ mats, const Work* __restrict__ work)
{
  const Work wi = work[blockIdx.x];
  if (wi.mat < 0) return;
  const DevMat& d = mats[wi.mat];
  const int rp = d.rpad;
  const int parts = d.gram_parts;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const GLOBAL double* __restrict__ gram = gbl(d.gram);
  GLOBAL double* __restrict__ tmat = gbl(d.tmat);

  __shared__ double W[kPackMax];
  __shared__ double T[kPackMax];
  __shared__ double diag0[128];
  __shared__ double rrow[128];

  // W = sum of the partial Gram matrices in part order; T = I.
  for (int i = ty; i < rp; i += 32) {
    const int base = i * rp - (i * (i - 1)) / 2 - i;
    for (int j = i + tx; j < rp; j += 32) {
      double sum = 0.0;
      for (int pt = 0; pt < parts; ++pt) sum += gram[((int64_t)pt * rp + i) * rp + j];
      W[base + j] = sum;
      T[base + j] = (i == j) ? 1.0 : 0.0;
    }
  }
  __syncthreads();
  if (threadIdx.x < rp) diag0[threadIdx.x] = W[pidx(threadIdx.x, threadIdx.x, rp)];
  __syncthreads();

  for (int j = 0; j < rp; ++j) {
    const double dj = W[pidx(j, j, rp)];
    const double d0 = diag0[j];
    const bool ok = (d0 > 0.0) && (dj > kDegenerate * d0) && (dj <= 1.0e300);
    const double inv = ok ? 1.0 / sqrt(dj) : 0.0;
    // r_jk = <q_j, v_k> = W[j][k] / ||v_j||; t_j = u_j / ||v_j||
    const int k1 = j + 1 + (int)threadIdx.x;
    if (k1 < rp) rrow[k1] = W[pidx(j, k1, rp)] * inv;
    if ((int)threadIdx.x <= j) T[pidx(threadIdx.x, j, rp)] *= inv;
    __syncthreads();
    // v_k -= r_jk q_j for k > j: Gram update and coefficient update
    for (int k = j + 1 + ty; k < rp; k += 32) {
      const int base = k * rp - (k * (k - 1)) / 2 - k;
      const double rk = rrow[k];
      for (int l = k + ((tx - (k - j - 1)) & 31); l < rp; l += 32) W[base + l] -= rk * rrow[l];
    }
    for (int i = ty; i <= j; i += 32) {
      const int base = i * rp - (i * (i - 1)) / 2 - i;
      const double tij = T[base + j];
      for (int k = j + 1 + tx; k < rp; k += 32) T[base + k] -= rrow[k] * tij;
    }
    __syncthreads();
  }

  for (int i = ty; i < rp; i += 32) {
    const int base = i * rp - (i * (i - 1)) / 2 - i;
    for (int j = tx; j < rp; j += 32) tmat[(int64_t)i * rp + j] = (j >= i) ? T[base + j] : 0.0;
  }
}

// ------------------------------------------------------------------------------------------
// P_hat = P T and the operand layouts of the two products that follow
// ------------------------------------------------------------------------------------------
constexpr int GSA_RA = 2;                          // 16-row tiles per wave
constexpr int GSA_ROWS = GSA_RA * 16 * (GS_THREADS / kWave);   // 128 rows per workgroup

template <int RT>
__global__ __launch_bounds__(GS_THREADS)
void k_gs_apply(const DevMat* __restrict__ mats, const Work* __restrict__ work)
{
  const Work wi = work[xcd_remap(blockIdx.x, gridDim.x)];
  if (wi.mat < 0) return;
  const DevMat& d = mats[wi.mat];
  const int m = d.m, r = d.r, rpad = d.rpad, mpad = d.mpad, kpad3 = d.kpad3;
  const GLOBAL float* __restrict__ P = gbl(d.p_raw);
  const GLOBAL double* __restrict__ Tm = gbl(d.tmat);
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int c = lane & 15, g = lane >> 4;
  const int row0 = wi.a;                   // this workgroup's GSA_ROWS rows
  constexpr int SP = RT * 16 + 1;          // LDS row pitch (floats); odd, so column reads spread over banks

  __shared__ float S[GSA_ROWS * SP];
  __shared__ int sexp[GSA_ROWS];

  f64x4 acc[GSA_RA][RT];
#pragma unroll
  for (int a = 0; a < GSA_RA; ++a)
#pragma unroll
    for (int t = 0; t < RT; ++t) acc[a][t] = f64x4{0, 0, 0, 0};

  // P_hat = P T with T upper triangular: k tile kt only feeds column tiles tj >= kt.
#pragma unroll
  for (int kt = 0; kt < RT; ++kt) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int k = kt * 16 + ks * 4 + g;
      double av[GSA_RA];
#pragma unroll
      for (int a = 0; a < GSA_RA; ++a) {
        const int rowA = row0 + (wv * GSA_RA + a) * 16 + c;     // A-fragment row of this lane
        av[a] = rowA < m ? (double)P[(int64_t)rowA * rpad + k] : 0.0;
      }
#pragma unroll
      for (int tj = kt; tj < RT; ++tj) {
        const double b = Tm[(int64_t)k * rpad + tj * 16 + c];
#pragma unroll
        for (int a = 0; a < GSA_RA; ++a) acc[a][tj] = mfma_f64(av[a], b, acc[a][tj]);
      }
    }
  }

  // C layout of v_mfma_f64_16x16x4f64: lane 16g + c, register i holds C[g + 4i][c].
#pragma unroll
  for (int a = 0; a < GSA_RA; ++a)
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S[((wv * GSA_RA + a) * 16 + g + 4 * i) * SP + t * 16 + c] = (float)acc[a][t][i];
  __syncthreads();

  // (a) fp32 P_hat, m x r row-major
  GLOBAL float* __restrict__ pout = gbl(d.p);
  for (int idx = threadIdx.x; idx < GSA_ROWS * r; idx += GS_THREADS) {
    const int rr = idx / r, cc = idx - rr * r;
    if (row0 + rr < m) pout[(int64_t)(row0 + rr) * r + cc] = S[rr * SP + cc];
  }
  // (b) P_hat^T split bf16 hi/lo, rpad x mpad: 8 consecutive rows of one column per store
  GLOBAL uint16_t* __restrict__ pth = gbl(d.pt_hi);
  GLOBAL uint16_t* __restrict__ ptl = gbl(d.pt_lo);
  for (int idx = threadIdx.x; idx < rpad * (GSA_ROWS / 8); idx += GS_THREADS) {
    const int col = idx / (GSA_ROWS / 8), r8 = (idx % (GSA_ROWS / 8)) * 8;
    if (row0 + r8 >= mpad) continue;
    uint32_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x0 = S[(r8 + 2 * e) * SP + col], x1 = S[(r8 + 2 * e + 1) * SP + col];
      const __bf16 h0 = (__bf16)x0, h1 = (__bf16)x1;
      h[e] = bf16_bits(h0) | ((uint32_t)bf16_bits(h1) << 16);
      l[e] = bf16_bits((__bf16)(x0 - (float)h0)) | ((uint32_t)bf16_bits((__bf16)(x1 - (float)h1)) << 16);
    }
    *gcast<u32x4>(pth + (int64_t)col * mpad + row0 + r8) = u32x4{h[0], h[1], h[2], h[3]};
    *gcast<u32x4>(ptl + (int64_t)col * mpad + row0 + r8) = u32x4{l[0], l[1], l[2], l[3]};
  }
  // (c) rows scaled by 2^e (largest entry in [2^13, 2^14)) and split fp16 hi/lo, m x kpad3
  if (threadIdx.x < GSA_ROWS) {
    float amax = 0.0f;
    for (int cc = 0; cc < RT * 16; ++cc) amax = fmaxf(amax, fabsf(S[threadIdx.x * SP + cc]));
    sexp[threadIdx.x] = fp16_row_exponent(amax);
  }
  __syncthreads();
  GLOBAL uint16_t* __restrict__ p3h = gbl(d.p3_hi);
  GLOBAL uint16_t* __restrict__ p3l = gbl(d.p3_lo);
  GLOBAL int32_t* __restrict__ p3e = gbl(d.p3_exp);
  constexpr int U8 = RT * 2;                         // 8-column units per row (rpad / 8)
  for (int idx = threadIdx.x; idx < GSA_ROWS * U8; idx += GS_THREADS) {
    const int rr = idx / U8, c8 = (idx % U8) * 8;
    if (row0 + rr >= m) continue;
    const int ex = sexp[rr];
    uint32_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x0 = ldexpf(S[rr * SP + c8 + 2 * e], ex), x1 = ldexpf(S[rr * SP + c8 + 2 * e + 1], ex);
      const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
      h[e] = f16_bits(h0) | ((uint32_t)f16_bits(h1) << 16);
      l[e] = f16_bits((_Float16)(x0 - (float)h0)) | ((uint32_t)f16_bits((_Float16)(x1 - (float)h1)) << 16);
    }
    *gcast<u32x4>(p3h + (int64_t)(row0 + rr) * kpad3 + c8) = u32x4{h[0], h[1], h[2], h[3]};
    *gcast<u32x4>(p3l + (int64_t)(row0 + rr) * kpad3 + c8) = u32x4{l[0], l[1], l[2], l[3]};
  }
  if (threadIdx.x < GSA_ROWS && row0 + (int)threadIdx.x < m) p3e[row0 + threadIdx.x] = sexp[threadIdx.x];
}

}  // namespace

hipError_t launch_gs_gram(int rt, const DevMat* mats, const Work* work, int n_work, hipStream_t s) {
  if (n_work <= 0) return hipSuccess;
  const dim3 grid(n_work), block(GS_THREADS);
  switch (rt) {
#define CASE(R) case R: k_gs_gram<R><<<grid, block, 0, s>>>(mats, work); break;
    CASE(1) CASE(2) CASE(3) CASE(4) CASE(5) CASE(6) CASE(7) CASE(8)
#undef CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gs_factor(const DevMat* mats, const Work* work, int n_work, hipStream_t s) {
  if (n_work <= 0) return hipSuccess;
  k_gs_factor<<<dim3(n_work), dim3(GSF_THREADS), 0, s>>>(mats, work);
  return hipGetLastError();
}

hipError_t launch_gs_apply(int rt, const DevMat* mats, const Work* work, int n_work, hipStream_t s) {
  if (n_work <= 0) return hipSuccess;
  const dim3 grid(n_work), block(GS_THREADS);
  switch (rt) {
#define CASE(R) case R: k_gs_apply<R><<<grid, block, 0, s>>>(mats, work); break;
    CASE(1) CASE(2) CASE(3) CASE(4) CASE(5) CASE(6) CASE(7) CASE(8)
#undef CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int gs_apply_rows_per_block() { return GSA_ROWS; }

}  // namespace psgd
