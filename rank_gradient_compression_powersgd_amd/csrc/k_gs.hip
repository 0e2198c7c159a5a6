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
  for (int ks = 0; ks < kGramRows / 4; ++ks) {
    const int row = row0 + 4 * ks + g;
    double v[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) v[t] = row < m ? (double)P[(int64_t)row * rpad + t * 16 + c] : 0.0;
    // lane supplies A[c][g] = P[row][ti*16 + c] and B[g][c] = P[row][tj*16 + c]
    int p = 0;
#pragma unroll
    for (int ti = 0; ti < RT; ++ti)
#pragma unroll
      for (int tj = ti; tj < RT; ++tj, ++p)
        if (p % NW == wv) acc[p / NW] = mfma_f64(v[ti], v[tj], acc[p / NW]);
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

__global__ __launch_bounds__(GS_THREADS)
void k_gs_factor(const DevMat* __restrict__ mats, const Work* __restrict__ work)
{
  const Work wi = work[blockIdx.x];
  if (wi.mat < 0) return;
  const DevMat& d = mats[wi.mat];
  const int rp = d.rpad;
  const int parts = d.gram_parts;
  const int tid = threadIdx.x;
  const GLOBAL double* __restrict__ gram = gbl(d.gram);
  GLOBAL double* __restrict__ tmat = gbl(d.tmat);

  __shared__ double W[kPackMax];
  __shared__ double T[kPackMax];
  __shared__ double diag0[128];
  __shared__ double rrow[128];

  // W = sum of the partial Gram matrices in part order; T = I.
  const int np = rp * (rp + 1) / 2;
  for (int i = 0; i < rp; ++i) {
    for (int j = i + tid; j < rp; j += GS_THREADS) {
      double sum = 0.0;
      for (int pt = 0; pt < parts; ++pt) sum += gram[((int64_t)pt * rp + i) * rp + j];
      W[pidx(i, j, rp)] = sum;
      T[pidx(i, j, rp)] = (i == j) ? 1.0 : 0.0;
    }
  }
  __syncthreads();
  for (int i = tid; i < rp; i += GS_THREADS) diag0[i] = W[pidx(i, i, rp)];
  __syncthreads();

  for (int j = 0; j < rp; ++j) {
    const double dj = W[pidx(j, j, rp)];
    const double d0 = diag0[j];
    const bool ok = (d0 > 0.0) && (dj > kDegenerate * d0) && (dj <= 1.0e300);
    const double inv = ok ? 1.0 / sqrt(dj) : 0.0;
    // r_jk = <q_j, v_k> = W[j][k] / ||v_j||; t_j = u_j / ||v_j||
    for (int k = j + 1 + tid; k < rp; k += GS_THREADS) rrow[k] = W[pidx(j, k, rp)] * inv;
    for (int i = tid; i <= j; i += GS_THREADS) T[pidx(i, j, rp)] *= inv;
    __syncthreads();
    // v_k -= r_jk q_j for k > j: Gram update and coefficient update
    const int L = rp - j - 1;
    for (int idx = tid; idx < L * L; idx += GS_THREADS) {
      const int k = j + 1 + idx / L, l = j + 1 + idx % L;
      if (l >= k) W[pidx(k, l, rp)] -= rrow[k] * rrow[l];
    }
    const int nt = (j + 1) * L;
    for (int idx = tid; idx < nt; idx += GS_THREADS) {
      const int i = idx / L, k = j + 1 + idx % L;
      T[pidx(i, k, rp)] -= rrow[k] * T[pidx(i, j, rp)];
    }
    __syncthreads();
  }

  for (int idx = tid; idx < rp * rp; idx += GS_THREADS) {
    const int i = idx / rp, j = idx % rp;
    tmat[idx] = (i <= j) ? T[pidx(i, j, rp)] : 0.0;
  }
  (void)np;
}

// ------------------------------------------------------------------------------------------
// P_hat = P T and the operand layouts of the two products that follow
// ------------------------------------------------------------------------------------------
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
  GLOBAL float* __restrict__ pout = gbl(d.p);
  GLOBAL uint16_t* __restrict__ pth = gbl(d.pt_hi);
  GLOBAL uint16_t* __restrict__ ptl = gbl(d.pt_lo);
  GLOBAL uint16_t* __restrict__ p3h = gbl(d.p3_hi);
  GLOBAL uint16_t* __restrict__ p3l = gbl(d.p3_lo);
  GLOBAL int32_t* __restrict__ p3e = gbl(d.p3_exp);
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int c = lane & 15, g = lane >> 4;
  const int rbase = wi.a + wv * 16;        // this wave's 16 rows
  const int rowA = rbase + c;              // A-fragment row supplied by this lane

  f64x4 acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = f64x4{0, 0, 0, 0};

#pragma unroll
  for (int kt = 0; kt < RT; ++kt) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int k = kt * 16 + ks * 4 + g;
      const double a = rowA < m ? (double)P[(int64_t)rowA * rpad + k] : 0.0;
#pragma unroll
      for (int tj = kt; tj < RT; ++tj) {       // T is upper triangular
        const double b = Tm[(int64_t)k * rpad + tj * 16 + c];
        acc[tj] = mfma_f64(a, b, acc[tj]);
      }
    }
  }

  // C layout of v_mfma_f64_16x16x4f64: lane 16g + c, register i holds P_hat[rbase + g + 4i][tj*16 + c]
  float x32[RT][4];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) x32[t][i] = (float)acc[t][i];

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = rbase + g + 4 * i;
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int col = t * 16 + c;
      // (a) fp32 P_hat, m x r row-major
      if (row < m && col < r) pout[(int64_t)row * r + col] = x32[t][i];
      // (b) P_hat^T split bf16 hi/lo, rpad x mpad (rows m..mpad hold zeros)
      if (row < mpad) {
        const __bf16 hb = (__bf16)x32[t][i];
        pth[(int64_t)col * mpad + row] = bf16_bits(hb);
        ptl[(int64_t)col * mpad + row] = bf16_bits((__bf16)(x32[t][i] - (float)hb));
      }
    }
  }
  // (c) rows scaled by 2^e (largest entry in [2^13, 2^14)) and split fp16 hi/lo, m x kpad3
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float amax = 0.0f;
#pragma unroll
    for (int t = 0; t < RT; ++t) amax = fmaxf(amax, fabsf(x32[t][i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    amax = fmaxf(amax, __shfl_xor(amax, 4));
    amax = fmaxf(amax, __shfl_xor(amax, 8));
    const int ex = fp16_row_exponent(amax);
    const int row = rbase + g + 4 * i;
    if (row < m) {
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const float x = ldexpf(x32[t][i], ex);
        const _Float16 h = (_Float16)x;
        p3h[(int64_t)row * kpad3 + t * 16 + c] = f16_bits(h);
        p3l[(int64_t)row * kpad3 + t * 16 + c] = f16_bits((_Float16)(x - (float)h));
      }
      if (c == 0) p3e[row] = ex;
    }
  }
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
  k_gs_factor<<<dim3(n_work), dim3(GS_THREADS), 0, s>>>(mats, work);
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

int gs_apply_rows_per_block() { return (GS_THREADS / kWave) * 16; }

}  // namespace psgd
